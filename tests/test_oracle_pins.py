"""Pins for the fp64 CPU oracle (oracle/paro_ref.c), CPU only.

The oracle is checked against things other than itself:
  * hand-worked values derived from the pages' formulas (tests/golden/*.json,
    each with its citation and derivation),
  * closed forms and invariants the pages state (inverse = reversed stages
    with negated angles, orthogonality, X_r W_r^T = X W^T, the equivalent
    weight, the identity state),
  * brute force (dense Givens matrices multiplied out; numpy's fp16 cast;
    exhaustive decode of all 2^16 bit patterns),
  * an independent vectorised numpy implementation fed with the generator's
    raw codes (not the packed words the oracle reads).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _angle(expr):
    return float(eval(expr, {"pi": math.pi, "sqrt": math.sqrt}))


def tiny_layer(I, G, krot, pairs, theta, cs, O=8):
    """A layer whose weights are irrelevant (rotation-only checks)."""
    ng = I // (I if G == -1 else G)
    return synth.Layer(
        I, O, G, krot,
        np.ascontiguousarray(np.asarray(pairs, dtype=np.int16).reshape(krot, I)),
        np.ascontiguousarray(np.asarray(theta, dtype=np.float32).reshape(krot, I // 2)),
        np.ascontiguousarray(np.asarray(cs, dtype=np.float32).reshape(I)),
        np.zeros((I, O // 8), np.int32), np.zeros((ng, O // 8), np.int32),
        np.zeros((ng, O), np.uint16), None)


def dense_rotation(layer):
    """Brute force: R = R_0 R_1 ... R_{krot-1}, each R_t an explicit matrix of
    disjoint Givens blocks acting on row vectors (x' = x R_t)."""
    I, krot = layer.in_features, layer.krot
    G = I if layer.group_size == -1 else layer.group_size
    R = np.eye(I)
    for t in range(krot):
        Rt = np.eye(I)
        for g in range(I // G):
            for p in range(G // 2):
                i = g * G + int(layer.pairs[t, g * G + 2 * p])
                j = g * G + int(layer.pairs[t, g * G + 2 * p + 1])
                th = float(layer.theta[t, g * (G // 2) + p])
                c, s = math.cos(th), math.sin(th)
                Rt[i, i], Rt[j, j] = c, c
                Rt[j, i], Rt[i, j] = s, -s
        R = R @ Rt
    return R


def random_layer(I, O, G=128, krot=8, seed=0, **kw):
    return synth.make_layer(100 + seed, 0, I, O, G, krot, **kw)


def x_to_f64(x, dt):
    if dt == synth.F16:
        return x.view(np.float16).astype(np.float64)
    if dt == synth.BF16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def numpy_linear(layer, x, dt):
    """Independent vectorised implementation from the generator's raw codes."""
    I, O, krot = layer.in_features, layer.out_features, layer.krot
    G = I if layer.group_size == -1 else layer.group_size
    ng = I // G
    xs = x_to_f64(x, dt) * layer.channel_scales.astype(np.float64)[None, :]
    base = (np.arange(ng) * G)[:, None]
    for t in range(krot):
        pr = layer.pairs[t].astype(np.int64).reshape(ng, G // 2, 2)
        ia, ib = (base + pr[:, :, 0]).ravel(), (base + pr[:, :, 1]).ravel()
        th = layer.theta[t].astype(np.float64)
        c, s = np.cos(th), np.sin(th)
        a, b = xs[:, ia].copy(), xs[:, ib].copy()
        xs[:, ia] = a * c + b * s
        xs[:, ib] = -a * s + b * c
    sc = layer.scales.view(np.float16).astype(np.float64)
    zrep = np.repeat(layer.z.astype(np.float64), G, axis=0)
    srep = np.repeat(sc, G, axis=0)
    w = (layer.q.astype(np.float64) - zrep) * srep
    y = xs @ w
    if layer.bias is not None:
        y = y + layer.bias.view(np.float16).astype(np.float64)[None, :]
    return y


# --------------------------------------------------------------------------
# Worked examples (tests/golden)
# --------------------------------------------------------------------------

def test_golden_rotation_g4_krot2():
    fx = golden("rotation_g4_krot2.json")
    theta = [[_angle(e) for e in row] for row in fx["theta_expr"]]
    L = tiny_layer(fx["in_features"], fx["group_size"], fx["krot"], fx["pairs"], theta,
                   fx["channel_scales"])
    x = np.asarray([fx["x"]], dtype=np.float64)
    xr = ref.scale_rotate(L, x, ref.F64)[0]
    np.testing.assert_allclose(xr, fx["x_r"], atol=fx["tol_abs"], rtol=0)
    assert abs(float(xr @ xr) - fx["norm2"]) < 1e-5
    # the first stage alone
    L1 = tiny_layer(4, 4, 1, fx["pairs"][0], theta[0], fx["channel_scales"])
    np.testing.assert_allclose(ref.scale_rotate(L1, x, ref.F64)[0], fx["after_stage0"], atol=1e-6)


def test_golden_rotation_two_groups():
    fx = golden("rotation_two_groups.json")
    theta = [[_angle(e) for e in row] for row in fx["theta_expr"]]
    L = tiny_layer(fx["in_features"], fx["group_size"], fx["krot"], fx["pairs"], theta,
                   fx["channel_scales"])
    xr = ref.scale_rotate(L, np.asarray([fx["x"]], np.float64), ref.F64)[0]
    np.testing.assert_allclose(xr, fx["x_r"], atol=fx["tol_abs"], rtol=0)


def test_golden_single_pair():
    fx = golden("single_pair.json")
    theta = [[_angle(e) for e in row] for row in fx["theta_expr"]]
    L = tiny_layer(2, 2, 1, fx["pairs"], theta, fx["channel_scales"])
    for case in fx["cases"]:
        xr = ref.scale_rotate(L, np.asarray([case["x"]], np.float64), ref.F64)[0]
        np.testing.assert_allclose(xr, case["x_r"], atol=fx["tol_abs"], rtol=0)


def test_golden_awq_words():
    fx = golden("awq_words.json")
    for case in fx["cases"]:
        word = np.array([int(case["word_hex"], 16)], dtype=np.uint32).view(np.int32)
        # the generator's packer produces the worked word ...
        assert synth.awq_pack(np.array([case["columns"]], np.uint8))[0, 0] == word[0]
        # ... and the oracle unpacks it to the columns
        L = synth.Layer(2, 8, 2, 1, np.array([[0, 1]], np.int16), np.zeros((1, 1), np.float32),
                        np.ones(2, np.float32), np.array([[word[0]], [0]], np.int32),
                        np.array([[word[0]]], np.int32), np.zeros((1, 8), np.uint16), None)
        q, z = ref.unpack(L)
        assert list(q[0]) == case["columns"]
        assert list(q[1]) == [0] * 8
        assert list(z[0]) == case["columns"]


def test_golden_dequant_tie():
    fx = golden("dequant_tie.json")
    qc = np.zeros((2, 8), np.uint8)
    zc = np.zeros((1, 8), np.uint8)
    qc[0, 5], zc[0, 5] = fx["q"], fx["z"]
    sc = np.zeros((1, 8), np.uint16)
    sc[0, 5] = int(fx["scale_bits_hex"], 16)
    L = synth.Layer(2, 8, 2, 1, np.array([[0, 1]], np.int16), np.zeros((1, 1), np.float32),
                    np.ones(2, np.float32), synth.awq_pack(qc), synth.awq_pack(zc), sc, None)
    assert ref.f16_to_double(int(fx["scale_bits_hex"], 16)) == fx["scale_value"]
    w = ref.dequant(L)
    assert w[0, 5] == fx["w_exact"]
    assert np.float32(w[0, 5]) == np.float32(fx["w_exact"])  # exact in fp32 too
    assert ref.round_array([w[0, 5]], ref.F16)[0] == int(fx["w_f16_bits_hex"], 16)
    assert ref.round_array([w[0, 5]], ref.BF16)[0] == int(fx["w_bf16_bits_hex"], 16)
    # row 1 shares the group: (0 - 8) * s; every other column has scale 0
    assert w[1, 5] == -8 * fx["scale_value"]
    assert np.count_nonzero(w) == 2


# --------------------------------------------------------------------------
# Number formats: exhaustive decode, rounding vs library routines
# --------------------------------------------------------------------------

def test_f16_decode_exhaustive():
    lib = ref.load()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([lib.paro_ref_f16_to_double(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_bf16_decode_exhaustive():
    lib = ref.load()
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        want = (bits << 16).view(np.float32).astype(np.float64)
    got = np.array([lib.paro_ref_bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def _rounding_probe_values(rng):
    v = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -24,
         2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
         1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -11 + 2.0 ** -40]
    v += list(rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5, 20000))
    # exact ties at several binades: k + 0.5 ulp
    for e in range(-24, 16):
        for k in range(0, 2048, 37):
            v.append((1024 + k + 0.5) * 2.0 ** (e - 10))
    return np.array(v, dtype=np.float64)


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(1)
    v = _rounding_probe_values(rng)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    got = ref.round_array(v, ref.F16)
    assert np.array_equal(got, want)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(2)
    v32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.uniform(-30, 30, 20000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895314e38, 3.4e38, 1e-39, -1e-40],
                 dtype=np.float32),
        # exact ties between bf16 neighbours (fp32 values with bit 15 set, low bits clear)
        ((rng.integers(0x00800000, 0x7F000000, 5000, dtype=np.uint64).astype(np.uint32) & 0xFFFF0000) | 0x8000).view(np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = ref.round_array(v32.astype(np.float64), ref.BF16)
    assert np.array_equal(got, want)
    # a double just above a tie rounds up (a fp32 pre-rounding would lose this)
    assert ref.round_array([1.0 + 2.0 ** -8 + 2.0 ** -40], ref.BF16)[0] == 0x3F81
    assert ref.round_array([1.0 + 2.0 ** -8], ref.BF16)[0] == 0x3F80


# --------------------------------------------------------------------------
# Rotation invariants and brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("G,krot,I", [(2, 1, 8), (4, 2, 8), (8, 3, 16), (16, 2, 32), (128, 8, 256),
                                      (-1, 3, 64)])
def test_staged_equals_dense_bruteforce(G, krot, I):
    L = random_layer(I, 8, G, krot, seed=G + krot)
    x = np.random.default_rng(abs(G)).standard_normal((5, I))
    want = (x * L.channel_scales.astype(np.float64)) @ dense_rotation(L)
    got = ref.scale_rotate(L, x, ref.F64)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())


def _inverse_layer(L):
    """The inverse per the pages: reverse the stage order and negate the angles."""
    return synth.Layer(L.in_features, L.out_features, L.group_size, L.krot,
                       np.ascontiguousarray(L.pairs[::-1]),
                       np.ascontiguousarray(-L.theta[::-1]),
                       np.ones(L.in_features, np.float32), L.qweight, L.qzeros, L.scales, None)


@pytest.mark.parametrize("G,krot", [(128, 8), (16, 3), (-1, 2)])
def test_inverse_restores_input(G, krot):
    L = random_layer(256, 8, G, krot, seed=3)
    x = np.random.default_rng(3).standard_normal((7, 256))
    xr = ref.scale_rotate(L, x, ref.F64)
    back = ref.scale_rotate(_inverse_layer(L), xr, ref.F64)
    want = x * L.channel_scales.astype(np.float64)
    np.testing.assert_allclose(back, want, rtol=0, atol=1e-13 * np.abs(want).max())


def test_orthogonality_and_norm():
    L = random_layer(256, 8, 128, 8, seed=4, identity=False)
    Lu = synth.Layer(256, 8, 128, 8, L.pairs, L.theta, np.ones(256, np.float32),
                     L.qweight, L.qzeros, L.scales, None)
    R = ref.scale_rotate(Lu, np.eye(256), ref.F64)  # rows of R
    np.testing.assert_allclose(R @ R.T, np.eye(256), rtol=0, atol=1e-13)
    # block diagonal: nothing crosses a group boundary
    assert np.abs(R[:128, 128:]).max() == 0.0 and np.abs(R[128:, :128]).max() == 0.0
    x = np.random.default_rng(4).standard_normal((9, 256))
    xr = ref.scale_rotate(Lu, x, ref.F64)
    np.testing.assert_allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


def test_group_locality():
    L = random_layer(384, 8, 128, 4, seed=5)
    x = np.random.default_rng(5).standard_normal((3, 384))
    base = ref.scale_rotate(L, x, ref.F64)
    th = L.theta.copy()
    th[2, 64:128] += 0.3  # angles of group 1 at stage 2
    L2 = synth.Layer(384, 8, 128, 4, L.pairs, th, L.channel_scales, L.qweight, L.qzeros,
                     L.scales, None)
    out = ref.scale_rotate(L2, x, ref.F64)
    diff = np.abs(out - base).max(axis=0)
    assert diff[:128].max() == 0.0 and diff[256:].max() == 0.0
    assert diff[128:256].max() > 1e-3


def test_stage_order_matters():
    L = random_layer(128, 8, 128, 2, seed=6)
    x = np.random.default_rng(6).standard_normal((2, 128))
    swapped = synth.Layer(128, 8, 128, 2, np.ascontiguousarray(L.pairs[::-1]),
                          np.ascontiguousarray(L.theta[::-1]), L.channel_scales, L.qweight,
                          L.qzeros, L.scales, None)
    assert np.abs(ref.scale_rotate(L, x, ref.F64) - ref.scale_rotate(swapped, x, ref.F64)).max() > 1e-3


def test_pairs_must_be_permutations():
    L = random_layer(256, 8, 128, 2, seed=7)
    assert ref.check_pairs(L) == ref.OK
    bad = L.pairs.copy()
    bad[1, 130] = bad[1, 131]  # duplicate inside group 1 of stage 1
    Lb = synth.Layer(256, 8, 128, 2, bad, L.theta, L.channel_scales, L.qweight, L.qzeros,
                     L.scales, None)
    assert ref.check_pairs(Lb) == ref.ERR_PAIRS
    with pytest.raises(RuntimeError):
        ref.scale_rotate(Lb, np.zeros((1, 256)), ref.F64)
    out_of_range = L.pairs.copy()
    out_of_range[0, 0] = 128
    Lo = synth.Layer(256, 8, 128, 2, out_of_range, L.theta, L.channel_scales, L.qweight,
                     L.qzeros, L.scales, None)
    assert ref.check_pairs(Lo) == ref.ERR_PAIRS


# --------------------------------------------------------------------------
# Transform identities of the pages
# --------------------------------------------------------------------------

def test_transform_equivalence_without_quantization():
    """X_r W_r^T = X W^T with X_r = X D^-1 R, W_r = W D R (stored cs = D^-1)."""
    I, O = 256, 48
    L = random_layer(I, O, 128, 8, seed=8)
    rng = np.random.default_rng(8)
    X = rng.standard_normal((6, I))
    W = rng.standard_normal((O, I))
    D = np.diag(1.0 / L.channel_scales.astype(np.float64))
    Xr = ref.scale_rotate(L, X, ref.F64)
    Wr = W @ D @ dense_rotation(L)
    lhs, rhs = Xr @ Wr.T, X @ W.T
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12 * np.abs(rhs).max())


def test_equivalent_weight_identity():
    """Y = X (Q(W_r) R^T D^-1)^T + b, the equivalent weight in input coordinates."""
    I, O = 256, 64
    L = random_layer(I, O, 128, 8, seed=9, keep_codes=True)
    x = synth.make_x(109, 0, 5, I, synth.F16)
    y = ref.linear(L, x, ref.F16)
    sc = L.scales.view(np.float16).astype(np.float64)
    Wdeq_t = (L.q.astype(np.float64) - np.repeat(L.z, 128, 0)) * np.repeat(sc, 128, 0)  # (I, O)
    Qwr = Wdeq_t.T                                   # Q(W_r), (O, I)
    Dinv = np.diag(L.channel_scales.astype(np.float64))
    W_eq = Qwr @ dense_rotation(L).T @ Dinv          # (O, I)
    want = x_to_f64(x, synth.F16) @ W_eq.T + L.bias.view(np.float16).astype(np.float64)
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_identity_state_is_plain_dequant_gemm():
    I, O = 384, 40
    L = random_layer(I, O, 128, 8, seed=10, identity=True, keep_codes=True)
    x = synth.make_x(110, 0, 4, I, synth.BF16)
    sc = L.scales.view(np.float16).astype(np.float64)
    W = (L.q.astype(np.float64) - np.repeat(L.z, 128, 0)) * np.repeat(sc, 128, 0)
    want = np.matmul(x_to_f64(x, synth.BF16), W) + L.bias.view(np.float16).astype(np.float64)
    np.testing.assert_allclose(ref.linear(L, x, ref.BF16), want, rtol=0,
                               atol=1e-13 * np.abs(want).max())


def test_unpack_roundtrip_and_dequant_bruteforce():
    I, O, G = 256, 96, 64
    L = random_layer(I, O, G, 2, seed=11, keep_codes=True)
    q, z = ref.unpack(L)
    assert np.array_equal(q, L.q) and np.array_equal(z, L.z)
    w = ref.dequant(L)
    sc = L.scales.view(np.float16).astype(np.float64)
    for k in range(0, I, 17):
        for n in range(0, O, 5):
            assert w[k, n] == (int(L.q[k, n]) - int(L.z[k // G, n])) * sc[k // G, n]


# --------------------------------------------------------------------------
# The whole linear against an independent numpy implementation, and the check
# --------------------------------------------------------------------------

@pytest.mark.parametrize("I,O,G,krot,M,dt", [(256, 256, 128, 8, 4, synth.F16),
                                              (384, 136, 128, 8, 3, synth.BF16),
                                              (256, 64, 32, 3, 2, synth.F32),
                                              (128, 16, -1, 1, 1, synth.F16)])
def test_linear_matches_numpy_mirror(I, O, G, krot, M, dt):
    L = random_layer(I, O, G, krot, seed=12 + I, keep_codes=True)
    x = synth.make_x(112, I, M, I, dt)
    want = numpy_linear(L, x, dt)
    got = ref.linear(L, x, dt)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_workload0_matches_numpy_mirror():
    (_, L, x), = list(synth.workload_layers(0, keep_codes=True))
    want = numpy_linear(L, x, synth.F16)
    got = ref.linear(L, x, ref.F16)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_ref_check_status():
    (_, L, x), = list(synth.workload_layers(0))
    rc, err, mref, yref = ref.paro_linear_ref_check(L, x, ref.F16, want_ref=True)
    assert rc == ref.OK and mref > 0
    y32 = yref.astype(np.float32)
    rc, err, _, _ = ref.paro_linear_ref_check(L, x, ref.F16, y32, ref.F32)
    assert rc == ref.OK and err < 1e-6 * mref
    y16 = ref.round_array(yref, ref.F16)
    rc, err, _, _ = ref.paro_linear_ref_check(L, x, ref.F16, y16, ref.F16)
    assert rc == ref.OK and err <= 2.0 ** -11 * mref
    bad = y32.copy()
    bad[1, 7] += np.float32(0.01 * mref)
    rc, err, _, _ = ref.paro_linear_ref_check(L, x, ref.F16, bad, ref.F32)
    assert rc == ref.ERR_CHECK_FAILED and err > 5e-3 * mref
    nan = y32.copy()
    nan[0, 0] = np.nan
    rc, _, _, _ = ref.paro_linear_ref_check(L, x, ref.F16, nan, ref.F32)
    assert rc == ref.ERR_CHECK_FAILED


def test_zero_tokens_and_bad_shapes():
    (_, L, x), = list(synth.workload_layers(0))
    assert ref.paro_linear_ref_check(L, x[:0], ref.F16)[0] == ref.OK
    bad = synth.Layer(256, 252, 128, 8, L.pairs, L.theta, L.channel_scales, L.qweight,
                      L.qzeros, L.scales, None)
    assert ref.paro_linear_ref_check(bad, x, ref.F16)[0] == ref.ERR_SHAPE
    odd = synth.Layer(256, 256, 127, 8, L.pairs, L.theta, L.channel_scales, L.qweight,
                      L.qzeros, L.scales, None)
    assert ref.paro_linear_ref_check(odd, x, ref.F16)[0] == ref.ERR_SHAPE


# ---------------------------------------------------------------------------
# Offline transform, group quantization and AWQ packing
# ---------------------------------------------------------------------------

def _frac(expr):
    return float(eval(expr, {}))


def test_golden_quantize_worked_examples():
    fx = golden("quantize_worked.json")
    for c in fx["cases"]:
        x = np.asarray([c["x"]], dtype=np.float64)
        q, z, s16, scale = ref.quantize(x, 4, c["sym"])
        assert q[:, 0].tolist() == c["q"], c
        assert int(z[0, 0]) == c["zero"], c
        assert scale[0, 0] == pytest.approx(_frac(c["scale"]), rel=1e-15), c
        assert int(s16[0, 0]) == int(np.float16(_frac(c["scale"])).view(np.uint16)), c


@pytest.mark.parametrize("sym", [True, False])
def test_quantize_is_round_to_nearest_on_its_grid(sym):
    """Every value lies within half a step of its dequantized code (the range
    fit makes clamping cost at most that half step), and grid points map to
    themselves."""
    rng = np.random.default_rng(11)
    O, I, G = 24, 256, 128
    w = rng.normal(0, 0.03, size=(O, I)) * rng.uniform(0.2, 3.0, size=(O, 1))
    q, z, _, scale = ref.quantize(w, G, sym)
    for g in range(I // G):
        s = scale[g][None, :]                                    # [1][O]
        xh = s * (q[g * G:(g + 1) * G].astype(np.float64) - z[g][None, :])
        err = np.abs(xh - w[:, g * G:(g + 1) * G].T)
        assert (err <= 0.5 * s * (1 + 1e-12)).all()
    # re-quantizing the dequantized grid points reproduces the codes when the
    # range is unchanged (affine: the extremes are grid points only where hit)
    if sym:
        xh_full = np.concatenate([(scale[g][None, :] * (q[g * G:(g + 1) * G].astype(np.float64) - z[g][None, :])).T
                                  for g in range(I // G)], axis=1)
        q2, z2, _, s2 = ref.quantize(xh_full, G, sym)
        same = np.isclose(s2, scale, rtol=1e-12)
        for g in range(I // G):
            cols = same[g]
            assert (q2[g * G:(g + 1) * G, cols] == q[g * G:(g + 1) * G, cols]).all()


def test_pack_is_the_inverse_of_unpack():
    rng = np.random.default_rng(12)
    I, O, G = 256, 48, 128
    q = rng.integers(0, 16, size=(I, O)).astype(np.uint8)
    z = rng.integers(0, 16, size=(I // G, O)).astype(np.uint8)
    qw, qz = ref.pack(q, z, G)
    L = synth.Layer(I, O, G, 1, np.zeros((1, I), np.int16), np.zeros((1, I // 2), np.float32),
                    np.ones(I, np.float32), qw, qz, np.zeros((I // G, O), np.uint16), None)
    q2, z2 = ref.unpack(L)
    assert np.array_equal(q2, q) and np.array_equal(z2, z)
    fx = golden("awq_words.json")
    for c in fx["cases"]:
        qq = np.zeros((128, 8), np.uint8)
        qq[0] = c["columns"]
        w, _ = ref.pack(qq, np.zeros((1, 8), np.uint8), 128)
        assert int(w[0, 0]) & 0xFFFFFFFF == int(c["word_hex"], 16)


def test_transform_weight_identity_and_channel_division():
    rng = np.random.default_rng(13)
    I, O, G, krot = 256, 16, 128, 3
    w = rng.normal(size=(O, I))
    pairs = np.stack([np.concatenate([rng.permutation(G) for _ in range(I // G)]) for _ in range(krot)])
    cs = rng.uniform(0.5, 2.0, size=I)
    L = tiny_layer(I, G, krot, pairs, np.zeros((krot, I // 2)), np.ones(I), O=O)
    assert np.array_equal(ref.transform_weight(L, w, ref.F64), w)     # identity state
    L = tiny_layer(I, G, krot, pairs, np.zeros((krot, I // 2)), cs, O=O)
    np.testing.assert_allclose(ref.transform_weight(L, w, ref.F64), w / cs.astype(np.float32), rtol=1e-15)


def test_transform_weight_keeps_the_product():
    """X_r W_r^T = X W^T: the activations are multiplied by the stored scales,
    the weight divided, both rotated by the same orthogonal R."""
    rng = np.random.default_rng(14)
    I, O, G, krot, M = 256, 24, 64, 5, 7
    pairs = np.stack([np.concatenate([rng.permutation(G) for _ in range(I // G)]) for _ in range(krot)])
    theta = rng.uniform(-np.pi / 4, np.pi / 4, size=(krot, I // 2))
    cs = rng.uniform(0.5, 2.0, size=I)
    L = tiny_layer(I, G, krot, pairs, theta, cs, O=O)
    x = rng.normal(size=(M, I))
    w = rng.normal(size=(O, I))
    xr = ref.scale_rotate(L, x, ref.F64)
    wr = ref.transform_weight(L, w, ref.F64)
    lhs, rhs = xr @ wr.T, x @ w.T
    assert np.abs(lhs - rhs).max() <= 1e-12 * np.abs(rhs).max()


@pytest.mark.parametrize("sym", [True, False])
def test_quantized_layer_reproduces_dense_linear_within_rounding(sym):
    """Transform, quantize and pack a dense weight, then run the oracle linear:
    |Y - (X W^T + b)| <= sum_k |x_r[k]| * scale_k / 2 (each weight is off by at
    most half a step, the rotation is exact up to fp64)."""
    rng = np.random.default_rng(15 + sym)
    I, O, G, krot, M = 256, 32, 128, 4, 5
    pairs = np.stack([np.concatenate([rng.permutation(G) for _ in range(I // G)]) for _ in range(krot)])
    theta = rng.uniform(-np.pi / 4, np.pi / 4, size=(krot, I // 2)).astype(np.float32)
    cs = rng.uniform(0.5, 2.0, size=I).astype(np.float32)
    w = rng.normal(0, 0.02, size=(O, I))
    L0 = tiny_layer(I, G, krot, pairs, theta, cs, O=O)
    wr = ref.transform_weight(L0, w, ref.F64)
    q, z, s16, scale = ref.quantize(wr, G, sym)
    qw, qz = ref.pack(q, z, G)
    # the layer stores fp16 scales; re-quantize against them so codes and
    # stored scales are consistent (a step of the fp16 scale differs from the
    # exact one by at most 2^-11 relative)
    s_eff = np.asarray([[ref.f16_to_double(h) for h in row] for row in s16])
    bias = synth.f16_bits(rng.normal(0, 0.01, size=O))
    L = synth.Layer(I, O, G, krot, L0.pairs, L0.theta, L0.channel_scales, qw, qz, s16, bias)
    x = rng.normal(size=(M, I))
    y = ref.linear(L, x, ref.F64)
    b = np.asarray([ref.f16_to_double(h) for h in bias])
    xr = ref.scale_rotate(L, x, ref.F64)
    step = np.repeat(np.maximum(s_eff, scale), G, axis=0)               # [I][O]
    extra = np.repeat(np.abs(s_eff - scale), G, axis=0) * 15            # scale rounding
    bound = np.abs(xr) @ (0.5 * step + extra)
    assert (np.abs(y - (x @ w.T + b)) <= bound * (1 + 1e-9) + 1e-12).all()


# ---------------------------------------------------------------------------
# Backward of the scaling and rotation
# ---------------------------------------------------------------------------

def _bwd_layer(rng, I, G, krot, grid=2.0 ** -10):
    """Angles and scales on a dyadic grid, so that +-2^-12 steps are exact in fp32."""
    pairs = np.stack([np.concatenate([rng.permutation(G) for _ in range(I // G)]) for _ in range(krot)])
    theta = np.round(rng.uniform(-np.pi / 4, np.pi / 4, size=(krot, I // 2)) / grid) * grid
    cs = np.round(rng.uniform(0.5, 2.0, size=I) / grid) * grid
    return tiny_layer(I, G, krot, pairs, theta, cs)


def _loss(layer, x, g):
    return float((ref.scale_rotate(layer, x, ref.F64) * g).sum())


def test_backward_matches_central_differences():
    rng = np.random.default_rng(21)
    I, G, krot, M = 8, 4, 3, 3
    L = _bwd_layer(rng, I, G, krot)
    x = rng.normal(size=(M, I))
    g = rng.normal(size=(M, I))
    gx, gth, gcs = ref.scale_rotate_backward(L, x, ref.F64, g)
    h = 2.0 ** -12
    for t in range(krot):
        for p in range(I // 2):
            thp, thm = L.theta.copy(), L.theta.copy()
            thp[t, p] += h
            thm[t, p] -= h
            Lp = synth.Layer(**{**L.__dict__, "theta": thp})
            Lm = synth.Layer(**{**L.__dict__, "theta": thm})
            num = (_loss(Lp, x, g) - _loss(Lm, x, g)) / (2 * h)
            assert gth[t, p] == pytest.approx(num, rel=2e-5, abs=1e-7), (t, p)
    for k in range(I):
        csp, csm = L.channel_scales.copy(), L.channel_scales.copy()
        csp[k] += h
        csm[k] -= h
        Lp = synth.Layer(**{**L.__dict__, "channel_scales": csp})
        Lm = synth.Layer(**{**L.__dict__, "channel_scales": csm})
        num = (_loss(Lp, x, g) - _loss(Lm, x, g)) / (2 * h)
        assert gcs[k] == pytest.approx(num, rel=2e-5, abs=1e-7), k
    for m in range(M):
        for k in range(I):
            xp, xm = x.copy(), x.copy()
            xp[m, k] += 1e-6
            xm[m, k] -= 1e-6
            num = (_loss(L, xp, g) - _loss(L, xm, g)) / 2e-6
            assert gx[m, k] == pytest.approx(num, rel=1e-6, abs=1e-9), (m, k)


def test_backward_closed_forms_with_dense_rotation():
    """x_r = (x * cs) R, so dL/dx = (g R^T) * cs and dL/dcs = sum_m (g R^T) * x."""
    rng = np.random.default_rng(22)
    I, G, krot, M = 64, 16, 5, 9
    L = _bwd_layer(rng, I, G, krot)
    x = rng.normal(size=(M, I))
    g = rng.normal(size=(M, I))
    gx, _, gcs = ref.scale_rotate_backward(L, x, ref.F64, g)
    R = dense_rotation(L)
    gs = g @ R.T
    np.testing.assert_allclose(gx, gs * L.channel_scales.astype(np.float64), rtol=0, atol=1e-12)
    np.testing.assert_allclose(gcs, (gs * x).sum(axis=0), rtol=0, atol=1e-11)


def test_backward_theta_at_zero_angle():
    """One stage at theta = 0 is the identity: dL/dtheta_p = sum_m (g_a x_b - g_b x_a) of the scaled rows."""
    rng = np.random.default_rng(23)
    I, G, M = 16, 8, 5
    pairs = np.concatenate([rng.permutation(G) for _ in range(I // G)])[None, :]
    cs = np.round(rng.uniform(0.5, 2.0, size=I) * 1024) / 1024
    L = tiny_layer(I, G, 1, pairs, np.zeros((1, I // 2)), cs)
    x = rng.normal(size=(M, I))
    g = rng.normal(size=(M, I))
    _, gth, _ = ref.scale_rotate_backward(L, x, ref.F64, g)
    xs = x * cs
    for gi in range(I // G):
        for p in range(G // 2):
            a = gi * G + pairs[0, gi * G + 2 * p]
            b = gi * G + pairs[0, gi * G + 2 * p + 1]
            want = (g[:, a] * xs[:, b] - g[:, b] * xs[:, a]).sum()
            assert gth[0, gi * G // 2 + p] == pytest.approx(want, rel=1e-13, abs=1e-13)


# ---------------------------------------------------------------------------
# mixture of experts with one shared rotation (the oracle's composition)
# ---------------------------------------------------------------------------

def test_moe_with_identical_experts_is_the_plain_linear():
    """E copies of one layer: every routing gives the plain linear on all rows."""
    I, O, M, E = 256, 64, 37, 3
    L = synth.make_layer(601, 0, I, O)
    stack = lambda a: np.ascontiguousarray(np.stack([a] * E))
    Lm = synth.Layer(I, O, 128, L.krot, L.pairs, L.theta, L.channel_scales, stack(L.qweight), stack(L.qzeros),
                     stack(L.scales), stack(L.bias))
    x = synth.make_x(601, 0, M, I, synth.F16)
    want = ref.linear(L, x, synth.F16)
    for offs in ([0, 10, 10, 37], [0, 37, 37, 37], [0, 1, 2, 37]):
        assert np.array_equal(ref.moe_linear(Lm, offs, x, synth.F16), want)


def test_moe_rows_depend_only_on_their_expert():
    I, O, M, E = 256, 64, 40, 4
    Lm = synth.make_moe_layer(602, E, I, O)
    x = synth.make_x(602, 0, M, I, synth.BF16)
    offs = np.array([0, 7, 7, 30, 40])
    y = ref.moe_linear(Lm, offs, x, synth.BF16)
    # expert 2's weights replaced: only rows 7..29 change
    other = synth.make_layer(603, 0, I, O)
    qw = Lm.qweight.copy(); qw[2] = other.qweight
    sc = Lm.scales.copy(); sc[2] = other.scales
    import dataclasses
    y2 = ref.moe_linear(dataclasses.replace(Lm, qweight=qw, scales=sc), offs, x, synth.BF16)
    assert np.array_equal(y2[:7], y[:7]) and np.array_equal(y2[30:], y[30:])
    assert not np.allclose(y2[7:30], y[7:30])
    # and each expert's rows are that expert's plain linear (empty expert 1 contributes nothing)
    for e, (lo, hi) in enumerate(zip(offs[:-1], offs[1:])):
        if hi > lo:
            assert np.array_equal(y[lo:hi], ref.linear(ref.expert_layer(Lm, e), x[lo:hi], synth.BF16))


def test_moe_routing_generator_covers_every_row():
    offs = synth.make_routing(5, 8, 2048, 2)
    assert offs[0] == 0 and offs[-1] == 4096 and (np.diff(offs) >= 0).all() and len(offs) == 9


# ---------------------------------------------------------------------------
# MXFP4 (32-element blocks, E8M0 scale, E2M1 elements)
# ---------------------------------------------------------------------------

E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def nibbles(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[0], -1)


def test_mxfp4_worked_block():
    """Hand-worked: max |v| = 6 gives floor(log2 6) - 2 = 0, scale 2^0 (byte
    127); the ties 0.25, 0.75, 1.25, 1.75, 2.5, 3.5 and 5 go to the even code
    (0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0); 7.9 saturates to 6 in the next block."""
    v = np.zeros((1, 64))
    vals = [6.0, -3.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.3, 0.0, 4.9, -0.1, 2.9, 1.1, -6.0]
    want = [7, 8 | 5, 0, 2, 2, 4, 4, 6, 6, 8 | 1, 0, 6, 0, 5, 2, 8 | 7]
    v[0, :16] = vals
    v[0, 32] = 7.9       # block 2: floor(log2 7.9) = 2, scale 1, 7.9 -> 6
    v[0, 33] = -0.24     # -> 0, stored as +0
    codes, scales = ref.mxfp4_quantize(v)
    assert list(scales[0]) == [127, 127]
    n = nibbles(codes)[0]
    assert list(n[:16]) == want
    assert n[32] == 7 and n[33] == 0
    assert codes[0, 0] == (7 | (13 << 4))  # element 0 low nibble, element 1 high nibble


def test_mxfp4_scale_exponent_and_zero_block():
    v = np.zeros((3, 32))
    v[0, 5] = 0.1        # floor(log2 0.1) = -4 -> exponent -6 -> byte 121; 0.1 / 2^-6 = 6.4 -> 6
    v[1, 0] = 1000.0     # floor(log2 1000) = 9 -> exponent 7 -> byte 134; 1000 / 128 = 7.8 -> 6
    codes, scales = ref.mxfp4_quantize(v)
    assert scales[0, 0] == 121 and scales[1, 0] == 134 and scales[2, 0] == 0
    back = ref.mxfp4_dequant(codes, scales)
    assert back[0, 5] == 6 * 2.0 ** -6 and back[1, 0] == 768.0
    assert not back[2].any() and not codes[2].any()


def test_mxfp4_elements_are_nearest_points_brute_force():
    rng = np.random.default_rng(11)
    v = rng.standard_normal((64, 64)) * np.exp(rng.uniform(-8, 8, size=(64, 1)))
    codes, scales = ref.mxfp4_quantize(v)
    back = ref.mxfp4_dequant(codes, scales)
    n = nibbles(codes)
    for r in range(64):
        for b in range(2):
            blk = v[r, 32 * b:32 * b + 32]
            X = 2.0 ** (int(scales[r, b]) - 127)
            amax = np.abs(blk).max()
            assert 4 <= amax / X < 8                       # the block exponent rule
            grid = np.array([s * m for m in E2M1_VALUES for s in (1, -1)]) * X
            for e in range(32):
                d = np.abs(grid - blk[e])
                assert abs(back[r, 32 * b + e] - blk[e]) == d.min()
                c = int(n[r, 32 * b + e])
                if (d == d.min()).sum() > 1 and abs(blk[e]) < 6 * X:  # a tie: the even code
                    assert c & 1 == 0


def test_mxfp4_round_trip_of_canonical_blocks():
    """A block whose largest magnitude code is 4 or 6 re-quantizes to itself."""
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 256, size=(16, 32), dtype=np.uint8)   # 64 elements: two blocks
    codes[:, 0] = 7 | (6 << 4)
    codes[:, 16] = 6 | (15 << 4)
    scales = rng.integers(100, 150, size=(16, 2), dtype=np.uint8)
    back = ref.mxfp4_dequant(codes, scales)
    c2, s2 = ref.mxfp4_quantize(back)
    # -0 (code 8) is stored as +0: compare the values they stand for
    assert np.array_equal(s2, scales)
    assert np.array_equal(ref.mxfp4_dequant(c2, s2), back)


def e2m1_decode_by_hand(codes, scales):
    """Values of MXFP4 rows from the format's definition (not the oracle's
    dequant): element 2j is the low nibble of byte j, bit 3 of a nibble is
    the sign and bits 0..2 index the E2M1 magnitudes; block b of 32 elements
    is scaled by 2^(scales[b] - 127)."""
    rows, K = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((rows, K))
    for r in range(rows):
        for e in range(K):
            nib = (int(codes[r, e // 2]) >> (4 * (e % 2))) & 15
            mag = E2M1_VALUES[nib & 7]
            out[r, e] = (-mag if nib & 8 else mag) * 2.0 ** (int(scales[r, e // 32]) - 127)
    return out


def mx_row(K, entries, scales):
    """codes and scales of one MXFP4 row with nibble `code` at element e."""
    codes = np.zeros(K // 2, dtype=np.uint8)
    for e, code in entries.items():
        codes[e // 2] |= code << (4 * (e % 2))
    return codes, np.asarray(scales, dtype=np.uint8)


def test_mxfp4_matmul_worked_one_block():
    """A (1 x 32): 6 (code 7) and -1.5 (code 11) at elements 0, 1, scale byte
    128 (x2): 12 and -3.  W (1 x 32): 0.5 (code 1) and 3 (code 5), scale 126
    (x0.5): 0.25 and 1.5.  y = 12 * 0.25 - 3 * 1.5 = -1.5, plus the fp16 bias
    1.0 (0x3C00): -0.5."""
    ac, as_ = mx_row(32, {0: 7, 1: 11}, [128])
    wc, ws = mx_row(32, {0: 1, 1: 5}, [126])
    y = ref.mxfp4_matmul(ac[None], as_[None], wc[None], ws[None], np.array([0x3C00], np.uint16))
    assert y.shape == (1, 1) and y[0, 0] == -0.5
    assert ref.mxfp4_matmul(ac[None], as_[None], wc[None], ws[None])[0, 0] == -1.5


def test_mxfp4_matmul_worked_two_by_two():
    """Two rows and two blocks each, so that a transposed product, a swapped
    block scale or a dropped bias all change the result.
      A row 0: 1.0 at k=0 (code 2, block scale 127), 1.0 at k=32 (code 2,
               block scale 129: x4)                    -> 1 at k=0, 4 at k=32
      A row 1: -2.0 at k=1 (code 12, scale 126: x0.5)  -> -1 at k=1
      W row 0: 0.5 at k=0 (code 1, scale 127), 6 at k=32 (code 7, scale 125:
               x0.25)                                   -> 0.5 at k=0, 1.5 at k=32
      W row 1: 4 at k=1 (code 6, scale 128: x2), -1 at k=32 (code 10, scale
               127)                                     -> 8 at k=1, -1 at k=32
    A . W^T = [[1*0.5 + 4*1.5, 4*-1], [0, -1*8]] = [[6.5, -4], [0, -8]];
    bias fp16 (0.25, -2) = (0x3400, 0xC000) -> [[6.75, -6], [0.25, -10]]."""
    a0 = mx_row(64, {0: 2, 32: 2}, [127, 129])
    a1 = mx_row(64, {1: 12}, [126, 127])
    w0 = mx_row(64, {0: 1, 32: 7}, [127, 125])
    w1 = mx_row(64, {1: 6, 32: 10}, [128, 127])
    ac, as_ = np.stack([a0[0], a1[0]]), np.stack([a0[1], a1[1]])
    wc, ws = np.stack([w0[0], w1[0]]), np.stack([w0[1], w1[1]])
    y = ref.mxfp4_matmul(ac, as_, wc, ws, np.array([0x3400, 0xC000], np.uint16))
    assert np.array_equal(y, np.array([[6.75, -6.0], [0.25, -10.0]]))


def test_mxfp4_matmul_brute_force():
    """Random codes and scales: a triple loop over values decoded by hand from
    the format equals the oracle's product (powers of two times E2M1 values
    multiply exactly; only the order of the fp64 sums differs)."""
    rng = np.random.default_rng(13)
    M, N, K = 3, 5, 64
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    as_ = rng.integers(120, 135, size=(M, K // 32), dtype=np.uint8)
    ws = rng.integers(120, 135, size=(N, K // 32), dtype=np.uint8)
    bias = np.array([0x3C00, 0xBC00, 0x0000, 0x4000, 0x3555], np.uint16)  # 1, -1, 0, 2, 0.333...
    bias_v = [1.0, -1.0, 0.0, 2.0, 1365.0 / 4096]                          # 0x3555 = 1.3330078125 / 4
    a, w = e2m1_decode_by_hand(ac, as_), e2m1_decode_by_hand(wc, ws)
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += a[m, k] * w[n, k]
            want[m, n] = s + bias_v[n]
    got = ref.mxfp4_matmul(ac, as_, wc, ws, bias)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13 * np.abs(want).max())
