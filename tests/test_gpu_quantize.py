"""GPU parity of paro_w4_quantize_pack (W_r = W D R, group quantization, AWQ
packing) against the fp64 oracle, through the C-ABI.

The kernel takes every decision in fp32 on its fp32 rotation of W; the oracle
in fp64 on its exact one.  The two W_r differ by fp32 rounding (~1e-7
relative), so a code, zero point or fp16 scale may differ only where the
oracle's own value sits within 1e-4 of a rounding tie; there the two must
differ by one step, and such places must be rare.  Everything else is
bit-exact.  The packed layer must also drive the linear to the oracle's gate.
Full-size shapes are checked on seeded blocks of 8 output rows (rows are
independent, so the oracle computes exactly those).
"""
import numpy as np
import pytest

import synth
from _helpers import LIN_TOL, say, x_to_device, torch_dtype
from oracle import ref

torch = pytest.importorskip("torch")
paro = pytest.importorskip("rotation_int4_weight_amd")

pytestmark = pytest.mark.gpu

TIE = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    paro.load()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.synchronize()


def gpu_quantize(D, w, dt, O, I, sym, G=128):
    wd = x_to_device(w, dt)
    qw = torch.full((I, O // 8), -1, dtype=torch.int32, device="cuda")
    qz = torch.full((I // G, O // 8), -1, dtype=torch.int32, device="cuda")
    sc = torch.full((I // G, O), -1, dtype=torch.int16, device="cuda")
    paro.paro_w4_quantize_pack(D, wd, sym, qw, qz, sc)
    torch.cuda.synchronize()
    return qw.cpu().numpy(), qz.cpu().numpy(), sc.cpu().numpy().view(np.uint16)


def sub_layer(L, O):
    """The rotation of L with O output rows (weights irrelevant)."""
    I, G = L.in_features, L.group_size
    return synth.Layer(I, O, G, L.krot, L.pairs, L.theta, L.channel_scales,
                       np.zeros((I, O // 8), np.int32), np.zeros((I // G, O // 8), np.int32),
                       np.zeros((I // G, O), np.uint16), None)


def unpack_cols(qw, qz, I, O, G=128):
    """Oracle unpack of GPU words -> q [I][O], z [I/G][O]."""
    L = synth.Layer(I, O, G, 1, np.zeros((1, I), np.int16), np.zeros((1, I // 2), np.float32),
                    np.ones(I, np.float32), np.ascontiguousarray(qw), np.ascontiguousarray(qz),
                    np.zeros((I // G, O), np.uint16), None)
    return ref.unpack(L)


def f16_tie(scale):
    """Oracle scales within 1e-6 (relative) of an fp16 rounding boundary."""
    s16 = scale.astype(np.float16).astype(np.float64)
    nxt = np.nextafter(scale.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    prv = np.nextafter(scale.astype(np.float16), np.float16(0)).astype(np.float64)
    mid = np.minimum(np.abs(scale - (s16 + nxt) / 2), np.abs(scale - (s16 + prv) / 2))
    return mid <= 1e-6 * scale


def compare(L, w, dt, sym, qw, qz, s16, rows):
    """Check the GPU's codes of output rows `rows` (multiple of 8 each block)."""
    I, O, G = L.in_features, L.out_features, L.group_size
    sub = sub_layer(L, len(rows))
    wr = ref.transform_weight(sub, np.ascontiguousarray(w[rows]), dt)        # [R][I]
    q_o, z_o, s_o, scale_o = ref.quantize(wr, G, sym)                         # [I][R], [I/G][R]
    q_g, z_g = unpack_cols(qw, qz, I, O, G)
    q_g, z_g, s_g = q_g[:, rows], z_g[:, rows], s16[:, rows]
    # scales: exact unless the oracle's scale is at an fp16 tie
    s_tie = f16_tie(scale_o)
    bad_s = (s_g != s_o) & ~(s_tie & (np.abs(s_g.astype(np.int64) - s_o.astype(np.int64)) == 1))
    assert not bad_s.any(), f"fp16 scales differ off ties at {np.argwhere(bad_s)[:5]}"
    # decision values of the oracle, per element: x / scale + zero
    xmin = np.minimum(wr.reshape(len(rows), I // G, G).min(axis=2), 0.0).T   # [I/G][R]
    zval = -xmin / scale_o
    z_tie = (np.abs(zval - np.floor(zval) - 0.5) < TIE) if not sym else np.zeros_like(zval, bool)
    bad_z = (z_g != z_o) & ~(z_tie & (np.abs(z_g.astype(int) - z_o.astype(int)) == 1))
    assert not bad_z.any(), f"zero points differ off ties at {np.argwhere(bad_z)[:5]}"
    v = wr.T / np.repeat(scale_o, G, axis=0)                                  # [I][R]
    frac = np.abs(v - np.floor(v) - 0.5)
    grp_tie = np.repeat(s_tie | z_tie, G, axis=0)
    tie = (frac < TIE) | grp_tie
    diff = q_g.astype(int) - q_o.astype(int)
    bad_q = (diff != 0) & ~(tie & (np.abs(diff) == 1))
    assert not bad_q.any(), f"codes differ off ties at {np.argwhere(bad_q)[:5]}"
    # rare: symmetric groups put one element per group on the 7.5 tie, so the
    # allowance scales with the number of groups (1e-3 at G = 128)
    assert (diff != 0).mean() < 1e-3 * 128 / G
    return (diff != 0).sum()


@pytest.mark.parametrize("I,O,dt,sym", [(256, 64, synth.F16, True), (1024, 200, synth.BF16, False),
                                        (384, 72, synth.F32, True), (128, 8, synth.F16, False),
                                        (512, 136, synth.F16, False)])
def test_quantize_pack_matches_oracle(I, O, dt, sym):
    L = synth.make_layer(301, 0, I, O)
    w = synth.make_w(301, 0, O, I, dt)
    say(f"quantize_pack I={I} O={O} dt={dt} sym={sym}")
    D = paro.DeviceLayer(L)
    qw, qz, s16 = gpu_quantize(D, w, dt, O, I, sym)
    ndiff = compare(L, w, dt, sym, qw, qz, s16, np.arange(O))
    say(f"  codes at ties that differ: {ndiff}")


@pytest.mark.parametrize("wl,li,dt,sym", [(3, 0, synth.BF16, True), (2, 0, synth.F16, True),
                                          (4, 1, synth.F16, False)])
def test_quantize_pack_full_size_sampled(wl, li, dt, sym):
    _, I, O = synth.WORKLOADS[wl]["layers"][li]
    L = synth.make_layer(wl, li, I, O)
    w = synth.make_w(wl, li, O, I, dt)
    say(f"quantize_pack workload {wl} layer {li}: I={I} O={O} dt={dt} sym={sym}")
    D = paro.DeviceLayer(L)
    qw, qz, s16 = gpu_quantize(D, w, dt, O, I, sym)
    rng = np.random.default_rng(wl * 10 + li)
    blocks = rng.choice(O // 8, size=4, replace=False)
    rows = np.sort(np.concatenate([np.arange(8 * b, 8 * b + 8) for b in blocks] + [np.arange(O - 8, O)]))
    compare(L, w, dt, sym, qw, qz, s16, np.unique(rows))


@pytest.mark.parametrize("sym", [True, False])
def test_quantized_layer_runs_through_the_linear(sym):
    """The packed outputs plus the rotation form a layer: the GPU linear over
    it meets the oracle gate on that layer, and stays within the quantization
    bound of the dense product X W^T + b."""
    I, O, M = 512, 256, 16
    L = synth.make_layer(302, 0, I, O)
    w = synth.make_w(302, 0, O, I, synth.F32)
    D = paro.DeviceLayer(L)
    qw, qz, s16 = gpu_quantize(D, w, synth.F32, O, I, sym)
    Q = synth.Layer(I, O, 128, L.krot, L.pairs, L.theta, L.channel_scales, np.ascontiguousarray(qw),
                    np.ascontiguousarray(qz), np.ascontiguousarray(s16), L.bias)
    x = synth.make_x(302, 0, M, I, synth.F16)
    DQ = paro.DeviceLayer(Q)
    xd = x_to_device(x, synth.F16)
    y = torch.empty((M, O), dtype=torch.float32, device="cuda")
    ws = paro.make_workspace(paro.paro_w4a16_linear_workspace_bytes(DQ, M, synth.F16, 0))
    paro.paro_w4a16_linear(DQ, xd, y, ws)
    torch.cuda.synchronize()
    yh = np.ascontiguousarray(y.cpu().numpy())
    rc, err, mref, _ = ref.paro_linear_ref_check(Q, x, synth.F16, yh, synth.F32, LIN_TOL)
    assert rc == ref.OK, f"linear on the packed layer off by {err / mref:.3e}"
    # against the dense product: each weight is within half a (fp16) step
    xs = ref.scale_rotate(Q, x, synth.F16)
    s_eff = np.asarray([[ref.f16_to_double(h) for h in row] for row in s16])
    bound = np.abs(xs) @ np.repeat(0.5 * s_eff * (1 + 2.0 ** -10), 128, axis=0)
    b = np.asarray([ref.f16_to_double(h) for h in L.bias])
    xv = np.asarray([[ref.f16_to_double(h) for h in row] for row in x])
    dense = xv @ w.astype(np.float64).T + b
    assert (np.abs(yh - dense) <= bound + LIN_TOL * np.abs(dense).max()).all()
