"""GPU parity of the MXFP4 (four-bit activations) path against the fp64
oracle, through the C-ABI.

Quantization: the kernel decides on its fp32 rotation of the rows (staged for
weights; for activations the dense R' = H + L on the matrix cores, good to
about 2^-16 relative), the oracle on its exact one.  A block scale may
differ (by one) only where the oracle's block maximum lies within 1e-4
(relative) of a power of two, and a code only where the oracle's v / scale
lies within 1e-4 of an E2M1 rounding boundary (then by one step); such places
must be rare.  Everything else is bit-exact.

GEMM: on the same codes and scales, the fp32 accumulation of exact FP4
products differs from the fp64 product by at most K * 2^-24 times the sum of
|products| per output (bound computed from the oracle's dequantized operands),
plus one output rounding for a 16-bit y.  The linear must equal its two steps
(quantize, GEMM) bit for bit.
"""
import numpy as np
import pytest

import synth
from _helpers import U, bits_to_f64, say, to_host_bits, torch_dtype, x_to_device
from oracle import ref

torch = pytest.importorskip("torch")
paro = pytest.importorskip("rotation_int4_weight_amd")

pytestmark = pytest.mark.gpu

TIE = 1e-4
# activations go through the dense R' = H + L (bf16 parts: each entry to about
# 2^-17), so a rotated value errs by up to about 2^-17 * sum |x_i R'_ij|, which
# for a group holding an x20 outlier column reaches ~1e-4 of the block scale:
# decisions within 2e-3 of a boundary may differ
TIE_ACT = 2e-3
BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    paro.load()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.synchronize()


def nibbles(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[0], -1).astype(int)


def magnitude_index(c):
    return np.where(c & 8, -(c & 7), c & 7)


def compare_quantized(v_ref, codes_g, scales_g, tie=TIE):
    """v_ref: the oracle's exact rotated rows [rows][K]; tie: the decision
    window (relative to the block scale) that the kernel's rotation error can
    reach."""
    codes_o, scales_o = ref.mxfp4_quantize(v_ref)
    rows, K = v_ref.shape
    amax = np.abs(v_ref.reshape(rows, K // 32, 32)).max(axis=2)
    frac = np.log2(np.where(amax > 0, amax, 1.0))
    near_pow2 = np.abs(frac - np.round(frac)) < tie / np.log(2)
    ds = scales_g.astype(int) - scales_o.astype(int)
    bad_s = (ds != 0) & ~(near_pow2 & (np.abs(ds) == 1))
    assert not bad_s.any(), f"block scales differ off powers of two at {np.argwhere(bad_s)[:5]}"
    X = np.repeat(2.0 ** (scales_o.astype(float) - 127), 32, axis=1)
    qv = np.abs(v_ref / X)
    near_b = (np.abs(qv[..., None] - BOUNDS) < tie).any(axis=-1)
    ng, no = nibbles(codes_g), nibbles(codes_o)
    diff = magnitude_index(ng) - magnitude_index(no)
    same_scale = np.repeat(ds == 0, 32, axis=1)
    bad_c = same_scale & (diff != 0) & ~(near_b & (np.abs(diff) == 1))
    assert not bad_c.any(), f"codes differ off rounding boundaries at {np.argwhere(bad_c)[:5]}"
    assert (diff != 0).mean() < 1e-3 and (ds != 0).mean() < 1e-3
    return int((diff != 0).sum()), int((ds != 0).sum())


def gpu_quant_acts(D, x, dt, I):
    M = x.shape[0]
    c = torch.full((M, I // 2), 0xAA, dtype=torch.uint8, device="cuda")
    s = torch.full((M, I // 32), 0xAA, dtype=torch.uint8, device="cuda")
    ws = torch.empty(paro.paro_mxfp4_activation_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    paro.paro_mxfp4_quantize_activations(D, x_to_device(x, dt), c, s, ws)
    torch.cuda.synchronize()
    return c, s


def gpu_quant_weight(D, w, dt, O, I):
    c = torch.full((O, I // 2), 0xAA, dtype=torch.uint8, device="cuda")
    s = torch.full((O, I // 32), 0xAA, dtype=torch.uint8, device="cuda")
    paro.paro_mxfp4_quantize_weight(D, x_to_device(w, dt), c, s)
    torch.cuda.synchronize()
    return c, s


@pytest.mark.parametrize("I,M,dt,G", [(256, 5, synth.F16, 128), (384, 100, synth.BF16, 128),
                                      (512, 64, synth.BF16, 64), (128, 1, synth.F16, 32)])
def test_activation_quantization_matches_oracle(I, M, dt, G):
    L = synth.make_layer(701, 0, I, 64, group_size=G)
    x = synth.make_x(701, 1, M, I, dt)
    say(f"mxfp4 activations I={I} M={M} dt={dt} G={G}")
    c, s = gpu_quant_acts(paro.DeviceLayer(L), x, dt, I)
    nc, ns = compare_quantized(ref.scale_rotate(L, x, dt), c.cpu().numpy(), s.cpu().numpy(), TIE_ACT)
    say(f"  codes at boundaries that differ: {nc}, scales at powers of two that differ: {ns}")


@pytest.mark.parametrize("I,O,dt", [(256, 64, synth.F16), (512, 200, synth.BF16), (384, 72, synth.F32)])
def test_weight_quantization_matches_oracle(I, O, dt):
    L = synth.make_layer(702, 0, I, O)
    w = synth.make_w(702, 0, O, I, dt)
    say(f"mxfp4 weight I={I} O={O} dt={dt}")
    c, s = gpu_quant_weight(paro.DeviceLayer(L), w, dt, O, I)
    compare_quantized(ref.transform_weight(L, w, dt), c.cpu().numpy(), s.cpu().numpy())


def random_mx(rng, rows, K, lo=118, hi=136):
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales


def check_gemm(ac, as_, wc, ws, bias, y_dt):
    M, K, O = ac.shape[0], ac.shape[1] * 2, wc.shape[0]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = torch.full((M, O), float("nan"), dtype=torch_dtype(y_dt), device="cuda")
    bd = None if bias is None else torch.from_numpy(bias.view(np.int16)).cuda()
    paro.paro_mxfp4_gemm(dev(ac), dev(as_), dev(wc), dev(ws), y, bd)
    torch.cuda.synchronize()
    got = bits_to_f64(to_host_bits(y), y_dt)
    want = ref.mxfp4_matmul(ac, as_, wc, ws, bias)
    B = np.abs(ref.mxfp4_dequant(ac, as_)) @ np.abs(ref.mxfp4_dequant(wc, ws)).T
    tol = K * 2.0 ** -24 * B + 1.01 * U[y_dt] * np.abs(want) + 1e-30
    d = np.abs(got - want)
    assert np.isfinite(got).all()
    assert (d <= tol).all(), f"off at {np.argwhere(d > tol)[:5]}: {d[d > tol][:5]}"
    return got


@pytest.mark.parametrize("M,O,K,y_dt,with_bias", [(1, 64, 128, synth.F32, False), (100, 200, 384, synth.F32, True),
                                                  (300, 256, 4096, synth.BF16, True),
                                                  (129, 136, 1024, synth.F16, False)])
def test_gemm_matches_oracle(M, O, K, y_dt, with_bias):
    rng = np.random.default_rng(M * 7 + O)
    # fp16 output: block scales small enough that |y| stays inside fp16's range
    lo, hi = (110, 124) if y_dt == synth.F16 else (118, 136)
    ac, as_ = random_mx(rng, M, K, lo, hi)
    wc, ws = random_mx(rng, O, K, lo, hi)
    bias = synth.f16_bits(rng.normal(0, 0.5, size=O)) if with_bias else None
    say(f"mxfp4 gemm M={M} O={O} K={K} y_dt={y_dt}")
    check_gemm(ac, as_, wc, ws, bias, y_dt)


def test_gemm_extreme_scales_and_zero_blocks():
    rng = np.random.default_rng(5)
    # A's scale bytes span 1..253 (2^-126 .. 2^126); W's keep every output
    # inside fp32's range (the largest is about 256 * 36 * 2^(126-17))
    ac, as_ = random_mx(rng, 40, 256, 1, 254)
    wc, ws = random_mx(rng, 64, 256, 100, 111)
    ac[3] = 0
    as_[3] = 0
    check_gemm(ac, as_, wc, ws, None, synth.F32)


@pytest.mark.parametrize("I,O,M,dt", [(512, 264, 70, synth.BF16), (256, 64, 3, synth.F16)])
def test_linear_is_quantize_then_gemm(I, O, M, dt):
    L = synth.make_layer(703, 0, I, O)
    x = synth.make_x(703, 1, M, I, dt)
    w = synth.make_w(703, 0, O, I, synth.F32)
    D = paro.DeviceLayer(L)
    wc, ws = gpu_quant_weight(D, w, synth.F32, O, I)
    y = torch.empty((M, O), dtype=torch.float32, device="cuda")
    work = torch.empty(paro.paro_mxfp4_linear_workspace_bytes(D, M), dtype=torch.uint8, device="cuda")
    paro.paro_mxfp4_linear(D, wc, ws, x_to_device(x, dt), y, work)
    ac, as_ = gpu_quant_acts(D, x, dt, I)
    y2 = torch.empty_like(y)
    bias = torch.from_numpy(L.bias.view(np.int16)).cuda()
    paro.paro_mxfp4_gemm(ac, as_, wc, ws, y2, bias)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    check_gemm(ac.cpu().numpy(), as_.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), L.bias, synth.F32)


@pytest.mark.parametrize("I,O,M,dt", [(512, 264, 70, synth.BF16), (256, 64, 3, synth.F16)])
def test_prepared_linear_equals_linear(I, O, M, dt):
    """The linear over a caller-built rotation matrix gives the same bits as
    the one that builds it in its workspace, on a workspace that holds no
    rotation matrix."""
    L = synth.make_layer(704, 0, I, O)
    x = synth.make_x(704, 1, M, I, dt)
    w = synth.make_w(704, 0, O, I, synth.F32)
    D = paro.DeviceLayer(L)
    wc, ws = gpu_quant_weight(D, w, synth.F32, O, I)
    xd = x_to_device(x, dt)
    y = torch.empty((M, O), dtype=torch_dtype(dt), device="cuda")
    work = torch.empty(paro.paro_mxfp4_linear_workspace_bytes(D, M), dtype=torch.uint8, device="cuda")
    paro.paro_mxfp4_linear(D, wc, ws, xd, y, work)
    hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device="cuda")
    paro.paro_rotation_matrix(D, dt, hl)
    need = paro.paro_mxfp4_linear_prepared_workspace_bytes(D, M)
    assert need < paro.paro_mxfp4_linear_workspace_bytes(D, M)
    y2 = torch.empty_like(y)
    work2 = torch.empty(need, dtype=torch.uint8, device="cuda")
    paro.paro_mxfp4_linear_prepared(D, hl, wc, ws, xd, y2, work2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_full_size_gemm_sampled_rows():
    """The down_proj shape at 2048 tokens: every output of 24 sampled rows."""
    M, K, O = 2048, 14336, 4096
    rng = np.random.default_rng(3)
    ac, as_ = random_mx(rng, M, K)
    wc, ws = random_mx(rng, O, K)
    dev = lambda a: torch.from_numpy(a).cuda()
    y = torch.empty((M, O), dtype=torch.float32, device="cuda")
    paro.paro_mxfp4_gemm(dev(ac), dev(as_), dev(wc), dev(ws), y)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 22, replace=False)]))
    got = y.cpu().numpy()[rows].astype(np.float64)
    wd = ref.mxfp4_dequant(wc, ws)
    ad = ref.mxfp4_dequant(ac[rows], as_[rows])
    want = ad @ wd.T
    B = np.abs(ad) @ np.abs(wd).T
    assert (np.abs(got - want) <= K * 2.0 ** -24 * B).all()
