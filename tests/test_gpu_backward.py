"""GPU parity of paro_scale_rotate_backward (dL/dx, dL/dtheta, dL/dcs of the
channel scaling and rotation) against the fp64 oracle, through the C-ABI.

Tolerances, from the arithmetic: dL/dx is g . R'^T on the matrix cores with g
and R' each split into a bf16 high part and remainder (each good to 2^-17)
and fp32 accumulation: |d| <= 2^-16 * row max |gx_ref| for an fp32 gx, plus
the output rounding (1.01 unit roundoffs of |gx_ref|) for a 16-bit gx.
dL/dtheta and dL/dcs come from the per-group Gram matrix g^T x, accumulated
in fp32 over the tokens and then walked through the stages in fp32; with
N(0, 1)-sized inputs the sums cancel to about sqrt(tokens) times a term while
fp32 accumulation errs by about 2^-24 * tokens times a term, so
1e-4 * max |ref| holds with room to spare at every size tested, and a dropped
or mis-signed term still breaks it.
"""
import numpy as np
import pytest

import synth
from _helpers import U, bits_to_f64, say, to_host_bits, torch_dtype, x_to_device
from oracle import ref

torch = pytest.importorskip("torch")
paro = pytest.importorskip("rotation_int4_weight_amd")

pytestmark = pytest.mark.gpu

GX_FP32 = 2.0 ** -16
SUM_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    paro.load()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.synchronize()


def gpu_backward(D, L, x, x_dt, g, g_dt, gx_dt, stream=None):
    M, I = x.shape
    xd = x_to_device(x, x_dt)
    gd = x_to_device(g, g_dt)
    gx = torch.full((M, I), float("nan"), dtype=torch_dtype(gx_dt), device="cuda")
    gth = torch.full((L.krot, I // 2), float("nan"), dtype=torch.float32, device="cuda")
    gcs = torch.full((I,), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((max(paro.paro_scale_rotate_backward_workspace_bytes(D, M), 16),), 0x7f, dtype=torch.uint8,
                    device="cuda")
    paro.paro_scale_rotate_backward(D, xd, gd, gx, gth, gcs, ws, stream)
    torch.cuda.synchronize()
    return to_host_bits(gx), gth.cpu().numpy().astype(np.float64), gcs.cpu().numpy().astype(np.float64)


def check(L, x, x_dt, g, g_dt, gx_dt, D=None):
    D = D or paro.DeviceLayer(L)
    gx_b, gth, gcs = gpu_backward(D, L, x, x_dt, g, g_dt, gx_dt)
    gx = bits_to_f64(gx_b, gx_dt)
    r_gx, r_gth, r_gcs = ref.scale_rotate_backward(L, x, x_dt, bits_to_f64(g, g_dt))
    rowmax = np.abs(r_gx).max(axis=1, keepdims=True)
    tol = GX_FP32 * rowmax + 1.01 * U[gx_dt] * np.abs(r_gx)
    d = np.abs(gx - r_gx)
    assert np.isfinite(gx).all()
    bad = d > tol
    assert not bad.any(), f"dL/dx off at {np.argwhere(bad)[:5]}: {d[bad][:5]} > {tol[bad][:5]}"
    for name, got, want in (("dL/dtheta", gth, r_gth), ("dL/dcs", gcs, r_gcs)):
        assert np.isfinite(got).all(), f"{name} not finite"
        err = np.abs(got - want).max()
        scale = np.abs(want).max()
        say(f"  {name}: max err {err:.3e} of max {scale:.3e}")
        assert err <= SUM_TOL * scale, f"{name} off by {err / scale:.3e} of its max"
    return d.max() / max(np.abs(r_gx).max(), 1e-300)


@pytest.mark.parametrize("I,M,krot,x_dt,g_dt,gx_dt", [
    (256, 1, 8, synth.F16, synth.F32, synth.F32),
    (256, 64, 8, synth.BF16, synth.BF16, synth.BF16),
    (384, 100, 8, synth.F16, synth.F16, synth.F32),      # ragged: two 64-row tiles, 36 rows in the last
    (256, 200, 1, synth.BF16, synth.F32, synth.BF16),
    (512, 77, 12, synth.F16, synth.F32, synth.F16),      # more stages than are held in registers
    (128, 16, 3, synth.BF16, synth.F32, synth.F32),
])
def test_backward_matches_oracle(I, M, krot, x_dt, g_dt, gx_dt):
    say(f"scale_rotate_backward I={I} M={M} krot={krot} x_dt={x_dt} g_dt={g_dt} gx_dt={gx_dt}")
    L = synth.make_layer(401, krot, I, 64, krot=krot)
    x = synth.make_x(401, krot, M, I, x_dt)
    g = synth.make_g(401, krot, M, I, g_dt)
    check(L, x, x_dt, g, g_dt, gx_dt)


def test_backward_zero_tokens_writes_zero_sums():
    I = 256
    L = synth.make_layer(402, 0, I, 64)
    D = paro.DeviceLayer(L)
    x = torch.empty((0, I), dtype=torch.float16, device="cuda")
    g = torch.empty((0, I), dtype=torch.float32, device="cuda")
    gx = torch.empty((0, I), dtype=torch.float32, device="cuda")
    gth = torch.full((L.krot, I // 2), float("nan"), device="cuda")
    gcs = torch.full((I,), float("nan"), device="cuda")
    ws = torch.empty(paro.paro_scale_rotate_backward_workspace_bytes(D, 0), dtype=torch.uint8, device="cuda")
    paro.paro_scale_rotate_backward(D, x, g, gx, gth, gcs, ws)
    torch.cuda.synchronize()
    assert (gth.cpu() == 0).all() and (gcs.cpu() == 0).all()


def test_backward_identity_rotation_reduces_to_scaling():
    """theta = 0: dL/dx = g * cs, dL/dcs = sum g * x and dL/dtheta = sum over
    tokens of g_a x_b cs_b - g_b x_a cs_a (the textbook derivative at 0)."""
    I, M = 256, 50
    L = synth.make_layer(403, 0, I, 64)
    L = synth.Layer(L.in_features, L.out_features, L.group_size, L.krot, L.pairs,
                    np.zeros_like(L.theta), L.channel_scales, L.qweight, L.qzeros, L.scales, L.bias)
    x = synth.make_x(403, 0, M, I, synth.F16)
    g = synth.make_g(403, 0, M, I, synth.F32)
    D = paro.DeviceLayer(L)
    gx_b, gth, gcs = gpu_backward(D, L, x, synth.F16, g, synth.F32, synth.F32)
    xv, gv, cs = bits_to_f64(x, synth.F16), g.astype(np.float64), L.channel_scales.astype(np.float64)
    # dL/dx runs through the matrix cores with g and R' each split into a bf16
    # high part and remainder (each to 2^-17): within 2^-15 of the row's scale
    want_gx = gv * cs
    assert (np.abs(gx_b - want_gx) <= 2.0 ** -15 * np.abs(want_gx).max(axis=1, keepdims=True)).all()
    assert np.abs(gcs - (gv * xv).sum(axis=0)).max() <= SUM_TOL * np.abs((gv * xv).sum(axis=0)).max()
    xs = xv * cs
    a = L.pairs[:, 0::2].astype(np.int64) + (np.arange(I // 2) // 64 * 128)[None, :]
    b = L.pairs[:, 1::2].astype(np.int64) + (np.arange(I // 2) // 64 * 128)[None, :]
    want = np.stack([(gv[:, a[t]] * xs[:, b[t]] - gv[:, b[t]] * xs[:, a[t]]).sum(axis=0) for t in range(L.krot)])
    assert np.abs(gth - want).max() <= SUM_TOL * np.abs(want).max()


@pytest.mark.parametrize("wl,x_dt,g_dt,gx_dt", [(3, synth.BF16, synth.BF16, synth.BF16),
                                               (2, synth.F16, synth.F32, synth.F32)])
def test_backward_full_size(wl, x_dt, g_dt, gx_dt):
    """The workload's layer input at full size (the sums cover every token, so
    the oracle runs on all of them)."""
    spec = synth.WORKLOADS[wl]
    _, I, O = spec["layers"][0]
    M = max(spec["tokens"], 256)
    say(f"scale_rotate_backward workload {wl}: I={I} M={M}")
    L = synth.make_layer(wl, 0, I, O)
    x = synth.make_x(wl, 0, M, I, x_dt)
    g = synth.make_g(wl, 0, M, I, g_dt)
    check(L, x, x_dt, g, g_dt, gx_dt)


def test_backward_is_deterministic():
    I, M = 1024, 300
    L = synth.make_layer(404, 0, I, 64)
    D = paro.DeviceLayer(L)
    x = synth.make_x(404, 0, M, I, synth.BF16)
    g = synth.make_g(404, 0, M, I, synth.F32)
    first = gpu_backward(D, L, x, synth.BF16, g, synth.F32, synth.F32)
    second = gpu_backward(D, L, x, synth.BF16, g, synth.F32, synth.F32)
    for a, b in zip(first, second):
        assert np.array_equal(a, b)
