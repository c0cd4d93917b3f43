"""GPU parity of libparo against the fp64 CPU oracle, through the C-ABI.

Every expected value comes from oracle/ (or from the exact format rules);
inputs come from the seeded generator in synth/.  Gates:
  * integers (unpacked codes, zero points): bit-exact;
  * dense dequant: bit-exact vs round-to-nearest-even of the exact product;
  * rotated activations: per row max|dX_r| <= 1e-3 * max|X_r,ref| (fp32
    output), plus the output dtype's unit roundoff for fp16/bf16 outputs;
  * linear: max|dY| <= 5e-3 * max|Y_ref| for fp32 output, plus the unit
    roundoff for fp16/bf16 output, which must also equal the
    round-to-nearest-even of the fp32 output (same kernels, deterministic).
Full-size workloads are run whole on the GPU and checked on a seeded sample
of rows (rows are independent, so the oracle computes exactly those rows).
"""
import numpy as np
import pytest

import synth
from _helpers import (LIN_TOL, ROT_TOL, U, bits_to_f64, sample_rows, say, stratified_rows, to_host_bits,
                      torch_dtype, workload, x_to_device)
from oracle import ref

torch = pytest.importorskip("torch")
paro = pytest.importorskip("rotation_int4_weight_amd")

pytestmark = pytest.mark.gpu

PATHS = {"fused": 1, "split": 2, "prefill": 3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    paro.load()  # raises when libparo.so is missing: no fallback exists
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.synchronize()


def run_linear(D, xd, O, out_dt, path, ws=None):
    M = xd.shape[0]
    y = torch.full((M, O), float("nan"), dtype=torch_dtype(out_dt), device="cuda")
    if ws is None:
        ws = paro.make_workspace(paro.paro_w4a16_linear_workspace_bytes(
            D, M, 0 if xd.dtype == torch.float16 else 1, path))
    paro.paro_w4a16_linear(D, xd, y, ws, path=path)
    torch.cuda.synchronize()
    return y


def check_linear(L, x, dt, path, rows=None, label=""):
    """Run one path in fp32 and activation-dtype output; check vs the oracle."""
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, dt)
    M, O = x.shape[0], L.out_features
    say(f"linear {label} path={path} I={L.in_features} O={O} M={M} dt={dt}")
    y32 = run_linear(D, xd, O, synth.F32, PATHS[path])
    ya = run_linear(D, xd, O, dt, PATHS[path])
    y32h, yah = to_host_bits(y32), to_host_bits(ya)
    rows = np.arange(M) if rows is None else rows
    rc, err, mref, _ = ref.paro_linear_ref_check(L, x[rows], dt, np.ascontiguousarray(y32h[rows]),
                                                 synth.F32, LIN_TOL)
    say(f"  fp32 out: max|dY|/max|Y| = {err / mref:.3e}")
    assert rc == ref.OK, f"fp32 output off by {err / mref:.3e} of max|Y|"
    rc, err2, _, _ = ref.paro_linear_ref_check(L, x[rows], dt, np.ascontiguousarray(yah[rows]), dt,
                                               LIN_TOL + U[dt])
    say(f"  act out:  max|dY|/max|Y| = {err2 / mref:.3e}")
    assert rc == ref.OK
    # the activation-dtype output is one RNE rounding of the fp32 result
    rne = torch.from_numpy(y32h).to(torch_dtype(dt)).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yah, rne)
    # deterministic: a second call gives identical bits
    y32b = to_host_bits(run_linear(D, xd, O, synth.F32, PATHS[path]))
    assert np.array_equal(y32h.view(np.uint32), y32b.view(np.uint32))
    return y32h


# ---------------------------------------------------------------------------
# unpack + dequant
# ---------------------------------------------------------------------------

UNPACK_CASES = [(0, 0), (1, 0), (2, 0), (3, 0)] + [(4, li) for li in range(7)]


@pytest.mark.parametrize("cfg,li", UNPACK_CASES)
def test_unpack_dequant_bitexact(cfg, li):
    lname, L, x, dt = workload(cfg, li)
    I, O = L.in_features, L.out_features
    say(f"unpack_dequant cfg{cfg} {lname} I={I} O={O}")
    D = paro.DeviceLayer(L)
    q = torch.empty((I, O), dtype=torch.uint8, device="cuda")
    z = torch.empty((I // 128, O), dtype=torch.uint8, device="cuda")
    w32 = torch.empty((I, O), dtype=torch.float32, device="cuda")
    paro.paro_w4_unpack_dequant(D, q, z, w32)
    torch.cuda.synchronize()
    q_ref, z_ref = ref.unpack(L)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(z.cpu().numpy(), z_ref)
    w_ref = ref.dequant(L)
    assert np.array_equal(w32.cpu().numpy().astype(np.float64), w_ref)
    del w32
    for wdt in (synth.F16, synth.BF16):
        w = torch.empty((I, O), dtype=torch_dtype(wdt), device="cuda")
        paro.paro_w4_unpack_dequant(D, None, None, w)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(w), ref.round_array(w_ref, wdt))


def test_unpack_dequant_ragged_and_partial_outputs():
    L = synth.make_layer(200, 0, 384, 136)
    D = paro.DeviceLayer(L)
    q_ref, z_ref = ref.unpack(L)
    z = torch.full((3, 136), 255, dtype=torch.uint8, device="cuda")
    paro.paro_w4_unpack_dequant(D, None, z, None)
    torch.cuda.synchronize()
    assert np.array_equal(z.cpu().numpy(), z_ref)
    w = torch.empty((384, 136), dtype=torch.float16, device="cuda")
    paro.paro_w4_unpack_dequant(D, None, None, w)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(w), ref.round_array(ref.dequant(L), synth.F16))


# ---------------------------------------------------------------------------
# scale + rotate
# ---------------------------------------------------------------------------

def check_rotation(L, x, dt, rows, label):
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, dt)
    M, I = x.shape
    say(f"scale_rotate {label} I={I} M={M} krot={L.krot} dt={dt}")
    xr_ref = ref.scale_rotate(L, np.ascontiguousarray(x[rows]), dt)
    rowmax = np.abs(xr_ref).max(axis=1)
    out32 = None
    for odt in (synth.F32, synth.F16, synth.BF16):
        out = torch.empty((M, I), dtype=torch_dtype(odt), device="cuda")
        paro.paro_scale_rotate(D, xd, out)
        torch.cuda.synchronize()
        h = to_host_bits(out)
        got = bits_to_f64(h[rows], odt)
        err = np.abs(got - xr_ref).max(axis=1)
        worst = float((err / rowmax).max())
        say(f"  out dt={odt}: worst row max|dX_r|/max|X_r| = {worst:.3e}")
        assert worst <= ROT_TOL + U[odt]
        if odt == synth.F32:
            out32 = h
        else:  # one RNE rounding of the fp32 result
            rne = torch.from_numpy(out32).to(torch_dtype(odt)).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(h, rne)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_scale_rotate_workloads(cfg):
    lname, L, x, dt = workload(cfg)
    check_rotation(L, x, dt, sample_rows(x.shape[0], 64, seed=cfg), f"cfg{cfg} {lname}")


@pytest.mark.parametrize("I,M,krot,dt", [(128, 1, 1, synth.F16), (384, 65, 9, synth.BF16),
                                         (256, 130, 64, synth.F16), (1024, 3, 8, synth.BF16)])
def test_scale_rotate_shapes(I, M, krot, dt):
    L = synth.make_layer(201, krot, I, 8, krot=krot)
    x = synth.make_x(201, krot, M, I, dt)
    check_rotation(L, x, dt, np.arange(M), f"I={I} M={M}")


def test_scale_rotate_in_place():
    L = synth.make_layer(202, 0, 256, 8)
    x = synth.make_x(202, 0, 70, 256, synth.F16)
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, synth.F16)
    sep = torch.empty_like(xd)
    paro.paro_scale_rotate(D, xd, sep)
    paro.paro_scale_rotate(D, xd, xd)
    torch.cuda.synchronize()
    assert torch.equal(sep.view(torch.int16), xd.view(torch.int16))


def test_identity_state_rotation_is_exact():
    L = synth.make_layer(203, 0, 256, 8, identity=True)
    x = synth.make_x(203, 0, 5, 256, synth.BF16)
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, synth.BF16)
    out = torch.empty((5, 256), dtype=torch.float32, device="cuda")
    paro.paro_scale_rotate(D, xd, out)
    torch.cuda.synchronize()
    # zero angles: cos = 1, sin = 0, unit scales -> the input, exactly
    assert np.array_equal(out.cpu().numpy().astype(np.float64), bits_to_f64(x, synth.BF16))


# ---------------------------------------------------------------------------
# the linear, on the five workloads (full size, sampled rows)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,path", [(0, "fused"), (0, "split"), (0, "prefill"),
                                      (1, "fused"), (1, "split"), (1, "prefill"),
                                      (2, "split"), (2, "fused"), (2, "prefill"),
                                      (3, "prefill")])
def test_linear_workloads(cfg, path):
    lname, L, x, dt = workload(cfg)
    # prefill at full size: rows in every 256-row M tile, all residues mod 16
    rows = stratified_rows(x.shape[0], 4, seed=cfg) if path == "prefill" else sample_rows(x.shape[0], 48, seed=cfg)
    check_linear(L, x, dt, path, rows, f"cfg{cfg} {lname}")


@pytest.mark.parametrize("li", range(7))
def test_linear_decoder_layer_prefill(li):
    lname, L, x, dt = workload(4, li)
    check_linear(L, x, dt, "prefill", stratified_rows(x.shape[0], 3, seed=40 + li), f"cfg4 {lname}")


def tiled_rows_of(bits, M, I, rows):
    """Rows `rows` of a tiled X_r buffer (layout of include/paro.h), row-major."""
    a = np.asarray(bits).reshape((M + 15) // 16, I // 32, 4, 16, 8)
    return np.stack([a[r // 16, :, :, r % 16, :].reshape(I) for r in rows])


@pytest.mark.parametrize("cfg,li", [(3, 0)] + [(4, li) for li in range(7)])
def test_dense_rotation_full_size(cfg, li):
    """The prefill rotation as the linear runs it (dense H + L on the matrix
    cores, the full token count, so the launch takes the large-workgroup
    row split) meets the rotated-activation gate on stratified rows."""
    lname, L, x, dt = workload(cfg, li)
    M, I = x.shape
    say(f"dense rotation cfg{cfg} {lname} I={I} M={M}")
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, dt)
    hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device="cuda")
    paro.paro_rotation_matrix(D, dt, hl)
    xt = torch.full((paro.paro_tiled_bytes(D, M) // 2,), -1, dtype=torch.int16, device="cuda")
    paro.paro_scale_rotate_tiled(D, hl, xd, xt)
    torch.cuda.synchronize()
    rows = stratified_rows(M, 3, seed=60 + 7 * cfg + li)
    got = bits_to_f64(tiled_rows_of(xt.cpu().numpy().view(np.uint16), M, I, rows), dt)
    want = ref.scale_rotate(L, np.ascontiguousarray(x[rows]), dt)
    err = np.abs(got - want).max(axis=1) / np.abs(want).max(axis=1)
    say(f"  worst row max|dX_r|/max|X_r| = {float(err.max()):.3e}")
    assert float(err.max()) <= ROT_TOL + U[dt]


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

EDGE = [
    # I, O, M, dt, krot, path
    (128, 136, 3, synth.F16, 8, "fused"),
    (128, 136, 3, synth.F16, 8, "split"),
    (128, 136, 3, synth.F16, 8, "prefill"),
    (384, 264, 17, synth.BF16, 1, "prefill"),
    (256, 8, 1, synth.F16, 9, "fused"),
    (256, 8, 2, synth.BF16, 9, "fused"),
    (640, 1000, 300, synth.BF16, 8, "prefill"),
    (1024, 520, 16, synth.F16, 64, "split"),
    (1024, 520, 16, synth.BF16, 8, "fused"),
    (1280, 392, 7, synth.F16, 8, "split"),
    (512, 256, 257, synth.F16, 8, "prefill"),
    # 128-row tiles, ragged rows and a partial last column tile
    (4096, 1000, 300, synth.BF16, 8, "prefill"),
]


@pytest.mark.parametrize("I,O,M,dt,krot,path", EDGE)
def test_linear_edge_shapes(I, O, M, dt, krot, path):
    L = synth.make_layer(300 + I % 97, O % 89, I, O, krot=krot, bias=(O % 3 != 0))
    x = synth.make_x(300 + I % 97, O % 89, M, I, dt)
    check_linear(L, x, dt, path, None, f"edge")


def test_linear_persistent_ragged_fp16():
    """297 output tiles on at most 256 workgroups (some take two), a ragged
    last row block and a last column tile of 8 columns, fp16.  check_linear
    compares the whole fp16 output bit for bit with the rounding of the fp32
    output (a fused bias-and-convert with a single rounding fails this)."""
    I, O, M = 2304, 4104, 2100
    L = synth.make_layer(77, 5, I, O, krot=8, bias=True)
    x = synth.make_x(77, 5, M, I, synth.F16)
    check_linear(L, x, synth.F16, "prefill", stratified_rows(M, 3, seed=77), "persistent ragged")


def test_linear_identity_state_no_bias():
    L = synth.make_layer(310, 0, 512, 256, identity=True, bias=False)
    x = synth.make_x(310, 0, 9, 512, synth.F16)
    for path in ("fused", "split", "prefill"):
        check_linear(L, x, synth.F16, path, None, "identity")


def test_fused_and_split_decode_agree_bitwise():
    lname, L, x, dt = workload(1)
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, dt)
    a = to_host_bits(run_linear(D, xd, L.out_features, synth.F32, PATHS["fused"]))
    b = to_host_bits(run_linear(D, xd, L.out_features, synth.F32, PATHS["split"]))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_zero_tokens_is_a_noop():
    L = synth.make_layer(311, 0, 256, 64)
    D = paro.DeviceLayer(L)
    x = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    y = torch.empty((0, 64), dtype=torch.float16, device="cuda")
    paro.paro_w4a16_linear(D, x, y, None)
    paro.paro_scale_rotate(D, x, torch.empty((0, 256), dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()


def test_one_workspace_serves_many_shapes_and_paths():
    """The split-K counters live in a fixed area that every call leaves zero."""
    cases = [(256, 512, 1, "fused"), (1024, 136, 16, "split"), (512, 264, 40, "prefill"),
             (4096, 1024, 2, "fused"), (256, 512, 1, "fused"), (1024, 136, 5, "split")]
    need = 0
    layers = []
    for I, O, M, path in cases:
        L = synth.make_layer(320, I + O, I, O)
        x = synth.make_x(320, I + O, M, I, synth.F16)
        D = paro.DeviceLayer(L)
        need = max(need, paro.paro_w4a16_linear_workspace_bytes(D, M, 0, PATHS[path]))
        layers.append((L, x, D, path))
    ws = paro.make_workspace(need)
    for L, x, D, path in layers:
        xd = x_to_device(x, synth.F16)
        y = run_linear(D, xd, L.out_features, synth.F32, PATHS[path], ws=ws)
        rc, err, mref, _ = ref.paro_linear_ref_check(L, x, synth.F16, to_host_bits(y), synth.F32, LIN_TOL)
        say(f"  shared ws I={L.in_features} O={L.out_features} M={x.shape[0]} {path}: {err / mref:.3e}")
        assert rc == ref.OK


@pytest.mark.parametrize("cfg,path", [(1, "split"), (2, "split"), (3, "prefill")])
def test_prerotated_projection_matches_linear(cfg, path):
    """The projection alone over the linear's own X_r == the linear, bit for bit
    (X_r from paro_scale_rotate for the split path, from the dense tiled
    rotation for PREFILL)."""
    lname, L, x, dt = workload(cfg)
    say(f"prerotated cfg{cfg} {lname} path={path}")
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, dt)
    M, O = x.shape[0], L.out_features
    full = to_host_bits(run_linear(D, xd, O, synth.F32, PATHS[path]))
    if path == "prefill":  # the PREFILL linear rotates with the dense matrix: take its X_r
        hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device="cuda")
        paro.paro_rotation_matrix(D, dt, hl)
        xt = torch.empty((paro.paro_tiled_bytes(D, M) // 2,), dtype=torch.int16, device="cuda")
        paro.paro_scale_rotate_tiled(D, hl, xd, xt)
        rows = untile(xt.cpu().numpy().view(np.uint16), M, L.in_features)[:M]
        xr = x_to_device(np.ascontiguousarray(rows), dt)
    else:
        xr = torch.empty_like(xd)
        paro.paro_scale_rotate(D, xd, xr)
    y = torch.empty((M, O), dtype=torch.float32, device="cuda")
    ws = paro.make_workspace(paro.paro_w4a16_linear_workspace_bytes(D, M, dt, PATHS[path]))
    paro.paro_w4a16_linear_prerotated(D, xr, y, ws, path=PATHS[path])
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(y).view(np.uint32), full.view(np.uint32))


def untile(bits, M, I):
    """Tiled X_r (layout of include/paro.h) -> row-major [rows][I], rows padded to 16.

    Element (m, k) sits at ((m/16)*(I/32) + k/32)*512 + (((k%32)/8)*16 + m%16)*8 + k%8,
    i.e. the flat buffer is an array [m/16][k/32][(k%32)/8][m%16][k%8].
    """
    rows = (M + 15) // 16 * 16
    a = np.asarray(bits).reshape(rows // 16, I // 32, 4, 16, 8)
    return a.transpose(0, 3, 1, 2, 4).reshape(rows, I)


def mfma_row_of_channel(j):
    """Row of output channel j (< 128) in the H / L matrices: the matrix cores
    take row 4q+r of 16-row tile 2b+h as channel 32b + 8q + 4h + r."""
    j = np.asarray(j)
    return (j & ~31) | (((j >> 2) & 1) << 4) | (((j >> 3) & 3) << 2) | (j & 3)


def within_one_ulp(a, b, dt):
    """Elementwise: a and b (values of dtype dt) are equal or adjacent."""
    mant, tiny = (10, 2.0 ** -14) if dt == synth.F16 else (7, 2.0 ** -126)
    mag = np.maximum(np.maximum(np.abs(a), np.abs(b)), tiny)
    return np.abs(a - b) <= 2.0 ** (np.floor(np.log2(mag)) - mant)


ONE_BITS = {synth.F16: 0x3C00, synth.BF16: 0x3F80}


@pytest.mark.parametrize("I,krot,dt", [(128, 1, synth.F16), (256, 8, synth.BF16), (512, 9, synth.F16),
                                       (384, 40, synth.BF16)])
def test_rotation_matrix_is_the_scaled_rotation(I, krot, dt):
    """H + L == diag(cs) . R per group: the oracle's scaling and rotation of
    the unit rows (x = identity, exact in either dtype) gives R' row by row."""
    L = synth.make_layer(207, krot, I, 8, krot=krot)
    say(f"rotation_matrix I={I} krot={krot} dt={dt}")
    D = paro.DeviceLayer(L)
    nbytes = paro.paro_rotation_matrix_bytes(D)
    assert nbytes == I * 512
    hl = torch.full((nbytes // 2,), -1, dtype=torch.int16, device="cuda")
    paro.paro_rotation_matrix(D, dt, hl)
    torch.cuda.synchronize()
    eye = np.zeros((I, I), dtype=np.uint16)
    eye[np.arange(I), np.arange(I)] = ONE_BITS[dt]
    r_ref = ref.scale_rotate(L, eye, dt)  # r_ref[i][k] = R'[i][k] (block diagonal)
    m = bits_to_f64(hl.cpu().numpy().view(np.uint16), dt).reshape(I // 128, 2, 128, 128)
    rows = mfma_row_of_channel(np.arange(128))
    tol = 4e-6 if dt == synth.F16 else 4e-5
    for g in range(I // 128):
        blk = r_ref[g * 128:(g + 1) * 128, g * 128:(g + 1) * 128]
        rec = (m[g, 0] + m[g, 1])[rows, :].T  # rec[i][j] = H_T[row(j)][i] + L_T[row(j)][i]
        assert np.abs(rec - blk).max() <= tol * np.abs(blk).max(), g
        h = m[g, 0][rows, :].T
        # H is R' rounded to the dtype: within one unit in the last place, or,
        # for entries near zero, within the fp32 error of the staged build
        # (about krot * 2^-24 of the block's scale)
        fp32_err = krot * 2.0 ** -23 * np.abs(blk).max()
        assert (within_one_ulp(h, blk, dt) | (np.abs(h - blk) <= fp32_err)).all()
    off = r_ref.copy()
    for g in range(I // 128):
        off[g * 128:(g + 1) * 128, g * 128:(g + 1) * 128] = 0
    assert not off.any()  # the oracle's rotation never mixes groups


@pytest.mark.parametrize("I,M,krot,dt", [(128, 1, 1, synth.F16), (4096, 17, 8, synth.F16),
                                         (384, 65, 9, synth.BF16), (1024, 48, 8, synth.BF16),
                                         (256, 600, 8, synth.F16), (128, 1040, 3, synth.BF16)])
def test_scale_rotate_tiled(I, M, krot, dt):
    """The tiled rotation (dense H + L on the matrix cores) meets the oracle's
    rotated-activation gate, is within one unit in the last place of the
    staged row-major rotation, and leaves the pad rows zero."""
    L = synth.make_layer(205, krot, I, 8, krot=krot)
    x = synth.make_x(205, krot, M, I, dt)
    say(f"scale_rotate_tiled I={I} M={M} krot={krot} dt={dt}")
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, dt)
    nbytes = paro.paro_tiled_bytes(D, M)
    assert nbytes == (M + 15) // 16 * 16 * I * 2
    hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device="cuda")
    paro.paro_rotation_matrix(D, dt, hl)
    xt = torch.full((nbytes // 2,), -1, dtype=torch.int16, device="cuda")  # poison
    paro.paro_scale_rotate_tiled(D, hl, xd, xt)
    rm = torch.empty_like(xd)
    paro.paro_scale_rotate(D, xd, rm)
    torch.cuda.synchronize()
    t = untile(xt.cpu().numpy().view(np.uint16), M, I)
    assert not t[M:].any()
    tv, rv = bits_to_f64(t[:M], dt), bits_to_f64(to_host_bits(rm), dt)
    # the dense and the staged rotation differ only in fp32 rounding: one unit
    # in the last place, except near zero (cancellation), where both sit
    # within 2^-12 of the row's scale of the exact value
    ulp1 = within_one_ulp(tv, rv, dt)
    near = np.abs(tv - rv) <= 2.0 ** -12 * np.abs(rv).max(axis=1, keepdims=True)
    assert (ulp1 | near).all()
    assert ulp1.mean() >= 0.999
    xr_ref = ref.scale_rotate(L, np.ascontiguousarray(x), dt)
    err = np.abs(tv - xr_ref).max(axis=1) / np.abs(xr_ref).max(axis=1)
    assert float(err.max()) <= ROT_TOL + U[dt]


@pytest.mark.parametrize("cfg,extra", [(0, None), (3, None), ("edge", (1024, 200, 40, synth.F16))])
def test_linear_tiled_matches_prefill_path(cfg, extra):
    """paro_rotation_matrix + paro_scale_rotate_tiled + paro_w4a16_linear_tiled
    == the PREFILL path, bit for bit."""
    if cfg == "edge":
        I, O, M, dt = extra
        L = synth.make_layer(206, 0, I, O)
        x = synth.make_x(206, 0, M, I, dt)
    else:
        _, L, x, dt = workload(cfg)
    M, I, O = x.shape[0], L.in_features, L.out_features
    say(f"linear_tiled cfg={cfg} I={I} O={O} M={M}")
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, dt)
    full = to_host_bits(run_linear(D, xd, O, synth.F32, PATHS["prefill"]))
    hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device="cuda")
    paro.paro_rotation_matrix(D, dt, hl)
    xt = torch.empty((paro.paro_tiled_bytes(D, M) // 2,), dtype=torch.int16, device="cuda")
    paro.paro_scale_rotate_tiled(D, hl, xd, xt)
    y = torch.empty((M, O), dtype=torch.float32, device="cuda")
    paro.paro_w4a16_linear_tiled(D, xt, dt, M, y)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(y).view(np.uint32), full.view(np.uint32))


@pytest.mark.parametrize("I,O,M,path", [(4096, 4096, 1, "fused"), (4096, 2048, 16, "split"),
                                        (2048, 1024, 3, "fused")])
def test_split_k_handoff_alternating_inputs(I, O, M, path):
    """Two inputs alternate on one workspace for many calls: every output must
    equal its first (oracle-checked) result bit for bit, so no call ever sees
    another call's partial sums or a counter left non-zero."""
    L = synth.make_layer(330, M, I, O)
    xa = synth.make_x(330, M, M, I, synth.F16)
    xb = synth.make_x(331, M, M, I, synth.F16)
    D = paro.DeviceLayer(L)
    ws = paro.make_workspace(paro.paro_w4a16_linear_workspace_bytes(D, M, 0, PATHS[path]))
    say(f"handoff stress I={I} O={O} M={M} path={path}")
    outs = []
    for x in (xa, xb):
        xd = x_to_device(x, synth.F16)
        y = run_linear(D, xd, O, synth.F32, PATHS[path], ws=ws)
        rc, err, mref, _ = ref.paro_linear_ref_check(L, x, synth.F16, to_host_bits(y), synth.F32, LIN_TOL)
        assert rc == ref.OK
        outs.append((xd, y.clone()))
    ys = [torch.empty((M, O), dtype=torch.float32, device="cuda") for _ in range(200)]
    for i, yi in enumerate(ys):
        paro.paro_w4a16_linear(D, outs[i % 2][0], yi, ws, path=PATHS[path])
    torch.cuda.synchronize()
    for i, yi in enumerate(ys):
        assert torch.equal(yi.view(torch.int32), outs[i % 2][1].view(torch.int32)), f"call {i} differs"


@pytest.mark.parametrize("cfg,li", [(0, 0), (1, 0), (2, 0), (3, 0), (4, 1), ("edge", 0)])
def test_prepared_linear_matches_linear(cfg, li):
    """paro_w4a16_linear_prepared with the layer's rotation matrix built once
    == paro_w4a16_linear, bit for bit, on every path the shape selects, and
    the matrix stays usable for later calls (it is read, never written)."""
    if cfg == "edge":
        L = synth.make_layer(208, 0, 640, 1000)
        x = synth.make_x(208, 0, 300, 640, synth.BF16)
        dt = synth.BF16
    else:
        _, L, x, dt = workload(cfg, li)
    M, I, O = x.shape[0], L.in_features, L.out_features
    say(f"prepared linear cfg={cfg} layer={li} I={I} O={O} M={M}")
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, dt)
    hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device="cuda")
    paro.paro_rotation_matrix(D, dt, hl)
    hl0 = hl.clone()
    ws = paro.make_workspace(paro.paro_w4a16_linear_prepared_workspace_bytes(D, M))
    for ydt in (synth.F32, dt):
        ref_y = to_host_bits(run_linear(D, xd, O, ydt, 0))
        for _ in range(2):
            y = torch.full((M, O), float("nan"), dtype=torch_dtype(ydt), device="cuda")
            paro.paro_w4a16_linear_prepared(D, hl, xd, y, ws)
            torch.cuda.synchronize()
            assert np.array_equal(to_host_bits(y).view(np.uint8), ref_y.view(np.uint8))
    assert torch.equal(hl, hl0)
