"""GPU parity of paro_w4a16_linear_prepared_multi (layers over the same
input, out_features possibly different, one GEMM launch on the prefill path)
through the C-ABI.

Each layer's output must equal, bit for bit, that of its own
paro_w4a16_linear_prepared call (the same tile arithmetic), which the parity
tests of the single-layer entry point hold to the oracle; one sampled row
set per layer is also checked against the fp64 oracle directly.
"""
import numpy as np
import pytest

import synth
from _helpers import LIN_TOL, say, stratified_rows, to_host_bits, torch_dtype, workload, x_to_device
from oracle import ref

torch = pytest.importorskip("torch")
paro = pytest.importorskip("rotation_int4_weight_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    paro.load()  # raises when libparo.so is missing: no fallback exists
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.synchronize()


def _rotation(D, dt):
    hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device="cuda")
    paro.paro_rotation_matrix(D, dt, hl)
    return hl


def check_multi(hosts, x, dt, label, rows=None, ydts=None):
    M = x.shape[0]
    Os = [L.out_features for L in hosts]
    Ds = [paro.DeviceLayer(L) for L in hosts]
    xd = x_to_device(x, dt)
    hls = [_rotation(D, dt) for D in Ds]
    ws = paro.make_workspace(paro.paro_w4a16_linear_prepared_multi_workspace_bytes(Ds, M))
    ws1 = paro.make_workspace(max(paro.paro_w4a16_linear_prepared_workspace_bytes(D, M) for D in Ds))
    say(f"multi linear {label}: {len(hosts)} layers I={hosts[0].in_features} O={Os} M={M} dt={dt}")
    for ydt in (ydts or (synth.F32, dt)):
        refs = []
        for D, hl, O in zip(Ds, hls, Os):
            y = torch.full((M, O), float("nan"), dtype=torch_dtype(ydt), device="cuda")
            paro.paro_w4a16_linear_prepared(D, hl, xd, y, ws1)
            refs.append(y)
        torch.cuda.synchronize()
        for rep in range(2):  # a second call on the same workspace
            ys = [torch.full((M, O), float("nan"), dtype=torch_dtype(ydt), device="cuda") for O in Os]
            paro.paro_w4a16_linear_prepared_multi(Ds, hls, xd, ys, ws)
            torch.cuda.synchronize()
            for i, (y, r) in enumerate(zip(ys, refs)):
                assert np.array_equal(to_host_bits(y).view(np.uint8), to_host_bits(r).view(np.uint8)), \
                    f"layer {i}, output dtype {ydt}, call {rep}"
        if ydt == synth.F32:
            rs = np.arange(M) if rows is None else rows
            for i, L in enumerate(hosts):
                yh = to_host_bits(ys[i])
                rc, err, mref, _ = ref.paro_linear_ref_check(L, x[rs], dt, np.ascontiguousarray(yh[rs]), synth.F32,
                                                             LIN_TOL)
                say(f"  layer {i}: max|dY|/max|Y| = {err / mref:.3e}")
                assert rc == ref.OK


def test_multi_key_value_projections_decoder_layer():
    """The decoder layer's k_proj and v_proj (4096 -> 1024 each, 4096 tokens,
    bf16): 2 x 128 tiles of 256 rows in one launch instead of two launches
    of 128-row tiles."""
    _, Lk, x, dt = workload(4, 1)
    _, Lv, _, _ = workload(4, 2)
    check_multi([Lk, Lv], x, dt, "cfg4 k+v", rows=stratified_rows(x.shape[0], 2, seed=71), ydts=(dt, synth.F32))


@pytest.mark.parametrize("I,O,M,dt,n", [
    (1024, 2048, 2100, synth.F16, 2),   # 288 tiles on 256 workgroups: some take tiles of two layers
    (512, 264, 300, synth.BF16, 3),     # a last column tile of 8 columns, ragged rows, three layers
    (384, 136, 17, synth.F16, 4),       # the smallest prefill token count, four layers
    (256, 128, 5, synth.F16, 2),        # split decode: the layers run one after another
    (256, 128, 1, synth.BF16, 3),       # fused decode
])
def test_multi_shapes(I, O, M, dt, n):
    hosts = [synth.make_layer(500 + 7 * i + I % 13, O % 11, I, O, krot=8, bias=(i % 2 == 0)) for i in range(n)]
    x = synth.make_x(500 + I % 13, O % 11, M, I, dt)
    rows = None if M * O * I <= (1 << 27) else stratified_rows(M, 3, seed=I)
    check_multi(hosts, x, dt, f"{n} layers", rows=rows)


def test_multi_query_key_value_projections_decoder_layer():
    """The decoder layer's q_proj (4096 -> 4096), k_proj and v_proj (4096 ->
    1024) over one input, 4096 tokens, bf16: 16 x (32 + 8 + 8) tiles of 256
    rows in one launch, the layers' column tiles one after another."""
    _, Lq, x, dt = workload(4, 0)
    _, Lk, _, _ = workload(4, 1)
    _, Lv, _, _ = workload(4, 2)
    check_multi([Lq, Lk, Lv], x, dt, "cfg4 q+k+v", rows=stratified_rows(x.shape[0], 2, seed=72),
                ydts=(dt, synth.F32))


@pytest.mark.parametrize("I,Os,M,dt", [
    (512, (264, 128, 2048), 300, synth.BF16),   # ragged last tile in the first layer, a wide last layer
    (1024, (128, 2048, 136), 2100, synth.F16),  # tiles of layers of several widths across persistent workgroups
    (384, (136, 64, 264, 8), 17, synth.F16),    # four widths, the smallest prefill token count
    (256, (128, 264), 5, synth.F16),            # split decode: one layer after another
    (256, (264, 128, 64), 1, synth.BF16),       # fused decode
])
def test_multi_mixed_widths(I, Os, M, dt):
    hosts = [synth.make_layer(540 + 3 * i + I % 7, O % 13, I, O, krot=8, bias=(i % 2 == 1)) for i, O in enumerate(Os)]
    x = synth.make_x(540 + I % 7, len(Os), M, I, dt)
    rows = None if M * max(Os) * I <= (1 << 27) else stratified_rows(M, 3, seed=I + 1)
    check_multi(hosts, x, dt, f"widths {Os}", rows=rows)
