"""The linear captured into a HIP graph and replayed (as bench.py replays
decode steps): every replay, with eager calls and synchronizations between
the replays, gives the eager result bit for bit, through the C-ABI."""
import numpy as np
import pytest

import synth
from _helpers import say, to_host_bits, torch_dtype, x_to_device

torch = pytest.importorskip("torch")
paro = pytest.importorskip("rotation_int4_weight_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    paro.load()  # raises when libparo.so is missing: no fallback exists
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,path,prepared", [(1, 0, False), (3, 1, False), (16, 2, False), (64, 0, True)])
def test_graph_replays_equal_eager(M, path, prepared):
    I, O, dt = 1024, 768, synth.F16
    L = synth.make_layer(610, M, I, O, bias=True)
    x = synth.make_x(610, M, M, I, dt)
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, dt)
    hl = None
    if prepared:
        hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device="cuda")
        paro.paro_rotation_matrix(D, dt, hl)
        ws = paro.make_workspace(paro.paro_w4a16_linear_prepared_workspace_bytes(D, M))
    else:
        ws = paro.make_workspace(paro.paro_w4a16_linear_workspace_bytes(D, M, dt, path))

    def call(y, stream=None):
        if prepared:
            paro.paro_w4a16_linear_prepared(D, hl, xd, y, ws, stream=stream)
        else:
            paro.paro_w4a16_linear(D, xd, y, ws, stream=stream, path=path)

    say(f"graph replay M={M} path={path} prepared={prepared}")
    y_eager = torch.full((M, O), float("nan"), dtype=torch_dtype(dt), device="cuda")
    call(y_eager)
    torch.cuda.synchronize()
    ref_bits = to_host_bits(y_eager).copy()
    y = torch.full((M, O), float("nan"), dtype=torch_dtype(dt), device="cuda")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        call(y)
    torch.cuda.synchronize()
    other = torch.empty_like(y_eager)
    for rep in range(4):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(y), ref_bits), f"replay {rep}"
        call(other)  # the program's own eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(other), ref_bits)
