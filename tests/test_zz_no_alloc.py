"""The allocation-free linear (paro_w4a16_linear_noalloc) against the
workspace variant, through the C-ABI: identical bits on two calls in a row on
one GPU, the second smaller, so the library-held scratch is reused; a shape
beyond the scratch is refused before anything is launched."""
import ctypes

import numpy as np
import pytest

import synth
from _helpers import say, to_host_bits, x_to_device

torch = pytest.importorskip("torch")
paro = pytest.importorskip("rotation_int4_weight_amd")
from rotation_int4_weight_amd import _lib  # noqa: E402

pytestmark = pytest.mark.gpu


def noalloc(D, xd, y):
    """paro_w4a16_linear_noalloc through the C-ABI; returns its status."""
    return _lib.load().paro_w4a16_linear_noalloc(D.ref, ctypes.c_void_p(xd.data_ptr()), _lib._dt(xd), xd.shape[0],
                                                 ctypes.c_void_p(y.data_ptr()), _lib._dt(y),
                                                 _lib._stream_handle(None))


def with_workspace(D, xd, y):
    ws = paro.make_workspace(paro.paro_w4a16_linear_workspace_bytes(D, xd.shape[0], _lib._dt(xd)))
    paro.paro_w4a16_linear(D, xd, y, ws)


CASES = [
    # (label, I, O, tokens, dtype): prefill then a smaller prefill, decode (split-K) after
    [("prefill", 640, 1000, 300, synth.BF16), ("prefill, smaller", 384, 264, 40, synth.BF16)],
    [("decode 16 tokens", 4096, 2048, 16, synth.F16), ("decode 1 token", 1024, 520, 1, synth.F16)],
    [("prefill Llama q_proj 2048 tokens", 4096, 4096, 2048, synth.BF16), ("prefill 17 tokens", 256, 136, 17, synth.BF16)],
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_workspace_variant(case):
    assert torch.cuda.is_available()
    for i, (label, I, O, M, dt) in enumerate(CASES[case]):
        L = synth.make_layer(600 + case, i, I, O)
        x = synth.make_x(600 + case, i, M, I, dt)
        D = paro.DeviceLayer(L)
        xd = x_to_device(x, dt)
        for ydt in (dt, synth.F32):
            tdt = {synth.F16: torch.float16, synth.BF16: torch.bfloat16, synth.F32: torch.float32}[ydt]
            say(f"noalloc case {case} call {i} ({label}): I={I} O={O} M={M} x dt={dt} y dt={ydt}")
            a = torch.full((M, O), float("nan"), dtype=tdt, device="cuda")
            b = torch.full((M, O), float("nan"), dtype=tdt, device="cuda")
            rc = noalloc(D, xd, a)
            assert rc == 0, _lib.paro_last_error()
            with_workspace(D, xd, b)
            torch.cuda.synchronize()
            ha, hb = to_host_bits(a), to_host_bits(b)
            assert np.array_equal(ha.view(np.uint8), hb.view(np.uint8)), f"{label}: outputs differ"


def test_noalloc_refuses_shapes_beyond_its_scratch():
    L = synth.make_layer(610, 0, 14336, 64)
    D = paro.DeviceLayer(L)
    xd = torch.zeros((4096, 14336), dtype=torch.bfloat16, device="cuda")  # tiled X_r alone is 117 MB
    y = torch.zeros((4096, 64), dtype=torch.bfloat16, device="cuda")
    assert noalloc(D, xd, y) == 5
    assert "allocation-free" in _lib.paro_last_error()
