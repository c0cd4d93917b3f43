"""GPU parity with one rotation and quantization group over the whole row
(group_size -1, i.e. G = in_features): the "ParoQuant" wiki's Concepts /
Pairwise Givens rotations take -1 to mean all in_features channels, and its
Backend reference lists -1 among the supported group sizes.

A stage's pairs may then join any two channels of the row, so the kernels
cannot rotate 128-channel blocks: the rotation runs in its own pass with
whole rows staged in LDS, and the contraction folds one scale and zero
point per column over all of K.  Same gates as at G = 128 against the fp64
oracle, which takes -1 as I."""
import ctypes

import numpy as np
import pytest

import synth
from _helpers import say, stratified_rows, to_host_bits, torch_dtype, x_to_device
from oracle import ref

torch = pytest.importorskip("torch")
paro = pytest.importorskip("rotation_int4_weight_amd")
from rotation_int4_weight_amd import _lib  # noqa: E402

from test_gpu_parity import PATHS, check_linear, check_rotation, run_linear  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    paro.load()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.synchronize()


def layer(I, O, krot=8, seed=0):
    return synth.make_layer(700, seed, I, O, group_size=-1, krot=krot)


@pytest.mark.parametrize("I,M,krot,dt", [(256, 3, 8, synth.F16), (384, 70, 5, synth.BF16), (128, 1, 1, synth.F16),
                                         (1024, 17, 8, synth.BF16), (4096, 2, 8, synth.F16)])
def test_rotation_over_the_whole_row(I, M, krot, dt):
    L = layer(I, 8, krot)
    x = synth.make_x(700, 1, M, I, dt)
    check_rotation(L, x, dt, np.arange(M), "G=-1")


def test_rotation_over_the_whole_row_in_place():
    L = layer(512, 8)
    x = synth.make_x(700, 2, 37, 512, synth.BF16)
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, synth.BF16)
    sep = torch.empty_like(xd)
    paro.paro_scale_rotate(D, xd, sep)
    paro.paro_scale_rotate(D, xd, xd)
    torch.cuda.synchronize()
    assert torch.equal(sep.view(torch.int16), xd.view(torch.int16))


@pytest.mark.parametrize("I,O,M,dt,path", [(256, 64, 1, synth.F16, "split"), (384, 136, 16, synth.BF16, "split"),
                                          (512, 264, 300, synth.BF16, "prefill"), (1024, 512, 40, synth.F16, "prefill"),
                                          (640, 1000, 7, synth.F16, "prefill"), (256, 136, 3, synth.BF16, "split")])
def test_linear_whole_row_group(I, O, M, dt, path):
    L = layer(I, O)
    x = synth.make_x(700, 3, M, I, dt)
    check_linear(L, x, dt, path, label="G=-1")


@pytest.mark.parametrize("cfg,tokens", [(1, 1), (1, 16), (3, 2048)])
def test_linear_whole_row_group_llama_shapes(cfg, tokens):
    """Llama-3-8B q_proj (4096 -> 4096) in decode and down_proj (14336 -> 4096)
    at 2048 tokens, with one group over the whole row; the oracle checks
    rows in every 256-row tile, at every residue mod 16."""
    spec = synth.WORKLOADS[cfg]
    _, I, O = spec["layers"][0]
    L = synth.make_layer(cfg, 0, I, O, group_size=-1)
    x = synth.make_x(cfg, 0, tokens, I, spec["act"])
    path = "prefill" if tokens > 16 else "split"
    check_linear(L, x, spec["act"], path, rows=stratified_rows(tokens, 3, seed=70 + cfg), label=f"cfg{cfg} G=-1")


def test_auto_path_and_fused_refusal():
    L = layer(256, 64)
    D = paro.DeviceLayer(L)
    assert paro.paro_w4a16_linear_choose_path(D, 1) == PATHS["split"]
    assert paro.paro_w4a16_linear_choose_path(D, 40) == PATHS["prefill"]
    x = synth.make_x(700, 4, 2, 256, synth.F16)
    xd = x_to_device(x, synth.F16)
    y = torch.empty((2, 64), dtype=torch.float32, device="cuda")
    ws = paro.make_workspace(1 << 22)
    with pytest.raises(paro.ParoError) as e:
        paro.paro_w4a16_linear(D, xd, y, ws, path=PATHS["fused"])
    assert e.value.status == 5
    # AUTO at 2 tokens takes the split path and meets the gate
    paro.paro_w4a16_linear(D, xd, y, ws)
    torch.cuda.synchronize()
    rc, err, mref, _ = ref.paro_linear_ref_check(L, x, synth.F16, to_host_bits(y), synth.F32, 5e-3)
    assert rc == ref.OK


@pytest.mark.parametrize("I,O", [(384, 136), (4096, 1024)])
def test_unpack_dequant_whole_row_group(I, O):
    L = layer(I, O)
    D = paro.DeviceLayer(L)
    q = torch.empty((I, O), dtype=torch.uint8, device="cuda")
    z = torch.full((1, O), 255, dtype=torch.uint8, device="cuda")
    w32 = torch.empty((I, O), dtype=torch.float32, device="cuda")
    paro.paro_w4_unpack_dequant(D, q, z, w32)
    torch.cuda.synchronize()
    q_ref, z_ref = ref.unpack(L)
    assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(z.cpu().numpy(), z_ref)
    assert np.array_equal(w32.cpu().numpy().astype(np.float64), ref.dequant(L))


@pytest.mark.parametrize("M,path", [(9, "split"), (70, "prefill")])
def test_prerotated_and_noalloc_match_the_linear(M, path):
    """The projection over paro_scale_rotate's X_r, and the allocation-free
    linear, equal the linear bit for bit at G = -1."""
    I, O = 512, 264
    L = layer(I, O)
    x = synth.make_x(700, 5, M, I, synth.BF16)
    D = paro.DeviceLayer(L)
    xd = x_to_device(x, synth.BF16)
    full = to_host_bits(run_linear(D, xd, O, synth.F32, PATHS[path]))
    if path == "split":
        xr = torch.empty_like(xd)
        paro.paro_scale_rotate(D, xd, xr)
        y = torch.empty((M, O), dtype=torch.float32, device="cuda")
        ws = paro.make_workspace(paro.paro_w4a16_linear_workspace_bytes(D, M, synth.BF16, PATHS[path]))
        paro.paro_w4a16_linear_prerotated(D, xr, y, ws, path=PATHS[path])
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(y).view(np.uint32), full.view(np.uint32))
    y2 = torch.empty((M, O), dtype=torch.float32, device="cuda")
    paro.paro_w4a16_linear_noalloc(D, xd, y2)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(y2).view(np.uint32), full.view(np.uint32))
