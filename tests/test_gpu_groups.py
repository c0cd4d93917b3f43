"""GPU parity at rotation / quantization group sizes G = 64 and 32 (the
"ParoQuant" wiki's group_size option; pairs never leave their group and each
group of G input channels has its own scale and zero point).

Every entry point runs against the fp64 oracle at these G with the same gates
as at G = 128: the staged and the dense (tiled) rotation, the linear on all
three paths, the dequantized weight, the offline quantizer and the rotation
backward.  The kernels rotate 128-channel blocks with the stored group-local
pair indices rebased into the block, so a pair schedule that crosses the
128-channel block's halves in the oracle's indexing would show up here.
"""
import numpy as np
import pytest

import synth
from _helpers import LIN_TOL, ROT_TOL, U, bits_to_f64, sample_rows, say, to_host_bits, torch_dtype, x_to_device
from oracle import ref

torch = pytest.importorskip("torch")
paro = pytest.importorskip("rotation_int4_weight_amd")

from test_gpu_backward import check as check_backward  # noqa: E402
from test_gpu_parity import PATHS, check_linear, check_rotation, untile  # noqa: E402
from test_gpu_quantize import compare as compare_quantize, gpu_quantize  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    paro.load()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.synchronize()


def layer(G, I, O, krot=8, seed=0):
    return synth.make_layer(500 + G, seed, I, O, group_size=G, krot=krot)


def test_group_variants_pass_host_validation():
    for G in (32, 64):
        paro.paro_validate_layer(layer(G, 256, 64))


@pytest.mark.parametrize("G", [64, 32])
@pytest.mark.parametrize("I,M,krot,dt", [(256, 3, 8, synth.F16), (384, 70, 5, synth.BF16), (128, 1, 1, synth.F16)])
def test_staged_rotation(G, I, M, krot, dt):
    L = layer(G, I, 8, krot)
    x = synth.make_x(500 + G, 1, M, I, dt)
    check_rotation(L, x, dt, np.arange(M), f"G={G}")


@pytest.mark.parametrize("G", [64, 32])
@pytest.mark.parametrize("I,M,dt", [(256, 40, synth.F16), (512, 300, synth.BF16)])
def test_dense_tiled_rotation(G, I, M, dt):
    L = layer(G, I, 8)
    x = synth.make_x(500 + G, 2, M, I, dt)
    say(f"scale_rotate_tiled G={G} I={I} M={M}")
    D = paro.DeviceLayer(L)
    hl = torch.empty((paro.paro_rotation_matrix_bytes(D) // 2,), dtype=torch.int16, device="cuda")
    paro.paro_rotation_matrix(D, dt, hl)
    xt = torch.full((paro.paro_tiled_bytes(D, M) // 2,), -1, dtype=torch.int16, device="cuda")
    paro.paro_scale_rotate_tiled(D, hl, x_to_device(x, dt), xt)
    torch.cuda.synchronize()
    t = untile(xt.cpu().numpy().view(np.uint16), M, I)
    assert not t[M:].any()
    xr_ref = ref.scale_rotate(L, np.ascontiguousarray(x), dt)
    err = np.abs(bits_to_f64(t[:M], dt) - xr_ref).max(axis=1) / np.abs(xr_ref).max(axis=1)
    assert float(err.max()) <= ROT_TOL + U[dt]


@pytest.mark.parametrize("G", [64, 32])
@pytest.mark.parametrize("I,O,M,dt,path", [(256, 64, 1, synth.F16, "fused"), (512, 200, 4, synth.BF16, "fused"),
                                          (384, 136, 16, synth.F16, "split"), (512, 256, 9, synth.BF16, "split"),
                                          (256, 264, 300, synth.BF16, "prefill"),
                                          (1024, 512, 40, synth.F16, "prefill")])
def test_linear_all_paths(G, I, O, M, dt, path):
    L = layer(G, I, O)
    x = synth.make_x(500 + G, 3, M, I, dt)
    check_linear(L, x, dt, path, label=f"G={G}")


@pytest.mark.parametrize("G,cfg", [(64, 1), (32, 3)])
def test_linear_full_size_sampled(G, cfg):
    """A Llama-3-8B-shaped layer at G: decode at 1 token, prefill at 2048
    (sampled rows for the oracle)."""
    spec = synth.WORKLOADS[cfg]
    _, I, O = spec["layers"][0]
    L = synth.make_layer(cfg, 0, I, O, group_size=G)
    x = synth.make_x(cfg, 0, spec["tokens"], I, spec["act"])
    path = "prefill" if spec["tokens"] > 16 else "fused"
    check_linear(L, x, spec["act"], path, rows=sample_rows(spec["tokens"], 24), label=f"cfg{cfg} G={G}")


@pytest.mark.parametrize("G", [64, 32])
def test_unpack_dequant(G):
    I, O = 384, 136
    L = layer(G, I, O)
    D = paro.DeviceLayer(L)
    z = torch.full((I // G, O), 255, dtype=torch.uint8, device="cuda")
    w32 = torch.empty((I, O), dtype=torch.float32, device="cuda")
    paro.paro_w4_unpack_dequant(D, None, z, w32)
    torch.cuda.synchronize()
    assert np.array_equal(z.cpu().numpy(), ref.unpack(L)[1])
    assert np.array_equal(w32.cpu().numpy().astype(np.float64), ref.dequant(L))


@pytest.mark.parametrize("G", [64, 32])
@pytest.mark.parametrize("I,O,dt,sym", [(256, 64, synth.F16, True), (512, 136, synth.BF16, False),
                                        (384, 72, synth.F32, False)])
def test_quantize_pack(G, I, O, dt, sym):
    L = layer(G, I, O)
    w = synth.make_w(500 + G, 4, O, I, dt)
    say(f"quantize_pack G={G} I={I} O={O} dt={dt} sym={sym}")
    D = paro.DeviceLayer(L)
    qw, qz, s16 = gpu_quantize(D, w, dt, O, I, sym, G)
    compare_quantize(L, w, dt, sym, qw, qz, s16, np.arange(O))


@pytest.mark.parametrize("G", [64, 32])
@pytest.mark.parametrize("I,M,x_dt,g_dt,gx_dt", [(256, 100, synth.F16, synth.F32, synth.F32),
                                                 (512, 64, synth.BF16, synth.BF16, synth.BF16)])
def test_rotation_backward(G, I, M, x_dt, g_dt, gx_dt):
    L = layer(G, I, 64)
    x = synth.make_x(500 + G, 5, M, I, x_dt)
    g = synth.make_g(500 + G, 5, M, I, g_dt)
    say(f"scale_rotate_backward G={G} I={I} M={M}")
    check_backward(L, x, x_dt, g, g_dt, gx_dt)
