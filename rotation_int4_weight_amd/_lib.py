"""ctypes binding of libparo (include/paro.h).

Argument marshalling only: every step of the rotated W4A16 linear runs in the
HIP kernels of libparo.so.  PyTorch provides device memory and streams.  The
library must have been built (rotation_int4_weight_amd.build); there is no
fallback of any kind: a missing library or a failing call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# PARO_LIB names another build of the same library (e.g. one with host-side
# sanitizers); by default the in-tree libparo.so is loaded.
LIB_PATH = os.environ.get("PARO_LIB") or os.path.join(PKG, "libparo.so")

F16, BF16, F32 = 0, 1, 2
PATH_AUTO, PATH_DECODE_FUSED, PATH_DECODE_SPLIT, PATH_PREFILL = 0, 1, 2, 3
STATUS = {0: "PARO_OK", 1: "PARO_ERR_NULL", 2: "PARO_ERR_SHAPE", 3: "PARO_ERR_DTYPE",
          4: "PARO_ERR_ALIGN", 5: "PARO_ERR_UNSUPPORTED", 6: "PARO_ERR_PAIRS",
          7: "PARO_ERR_WORKSPACE", 8: "PARO_ERR_HIP"}
EXPORTS = ("paro_scale_rotate", "paro_w4_unpack_dequant", "paro_w4a16_linear",
           "paro_w4a16_linear_path", "paro_w4a16_linear_prerotated",
           "paro_w4a16_linear_prepared", "paro_w4a16_linear_prepared_workspace_bytes",
           "paro_w4a16_linear_prepared_multi", "paro_w4a16_linear_prepared_multi_workspace_bytes",
           "paro_w4a16_linear_tiled_multi",
           "paro_w4a16_linear_noalloc",
           "paro_w4_quantize_pack", "paro_scale_rotate_backward", "paro_w4a16_moe_linear",
           "paro_w4a16_moe_linear_workspace_bytes", "paro_mxfp4_quantize_weight",
           "paro_mxfp4_quantize_activations", "paro_mxfp4_gemm", "paro_mxfp4_linear",
           "paro_mxfp4_linear_workspace_bytes", "paro_mxfp4_activation_workspace_bytes",
           "paro_mxfp4_linear_prepared", "paro_mxfp4_linear_prepared_workspace_bytes",
           "paro_scale_rotate_backward_workspace_bytes",
           "paro_tiled_bytes", "paro_rotation_matrix_bytes", "paro_rotation_matrix",
           "paro_scale_rotate_tiled", "paro_w4a16_linear_tiled",
           "paro_w4a16_linear_workspace_bytes",
           "paro_w4a16_linear_choose_path", "paro_validate_layer", "paro_last_error",
           "paro_abi_version")


class ParoError(RuntimeError):
    def __init__(self, status: int, what: str, msg: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}: {msg}")
        self.status = status


class ParoLayerC(ctypes.Structure):
    _fields_ = [("in_features", ctypes.c_int64), ("out_features", ctypes.c_int64),
                ("group_size", ctypes.c_int32), ("krot", ctypes.c_int32),
                ("pairs", ctypes.c_void_p), ("theta", ctypes.c_void_p),
                ("channel_scales", ctypes.c_void_p), ("qweight", ctypes.c_void_p),
                ("qzeros", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("bias", ctypes.c_void_p)]


_lib = None


def load(path: str | None = None):
    """Load libparo.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m rotation_int4_weight_amd.build`")
    lib = ctypes.CDLL(path)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.paro_scale_rotate.argtypes = [P, P, I32, I64, P, I32, P]
    lib.paro_w4_unpack_dequant.argtypes = [P, P, P, P, I32, P]
    lib.paro_w4a16_linear.argtypes = [P, P, I32, I64, P, I32, P, SZ, P]
    lib.paro_w4a16_linear_path.argtypes = [P, P, I32, I64, P, I32, P, SZ, P, I32]
    lib.paro_w4a16_linear_prerotated.argtypes = [P, P, I32, I64, P, I32, P, SZ, P, I32]
    lib.paro_w4a16_linear_prepared.argtypes = [P, P, P, I32, I64, P, I32, P, SZ, P]
    lib.paro_w4a16_linear_prepared_workspace_bytes.argtypes = [P, I64]
    lib.paro_w4a16_linear_prepared_workspace_bytes.restype = SZ
    lib.paro_w4a16_linear_prepared_multi.argtypes = [P, ctypes.c_int, P, P, I32, I64, P, I32, P, SZ, P]
    lib.paro_w4a16_linear_prepared_multi_workspace_bytes.argtypes = [P, ctypes.c_int, I64]
    lib.paro_w4a16_linear_prepared_multi_workspace_bytes.restype = SZ
    lib.paro_w4a16_linear_tiled_multi.argtypes = [P, ctypes.c_int, P, I32, I64, P, I32, P]
    lib.paro_w4a16_linear_noalloc.argtypes = [P, P, I32, I64, P, I32, P]
    lib.paro_tiled_bytes.argtypes = [P, I64]
    lib.paro_tiled_bytes.restype = SZ
    lib.paro_w4_quantize_pack.argtypes = [P, P, I32, I32, P, P, P, P]
    lib.paro_w4a16_moe_linear.argtypes = [P, I32, P, P, I32, I64, P, I32, P, SZ, P]
    lib.paro_w4a16_moe_linear_workspace_bytes.argtypes = [P, I64, I32]
    lib.paro_w4a16_moe_linear_workspace_bytes.restype = SZ
    lib.paro_mxfp4_quantize_weight.argtypes = [P, P, I32, P, P, P]
    lib.paro_mxfp4_quantize_activations.argtypes = [P, P, I32, I64, P, P, P, SZ, P]
    lib.paro_mxfp4_activation_workspace_bytes.argtypes = [P]
    lib.paro_mxfp4_activation_workspace_bytes.restype = SZ
    lib.paro_mxfp4_gemm.argtypes = [P, P, I64, P, P, I64, I64, P, P, I32, P]
    lib.paro_mxfp4_linear.argtypes = [P, P, P, P, I32, I64, P, I32, P, SZ, P]
    lib.paro_mxfp4_linear_workspace_bytes.argtypes = [P, I64]
    lib.paro_mxfp4_linear_workspace_bytes.restype = SZ
    lib.paro_mxfp4_linear_prepared.argtypes = [P, P, P, P, P, I32, I64, P, I32, P, SZ, P]
    lib.paro_mxfp4_linear_prepared_workspace_bytes.argtypes = [P, I64]
    lib.paro_mxfp4_linear_prepared_workspace_bytes.restype = SZ
    lib.paro_scale_rotate_backward.argtypes = [P, P, I32, P, I32, I64, P, I32, P, P, P, SZ, P]
    lib.paro_scale_rotate_backward_workspace_bytes.argtypes = [P, I64]
    lib.paro_scale_rotate_backward_workspace_bytes.restype = SZ
    lib.paro_rotation_matrix_bytes.argtypes = [P]
    lib.paro_rotation_matrix_bytes.restype = SZ
    lib.paro_rotation_matrix.argtypes = [P, I32, P, P]
    lib.paro_scale_rotate_tiled.argtypes = [P, P, P, I32, I64, P, P]
    lib.paro_w4a16_linear_tiled.argtypes = [P, P, I32, I64, P, I32, P]
    lib.paro_w4a16_linear_workspace_bytes.argtypes = [P, I64, I32, I32]
    lib.paro_w4a16_linear_workspace_bytes.restype = SZ
    lib.paro_w4a16_linear_choose_path.argtypes = [P, I64]
    lib.paro_validate_layer.argtypes = [P]
    lib.paro_last_error.argtypes = []
    lib.paro_last_error.restype = ctypes.c_char_p
    lib.paro_abi_version.argtypes = []
    for name in ("paro_scale_rotate", "paro_w4_unpack_dequant", "paro_w4a16_linear",
                 "paro_w4a16_linear_path", "paro_w4a16_linear_prerotated", "paro_w4a16_linear_prepared",
                 "paro_w4a16_linear_prepared_multi", "paro_w4a16_linear_tiled_multi", "paro_w4a16_linear_noalloc",
                 "paro_w4_quantize_pack", "paro_scale_rotate_backward", "paro_w4a16_moe_linear",
                 "paro_mxfp4_quantize_weight", "paro_mxfp4_quantize_activations", "paro_mxfp4_gemm",
                 "paro_mxfp4_linear",
                 "paro_rotation_matrix", "paro_scale_rotate_tiled", "paro_w4a16_linear_tiled",
                 "paro_w4a16_linear_choose_path",
                 "paro_validate_layer", "paro_abi_version"):
        getattr(lib, name).restype = I32
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        raise ParoError(rc, what, load().paro_last_error().decode())


def paro_abi_version() -> int:
    return load().paro_abi_version()


def paro_last_error() -> str:
    return load().paro_last_error().decode()


def _stream_handle(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t) -> int:
    import torch
    return {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}[t.dtype]


class DeviceLayer:
    """A layer's stored tensors in device memory plus its C descriptor.

    Built from any object with the synth.Layer fields (numpy host arrays);
    torch allocates and owns the device copies.
    """

    def __init__(self, host, device="cuda"):
        import torch
        self.in_features = int(host.in_features)
        self.out_features = int(host.out_features)
        self.group_size = int(host.group_size)
        self.krot = int(host.krot)

        def up(a, dtype):
            return None if a is None else torch.from_numpy(a).to(device=device).view(dtype).contiguous()

        self.pairs = up(host.pairs, torch.int16)
        self.theta = up(host.theta, torch.float32)
        self.channel_scales = up(host.channel_scales, torch.float32)
        self.qweight = up(host.qweight, torch.int32)
        self.qzeros = up(host.qzeros, torch.int32)
        self.scales = up(host.scales.view("int16"), torch.float16)
        self.bias = None if host.bias is None else up(host.bias.view("int16"), torch.float16)
        self.c = ParoLayerC(self.in_features, self.out_features, self.group_size, self.krot,
                            self.pairs.data_ptr(), self.theta.data_ptr(),
                            self.channel_scales.data_ptr(), self.qweight.data_ptr(),
                            self.qzeros.data_ptr(), self.scales.data_ptr(),
                            None if self.bias is None else self.bias.data_ptr())

    @property
    def ref(self):
        return ctypes.byref(self.c)


def paro_validate_layer(host) -> None:
    """Host-side check of a layer's pair schedule and shape rules (numpy arrays)."""
    import numpy as np
    pairs = np.ascontiguousarray(host.pairs, dtype=np.int16)
    c = ParoLayerC(int(host.in_features), int(host.out_features), int(host.group_size),
                   int(host.krot), pairs.ctypes.data, None, None, None, None, None, None)
    _check(load().paro_validate_layer(ctypes.byref(c)), "paro_validate_layer")


def paro_scale_rotate(layer: DeviceLayer, x, x_r, stream=None) -> None:
    """x: (tokens, I) fp16/bf16 cuda tensor; x_r: (tokens, I) fp16/bf16/fp32 output."""
    _check(load().paro_scale_rotate(layer.ref, _ptr(x), _dt(x), x.shape[0], _ptr(x_r), _dt(x_r),
                                    _stream_handle(stream)), "paro_scale_rotate")


def paro_w4_unpack_dequant(layer: DeviceLayer, q_out=None, z_out=None, w_out=None, stream=None) -> None:
    w_dt = _dt(w_out) if w_out is not None else F32
    _check(load().paro_w4_unpack_dequant(layer.ref, _ptr(q_out), _ptr(z_out), _ptr(w_out), w_dt,
                                         _stream_handle(stream)), "paro_w4_unpack_dequant")


def paro_w4a16_linear_workspace_bytes(layer: DeviceLayer, tokens: int, x_dt: int = F16,
                                      path: int = PATH_AUTO) -> int:
    return int(load().paro_w4a16_linear_workspace_bytes(layer.ref, tokens, x_dt, path))


def paro_w4a16_linear_choose_path(layer: DeviceLayer, tokens: int) -> int:
    return int(load().paro_w4a16_linear_choose_path(layer.ref, tokens))


def make_workspace(nbytes: int, device="cuda"):
    """A zero-filled workspace (the contract requires zeros before first use)."""
    import torch
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def paro_w4a16_linear(layer: DeviceLayer, x, y, workspace=None, stream=None, path: int = PATH_AUTO) -> None:
    """y = rotated W4A16 linear of x.  x: (tokens, I) fp16/bf16; y: (tokens, O) x dtype or fp32."""
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load()
    if path == PATH_AUTO:
        rc = lib.paro_w4a16_linear(layer.ref, _ptr(x), _dt(x), x.shape[0], _ptr(y), _dt(y), ws_ptr,
                                   ws_bytes, _stream_handle(stream))
    else:
        rc = lib.paro_w4a16_linear_path(layer.ref, _ptr(x), _dt(x), x.shape[0], _ptr(y), _dt(y), ws_ptr,
                                        ws_bytes, _stream_handle(stream), path)
    _check(rc, "paro_w4a16_linear")


def paro_w4a16_linear_prepared_workspace_bytes(layer: DeviceLayer, tokens: int) -> int:
    return int(load().paro_w4a16_linear_prepared_workspace_bytes(layer.ref, tokens))


def paro_w4a16_linear_prepared(layer: DeviceLayer, hl, x, y, workspace=None, stream=None) -> None:
    """The linear with the layer's dense rotation hl prebuilt by paro_rotation_matrix (for x's dtype)."""
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().paro_w4a16_linear_prepared(layer.ref, _ptr(hl), _ptr(x), _dt(x), x.shape[0], _ptr(y), _dt(y),
                                             ws_ptr, ws_bytes, _stream_handle(stream)), "paro_w4a16_linear_prepared")


def _layer_array(layers):
    """A contiguous C array of the layers' descriptors (copies of their structs)."""
    arr = (ParoLayerC * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = L.c
    return arr


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def paro_w4a16_linear_prepared_multi_workspace_bytes(layers, tokens: int) -> int:
    return int(load().paro_w4a16_linear_prepared_multi_workspace_bytes(_layer_array(layers), len(layers), tokens))


def paro_w4a16_linear_prepared_multi(layers, hls, x, ys, workspace=None, stream=None) -> None:
    """Layers of one shape over the same input x, each with its rotation matrix hls[i] and output ys[i]."""
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().paro_w4a16_linear_prepared_multi(_layer_array(layers), len(layers), _ptr_array(hls), _ptr(x),
                                                   _dt(x), x.shape[0], _ptr_array(ys), _dt(ys[0]), ws_ptr,
                                                   ws_bytes, _stream_handle(stream)),
           "paro_w4a16_linear_prepared_multi")


def paro_w4a16_linear_tiled_multi(layers, x_ts, x_dt: int, tokens: int, ys, stream=None) -> None:
    """The prefill GEMM alone for layers of one shape, each over its tiled X_r, in one launch."""
    _check(load().paro_w4a16_linear_tiled_multi(_layer_array(layers), len(layers), _ptr_array(x_ts), x_dt, tokens,
                                                _ptr_array(ys), _dt(ys[0]), _stream_handle(stream)),
           "paro_w4a16_linear_tiled_multi")


def paro_w4a16_linear_noalloc(layer: DeviceLayer, x, y, stream=None) -> None:
    """The linear with the library-held workspace (no allocation in the call)."""
    _check(load().paro_w4a16_linear_noalloc(layer.ref, _ptr(x), _dt(x), x.shape[0], _ptr(y), _dt(y),
                                            _stream_handle(stream)), "paro_w4a16_linear_noalloc")


def paro_w4a16_linear_prerotated(layer: DeviceLayer, x_r, y, workspace=None, stream=None,
                                 path: int = PATH_AUTO) -> None:
    """The quantized projection alone over already rotated activations x_r."""
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().paro_w4a16_linear_prerotated(layer.ref, _ptr(x_r), _dt(x_r), x_r.shape[0], _ptr(y), _dt(y),
                                               ws_ptr, ws_bytes, _stream_handle(stream), path),
           "paro_w4a16_linear_prerotated")


def paro_tiled_bytes(layer: DeviceLayer, tokens: int) -> int:
    """Bytes of an X_r buffer in the prefill GEMM's tiled layout."""
    return int(load().paro_tiled_bytes(layer.ref, tokens))


def paro_w4_quantize_pack(layer: DeviceLayer, w, symmetric: bool, qweight, qzeros, scales, stream=None) -> None:
    """w: (O, I) fp16/bf16/fp32 device tensor; qweight int32 (I, O/8), qzeros int32 (I/128, O/8),
    scales fp16/int16 view (I/128, O)."""
    _check(load().paro_w4_quantize_pack(layer.ref, _ptr(w), _dt(w), int(bool(symmetric)), _ptr(qweight),
                                        _ptr(qzeros), _ptr(scales), _stream_handle(stream)), "paro_w4_quantize_pack")


def paro_mxfp4_quantize_weight(layer: DeviceLayer, w, codes, scales, stream=None) -> None:
    """w: (O, I) fp16/bf16/fp32; codes uint8 (O, I/2); scales uint8 (O, I/32)."""
    _check(load().paro_mxfp4_quantize_weight(layer.ref, _ptr(w), _dt(w), _ptr(codes), _ptr(scales),
                                             _stream_handle(stream)), "paro_mxfp4_quantize_weight")


def paro_mxfp4_activation_workspace_bytes(layer: DeviceLayer) -> int:
    return int(load().paro_mxfp4_activation_workspace_bytes(layer.ref))


def paro_mxfp4_quantize_activations(layer: DeviceLayer, x, codes, scales, workspace, stream=None) -> None:
    """x: (tokens, I) fp16/bf16; codes uint8 (tokens, I/2); scales uint8 (tokens, I/32); workspace: device
    buffer of paro_mxfp4_activation_workspace_bytes() bytes."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().paro_mxfp4_quantize_activations(layer.ref, _ptr(x), _dt(x), x.shape[0], _ptr(codes),
                                                  _ptr(scales), _ptr(workspace), ws_bytes, _stream_handle(stream)),
           "paro_mxfp4_quantize_activations")


def paro_mxfp4_gemm(a_codes, a_scales, w_codes, w_scales, y, bias=None, stream=None) -> None:
    """y (tokens, O) = A . W^T (+ bias) from MXFP4 codes/scales (uint8 device tensors)."""
    tokens, O, I = a_codes.shape[0], w_codes.shape[0], w_codes.shape[1] * 2
    _check(load().paro_mxfp4_gemm(_ptr(a_codes), _ptr(a_scales), tokens, _ptr(w_codes), _ptr(w_scales), O, I,
                                  _ptr(bias), _ptr(y), _dt(y), _stream_handle(stream)), "paro_mxfp4_gemm")


def paro_mxfp4_linear_workspace_bytes(layer: DeviceLayer, tokens: int) -> int:
    return int(load().paro_mxfp4_linear_workspace_bytes(layer.ref, tokens))


def paro_mxfp4_linear(layer: DeviceLayer, w_codes, w_scales, x, y, workspace, stream=None) -> None:
    """The W4A4 MXFP4 linear (rotation, activation quantization, FP4 GEMM, layer bias)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().paro_mxfp4_linear(layer.ref, _ptr(w_codes), _ptr(w_scales), _ptr(x), _dt(x), x.shape[0], _ptr(y),
                                    _dt(y), _ptr(workspace), ws_bytes, _stream_handle(stream)), "paro_mxfp4_linear")


def paro_mxfp4_linear_prepared_workspace_bytes(layer: DeviceLayer, tokens: int) -> int:
    return int(load().paro_mxfp4_linear_prepared_workspace_bytes(layer.ref, tokens))


def paro_mxfp4_linear_prepared(layer: DeviceLayer, hl, w_codes, w_scales, x, y, workspace, stream=None) -> None:
    """The W4A4 MXFP4 linear with the layer's dense rotation hl prebuilt by paro_rotation_matrix."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().paro_mxfp4_linear_prepared(layer.ref, _ptr(hl), _ptr(w_codes), _ptr(w_scales), _ptr(x), _dt(x),
                                             x.shape[0], _ptr(y), _dt(y), _ptr(workspace), ws_bytes,
                                             _stream_handle(stream)), "paro_mxfp4_linear_prepared")


def paro_w4a16_moe_linear_workspace_bytes(layer: DeviceLayer, tokens: int, x_dt: int = F16) -> int:
    """Workspace bytes of paro_w4a16_moe_linear for this many routed rows."""
    return int(load().paro_w4a16_moe_linear_workspace_bytes(layer.ref, tokens, x_dt))


def paro_w4a16_moe_linear(layer: DeviceLayer, num_experts: int, expert_offsets, x, y, workspace=None,
                          stream=None) -> None:
    """Experts stacked in `layer`'s weight tensors share its rotation.  expert_offsets: int64 device
    tensor (E+1,); x: (rows, I) fp16/bf16 grouped by expert; y: (rows, O) x dtype or fp32."""
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().paro_w4a16_moe_linear(layer.ref, int(num_experts), _ptr(expert_offsets), _ptr(x), _dt(x),
                                        x.shape[0], _ptr(y), _dt(y), ws_ptr, ws_bytes, _stream_handle(stream)),
           "paro_w4a16_moe_linear")


def paro_scale_rotate_backward_workspace_bytes(layer: DeviceLayer, tokens: int) -> int:
    """Workspace bytes of paro_scale_rotate_backward for this many tokens."""
    return int(load().paro_scale_rotate_backward_workspace_bytes(layer.ref, tokens))


def paro_scale_rotate_backward(layer: DeviceLayer, x, g, gx, gtheta, gcs, workspace, stream=None) -> None:
    """x: (tokens, I) fp16/bf16; g = dL/dx_r: (tokens, I) fp32 or x's dtype; gx: (tokens, I) fp32 or x's
    dtype; gtheta: fp32 (krot, I/2); gcs: fp32 (I,); workspace: device buffer of
    paro_scale_rotate_backward_workspace_bytes() bytes."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().paro_scale_rotate_backward(layer.ref, _ptr(x), _dt(x), _ptr(g), _dt(g), x.shape[0], _ptr(gx),
                                             _dt(gx), _ptr(gtheta), _ptr(gcs), _ptr(workspace), ws_bytes,
                                             _stream_handle(stream)), "paro_scale_rotate_backward")


def paro_rotation_matrix_bytes(layer: DeviceLayer) -> int:
    """Bytes of the dense rotation (H and L) that paro_rotation_matrix writes."""
    return int(load().paro_rotation_matrix_bytes(layer.ref))


def paro_rotation_matrix(layer: DeviceLayer, x_dt: int, hl, stream=None) -> None:
    """Build H + L = diag(cs) . R per group into hl (device buffer of paro_rotation_matrix_bytes())."""
    _check(load().paro_rotation_matrix(layer.ref, x_dt, _ptr(hl), _stream_handle(stream)),
           "paro_rotation_matrix")


def paro_scale_rotate_tiled(layer: DeviceLayer, hl, x, x_t, stream=None) -> None:
    """x: (tokens, I) fp16/bf16; hl: from paro_rotation_matrix for x's dtype;
    x_t: device buffer of paro_tiled_bytes() bytes (any dtype view)."""
    _check(load().paro_scale_rotate_tiled(layer.ref, _ptr(hl), _ptr(x), _dt(x), x.shape[0], _ptr(x_t),
                                          _stream_handle(stream)), "paro_scale_rotate_tiled")


def paro_w4a16_linear_tiled(layer: DeviceLayer, x_t, x_dt: int, tokens: int, y, stream=None) -> None:
    """The prefill contraction over X_r in the tiled layout; y: (tokens, O) x dtype or fp32."""
    _check(load().paro_w4a16_linear_tiled(layer.ref, _ptr(x_t), x_dt, tokens, _ptr(y), _dt(y),
                                          _stream_handle(stream)), "paro_w4a16_linear_tiled")
