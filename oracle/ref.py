"""ctypes binding of the fp64 CPU oracle (oracle/paro_ref.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg call this; the product package never imports it.  Argument
marshalling only -- every number is computed by the C oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libparo_ref.so")
SRC_PATH = os.path.join(HERE, "paro_ref.c")

F16, BF16, F32, F64 = 0, 1, 2, 3
OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_PAIRS, ERR_CHECK_FAILED, ERR_NOMEM = range(7)


def build(out_path: str = LIB_PATH, src_path: str = SRC_PATH, extra=(), openmp: bool = True) -> str:
    """Compile the oracle with gcc (plain C99, threaded with OpenMP unless
    openmp is False)."""
    cmd = ["gcc", "-std=gnu99", "-O2", *(["-fopenmp"] if openmp else []), "-fPIC", "-shared", "-Wall",
           "-I", os.path.join(ROOT, "include"), src_path, "-o", out_path, "-lm", *extra]
    subprocess.run(cmd, check=True)
    return out_path


class RefLayer(ctypes.Structure):
    _fields_ = [("in_features", ctypes.c_int64), ("out_features", ctypes.c_int64),
                ("group_size", ctypes.c_int32), ("krot", ctypes.c_int32),
                ("pairs", ctypes.c_void_p), ("theta", ctypes.c_void_p),
                ("channel_scales", ctypes.c_void_p), ("qweight", ctypes.c_void_p),
                ("qzeros", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("bias", ctypes.c_void_p)]


_lib = None
_lib_path = None


def load(path: str | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib, _lib_path
    path = path or os.environ.get("PARO_REF_LIB") or LIB_PATH
    if _lib is not None and _lib_path == path:
        return _lib
    if path == LIB_PATH and (not os.path.exists(path) or
                             os.path.getmtime(path) < max(os.path.getmtime(SRC_PATH), os.path.getmtime(
                                 os.path.join(ROOT, "include", "paro_ref.h")))):
        build(path)
    lib = ctypes.CDLL(path)
    P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.paro_ref_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.paro_ref_f16_to_double.restype = D
    lib.paro_ref_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.paro_ref_bf16_to_double.restype = D
    lib.paro_ref_round_f16.argtypes = [D]
    lib.paro_ref_round_f16.restype = ctypes.c_uint16
    lib.paro_ref_round_bf16.argtypes = [D]
    lib.paro_ref_round_bf16.restype = ctypes.c_uint16
    lib.paro_ref_round_array.argtypes = [P, I64, I32, P]
    lib.paro_ref_check_pairs.argtypes = [P]
    lib.paro_ref_scale_rotate.argtypes = [P, P, I32, I64, P, I32]
    lib.paro_ref_unpack.argtypes = [P, P, P]
    lib.paro_ref_dequant.argtypes = [P, P, I32]
    lib.paro_ref_linear.argtypes = [P, P, I32, I64, P, I32]
    lib.paro_linear_ref_check.argtypes = [P, P, I32, I64, P, I32, P, D, I32, P, P]
    lib.paro_ref_threads.argtypes = [I32]
    lib.paro_ref_transform_weight.argtypes = [P, P, I32, P, I32]
    lib.paro_ref_scale_rotate_backward.argtypes = [P, P, I32, P, I64, P, P, P, I32]
    lib.paro_ref_mxfp4_quantize.argtypes = [I64, I64, P, P, P]
    lib.paro_ref_mxfp4_dequant.argtypes = [I64, I64, P, P, P]
    lib.paro_ref_e2m1_to_double.argtypes = [I32]
    lib.paro_ref_e2m1_to_double.restype = ctypes.c_double
    lib.paro_ref_quantize.argtypes = [I64, I64, ctypes.c_int32, P, I32, P, P, P, P]
    lib.paro_ref_pack.argtypes = [I64, I64, ctypes.c_int32, P, P, P, P]
    for name in ("paro_ref_round_array", "paro_ref_check_pairs", "paro_ref_scale_rotate",
                 "paro_ref_unpack", "paro_ref_dequant", "paro_ref_linear",
                 "paro_linear_ref_check", "paro_ref_threads", "paro_ref_transform_weight",
                 "paro_ref_quantize", "paro_ref_pack", "paro_ref_scale_rotate_backward",
                 "paro_ref_mxfp4_quantize", "paro_ref_mxfp4_dequant"):
        getattr(lib, name).restype = I32
    _lib, _lib_path = lib, path
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def ref_layer(layer):
    """RefLayer struct for a synth.Layer-like object (arrays stay owned by it)."""
    for name in ("pairs", "theta", "channel_scales", "qweight", "qzeros", "scales", "bias"):
        a = getattr(layer, name)
        if a is not None and not a.flags["C_CONTIGUOUS"]:
            raise ValueError(f"{name} must be C-contiguous")
    return RefLayer(layer.in_features, layer.out_features, layer.group_size, layer.krot,
                    _ptr(layer.pairs), _ptr(layer.theta), _ptr(layer.channel_scales),
                    _ptr(layer.qweight), _ptr(layer.qzeros), _ptr(layer.scales),
                    _ptr(layer.bias))


def _group(layer):
    return layer.in_features if layer.group_size == -1 else layer.group_size


def _check(rc, what):
    if rc != OK:
        raise RuntimeError(f"{what} failed with oracle status {rc}")


def threads(n_threads: int = 0) -> int:
    return load().paro_ref_threads(n_threads)


def f16_to_double(h) -> float:
    return load().paro_ref_f16_to_double(int(h))


def bf16_to_double(h) -> float:
    return load().paro_ref_bf16_to_double(int(h))


def round_array(v, dt: int) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _check(load().paro_ref_round_array(_ptr(v), v.size, dt, _ptr(out)), "round_array")
    return out


def check_pairs(layer) -> int:
    return load().paro_ref_check_pairs(ctypes.byref(ref_layer(layer)))


def scale_rotate(layer, x, x_dt: int, n_threads: int = 0) -> np.ndarray:
    x = np.ascontiguousarray(x)
    tokens = x.shape[0]
    out = np.empty((tokens, layer.in_features), dtype=np.float64)
    _check(load().paro_ref_scale_rotate(ctypes.byref(ref_layer(layer)), _ptr(x), x_dt,
                                        tokens, _ptr(out), n_threads), "scale_rotate")
    return out


def unpack(layer):
    I, O = layer.in_features, layer.out_features
    q = np.empty((I, O), dtype=np.uint8)
    z = np.empty((I // _group(layer), O), dtype=np.uint8)
    _check(load().paro_ref_unpack(ctypes.byref(ref_layer(layer)), _ptr(q), _ptr(z)), "unpack")
    return q, z


def dequant(layer, n_threads: int = 0) -> np.ndarray:
    w = np.empty((layer.in_features, layer.out_features), dtype=np.float64)
    _check(load().paro_ref_dequant(ctypes.byref(ref_layer(layer)), _ptr(w), n_threads), "dequant")
    return w


def linear(layer, x, x_dt: int, n_threads: int = 0) -> np.ndarray:
    x = np.ascontiguousarray(x)
    y = np.empty((x.shape[0], layer.out_features), dtype=np.float64)
    _check(load().paro_ref_linear(ctypes.byref(ref_layer(layer)), _ptr(x), x_dt, x.shape[0],
                                  _ptr(y), n_threads), "linear")
    return y


def paro_linear_ref_check(layer, x, x_dt: int, y=None, y_dt: int = F32,
                          rel_tol: float = 5e-3, n_threads: int = 0, want_ref: bool = False):
    """Run the oracle's check.  Returns (status, max_abs_err, max_abs_ref, y_ref|None)."""
    x = np.ascontiguousarray(x)
    tokens = x.shape[0]
    yref = np.empty((tokens, layer.out_features), dtype=np.float64) if want_ref else None
    if y is not None:
        y = np.ascontiguousarray(y)
    err, ref = ctypes.c_double(0.0), ctypes.c_double(0.0)
    rc = load().paro_linear_ref_check(ctypes.byref(ref_layer(layer)), _ptr(x), x_dt, tokens,
                                      _ptr(y), y_dt, _ptr(yref), rel_tol, n_threads,
                                      ctypes.byref(err), ctypes.byref(ref))
    return rc, err.value, ref.value, yref


def transform_weight(layer, w, w_dt: int, n_threads: int = 0) -> np.ndarray:
    """W_r = W . D . R as double [O][I] (w: [O][I] bits of w_dt, or float64 for F64)."""
    O, I = layer.out_features, layer.in_features
    w = np.ascontiguousarray(w)
    assert w.shape == (O, I)
    out = np.empty((O, I), dtype=np.float64)
    L = ref_layer(layer)
    _check(load().paro_ref_transform_weight(ctypes.byref(L), _ptr(w), w_dt, _ptr(out), n_threads),
           "paro_ref_transform_weight")
    return out


def quantize(w_r, group_size: int, sym: bool):
    """Group RTN of w_r [O][I]: (q [I][O] uint8, z [I/G][O] uint8, s16 [I/G][O] uint16, scale [I/G][O])."""
    w_r = np.ascontiguousarray(w_r, dtype=np.float64)
    O, I = w_r.shape
    G = I if group_size == -1 else group_size
    q = np.empty((I, O), dtype=np.uint8)
    z = np.empty((I // G, O), dtype=np.uint8)
    s16 = np.empty((I // G, O), dtype=np.uint16)
    scale = np.empty((I // G, O), dtype=np.float64)
    _check(load().paro_ref_quantize(O, I, group_size, _ptr(w_r), int(bool(sym)), _ptr(q), _ptr(z), _ptr(s16),
                                    _ptr(scale)), "paro_ref_quantize")
    return q, z, s16, scale


def pack(q, z, group_size: int):
    """AWQ pack of q [I][O], z [I/G][O] -> (qweight int32 [I][O/8], qzeros int32 [I/G][O/8])."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    z = np.ascontiguousarray(z, dtype=np.uint8)
    I, O = q.shape
    G = I if group_size == -1 else group_size
    qw = np.empty((I, O // 8), dtype=np.int32)
    qz = np.empty((I // G, O // 8), dtype=np.int32)
    _check(load().paro_ref_pack(I, O, group_size, _ptr(q), _ptr(z), _ptr(qw), _ptr(qz)), "paro_ref_pack")
    return qw, qz


def mxfp4_quantize(v):
    """MXFP4 codes [rows][K/2] (uint8) and E8M0 scales [rows][K/32] of double v [rows][K]."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    rows, K = v.shape
    codes = np.empty((rows, K // 2), dtype=np.uint8)
    scales = np.empty((rows, K // 32), dtype=np.uint8)
    _check(load().paro_ref_mxfp4_quantize(rows, K, _ptr(v), _ptr(codes), _ptr(scales)), "paro_ref_mxfp4_quantize")
    return codes, scales


def mxfp4_dequant(codes, scales):
    """double [rows][K] from MXFP4 codes and scales."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, K = codes.shape[0], codes.shape[1] * 2
    out = np.empty((rows, K), dtype=np.float64)
    _check(load().paro_ref_mxfp4_dequant(rows, K, _ptr(codes), _ptr(scales), _ptr(out)), "paro_ref_mxfp4_dequant")
    return out


def mxfp4_weight(layer, w, w_dt: int):
    """MXFP4 codes and scales of the transformed weight W_r = W D R ([O][I] rows)."""
    return mxfp4_quantize(transform_weight(layer, w, w_dt))


def mxfp4_activations(layer, x, x_dt: int):
    """MXFP4 codes and scales of the rotated activations X_r = X D^-1 R."""
    return mxfp4_quantize(scale_rotate(layer, x, x_dt))


def mxfp4_matmul(a_codes, a_scales, w_codes, w_scales, bias=None):
    """Y = dequant(A) . dequant(W)^T (+ fp16 bias), double [rows][O]."""
    y = mxfp4_dequant(a_codes, a_scales) @ mxfp4_dequant(w_codes, w_scales).T
    if bias is not None:
        y = y + np.asarray([f16_to_double(h) for h in bias])
    return y


def expert_layer(layer, e: int):
    """Expert e of a stacked mixture-of-experts layer as an ordinary layer
    (the shared rotation and expert e's quantized weights and bias)."""
    import dataclasses
    return dataclasses.replace(layer, qweight=np.ascontiguousarray(layer.qweight[e]),
                               qzeros=np.ascontiguousarray(layer.qzeros[e]),
                               scales=np.ascontiguousarray(layer.scales[e]),
                               bias=None if layer.bias is None else np.ascontiguousarray(layer.bias[e]))


def moe_linear(layer, offsets, x, x_dt: int):
    """Mixture-of-experts projection with one shared rotation ("ParoQuant" blog
    on the MLX port, technical notes: stacked expert weights, rotations shared
    between experts): rows offsets[e] .. offsets[e+1]-1 of x go through
    expert e's linear, y double [rows][O].  Rows outside every range stay 0."""
    offsets = np.asarray(offsets, dtype=np.int64)
    y = np.zeros((x.shape[0], layer.out_features), dtype=np.float64)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y[lo:hi] = linear(expert_layer(layer, e), np.ascontiguousarray(x[lo:hi]), x_dt)
    return y


def scale_rotate_backward(layer, x, x_dt: int, g, n_threads: int = 0):
    """(gx [M][I], gtheta [krot][I/2], gcs [I]) for dL/dx_r = g (double [M][I])."""
    x = np.ascontiguousarray(x)
    g = np.ascontiguousarray(g, dtype=np.float64)
    M, I = g.shape
    gx = np.empty((M, I), dtype=np.float64)
    gth = np.empty((layer.krot, I // 2), dtype=np.float64)
    gcs = np.empty(I, dtype=np.float64)
    L = ref_layer(layer)
    _check(load().paro_ref_scale_rotate_backward(ctypes.byref(L), _ptr(x), x_dt, _ptr(g), M, _ptr(gx), _ptr(gth),
                                                 _ptr(gcs), n_threads), "paro_ref_scale_rotate_backward")
    return gx, gth, gcs
