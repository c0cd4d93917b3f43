"""rotation_int4_weight_amd: the rotated W4A16 linear of ParoQuant on MI355X.

    Y = (X . D^-1 . R) . Q(W_r)^T + b

computed by hand-written HIP kernels for gfx950 behind the C-ABI of
include/paro.h (libparo.so).  This package is the thin ctypes binding with the
same entry-point names; PyTorch supplies device memory and streams only.
"""
from ._lib import (BF16, EXPORTS, F16, F32, PATH_AUTO, PATH_DECODE_FUSED, PATH_DECODE_SPLIT,
                   PATH_PREFILL, DeviceLayer, ParoError, load, make_workspace,
                   paro_abi_version, paro_last_error, paro_scale_rotate,
                   paro_validate_layer, paro_w4_unpack_dequant, paro_w4a16_linear,
                   paro_w4a16_linear_choose_path, paro_w4a16_linear_prerotated,
                   paro_w4a16_linear_prepared, paro_w4a16_linear_prepared_workspace_bytes,
                   paro_w4a16_linear_prepared_multi, paro_w4a16_linear_prepared_multi_workspace_bytes,
                   paro_w4a16_linear_tiled_multi, paro_w4a16_linear_noalloc, paro_w4a16_linear_workspace_bytes, paro_tiled_bytes, paro_rotation_matrix_bytes,
                   paro_rotation_matrix, paro_scale_rotate_tiled, paro_w4a16_linear_tiled,
                   paro_w4_quantize_pack, paro_scale_rotate_backward,
                   paro_scale_rotate_backward_workspace_bytes, paro_w4a16_moe_linear,
                   paro_w4a16_moe_linear_workspace_bytes, paro_mxfp4_quantize_weight,
                   paro_mxfp4_quantize_activations, paro_mxfp4_gemm, paro_mxfp4_linear,
                   paro_mxfp4_linear_workspace_bytes, paro_mxfp4_activation_workspace_bytes,
                   paro_mxfp4_linear_prepared, paro_mxfp4_linear_prepared_workspace_bytes)

__all__ = ["BF16", "EXPORTS", "F16", "F32", "PATH_AUTO", "PATH_DECODE_FUSED", "PATH_DECODE_SPLIT",
           "PATH_PREFILL", "DeviceLayer", "ParoError", "load", "make_workspace", "paro_abi_version",
           "paro_last_error", "paro_scale_rotate", "paro_validate_layer", "paro_w4_unpack_dequant",
           "paro_w4a16_linear", "paro_w4a16_linear_choose_path", "paro_w4a16_linear_prerotated",
           "paro_w4a16_linear_prepared", "paro_w4a16_linear_prepared_workspace_bytes",
           "paro_w4a16_linear_prepared_multi", "paro_w4a16_linear_prepared_multi_workspace_bytes",
           "paro_w4a16_linear_tiled_multi", "paro_w4a16_linear_noalloc",
           "paro_w4a16_linear_workspace_bytes", "paro_tiled_bytes", "paro_rotation_matrix_bytes",
           "paro_rotation_matrix", "paro_scale_rotate_tiled", "paro_w4a16_linear_tiled",
           "paro_w4_quantize_pack", "paro_scale_rotate_backward",
           "paro_scale_rotate_backward_workspace_bytes", "paro_w4a16_moe_linear",
           "paro_w4a16_moe_linear_workspace_bytes", "paro_mxfp4_quantize_weight",
           "paro_mxfp4_quantize_activations", "paro_mxfp4_gemm", "paro_mxfp4_linear",
           "paro_mxfp4_linear_workspace_bytes", "paro_mxfp4_activation_workspace_bytes",
           "paro_mxfp4_linear_prepared", "paro_mxfp4_linear_prepared_workspace_bytes"]
