"""libmxq: float8 quantization kernels for MoE token and expert buffers on MI355X.

The kernels are hand-written HIP for gfx950, exported through the C ABI of
include/mxq.h; ``mxq`` is the thin ctypes binding with the same names.
"""
from .mxq import (  # noqa: F401
    EXPORTED, LIB_PATH, MXQ_LAYOUT_COL, MXQ_LAYOUT_ROW, MxqError, dequantize_mx, group_scale_fp8, lib,
    mxq_abi_version, mxq_dequantize_mx, mxq_group_scale_fp8, mxq_group_scale_workspace_bytes,
    mxq_quantize_mx, mxq_transpose_u8, quantize_mx, transpose_u8,
)
