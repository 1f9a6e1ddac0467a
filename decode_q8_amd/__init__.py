"""decode_q8_amd: the Q8_0 block-quantized matmul on MI355X (gfx950).

The computation lives in libq8.so (HIP kernels + a C ABI, include/q8.h);
``decode_q8_amd.q8`` is its ctypes binding.
"""
from .q8 import (  # noqa: F401
    Q8_BLOCK,
    Q8_BLOCK_BYTES,
    Q8_ERR_ALIGN,
    Q8_ERR_ARG,
    Q8_ERR_DEVICE,
    Q8_ERR_LAUNCH,
    Q8_ERR_SHAPE,
    Q8_ERR_WORKSPACE,
    Q8_GEMV_MAX_ROWS,
    Q8_LAYOUT_ACT,
    Q8_LAYOUT_PACKED,
    Q8_LAYOUT_ROWS,
    Q8_OK,
    Q8Error,
    lib,
    matmul,
    q8_abi_version,
    q8_grouped_matmul,
    q8_grouped_workspace_bytes,
    q8_matmul,
    q8_matmul_workspace_bytes,
    q8_quantize_matmul,
    q8_quantize_rows,
    q8_quantized_bytes,
    q8_repack_weights,
    q8_rmsnorm_quantize,
    q8_status_str,
    quantize,
    quantize_matmul,
    repack,
    rmsnorm_quantize,
    workspace,
)
