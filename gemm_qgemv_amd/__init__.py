"""Dequantize-fused low-bit matrix-vector / matrix-matrix products, a fused
greedy (argmax) head and the embedding-row gather for AMD MI355X (gfx950).

The computation lives in ``libqg.so`` (HIP kernels behind the C ABI of
``include/qg.h``); this package is its thin ctypes binding, plus the seeded
synthetic-input generator (``gemm_qgemv_amd.synth``) and device-buffer helpers
(``gemm_qgemv_amd.tensors``).
"""
from ._binding import (QG_B1_G128, QG_ERR_ALIAS, QG_ERR_ALIGN, QG_ERR_FORMAT,  # noqa: F401
                       QG_ERR_LAUNCH, QG_ERR_NULL, QG_ERR_SCRATCH, QG_ERR_SHAPE, QG_ERR_UNSUPPORTED,
                       QG_ERR_WORKSPACE, QG_I8_G64, QG_I8_ROW, QG_MAX_ARGMAX_BATCH, QG_MAX_GEMV_BATCH, QG_OK, QG_OP_GEMM,
                       QG_OP_GEMV, QG_OP_GEMV_ARGMAX, QG_STATIC_SCRATCH_BYTES, QG_U4_G64, QG_WS_CONTROL_BYTES,
                       QGError, qg_abi_version, qg_status_str, qg_workspace_bytes, qembed, qgemm,
                       qgemv, qgemv_argmax, qgemv_argmax_noalloc)
