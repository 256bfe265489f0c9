"""ctypes binding of libqg (include/qg.h): the same entry points, the same
argument order. It only marshals arguments; every step of the computation
runs in the library's HIP kernels.

Buffers may be passed as torch tensors (their device pointer is used) or as
integer device addresses. ``stream=None`` means torch's current stream.
Non-zero status codes raise ``QGError``.
"""
from __future__ import annotations

import ctypes
import os

QG_I8_ROW, QG_U4_G64, QG_B1_G128, QG_I8_G64 = 1, 2, 3, 4
QG_OP_GEMV, QG_OP_GEMM, QG_OP_GEMV_ARGMAX = 1, 2, 3
QG_OK = 0
QG_ERR_NULL, QG_ERR_FORMAT, QG_ERR_SHAPE, QG_ERR_ALIGN = -1, -2, -3, -4
QG_ERR_WORKSPACE, QG_ERR_ALIAS, QG_ERR_LAUNCH, QG_ERR_UNSUPPORTED = -5, -6, -7, -8
QG_ERR_SCRATCH = -9
QG_STATIC_SCRATCH_BYTES = 8 << 20
QG_MAX_GEMV_BATCH = 16
QG_MAX_ARGMAX_BATCH = 256
QG_WS_CONTROL_BYTES = 8192

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqg.so")

EXPORTS = ("qgemv", "qgemm", "qgemv_argmax", "qgemv_argmax_noalloc", "qembed",
           "qg_workspace_bytes", "qg_status_str", "qg_abi_version")

_lib = None


class QGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built: there is no
    other implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m gemm_qgemv_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.qgemv.argtypes = [I32, P, P, P, P, P, I64, I64, I32, P, SZ, P]
        L.qgemm.argtypes = [I32, P, P, P, P, P, I64, I64, I64, P, SZ, P]
        L.qgemv_argmax.argtypes = [I32, P, P, P, P, P, P, I64, I64, I32, P, SZ, P]
        L.qgemv_argmax_noalloc.argtypes = [I32, P, P, P, P, P, P, I64, I64, I32, P]
        L.qembed.argtypes = [I32, P, P, P, P, P, I64, I64, I64, P]
        L.qg_workspace_bytes.argtypes = [I32, I32, I64, I64, I64]
        L.qg_workspace_bytes.restype = SZ
        L.qg_status_str.argtypes = [I32]
        L.qg_status_str.restype = ctypes.c_char_p
        L.qg_abi_version.argtypes = []
        for f in (L.qgemv, L.qgemm, L.qgemv_argmax, L.qgemv_argmax_noalloc, L.qembed,
                  L.qg_abi_version):
            f.restype = I32
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(ws, ws_bytes):
    if ws_bytes is not None:
        return int(ws_bytes)
    if ws is None or isinstance(ws, int):
        return 0
    return ws.numel() * ws.element_size()


def _check(status, where):
    if status != QG_OK:
        raise QGError(status, where)


def qgemv(fmt, codes, scales, biases, x, y, M, K, batch, ws=None, ws_bytes=None, stream=None):
    _check(lib().qgemv(fmt, _ptr(codes), _ptr(scales), _ptr(biases), _ptr(x), _ptr(y),
                       M, K, batch, _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream)), "qgemv")


def qgemm(fmt, codes, scales, biases, x, y, M, K, N, ws=None, ws_bytes=None, stream=None):
    _check(lib().qgemm(fmt, _ptr(codes), _ptr(scales), _ptr(biases), _ptr(x), _ptr(y),
                       M, K, N, _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream)), "qgemm")


def qgemv_argmax(fmt, codes, scales, biases, x, logits, idx, M, K, batch, ws=None,
                 ws_bytes=None, stream=None):
    _check(lib().qgemv_argmax(fmt, _ptr(codes), _ptr(scales), _ptr(biases), _ptr(x),
                              _ptr(logits), _ptr(idx), M, K, batch, _ptr(ws),
                              _nbytes(ws, ws_bytes), _stream(stream)), "qgemv_argmax")


def qgemv_argmax_noalloc(fmt, codes, scales, biases, x, logits, idx, M, K, batch, stream=None):
    _check(lib().qgemv_argmax_noalloc(fmt, _ptr(codes), _ptr(scales), _ptr(biases), _ptr(x),
                                      _ptr(logits), _ptr(idx), M, K, batch, _stream(stream)),
           "qgemv_argmax_noalloc")


def qembed(fmt, codes, scales, biases, ids, out, M, K, n, stream=None):
    _check(lib().qembed(fmt, _ptr(codes), _ptr(scales), _ptr(biases), _ptr(ids), _ptr(out),
                        M, K, n, _stream(stream)), "qembed")


def qg_workspace_bytes(op, fmt, M, K, rows) -> int:
    return int(lib().qg_workspace_bytes(op, fmt, M, K, rows))


def qg_status_str(status) -> str:
    return lib().qg_status_str(status).decode()


def status_str(status) -> str:
    try:
        return qg_status_str(status)
    except Exception:  # library missing: still name the code
        return f"status {status}"


def qg_abi_version() -> int:
    return int(lib().qg_abi_version())
