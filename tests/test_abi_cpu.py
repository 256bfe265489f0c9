"""The C-ABI library on the CPU (no GPU needed): it loads, exports every
function include/qg.h declares, reports its version and status strings, sizes
its workspace, and rejects bad arguments on the host before anything is
enqueued. Every call here fails validation, so none reaches the GPU."""
import os
import re

import pytest

import gemm_qgemv_amd as q
from gemm_qgemv_amd import _binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "qg.h")

A = 1 << 20   # fake, 16-byte aligned "device" addresses (never dereferenced)


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(q\w+)\s*\(", text, re.M)))


def test_header_declares_the_expected_entry_points():
    assert header_functions() == sorted(_binding.EXPORTS)


def test_library_exports_every_declared_function():
    lib = _binding.lib()
    for name in header_functions():
        assert hasattr(lib, name), name


def test_probe_library_exports_and_rejects_bad_arguments():
    """The measurement-only probe library loads and checks its arguments on
    the host (these calls fail validation, so nothing is launched)."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "gemm_qgemv_amd", "libqgprobe.so")
    if not os.path.exists(path):
        pytest.skip("libqgprobe.so not built")
    lib = ctypes.CDLL(path)
    for name in ("qg_probe_read", "qg_probe_read_blocked", "qg_probe_copy"):
        assert hasattr(lib, name), name
    lib.qg_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    assert lib.qg_probe_read(A, 1000, A, 256, None) == -1     # not a multiple of 16 bytes
    assert lib.qg_probe_read(None, 1024, A, 256, None) == -1
    assert lib.qg_probe_read(A, 1024, A, 0, None) == -1       # no grid


def test_version_and_status_strings():
    assert q.qg_abi_version() == 2
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert q.qg_status_str(st) and q.qg_status_str(st) != "unknown status"
    assert q.qg_status_str(12345) == "unknown status"


def test_workspace_sizes():
    # the greedy head needs at least the control words; plain GEMV at these
    # shapes needs no workspace
    assert q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, 151936, 2048, 1) >= \
        q.QG_WS_CONTROL_BYTES
    assert q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, 151936, 2048, 8) >= \
        q.QG_WS_CONTROL_BYTES
    assert q.qg_workspace_bytes(q.QG_OP_GEMV, q.QG_U4_G64, 6144, 2048, 1) == 0
    # invalid requests report 0 (the entry point reports the error)
    assert q.qg_workspace_bytes(q.QG_OP_GEMV, 9, 10, 64, 1) == 0
    assert q.qg_workspace_bytes(q.QG_OP_GEMV, q.QG_U4_G64, 10, 65, 1) == 0
    assert q.qg_workspace_bytes(q.QG_OP_GEMV, q.QG_U4_G64, 10, 64, 17) == 0
    assert q.qg_workspace_bytes(77, q.QG_U4_G64, 10, 64, 1) == 0


def test_prefill_split_tail_planning():
    """The host cuts the short last round of a prefill grid into pieces of K
    (their partial tiles need workspace) only where that round is at most a
    quarter full: the shapes of the exact split-tail GPU test take that
    path, the configurations whose last round is fuller do not."""
    tile_bytes = {q.QG_I8_ROW: 256 * 64 * 4, q.QG_U4_G64: 128 * 64 * 4, q.QG_B1_G128: 128 * 64 * 4,
                  q.QG_I8_G64: 128 * 64 * 4}
    for fmt, M, K, N in [(q.QG_I8_ROW, 1000, 272, 12800), (q.QG_U4_G64, 2100, 576, 2000),
                         (q.QG_B1_G128, 1100, 1152, 3900), (q.QG_I8_G64, 2100, 576, 2900),
                         (q.QG_B1_G128, 17408, 5120, 512),
                         (q.QG_U4_G64, 2101, 576, 2000), (q.QG_I8_G64, 2099, 576, 2900),
                         (q.QG_I8_ROW, 1001, 272, 12290)]:
        ws = q.qg_workspace_bytes(q.QG_OP_GEMM, fmt, M, K, N)
        # control words plus at least two pieces of one tile
        assert ws >= q.QG_WS_CONTROL_BYTES + 2 * tile_bytes[fmt], (fmt, M, K, N, ws)
    for fmt, M, K, N in [(q.QG_I8_ROW, 3584, 1024, 10240), (q.QG_I8_ROW, 1024, 3584, 10240),
                         (q.QG_U4_G64, 6144, 2048, 2048), (q.QG_I8_ROW, 3584, 1024, 2048),
                         (q.QG_I8_ROW, 2000, 272, 3100)]:
        assert q.qg_workspace_bytes(q.QG_OP_GEMM, fmt, M, K, N) == 0, (fmt, M, K, N)


def test_prefill_split_k_planning():
    """Grids too small for the chip are cut along K into as many pieces as
    the host planner chooses for the format (their float32 partials fill the
    workspace after the control words): two for the 8-bit per-row 1024 x
    3584 grid at 2048 token rows, three for the 8-bit group-64 one, four for
    the 1-bit 5120 x 17408 grid at 512 rows; grids that fill the chip in
    whole rounds are not cut."""
    for fmt, M, K, N, pieces in [(q.QG_I8_ROW, 1024, 3584, 2048, 2), (q.QG_I8_G64, 1024, 3584, 2048, 3),
                                 (q.QG_B1_G128, 5120, 17408, 512, 4)]:
        ws = q.qg_workspace_bytes(q.QG_OP_GEMM, fmt, M, K, N)
        assert ws == q.QG_WS_CONTROL_BYTES + pieces * N * M * 4, (fmt, M, K, N, ws)
    for fmt, M, K, N in [(q.QG_I8_ROW, 3584, 1024, 2048), (q.QG_I8_G64, 3584, 1024, 10240),
                         (q.QG_U4_G64, 2048, 6144, 2048)]:
        assert q.qg_workspace_bytes(q.QG_OP_GEMM, fmt, M, K, N) == 0, (fmt, M, K, N)


def _err(fn, *args, **kw):
    with pytest.raises(q.QGError) as e:
        fn(*args, stream=0, **kw)
    return e.value.status


def test_bad_format():
    assert _err(q.qgemv, 9, A, A + 4096, None, A + 8192, A + 16384, 4, 64, 1) == q.QG_ERR_FORMAT


def test_null_pointers():
    assert _err(q.qgemv, q.QG_I8_ROW, None, A, None, A, A, 4, 64, 1) == q.QG_ERR_NULL
    assert _err(q.qgemv, q.QG_I8_ROW, A, A, None, A, None, 4, 64, 1) == q.QG_ERR_NULL
    # biases are required for the affine format and forbidden for the others
    assert _err(q.qgemv, q.QG_U4_G64, A, A + 4096, None, A + 8192, A + 16384, 4, 64, 1) == q.QG_ERR_NULL
    assert _err(q.qgemv, q.QG_I8_ROW, A, A + 4096, A + 12288, A + 8192, A + 16384, 4, 64, 1) == q.QG_ERR_NULL
    assert _err(q.qgemv_argmax, q.QG_U4_G64, A, A + 4096, A + 12288, A + 8192, A + 16384, None,
                4, 64, 1) == q.QG_ERR_NULL


def test_bad_shapes():
    for fmt, K in ((q.QG_I8_ROW, 24), (q.QG_U4_G64, 96), (q.QG_B1_G128, 192), (q.QG_U4_G64, 0)):
        b = A + 12288 if fmt == q.QG_U4_G64 else None
        assert _err(q.qgemv, fmt, A, A + 4096, b, A + 8192, A + 65536, 4, K, 1) == q.QG_ERR_SHAPE
    assert _err(q.qgemv, q.QG_I8_ROW, A, A + 4096, None, A + 8192, A + 65536, 0, 64, 1) == q.QG_ERR_SHAPE
    assert _err(q.qgemv, q.QG_I8_ROW, A, A + 4096, None, A + 8192, A + 65536, 4, 64, 0) == q.QG_ERR_SHAPE
    assert _err(q.qgemv, q.QG_I8_ROW, A, A + 4096, None, A + 8192, A + 65536, 4, 64, 17) == q.QG_ERR_SHAPE
    assert _err(q.qgemm, q.QG_I8_ROW, A, A + 4096, None, A + 8192, A + 65536, 4, 64, 0) == q.QG_ERR_SHAPE


def test_misaligned_pointers():
    assert _err(q.qgemv, q.QG_I8_ROW, A + 4, A + 4096, None, A + 8192, A + 65536, 4, 64, 1) == q.QG_ERR_ALIGN
    assert _err(q.qgemv, q.QG_I8_ROW, A, A + 4096, None, A + 8200, A + 65536, 4, 64, 1) == q.QG_ERR_ALIGN
    assert _err(q.qgemv, q.QG_I8_ROW, A, A + 4096, None, A + 8192, A + 65544, 4, 64, 1) == q.QG_ERR_ALIGN
    assert _err(q.qgemv_argmax, q.QG_I8_ROW, A, A + 4096, None, A + 8192, A + 65536, A + 90002,
                4, 64, 1, ws=A + 131072, ws_bytes=1 << 20) == q.QG_ERR_ALIGN


def test_workspace_too_small():
    M, K = 151936, 2048
    need = q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, M, K, 1)
    codes, scales, biases = A, A + (1 << 28), A + (1 << 29)
    x, y, idx, ws = A + (1 << 30), A + (1 << 31), A + (1 << 32), A + (1 << 33)
    assert _err(q.qgemv_argmax, q.QG_U4_G64, codes, scales, biases, x, y, idx, M, K, 1,
                ws=ws, ws_bytes=need - 1) == q.QG_ERR_WORKSPACE
    assert _err(q.qgemv_argmax, q.QG_U4_G64, codes, scales, biases, x, y, idx, M, K, 1,
                ws=None, ws_bytes=0) == q.QG_ERR_WORKSPACE


def test_aliasing_outputs():
    # y overlapping x, y overlapping the codes, idx inside y
    assert _err(q.qgemv, q.QG_I8_ROW, A, A + 4096, None, A + 8192, A + 8192, 4, 64, 1) == q.QG_ERR_ALIAS
    assert _err(q.qgemv, q.QG_I8_ROW, A, A + 4096, None, A + 8192, A + 128, 4, 64, 1) == q.QG_ERR_ALIAS
    M, K = 4096, 64
    need = q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_I8_ROW, M, K, 1)
    base = 1 << 30
    assert _err(q.qgemv_argmax, q.QG_I8_ROW, A, base, None, base + 65536, base + 131072,
                base + 131072 + 64, M, K, 1, ws=base + (1 << 24), ws_bytes=need) == q.QG_ERR_ALIAS


def test_exact_alias_is_rejected():
    """A written buffer that coincides exactly with an input (same start,
    same length) is an overlap like any other: y == x with M == K, and the
    gather's output on top of its codes."""
    M = K = 64
    codes, scales, x = A, A + 65536, A + 131072
    # 8-bit per-row: y == x (M * 4 bytes == K * 4 bytes)
    assert _err(q.qgemv, q.QG_I8_ROW, codes, scales, None, x, x, M, K, 1) == q.QG_ERR_ALIAS
    assert _err(q.qgemm, q.QG_I8_ROW, codes, scales, None, x, x, M, K, 20, ws=A + (1 << 24),
                ws_bytes=1 << 22) == q.QG_ERR_ALIAS
    need = q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_I8_ROW, M, K, 1)
    ws = A + (1 << 24)
    assert _err(q.qgemv_argmax, q.QG_I8_ROW, codes, scales, None, x, x, A + (1 << 23), M, K, 1,
                ws=ws, ws_bytes=need) == q.QG_ERR_ALIAS
    # idx exactly on top of x (batch * 4 bytes == K * 4 bytes needs batch == K: use K = 16)
    need16 = q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_I8_ROW, 4, 16, 16)
    assert _err(q.qgemv_argmax, q.QG_I8_ROW, codes, scales, None, x, A + (1 << 22), x, 4, 16, 1,
                ws=ws, ws_bytes=need16) == q.QG_ERR_ALIAS
    # y exactly on top of the codes: 8-bit codes of 16 x 64 bytes, y of 16 x 64 floats
    # needs batch * M * 4 == M * K: M = 16, K = 64, batch = 16
    assert _err(q.qgemv, q.QG_I8_ROW, codes, scales, None, x, codes, 16, 64, 16,
                ws=ws, ws_bytes=1 << 20) == q.QG_ERR_ALIAS
    # the gather writing over its own codes: n * K * 4 == M * K / 2 for M = 8 n
    M2, K2, n = 64, 128, 8
    with pytest.raises(q.QGError) as e:
        q.qembed(q.QG_U4_G64, codes, A + (1 << 21), A + (1 << 22), A + (1 << 23), codes,
                 M2, K2, n, stream=0)
    assert e.value.status == q.QG_ERR_ALIAS


def test_noalloc_greedy_checks():
    """qgemv_argmax_noalloc: argument errors as qgemv_argmax (reported
    before the library's scratch is touched), and calls that need more than
    QG_STATIC_SCRATCH_BYTES of scratch rejected with QG_ERR_SCRATCH."""
    codes, scales, biases = A, A + (1 << 28), A + (1 << 29)
    x, y, idx = A + (1 << 30), A + (1 << 31), A + (1 << 32)

    def err(*a):
        with pytest.raises(q.QGError) as e:
            q.qgemv_argmax_noalloc(*a, stream=0)
        return e.value.status

    assert err(9, codes, scales, None, x, y, idx, 64, 64, 1) == q.QG_ERR_FORMAT
    assert err(q.QG_U4_G64, codes, scales, None, x, y, idx, 64, 64, 1) == q.QG_ERR_NULL
    assert err(q.QG_U4_G64, codes, scales, biases, x, y, None, 64, 64, 1) == q.QG_ERR_NULL
    assert err(q.QG_U4_G64, codes, scales, biases, x, y, idx, 64, 96, 1) == q.QG_ERR_SHAPE
    assert err(q.QG_U4_G64, codes, scales, biases, x, y, idx, 64, 64, 0) == q.QG_ERR_SHAPE
    M, K, n = 10_000_000, 64, 256
    assert q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, M, K, n) > q.QG_STATIC_SCRATCH_BYTES
    assert err(q.QG_U4_G64, codes, scales, biases, x, y, idx, M, K, n) == q.QG_ERR_SCRATCH
    assert "QG_STATIC_SCRATCH_BYTES" in q.qg_status_str(q.QG_ERR_SCRATCH)
    hdr = open(HEADER).read()
    assert "#define QG_STATIC_SCRATCH_BYTES (8u << 20)" in hdr
    assert q.QG_STATIC_SCRATCH_BYTES == 8 << 20
    # the configurations' greedy heads fit
    for rows in (1, 8, 16, 64, 128, 256):
        assert q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, 151936, 2048, rows) <= \
            q.QG_STATIC_SCRATCH_BYTES


def test_prefill_affine_format_checks():
    # the 4-bit prefill needs its biases, and its biases must not overlap Y
    assert _err(q.qgemm, q.QG_U4_G64, A, A + 4096, None, A + 8192, A + 65536, 4, 64, 8) == \
        q.QG_ERR_NULL
    assert _err(q.qgemm, q.QG_U4_G64, A, A + 4096, A + 65536, A + 8192, A + 65536, 4, 64, 8,
                ws=A + (1 << 24), ws_bytes=1 << 22) == q.QG_ERR_ALIAS


def test_wide_greedy_head_checks():
    """More than QG_MAX_GEMV_BATCH rows of the greedy head: tile keys in the
    workspace (after the control words), at most QG_MAX_ARGMAX_BATCH rows;
    logits may be NULL there as for small batches, but plain qgemv needs y."""
    hdr = open(HEADER).read()
    assert f"#define QG_MAX_ARGMAX_BATCH {q.QG_MAX_ARGMAX_BATCH}" in hdr
    M, K = 151936, 2048
    for n in (64, 128, q.QG_MAX_ARGMAX_BATCH):
        need = q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, M, K, n)
        assert need >= q.QG_WS_CONTROL_BYTES + n * (M // 128) * 8   # one key per 128-row tile
    # 17..48 rows of this 4-bit head run as launches of up to 16 rows of the
    # matrix-vector kernels: control words plus 16 keys per workgroup
    for n in (17, 33, 48):
        need = q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, M, K, n)
        assert need >= q.QG_WS_CONTROL_BYTES + 16 * 8
    assert q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, M, K,
                                q.QG_MAX_ARGMAX_BATCH + 1) == 0
    codes, scales, biases = A, A + (1 << 28), A + (1 << 29)
    x, idx, ws = A + (1 << 30), A + (1 << 32), A + (1 << 33)
    for n in (17, 64):
        need = q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, M, K, n)
        assert _err(q.qgemv_argmax, q.QG_U4_G64, codes, scales, biases, x, None, idx, M, K, n,
                    ws=ws, ws_bytes=need - 1) == q.QG_ERR_WORKSPACE
    need = q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, M, K, 64)
    assert _err(q.qgemv_argmax, q.QG_U4_G64, codes, scales, biases, x, None, idx, M, K,
                q.QG_MAX_ARGMAX_BATCH + 1, ws=ws, ws_bytes=1 << 30) == q.QG_ERR_SHAPE
    # idx inside the keys area of the workspace
    assert _err(q.qgemv_argmax, q.QG_U4_G64, codes, scales, biases, x, None, ws + 8192, M, K, 64,
                ws=ws, ws_bytes=need) == q.QG_ERR_ALIAS
    # qgemv without an output
    assert _err(q.qgemv, q.QG_U4_G64, codes, scales, biases, x, None, M, K, 1) == q.QG_ERR_NULL


def test_embed_checks():
    """qembed: 4-bit rows only (the other known formats are not implemented
    for the gather), ids and out required, out 16-byte and ids 4-byte
    aligned, out overlapping nothing."""
    M, K, n = 1000, 128, 8
    codes, scales, biases = A, A + (1 << 20), A + (1 << 21)
    ids, out = A + (1 << 22), A + (1 << 23)
    ok = dict(fmt=q.QG_U4_G64, codes=codes, scales=scales, biases=biases, ids=ids, out=out,
              M=M, K=K, n=n)

    def err(**kw):
        a = dict(ok, **kw)
        with pytest.raises(q.QGError) as e:
            q.qembed(a["fmt"], a["codes"], a["scales"], a["biases"], a["ids"], a["out"],
                     a["M"], a["K"], a["n"], stream=0)
        return e.value.status

    assert err(fmt=9) == q.QG_ERR_FORMAT
    assert err(fmt=q.QG_I8_ROW, biases=None) == q.QG_ERR_UNSUPPORTED
    assert err(fmt=q.QG_B1_G128, biases=None) == q.QG_ERR_UNSUPPORTED
    assert err(fmt=q.QG_I8_ROW) == q.QG_ERR_NULL            # biases where none belong
    assert err(biases=None) == q.QG_ERR_NULL
    assert err(ids=None) == q.QG_ERR_NULL
    assert err(out=None) == q.QG_ERR_NULL
    assert err(codes=None) == q.QG_ERR_NULL
    assert err(K=96) == q.QG_ERR_SHAPE
    assert err(K=0) == q.QG_ERR_SHAPE
    assert err(M=0) == q.QG_ERR_SHAPE
    assert err(n=0) == q.QG_ERR_SHAPE
    assert err(n=-3) == q.QG_ERR_SHAPE
    assert err(out=out + 4) == q.QG_ERR_ALIGN
    assert err(ids=ids + 2) == q.QG_ERR_ALIGN
    assert err(scales=scales + 8) == q.QG_ERR_ALIGN
    assert err(out=codes + 4096) == q.QG_ERR_ALIAS          # inside the codes
    assert err(out=ids - 16) == q.QG_ERR_ALIAS              # covers the ids
    assert err(ids=out + 64) == q.QG_ERR_ALIAS              # ids inside out
    assert "format" in q.qg_status_str(q.QG_ERR_UNSUPPORTED)


def test_i8_group64_format_checks():
    """8-bit weights with a float32 scale per 64 inputs: K a multiple of 64,
    no biases; the workspace rules are those of the other formats."""
    assert _err(q.qgemv, q.QG_I8_G64, A, A + 4096, None, A + 8192, A + 65536, 4, 48, 1) == \
        q.QG_ERR_SHAPE
    assert _err(q.qgemv, q.QG_I8_G64, A, A + 4096, A + 12288, A + 8192, A + 65536, 4, 64, 1) == \
        q.QG_ERR_NULL
    assert _err(q.qgemm, q.QG_I8_G64, A, A + 4096, None, A + 8192, A + 65536, 4, 96, 32) == \
        q.QG_ERR_SHAPE
    # y overlapping the scales ([M][K/64] floats = 4 * 2 * 4 bytes here)
    assert _err(q.qgemv, q.QG_I8_G64, A, A + 4096, None, A + 8192, A + 4096, 4, 128, 1) == \
        q.QG_ERR_ALIAS
    assert q.qg_workspace_bytes(q.QG_OP_GEMV, q.QG_I8_G64, 10, 96, 1) == 0
    assert q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_I8_G64, 3584, 1024, 1) >= \
        q.QG_WS_CONTROL_BYTES
    assert q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_I8_G64, 3584, 1024, 64) >= \
        q.QG_WS_CONTROL_BYTES + 64 * (3584 // 64) * 8


def test_prefill_k_limit():
    """Above 16 token rows the matrix-core kernels take K up to 2^21 (their
    buffer loads use 32-bit offsets within a tile); the matrix-vector path
    below that keeps the full range."""
    K = (1 << 21) + 64
    assert _err(q.qgemm, q.QG_U4_G64, A, A + (1 << 32), A + (1 << 33), A + (1 << 34),
                A + (1 << 36), 4, K, 17) == q.QG_ERR_SHAPE
    assert q.qg_workspace_bytes(q.QG_OP_GEMM, q.QG_U4_G64, 4, K, 17) == 0
    assert q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, q.QG_U4_G64, 4, K, 64) == 0
    assert _err(q.qgemv_argmax, q.QG_U4_G64, A, A + (1 << 32), A + (1 << 33), A + (1 << 34),
                None, A + (1 << 36), 4, K, 64, ws=A + (1 << 37), ws_bytes=1 << 20) == q.QG_ERR_SHAPE
