"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: every output finite and within 1e-5 * sum_k |w[m][k] x[n][k]| of the
oracle's exact value; argmax indices equal to the oracle's, and equal to the
lowest-index maximum of the float32 logits the call returned; exact-arithmetic
inputs (power-of-two scales, small integer activations) bit-exact; repeated
calls bit-identical; guard bands around outputs untouched.
"""
import numpy as np
import pytest

import gemm_qgemv_amd as q
import oracle
import pins
from gemm_qgemv_amd import synth, tensors

pytestmark = pytest.mark.gpu
TOL = 1e-5
PAD = 64          # guard floats on each side of every output
CANARY = 1234.5


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "these tests need the GPU"
    return t


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

class Out:
    """An output buffer with guard bands."""

    def __init__(self, torch, n, dtype="float32"):
        dt = getattr(torch, dtype)
        self.full = torch.full((n + 2 * PAD,), CANARY if dtype == "float32" else -7,
                               dtype=dt, device="cuda")
        self.t = self.full[PAD:PAD + n]

    def check_guards(self):
        f = self.full.cpu().numpy()
        assert np.all(f[:PAD] == f[0]) and np.all(f[-PAD:] == f[0]), "guard band overwritten"


def gpu_gemv(torch, w, x, argmax=False, ws_fill=0xA5):
    """Run qgemv (or qgemv_argmax) on device weights w for x [batch][K];
    returns (y [batch][M] float32, idx or None). The workspace, control
    words included, starts filled with ws_fill: its contents on entry must
    not matter."""
    batch = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    y = Out(torch, batch * w.M)
    op = q.QG_OP_GEMV_ARGMAX if argmax else q.QG_OP_GEMV
    ws = tensors.workspace(op, w.fmt, w.M, w.K, batch)
    if ws is not None and ws_fill is not None:
        ws.fill_(ws_fill)
    idx = None
    if argmax:
        idx = Out(torch, batch, "int32")
        q.qgemv_argmax(w.fmt, w.codes, w.scales, w.biases, xd, y.t, idx.t, w.M, w.K, batch, ws)
    else:
        q.qgemv(w.fmt, w.codes, w.scales, w.biases, xd, y.t, w.M, w.K, batch, ws)
    torch.cuda.synchronize()
    y.check_guards()
    yh = y.t.cpu().numpy().reshape(batch, w.M)
    ih = None
    if argmax:
        idx.check_guards()
        ih = idx.t.cpu().numpy()
    return yh, ih


def gpu_gemm(torch, w, x):
    N = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    y = Out(torch, N * w.M)
    ws = tensors.workspace(q.QG_OP_GEMM, w.fmt, w.M, w.K, N)
    q.qgemm(w.fmt, w.codes, w.scales, w.biases, xd, y.t, w.M, w.K, N, ws)
    torch.cuda.synchronize()
    y.check_guards()
    return y.t.cpu().numpy().reshape(N, w.M)


def check_bound(y, ref, absdot, what):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - ref)
    bound = TOL * absdot
    bad = err > bound
    ratio = np.max(np.where(bound > 0, err / np.where(bound > 0, bound, 1), np.where(err > 0, np.inf, 0)))
    say(f"  {what}: max err/bound = {ratio:.3g}")
    assert not bad.any(), f"{what}: {bad.sum()} outputs outside the bound (worst ratio {ratio:.3g})"


def check_argmax(idx, y_gpu, ref, absdot, orc, what):
    want, gap = orc.argmax(ref)
    lowest = np.array([int(np.argmax(r)) for r in y_gpu])   # first occurrence of the max
    for n in range(len(idx)):
        bound = TOL * absdot[n, want[n]]
        margin = gap[n] / (2 * bound) if bound > 0 else np.inf
        say(f"  {what} row {n}: idx {idx[n]} oracle {want[n]} margin {margin:.3g}")
    assert np.array_equal(idx, lowest), f"{what}: idx is not the lowest-index max of the logits"
    assert np.array_equal(idx, want), f"{what}: idx differs from the oracle"


def dev(w):
    return tensors.to_device(w)


# ---------------------------------------------------------------------------
# hand-worked fixtures and exact arithmetic
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", pins.hand_fixtures())
def test_hand_fixture(torch, orc, name):
    say(f"hand fixture {name}")
    d, codes, scales, biases = pins.load_fixture(name)
    w = dev(synth.QWeights(d["fmt"], d["M"], d["K"], codes, scales, biases))
    x = np.asarray(d["x"], np.float32)
    ref, a = orc.qgemv(d["fmt"], codes, scales, biases, x, d["M"], d["K"])
    y, idx = gpu_gemv(torch, w, x, argmax=True)
    check_bound(y, ref, a, name)
    assert list(idx) == d["idx"]


def exact_inputs(fmt, M, K, N, rng):
    """Power-of-two scales, biases on a 2^-8 grid, integer activations in
    [-8, 8]: every partial sum is exact in float32 at these sizes, so any
    correct kernel, in any summation order, matches the oracle bit for bit."""
    x = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    if fmt == synth.I8_ROW:
        codes = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        scales = (2.0 ** -rng.integers(4, 8, size=M)).astype(np.float32)
        return synth.QWeights(fmt, M, K, codes, scales, None), x
    if fmt == synth.I8_G64:
        codes = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        scales = (2.0 ** -rng.integers(4, 8, size=(M, K // 64))).astype(np.float32)
        return synth.QWeights(fmt, M, K, codes, scales, None), x
    if fmt == synth.U4_G64:
        codes = rng.integers(0, 256, size=(M, K // 2)).astype(np.uint8)
        s = (2.0 ** -rng.integers(4, 8, size=(M, K // 64))).astype(np.float32)
        b = (rng.integers(-64, 65, size=(M, K // 64)) / 256.0).astype(np.float32)
        return synth.QWeights(fmt, M, K, codes, synth.to_bf16_bits(s), synth.to_bf16_bits(b)), x
    codes = rng.integers(0, 256, size=(M, K // 8)).astype(np.uint8)
    s = (2.0 ** -rng.integers(0, 8, size=(M, K // 128))).astype(np.float32)
    return synth.QWeights(fmt, M, K, codes, synth.to_fp16_bits(s), None), x


@pytest.mark.parametrize("fmt,M,K,N", [
    (synth.I8_ROW, 129, 1024, 1), (synth.I8_ROW, 70, 528, 5), (synth.I8_ROW, 33, 1024, 16),
    (synth.U4_G64, 129, 1024, 1), (synth.U4_G64, 65, 576, 3), (synth.U4_G64, 300, 1024, 8),
    (synth.B1_G128, 129, 1024, 1), (synth.B1_G128, 17, 1152, 6), (synth.B1_G128, 257, 1024, 16),
    (synth.I8_G64, 129, 1024, 1), (synth.I8_G64, 70, 576, 5), (synth.I8_G64, 33, 1024, 16),
    (synth.I8_G64, 100, 4160, 1), (synth.I8_ROW, 300, 2048, 7), (synth.I8_G64, 4099, 2048, 13),
    (synth.U4_G64, 300, 6144, 5), (synth.I8_ROW, 129, 4096, 11), (synth.I8_G64, 40, 3072, 16),
    (synth.B1_G128, 300, 5120, 5), (synth.B1_G128, 33, 2048, 3),
    (synth.I8_ROW, 77, 3584, 9), (synth.I8_G64, 1000, 2560, 7), (synth.I8_G64, 99, 512, 4),
    (synth.U4_G64, 1003, 2048, 1), (synth.U4_G64, 259, 6144, 1), (synth.U4_G64, 70, 8192, 1),
])
def test_exact_arithmetic_bit_exact(torch, orc, fmt, M, K, N):
    say(f"exact fmt={fmt} M={M} K={K} N={N}")
    rng = np.random.default_rng([fmt, M, K, N])
    w, x = exact_inputs(fmt, M, K, N, rng)
    ref, _ = orc.qgemv(fmt, w.codes, w.scales, w.biases, x, M, K)
    want = ref.astype(np.float32)
    assert np.array_equal(want.astype(np.float64), ref), "fixture is not exact in float32"
    y, _ = gpu_gemv(torch, dev(w), x)
    assert np.array_equal(y, want), f"gemv not bit-exact: max diff {np.max(np.abs(y - want))}"
    yg = gpu_gemm(torch, dev(w), x)
    assert np.array_equal(yg, want), "gemm not bit-exact"


@pytest.mark.parametrize("fmt,M,K,N", [
    (synth.I8_ROW, 129, 1024, 17), (synth.I8_ROW, 300, 1040, 130), (synth.I8_ROW, 7, 48, 257),
    (synth.I8_ROW, 1024, 3584, 64), (synth.B1_G128, 129, 1024, 17), (synth.B1_G128, 260, 640, 300),
    (synth.B1_G128, 5, 128, 129), (synth.U4_G64, 129, 1024, 17), (synth.U4_G64, 300, 1088, 130),
    (synth.U4_G64, 7, 64, 257), (synth.U4_G64, 1024, 2048, 64), (synth.U4_G64, 4001, 192, 1503),
    (synth.I8_G64, 129, 1024, 17), (synth.I8_G64, 300, 1088, 130), (synth.I8_G64, 7, 64, 257),
    (synth.I8_G64, 4001, 192, 1503), (synth.I8_G64, 1024, 3584, 64),
    # 288 tiles of 128 x 64, K split in two
    (synth.I8_ROW, 1025, 1040, 2000), (synth.I8_G64, 1025, 1088, 2000),
])
def test_exact_arithmetic_prefill_bit_exact(torch, orc, fmt, M, K, N):
    """The matrix-core prefill path (more than 16 token rows) on exact inputs."""
    say(f"exact prefill fmt={fmt} M={M} K={K} N={N}")
    rng = np.random.default_rng([fmt, M, K, N, 1])
    w, x = exact_inputs(fmt, M, K, N, rng)
    ref, _ = orc.qgemv(fmt, w.codes, w.scales, w.biases, x, M, K)
    want = ref.astype(np.float32)
    assert np.array_equal(want.astype(np.float64), ref), "fixture is not exact in float32"
    yg = gpu_gemm(torch, dev(w), x)
    assert np.array_equal(yg, want), f"prefill not bit-exact: max diff {np.max(np.abs(yg - want))}"


@pytest.mark.parametrize("M,K,N", [(4001, 160, 1503), (4096, 176, 1536), (3841, 1040, 1665),
                                   (4097, 176, 8001)])
def test_exact_arithmetic_prefill_large_grid(torch, orc, M, K, N):
    """8-bit prefill on grids of several hundred 128 x 128 tiles, and of
    two thousand 256 x 64 tiles (4097 x 8001): ragged M and N, K with a half
    step at the end."""
    say(f"exact prefill large grid M={M} K={K} N={N}")
    rng = np.random.default_rng([11, M, K, N])
    w, x = exact_inputs(synth.I8_ROW, M, K, N, rng)
    ref, _ = orc.qgemv(synth.I8_ROW, w.codes, w.scales, w.biases, x, M, K)
    want = ref.astype(np.float32)
    assert np.array_equal(want.astype(np.float64), ref), "fixture is not exact in float32"
    yg = gpu_gemm(torch, dev(w), x)
    assert np.array_equal(yg, want), f"prefill not bit-exact: max diff {np.max(np.abs(yg - want))}"


@pytest.mark.parametrize("fmt,M,K,N", [
    (synth.I8_ROW, 1000, 272, 12800), (synth.U4_G64, 2100, 576, 2000), (synth.B1_G128, 1100, 1152, 3900),
    (synth.I8_G64, 2100, 576, 2900),
    # M not a multiple of 4: the combine's scalar stores
    (synth.U4_G64, 2101, 576, 2000), (synth.I8_G64, 2099, 576, 2900), (synth.I8_ROW, 1001, 272, 12290),
])
def test_exact_arithmetic_prefill_split_tail(torch, orc, fmt, M, K, N):
    """Grids of one or more full rounds of tiles plus a short last round,
    whose tiles are computed in pieces of K and added by a second launch:
    ragged M and N in the last round, a short last piece of K."""
    say(f"exact prefill split tail fmt={fmt} M={M} K={K} N={N}")
    rng = np.random.default_rng([13, fmt, M, K, N])
    w, x = exact_inputs(fmt, M, K, N, rng)
    ref, _ = orc.qgemv(fmt, w.codes, w.scales, w.biases, x, M, K)
    want = ref.astype(np.float32)
    assert np.array_equal(want.astype(np.float64), ref), "fixture is not exact in float32"
    yg = gpu_gemm(torch, dev(w), x)
    assert np.array_equal(yg, want), f"prefill not bit-exact: max diff {np.max(np.abs(yg - want))}"


@pytest.mark.parametrize("fmt,M,K,N", [
    (synth.I8_ROW, 1, 16, 17), (synth.I8_ROW, 127, 1040, 129), (synth.I8_ROW, 1000, 1024, 300),
    (synth.I8_ROW, 4001, 1040, 1503),
    (synth.I8_ROW, 130, 3584, 33), (synth.B1_G128, 1, 128, 40), (synth.B1_G128, 250, 5120, 131),
    (synth.B1_G128, 129, 1152, 256), (synth.U4_G64, 1, 64, 40), (synth.U4_G64, 1000, 2048, 300),
    (synth.U4_G64, 127, 6144, 129), (synth.U4_G64, 6144, 2048, 2048),
    (synth.I8_G64, 1, 64, 40), (synth.I8_G64, 1000, 1024, 300), (synth.I8_G64, 127, 3584, 129),
    (synth.I8_G64, 3584, 1024, 2048),
    # narrow tiles: 16 or 32 token rows wide, waves along the weight rows;
    # 128-row tiles once M gives every compute unit two of them
    (synth.I8_ROW, 66001, 256, 24), (synth.U4_G64, 70001, 512, 20), (synth.B1_G128, 66000, 256, 32),
    (synth.I8_G64, 66001, 192, 29), (synth.U4_G64, 3000, 2048, 32), (synth.I8_ROW, 2049, 3584, 25),
    (synth.B1_G128, 700, 5120, 21), (synth.I8_G64, 1000, 3584, 18),
    # 4-bit rows run as launches of 16 on the one-pass kernel (the last one
    # a single row on the batch-1 kernel, or 8 rows on the 8-row kernel)
    (synth.U4_G64, 30001, 2048, 17), (synth.U4_G64, 40000, 1024, 40),
])
def test_random_prefill_small(torch, orc, fmt, M, K, N):
    say(f"random prefill fmt={fmt} M={M} K={K} N={N}")
    rng = synth.rng_for(200 + fmt, M * 11 + N)
    w = synth.draw_weights(fmt, M, K, rng)
    x = synth.draw_x(N, K, rng)
    ref, a = orc.qgemv(fmt, w.codes, w.scales, w.biases, x, M, K)
    yg = gpu_gemm(torch, dev(w), x)
    check_bound(yg, ref, a, f"prefill {fmt} {M}x{K} n{N}")


# ---------------------------------------------------------------------------
# random inputs at small sizes: several tiles, ragged tails, every batch
# ---------------------------------------------------------------------------

SMALL = [
    (synth.I8_ROW, 1, 16, 1), (synth.I8_ROW, 63, 1040, 2), (synth.I8_ROW, 1000, 1024, 1),
    (synth.I8_ROW, 127, 3072, 3), (synth.I8_ROW, 129, 16384, 1), (synth.I8_ROW, 45, 20000, 2),
    (synth.U4_G64, 1, 64, 1), (synth.U4_G64, 127, 2112, 1), (synth.U4_G64, 1187, 2048, 4),
    (synth.U4_G64, 129, 6144, 5), (synth.U4_G64, 64, 8192, 16), (synth.U4_G64, 31, 18048, 7),
    (synth.U4_G64, 5, 2048, 1), (synth.U4_G64, 1003, 2048, 1), (synth.U4_G64, 333, 4096, 1),
    (synth.U4_G64, 130, 6144, 1), (synth.U4_G64, 77, 8192, 1), (synth.U4_G64, 4099, 4096, 1),
    (synth.B1_G128, 1, 128, 1), (synth.B1_G128, 129, 5120, 1), (synth.B1_G128, 1000, 1152, 2),
    (synth.B1_G128, 63, 17408, 1), (synth.B1_G128, 33, 2048, 16), (synth.B1_G128, 8, 640, 9),
    (synth.B1_G128, 3000, 5120, 5), (synth.B1_G128, 700, 17408, 12), (synth.B1_G128, 129, 1536, 3),
    (synth.B1_G128, 65, 4096, 7),
    (synth.I8_G64, 1, 64, 1), (synth.I8_G64, 127, 1088, 1), (synth.I8_G64, 1000, 1024, 3),
    (synth.I8_G64, 129, 16384, 1), (synth.I8_G64, 45, 20032, 2), (synth.I8_G64, 64, 4096, 16),
    (synth.I8_G64, 3584, 1024, 1), (synth.I8_G64, 1024, 3584, 1),
    # batches that the host routes to the prefill kernel's narrow tiles
    (synth.U4_G64, 6144, 2048, 12), (synth.U4_G64, 2048, 6144, 6), (synth.I8_ROW, 1024, 3584, 8),
    (synth.B1_G128, 17408, 5120, 16), (synth.I8_G64, 1024, 3584, 11), (synth.B1_G128, 5120, 17408, 6),
    (synth.B1_G128, 17408, 5120, 7),
    # 8-bit batches on the one-pass matrix-core kernel (K = 1024 or 2048)
    (synth.I8_ROW, 3000, 2048, 12), (synth.I8_G64, 70001, 2048, 5), (synth.I8_ROW, 1, 1024, 2),
    (synth.I8_G64, 17, 1024, 16), (synth.I8_ROW, 3584, 1024, 9),
    # longer K on the one-pass kernel in slices of 2048 or 1024 inputs
    (synth.U4_G64, 5000, 3072, 2), (synth.U4_G64, 2048, 6144, 16), (synth.I8_ROW, 4096, 4096, 9),
    (synth.I8_G64, 1000, 3072, 4), (synth.U4_G64, 70001, 16384, 3), (synth.I8_ROW, 7, 8192, 2),
    # 1-bit batches on the one-pass kernel (4-byte code loads per 128 inputs)
    (synth.B1_G128, 4096, 2048, 8), (synth.B1_G128, 1000, 1024, 3), (synth.B1_G128, 2000, 16384, 13),
    # 8-bit in slices of 512 inputs (one group per wave)
    (synth.I8_ROW, 1024, 3584, 12), (synth.I8_G64, 1024, 3584, 5), (synth.I8_ROW, 33, 1536, 16),
]


@pytest.mark.parametrize("fmt,M,K,N", SMALL)
def test_random_small(torch, orc, fmt, M, K, N):
    say(f"random fmt={fmt} M={M} K={K} N={N}")
    rng = synth.rng_for(100 + fmt, M * 7 + N)
    w = synth.draw_weights(fmt, M, K, rng)
    x = synth.draw_x(N, K, rng)
    ref, a = orc.qgemv(fmt, w.codes, w.scales, w.biases, x, M, K)
    y, idx = gpu_gemv(torch, dev(w), x, argmax=True, ws_fill=0xA5)
    check_bound(y, ref, a, f"gemv {fmt} {M}x{K} b{N}")
    check_argmax(idx, y, ref, a, orc, "argmax")
    yg = gpu_gemm(torch, dev(w), x)
    check_bound(yg, ref, a, "gemm")


def test_argmax_ties_and_signed_zero(torch, orc):
    """Duplicate maximum rows (first row, last row, across workgroups, in the
    tail), all-equal logits, and -0 against +0."""
    say("argmax ties")
    rng = np.random.default_rng(7)
    M, K = 9000, 256
    w = synth.draw_weights(synth.U4_G64, M, K, rng)
    x = synth.draw_x(3, K, rng)
    ref, _ = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    top = int(np.argmax(ref[0]))
    for dst in (0, M - 1, 4500, 8999 - 130):
        for arr in (w.codes, w.scales, w.biases):
            arr[dst] = arr[top]
    ref, a = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    y, idx = gpu_gemv(torch, dev(w), x, argmax=True)
    check_bound(y, ref, a, "ties")
    assert y[0, 0] == y[0, M - 1] == y[0, top], "duplicate rows must give identical logits"
    check_argmax(idx, y, ref, a, orc, "ties")
    assert idx[0] == 0
    # all-equal logits: x = 0
    y, idx = gpu_gemv(torch, dev(w), np.zeros((2, K), np.float32), argmax=True)
    assert np.all(y == 0) and list(idx) == [0, 0]
    # -0 against +0: zero codes with a negative scale give -0, a positive scale +0
    M, K = 12, 64
    codes = np.zeros((M, K), np.int8)
    codes[[0, 1, 2, 4, 5, 6, 8, 9, 10, 11]] = -1
    scales = np.ones(M, np.float32)
    scales[3] = -1.0
    wi = synth.QWeights(synth.I8_ROW, M, K, codes, scales, None)
    y, idx = gpu_gemv(torch, dev(wi), np.ones((1, K), np.float32), argmax=True)
    assert np.signbit(y[0, 3]) and y[0, 3] == 0 and y[0, 7] == 0 and not np.signbit(y[0, 7])
    assert idx[0] == 3


@pytest.mark.parametrize("M,K", [(9001, 2048), (3003, 6144)])
def test_batch1_argmax_ties(torch, orc, M, K):
    """One activation row: the maximum row duplicated at the first row, the
    last row, across waves and in a wave's final, partial block; the lowest
    index wins."""
    say(f"batch-1 ties M={M} K={K}")
    rng = np.random.default_rng([13, M, K])
    w = synth.draw_weights(synth.U4_G64, M, K, rng)
    x = synth.draw_x(1, K, rng)
    ref, _ = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    top = int(np.argmax(ref[0]))
    dups = [d for d in (0, M - 1, M // 2, M // 2 + 9, M - 2) if d != top]
    for dst in dups:
        for arr in (w.codes, w.scales, w.biases):
            arr[dst] = arr[top]
    ref, a = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    y, idx = gpu_gemv(torch, dev(w), x, argmax=True)
    check_bound(y, ref, a, "batch-1 ties")
    assert all(y[0, d] == y[0, top] for d in dups), "duplicate rows must give identical logits"
    check_argmax(idx, y, ref, a, orc, "batch-1 ties")
    assert idx[0] == 0


def test_zero_codes_give_bias_times_sum(torch, orc):
    say("zero codes")
    rng = np.random.default_rng(8)
    M, K = 300, 2048
    w = synth.draw_weights(synth.U4_G64, M, K, rng)
    w.codes[:] = 0
    x = synth.draw_x(2, K, rng)
    ref, a = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    y, _ = gpu_gemv(torch, dev(w), x)
    check_bound(y, ref, a, "zero codes")


# ---------------------------------------------------------------------------
# the small-batch 4-bit matrix-core paths: 2..8 rows, K a multiple of 512 up
# to 3072 (16-row tiles, up to several per wave, chunks of 512 inputs); 9..16
# rows in one pass for K = 1024 and 2048 (K cut across the waves), in two
# launches of up to 8 rows for other K; K = 3584 takes the vector path
# ---------------------------------------------------------------------------

MFMA_SHAPES = [
    (16, 512, 8), (17, 1024, 5), (300, 1536, 2), (40007, 512, 3), (70001, 2048, 8),
    (5000, 3072, 2), (9001, 3072, 7), (1000, 3584, 4), (2049, 2048, 9),
    (70001, 2048, 16), (3000, 3072, 12), (40007, 512, 10),
    (16, 1024, 9), (1000, 1024, 16), (17, 2048, 13), (70001, 1024, 11), (4097, 2048, 15),
    # more 16-row tiles per workgroup than LDS can stage: outputs stored directly
    (400003, 1024, 12),
    # a single weight row (every tile row but the first clamps to it)
    (1, 2048, 16), (1, 1024, 3), (5, 2048, 2),
]


@pytest.mark.parametrize("M,K,N", MFMA_SHAPES)
def test_small_batch_u4_exact(torch, orc, M, K, N):
    say(f"small-batch exact M={M} K={K} N={N}")
    rng = np.random.default_rng([9, M, K, N])
    w, x = exact_inputs(synth.U4_G64, M, K, N, rng)
    ref, a = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    want = ref.astype(np.float32)
    assert np.array_equal(want.astype(np.float64), ref), "fixture is not exact in float32"
    y, idx = gpu_gemv(torch, dev(w), x, argmax=True, ws_fill=0x5A)
    assert np.array_equal(y, want), f"not bit-exact: max diff {np.max(np.abs(y - want))}"
    assert list(idx) == [int(np.argmax(r)) for r in want]


@pytest.mark.parametrize("M,K,N", MFMA_SHAPES)
def test_small_batch_u4_random(torch, orc, M, K, N):
    say(f"small-batch random M={M} K={K} N={N}")
    rng = synth.rng_for(400, M * 13 + K + N)
    w = synth.draw_weights(synth.U4_G64, M, K, rng)
    x = synth.draw_x(N, K, rng)
    ref, a = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    y, idx = gpu_gemv(torch, dev(w), x, argmax=True, ws_fill=0xA5)
    check_bound(y, ref, a, f"small-batch {M}x{K} b{N}")
    check_argmax(idx, y, ref, a, orc, "argmax")
    y2, idx2 = gpu_gemv(torch, dev(w), x, argmax=True)
    assert np.array_equal(y, y2) and np.array_equal(idx, idx2), "repeated call differs"


def test_small_batch_u4_ties(torch, orc):
    """Equal maxima in different waves and workgroups (first row, last row,
    the middle), per activation row."""
    say("small-batch ties")
    rng = np.random.default_rng(10)
    M, K, N = 40000, 512, 4
    w = synth.draw_weights(synth.U4_G64, M, K, rng)
    x = synth.draw_x(N, K, rng)
    ref, _ = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    tops = [int(np.argmax(ref[n])) for n in range(N)]
    dsts = {0: [M - 1, 20011], 1: [0], 2: [30001], 3: [19999, 20000]}
    for n, ds in dsts.items():
        for dst in ds:
            if dst in tops:
                continue
            for arr in (w.codes, w.scales, w.biases):
                arr[dst] = arr[tops[n]]
    ref, a = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    y, idx = gpu_gemv(torch, dev(w), x, argmax=True)
    check_bound(y, ref, a, "ties")
    check_argmax(idx, y, ref, a, orc, "ties")


# ---------------------------------------------------------------------------
# the greedy head without logits, and over more rows than the matrix-vector
# kernels take (prefill kernels with per-tile keys)
# ---------------------------------------------------------------------------

def gpu_greedy(torch, w, x, logits=True):
    """qgemv_argmax through the C ABI; returns (logits or None, idx)."""
    batch = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    y = Out(torch, batch * w.M) if logits else None
    idx = Out(torch, batch, "int32")
    ws = tensors.workspace(q.QG_OP_GEMV_ARGMAX, w.fmt, w.M, w.K, batch)
    ws.fill_(0x3C)   # the whole workspace, control words included, may hold anything
    q.qgemv_argmax(w.fmt, w.codes, w.scales, w.biases, xd, None if y is None else y.t, idx.t,
                   w.M, w.K, batch, ws)
    torch.cuda.synchronize()
    idx.check_guards()
    if y is None:
        return None, idx.t.cpu().numpy()
    y.check_guards()
    return y.t.cpu().numpy().reshape(batch, w.M), idx.t.cpu().numpy()


@pytest.mark.parametrize("fmt,M,K,N", [
    (synth.U4_G64, 9000, 2048, 1), (synth.I8_ROW, 5000, 1024, 1), (synth.B1_G128, 3000, 1280, 1),
    (synth.U4_G64, 9001, 2048, 1), (synth.U4_G64, 4097, 4096, 1), (synth.U4_G64, 3001, 6144, 1),
    (synth.U4_G64, 40007, 512, 3), (synth.I8_ROW, 777, 1040, 5), (synth.B1_G128, 1000, 6144, 9),
    (synth.U4_G64, 30001, 2048, 64), (synth.I8_ROW, 9000, 1024, 100), (synth.B1_G128, 5000, 1280, 17),
    (synth.U4_G64, 20000, 2048, 128), (synth.U4_G64, 4099, 1024, 256),
    (synth.U4_G64, 30001, 2048, 16), (synth.U4_G64, 9000, 1024, 11),
    (synth.U4_G64, 30001, 2048, 24), (synth.I8_ROW, 70001, 256, 32), (synth.I8_G64, 70001, 192, 19),
    (synth.B1_G128, 66001, 256, 30),
    (synth.U4_G64, 40000, 1024, 33), (synth.U4_G64, 60000, 2048, 48),
    (synth.B1_G128, 3000, 2048, 7), (synth.I8_ROW, 20000, 1024, 12),
    # 8-bit per-row 256 x 64 tiles with per-tile keys (628 tiles, ragged M and N)
    (synth.I8_ROW, 40001, 256, 200),
])
def test_greedy_head_with_and_without_logits(torch, orc, fmt, M, K, N):
    say(f"greedy fmt={fmt} M={M} K={K} N={N}")
    rng = synth.rng_for(500 + fmt, M * 3 + N)
    w = synth.draw_weights(fmt, M, K, rng)
    x = synth.draw_x(N, K, rng)
    ref, a = orc.qgemv(fmt, w.codes, w.scales, w.biases, x, M, K)
    wd = dev(w)
    y, idx = gpu_greedy(torch, wd, x, logits=True)
    check_bound(y, ref, a, f"greedy {fmt} {M}x{K} n{N}")
    check_argmax(idx, y, ref, a, orc, "greedy")
    _, idx2 = gpu_greedy(torch, wd, x, logits=False)
    assert np.array_equal(idx, idx2), "logits-free call chose other rows"


@pytest.mark.parametrize("N", [64, 20])
def test_wide_greedy_head_ties(N):
    """Equal maxima in different 64-row tiles (first row, last row, the
    middle), and in the two halves of one tile (20 rows of activations:
    32-token tiles whose two waves each cover 32 of the 64 weight rows)."""
    import torch as t
    orc = oracle.get()
    say(f"wide greedy ties N={N}")
    rng = np.random.default_rng(12)
    M, K = 20000, 1024
    w = synth.draw_weights(synth.U4_G64, M, K, rng)
    x = synth.draw_x(N, K, rng)
    ref, _ = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    top = int(np.argmax(ref[0]))
    for dst in (0, M - 1, 10000, 10040, 10063):
        if dst != top:
            for arr in (w.codes, w.scales, w.biases):
                arr[dst] = arr[top]
    ref, a = orc.qgemv(synth.U4_G64, w.codes, w.scales, w.biases, x, M, K)
    y, idx = gpu_greedy(t, dev(w), x, logits=True)
    check_bound(y, ref, a, "wide ties")
    check_argmax(idx, y, ref, a, orc, "wide ties")
    assert idx[0] == min(0, top) == 0
    _, idx2 = gpu_greedy(t, dev(w), x, logits=False)
    assert np.array_equal(idx, idx2)


# ---------------------------------------------------------------------------
# seeded random shapes: every entry point on shapes drawn across the host's
# kernel choices (batch-1 kernels, small-batch kernels, the prefill kernel's
# narrow and wide tiles, split K, routed batches, the wide greedy head)
# ---------------------------------------------------------------------------

ROWS_DRAWN = [1, 2, 3, 4, 5, 6, 7, 8, 9, 11, 12, 13, 15, 16, 17, 19, 24, 31, 32, 33, 47, 64, 65, 100, 129]


def drawn_shapes(fmt, count, seed, budget=12e6, min_m=1.0, max_m=40000.0, ks=None):
    """(M, K, N) with M and K log-uniform (K a multiple of the format's
    unit, up to 8192, or drawn from `ks`) and N from ROWS_DRAWN, at most
    `budget` multiply-adds."""
    rng = np.random.default_rng([seed, fmt])
    unit = synth.K_UNIT[fmt]
    shapes = []
    while len(shapes) < count:
        M = int(np.exp(rng.uniform(np.log(min_m), np.log(max_m))))
        if ks is None:
            K = unit * max(1, int(round(np.exp(rng.uniform(0.0, np.log(8192 / unit))))))
        else:
            K = int(rng.choice(ks))
        N = int(rng.choice(ROWS_DRAWN))
        if M * K * N <= budget:
            shapes.append((M, K, N))
    return shapes


# the drawn sets: small shapes of any K, and larger ones at the K values
# where the host has the most kernel choices (the one-pass 4-bit kernel at
# K = 1024 and 2048, the batch-8 kernel up to 3072, long-K 1-bit tables)
DRAWN_SETS = {
    "small": dict(count=32, seed=77),
    "large": dict(count=12, seed=78, budget=2.5e8, min_m=2000.0, max_m=200000.0,
                  ks=[512, 1024, 2048, 3072, 4096, 5120]),
}


@pytest.mark.parametrize("fmt", [synth.I8_ROW, synth.U4_G64, synth.B1_G128, synth.I8_G64])
@pytest.mark.parametrize("drawn", sorted(DRAWN_SETS))
def test_drawn_shapes_all_entry_points(torch, orc, fmt, drawn):
    for i, (M, K, N) in enumerate(drawn_shapes(fmt, **DRAWN_SETS[drawn])):
        say(f"drawn {drawn} fmt={fmt} #{i} M={M} K={K} N={N}")
        rng = synth.rng_for(700 + fmt + (0 if drawn == "small" else 10), i)
        w = synth.draw_weights(fmt, M, K, rng)
        x = synth.draw_x(N, K, rng)
        ref, a = orc.qgemv(fmt, w.codes, w.scales, w.biases, x, M, K)
        wd = dev(w)
        check_bound(gpu_gemm(torch, wd, x), ref, a, f"qgemm {M}x{K} n{N}")
        if N <= q.QG_MAX_GEMV_BATCH:
            y, _ = gpu_gemv(torch, wd, x, ws_fill=0x77)
            check_bound(y, ref, a, f"qgemv {M}x{K} b{N}")
        y, idx = gpu_greedy(torch, wd, x, logits=True)
        check_bound(y, ref, a, f"greedy {M}x{K} b{N}")
        check_argmax(idx, y, ref, a, orc, "greedy")


# ---------------------------------------------------------------------------
# the thirteen measured workloads at full size
# ---------------------------------------------------------------------------

# those workloads, the measured cases of the 8-bit group-64 format and the
# 16-row head
MEASURED = synth.CASES + [c for c in synth.NEXT_CASES
                          if c.fmt == synth.I8_G64 or c.name == "n4_u4_head_151936x2048_b16"]
GEMV_CASES = [c for c in MEASURED if c.op != "gemm"]
GEMM_CASES = [c for c in MEASURED if c.op == "gemm"]


@pytest.mark.parametrize("case", GEMV_CASES, ids=lambda c: c.name)
def test_config_gemv_full(torch, orc, case):
    say(f"config {case.name}")
    w, x = synth.case_inputs(case)
    ref, a = orc.qgemv(case.fmt, w.codes, w.scales, w.biases, x, case.M, case.K)
    wd = dev(w)
    argmax = case.op == "gemv_argmax"
    y, idx = gpu_gemv(torch, wd, x, argmax=argmax)
    check_bound(y, ref, a, case.name)
    if argmax:
        check_argmax(idx, y, ref, a, orc, case.name)
    # a second call gives identical bits
    y2, idx2 = gpu_gemv(torch, wd, x, argmax=argmax)
    assert np.array_equal(y, y2), "repeated call differs"
    if argmax:
        assert np.array_equal(idx, idx2)


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: c.name)
def test_config_gemm_full(torch, orc, case):
    """Every output of the full-size prefill case against the oracle (exact
    weights times the activations in float64), within the bound."""
    say(f"config {case.name}")
    w, x = synth.case_inputs(case)
    y = gpu_gemm(torch, dev(w), x)
    ref, a = orc.qgemm_dense(case.fmt, w.codes, w.scales, w.biases, x, case.M, case.K)
    check_bound(y, ref, a, case.name)
    del ref, a
    # whole rows: prefill row n equals the matvec of x[n] (both within bound)
    for nn in (0, case.rows // 2, case.rows - 1):
        yv, _ = gpu_gemv(torch, dev(w), x[nn:nn + 1])
        refr, ar = orc.qgemv(case.fmt, w.codes, w.scales, w.biases, x[nn:nn + 1], case.M, case.K)
        check_bound(y[nn:nn + 1], refr, ar, f"{case.name} row {nn}")
        check_bound(yv, refr, ar, f"{case.name} gemv row {nn}")


@pytest.mark.parametrize("M,K", [(17408, 5120), (5120, 17408)])
def test_exact_arithmetic_b1_prefill_config_shape(torch, orc, M, K):
    """The 1-bit prefill at the configurations' shapes and 512 token rows on
    exact inputs (fp16 scales 2^-4 .. 2^-7, integer activations in [-8, 8]):
    every partial sum is a multiple of 2^-7 below 2^17 in magnitude, so any
    correct kernel, with or without its K split, is bit-exact."""
    N = 512
    say(f"exact 1-bit prefill M={M} K={K} N={N}")
    rng = np.random.default_rng([3, M, K, N])
    codes = rng.integers(0, 256, size=(M, K // 8)).astype(np.uint8)
    s = (2.0 ** -rng.integers(4, 8, size=(M, K // 128))).astype(np.float32)
    w = synth.QWeights(synth.B1_G128, M, K, codes, synth.to_fp16_bits(s), None)
    x = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    ref, _ = orc.qgemm_dense(synth.B1_G128, w.codes, w.scales, None, x, M, K)
    want = ref.astype(np.float32)
    assert np.array_equal(want.astype(np.float64), ref), "fixture is not exact in float32"
    yg = gpu_gemm(torch, dev(w), x)
    assert np.array_equal(yg, want), f"prefill not bit-exact: max diff {np.max(np.abs(yg - want))}"


# ---------------------------------------------------------------------------
# one workspace across many calls, and HIP graph replay
# ---------------------------------------------------------------------------

def test_shared_workspace_sequence(torch, orc):
    """One workspace (sized for the largest call, never cleared) serves a
    sequence of greedy-head calls of different shapes and batches and
    prefill calls that split K (their partial products live after the
    control words)."""
    say("shared workspace")
    calls = [(q.QG_OP_GEMV_ARGMAX, synth.U4_G64, 5000, 2048, 1),
             (q.QG_OP_GEMV_ARGMAX, synth.U4_G64, 3000, 1024, 8),
             (q.QG_OP_GEMM, synth.I8_ROW, 1024, 3584, 40),
             (q.QG_OP_GEMV_ARGMAX, synth.I8_ROW, 7000, 1024, 1),
             (q.QG_OP_GEMV_ARGMAX, synth.B1_G128, 2000, 1280, 3),
             (q.QG_OP_GEMM, synth.U4_G64, 500, 2048, 100),
             (q.QG_OP_GEMV_ARGMAX, synth.U4_G64, 5000, 2048, 1)]
    assert q.qg_workspace_bytes(q.QG_OP_GEMM, synth.I8_ROW, 1024, 3584, 40) > q.QG_WS_CONTROL_BYTES
    need = max(q.qg_workspace_bytes(op, f, M, K, n) for op, f, M, K, n in calls)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    for i, (op, fmt, M, K, n) in enumerate(calls):
        rng = synth.rng_for(300, i)
        w = synth.draw_weights(fmt, M, K, rng)
        x = synth.draw_x(n, K, rng)
        wd = dev(w)
        xd = torch.from_numpy(x).cuda()
        y = torch.empty(n * M, device="cuda")
        idx = torch.empty(n, dtype=torch.int32, device="cuda")
        if op == q.QG_OP_GEMM:
            q.qgemm(fmt, wd.codes, wd.scales, wd.biases, xd, y, M, K, n, ws)
        else:
            q.qgemv_argmax(fmt, wd.codes, wd.scales, wd.biases, xd, y, idx, M, K, n, ws)
        torch.cuda.synchronize()
        ref, a = orc.qgemv(fmt, w.codes, w.scales, w.biases, x, M, K)
        yh = y.cpu().numpy().reshape(n, M)
        check_bound(yh, ref, a, f"call {i}")
        if op != q.QG_OP_GEMM:
            check_argmax(idx.cpu().numpy(), yh, ref, a, orc, f"call {i}")


def test_graph_replay_matches_eager(torch, orc):
    """A HIP graph holding a greedy-head call, a matvec and a prefill call,
    replayed several times with eager work and synchronizations between
    replays: every replay equals the eager result bit for bit."""
    say("graph replay")
    rng = synth.rng_for(301, 0)
    wu = synth.draw_weights(synth.U4_G64, 20000, 2048, rng)
    wi = synth.draw_weights(synth.I8_ROW, 3000, 1024, rng)
    xu = torch.from_numpy(synth.draw_x(1, 2048, rng)).cuda()
    xi = torch.from_numpy(synth.draw_x(200, 1024, rng)).cuda()
    du, di = dev(wu), dev(wi)
    logits = torch.empty(20000, device="cuda")
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    yv = torch.empty(3000, device="cuda")
    yg = torch.empty(200 * 3000, device="cuda")
    ws = tensors.workspace(q.QG_OP_GEMV_ARGMAX, wu.fmt, 20000, 2048, 1)
    # the prefill call at this size splits K (too few tiles for the chip):
    # partial products in a workspace of its own size
    wsg = tensors.workspace(q.QG_OP_GEMM, wi.fmt, 3000, 1024, 200)
    assert wsg is not None
    s = torch.cuda.Stream()

    def work(stream):
        q.qgemv_argmax(wu.fmt, du.codes, du.scales, du.biases, xu, logits, idx, 20000, 2048, 1, ws,
                       stream=stream)
        q.qgemv(wi.fmt, di.codes, di.scales, None, xi[:1], yv, 3000, 1024, 1, stream=stream)
        q.qgemm(wi.fmt, di.codes, di.scales, None, xi, yg, 3000, 1024, 200, wsg, stream=stream)

    work(s)
    torch.cuda.synchronize()
    want = [t.clone() for t in (logits, idx, yv, yg)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        work(s)
    for rep in range(4):
        for t in (logits, yv, yg):
            t.fill_(float("nan"))
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((logits, idx, yv, yg), want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager result"
        # eager work between replays, and stale control words
        work(s)
        torch.cuda.synchronize()
        ws[:q.QG_WS_CONTROL_BYTES].random_(0, 256)


def test_graph_replay_counters_and_gather(torch, orc):
    """The paths that keep counters in the workspace, and the gather, in one
    HIP graph: the batch-8 matrix-core head (per-workgroup key rows), the
    64-row greedy head without logits (tile keys and their reduction), the
    1-bit batch-1 product with its K chunks combined in the kernel (row-tile
    counters), and qembed of the chosen tokens. Each replay, with eager calls
    and overwritten control words between replays, equals the eager result
    bit for bit."""
    say("graph replay: counters and gather")
    rng = synth.rng_for(302, 0)
    M, K = 30000, 2048
    wu = synth.draw_weights(synth.U4_G64, M, K, rng)
    wb = synth.draw_weights(synth.B1_G128, 5000, 5120, rng)
    du, db = dev(wu), dev(wb)
    x8 = torch.from_numpy(synth.draw_x(8, K, rng)).cuda()
    x64 = torch.from_numpy(synth.draw_x(64, K, rng)).cuda()
    xb = torch.from_numpy(synth.draw_x(1, 5120, rng)).cuda()
    logits8 = torch.empty(8 * M, device="cuda")
    idx8 = torch.empty(8, dtype=torch.int32, device="cuda")
    idx64 = torch.empty(64, dtype=torch.int32, device="cuda")
    yb = torch.empty(5000, device="cuda")
    rows = torch.empty(8 * K, device="cuda")
    ws8 = tensors.workspace(q.QG_OP_GEMV_ARGMAX, wu.fmt, M, K, 8)
    ws64 = tensors.workspace(q.QG_OP_GEMV_ARGMAX, wu.fmt, M, K, 64)
    wsb = tensors.workspace(q.QG_OP_GEMV, wb.fmt, 5000, 5120, 1)
    assert wsb is not None, "the 1-bit product at this K combines chunks in a workspace"
    s = torch.cuda.Stream()

    def work(stream):
        q.qgemv_argmax(wu.fmt, du.codes, du.scales, du.biases, x8, logits8, idx8, M, K, 8, ws8,
                       stream=stream)
        q.qgemv_argmax(wu.fmt, du.codes, du.scales, du.biases, x64, None, idx64, M, K, 64, ws64,
                       stream=stream)
        q.qgemv(wb.fmt, db.codes, db.scales, None, xb, yb, 5000, 5120, 1, wsb, stream=stream)
        q.qembed(wu.fmt, du.codes, du.scales, du.biases, idx8, rows, M, K, 8, stream=stream)

    work(s)
    torch.cuda.synchronize()
    outs = (logits8, idx8, idx64, yb, rows)
    want = [t.clone() for t in outs]
    # the eager results themselves are right
    ref8, _ = orc.qgemv(wu.fmt, wu.codes, wu.scales, wu.biases, x8.cpu().numpy(), M, K)
    assert np.array_equal(idx8.cpu().numpy(), orc.argmax(ref8)[0])
    e = orc.embed(wu.codes, wu.scales, wu.biases, idx8.cpu().numpy(), M, K)
    assert np.array_equal(rows.cpu().numpy().reshape(8, K).view(np.uint32), e.view(np.uint32))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        work(s)
    for rep in range(4):
        for t in (logits8, yb, rows):
            t.fill_(float("nan"))
        idx8.fill_(-1)
        idx64.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager result"
        work(s)
        torch.cuda.synchronize()
        for w in (ws8, ws64, wsb):
            w[:q.QG_WS_CONTROL_BYTES].random_(0, 256)


# ---------------------------------------------------------------------------
# workspaces whose control words hold anything on entry
# ---------------------------------------------------------------------------

GARBAGE_CASES = [
    # (fmt, M, K, batch): the greedy path each one takes
    (synth.U4_G64, 151936, 2048, 1),     # batch-1 kernel, 8-wave workgroups
    (synth.U4_G64, 6000, 6144, 1),       # batch-1 kernel, 4-wave workgroups
    (synth.I8_ROW, 3000, 1024, 1),       # batch-1 8-bit
    (synth.U4_G64, 100000, 2048, 1),     # batch-1 streaming head
    (synth.U4_G64, 40000, 2048, 8),      # batch-8 matrix-core head (parked key rows)
    (synth.U4_G64, 40000, 2048, 4),      # the same at 4 rows
    (synth.I8_ROW, 3000, 1024, 4),       # small-batch kernel, 4 parked key rows
    (synth.U4_G64, 5000, 2048, 16),      # one-pass 16-row head
    (synth.B1_G128, 5000, 5120, 1),      # 1-bit lookup, K chunks combined in the kernel
    (synth.B1_G128, 70000, 5120, 3),     # 1-bit lookup, more tiles than completion words
    (synth.I8_ROW, 2000, 20000, 2),      # vector-ALU kernel with K split: combine launch
    (synth.I8_ROW, 3000, 1040, 2),       # vector-ALU kernel, one K range
]


@pytest.mark.parametrize("fmt,M,K,N", GARBAGE_CASES)
def test_greedy_with_garbage_control_words(torch, orc, fmt, M, K, N):
    """Control words and scratch that hold anything on entry (all ones,
    random bytes, words left by a call of another shape, the previous call's
    own leftovers) still give the oracle's indices on every call."""
    say(f"garbage control words fmt={fmt} M={M} K={K} N={N}")
    rng = synth.rng_for(500 + fmt, M + N)
    w = synth.draw_weights(fmt, M, K, rng)
    x = synth.draw_x(N, K, rng)
    ref, a = orc.qgemv(fmt, w.codes, w.scales, w.biases, x, M, K)
    want, _ = orc.argmax(ref)
    wd = dev(w)
    xd = torch.from_numpy(x).cuda()
    need = max(q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, fmt, M, K, N),
               q.qg_workspace_bytes(q.QG_OP_GEMV_ARGMAX, synth.U4_G64, 4000, 1024, 1))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    other = synth.draw_weights(synth.U4_G64, 4000, 1024, rng)
    od = dev(other)
    ox = torch.from_numpy(synth.draw_x(1, 1024, rng)).cuda()
    oy = torch.empty(4000, device="cuda")
    oi = torch.empty(1, dtype=torch.int32, device="cuda")
    fills = ["ones", "random", "other call", "previous call", "random"]
    for i, how in enumerate(fills):
        if how == "ones":
            ws.fill_(0xFF)
        elif how == "random":
            ws.random_(0, 256)
        elif how == "other call":
            q.qgemv_argmax(other.fmt, od.codes, od.scales, od.biases, ox, oy, oi, 4000, 1024, 1, ws)
        y = torch.empty(N * M, device="cuda")
        idx = torch.full((N,), -7, dtype=torch.int32, device="cuda")
        q.qgemv_argmax(fmt, wd.codes, wd.scales, wd.biases, xd, y, idx, M, K, N, ws)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        say(f"  {how}: idx {got.tolist()} oracle {want.tolist()}")
        assert np.array_equal(got, want), f"{how}: idx differs from the oracle"
        if i == 0:
            check_bound(y.cpu().numpy().reshape(N, M), ref, a, f"garbage {how}")


# ---------------------------------------------------------------------------
# the batch-1 4-bit kernel with loader waves (large M, K = 2048, 4096, 8192)
# ---------------------------------------------------------------------------

STREAM_SHAPES = [(32768, 2048), (151937, 2048), (40001, 2048), (16384 + 5, 4096), (8192 * 3 + 7, 8192)]


@pytest.mark.parametrize("M,K", STREAM_SHAPES)
def test_stream_kernel_random(torch, orc, M, K):
    """Random inputs, with and without the greedy index and logits; every
    workgroup's run of rows ends in a partial stage at these M."""
    say(f"stream kernel M={M} K={K}")
    rng = synth.rng_for(600, M + K)
    w = synth.draw_weights(synth.U4_G64, M, K, rng)
    x = synth.draw_x(1, K, rng)
    ref, a = orc.qgemv(w.fmt, w.codes, w.scales, w.biases, x, M, K)
    wd = dev(w)
    y, _ = gpu_gemv(torch, wd, x)
    check_bound(y, ref, a, f"stream {M}x{K}")
    y2, idx = gpu_gemv(torch, wd, x, argmax=True)
    assert np.array_equal(y, y2), "logits differ from the plain product"
    check_argmax(idx, y2, ref, a, orc, f"stream {M}x{K}")
    _, idx3 = gpu_greedy(torch, wd, x, logits=False)
    assert np.array_equal(idx, idx3), "greedy index without logits differs"


@pytest.mark.parametrize("M,K", [(40000, 2048), (100000, 2048), (20000, 4096), (9000, 8192), (50001, 8192)])
def test_stream_kernel_exact(torch, orc, M, K):
    """Exact-arithmetic inputs: bit-exact against the oracle, the plain
    product and the greedy head's logits and index."""
    say(f"stream kernel exact M={M} K={K}")
    rng = np.random.default_rng([7, M, K])
    w, x = exact_inputs(synth.U4_G64, M, K, 1, rng)
    ref, _ = orc.qgemv(w.fmt, w.codes, w.scales, w.biases, x, M, K)
    want = ref.astype(np.float32)
    assert np.array_equal(want.astype(np.float64), ref), "fixture is not exact in float32"
    wd = dev(w)
    y, _ = gpu_gemv(torch, wd, x)
    assert np.array_equal(y, want), f"not bit-exact: max diff {np.max(np.abs(y - want))}"
    y2, idx = gpu_gemv(torch, wd, x, argmax=True)
    assert np.array_equal(y2, want), f"greedy logits not bit-exact: max diff {np.max(np.abs(y2 - want))}"
    assert idx[0] == int(np.argmax(want[0])), "greedy index"


def test_stream_kernel_ties(torch, orc):
    """Ties of the maximum across workgroups and within a stage: rows
    duplicated at the first row, in the middle of a stage, at the last row
    of a workgroup's run and at the last row; the lowest index wins."""
    M, K = 151936, 2048
    say("stream kernel ties")
    rng = synth.rng_for(601, 0)
    w = synth.draw_weights(synth.U4_G64, M, K, rng)
    x = synth.draw_x(1, K, rng)
    ref, _ = orc.qgemv(w.fmt, w.codes, w.scales, w.biases, x, M, K)
    best = int(np.argmax(ref[0]))
    codes, scales, biases = w.codes.copy(), w.scales.copy(), w.biases.copy()
    per_wg = M // 256
    for dst in (per_wg * 37 - 1, per_wg * 37 + 13, M - 1, 5, 131072, 140000 + 17, best):
        codes[dst], scales[dst], biases[dst] = codes[best], scales[best], biases[best]
    w2 = synth.QWeights(w.fmt, M, K, codes, scales, biases)
    ref2, a2 = orc.qgemv(w2.fmt, w2.codes, w2.scales, w2.biases, x, M, K)
    y, idx = gpu_gemv(torch, dev(w2), x, argmax=True)
    check_bound(y, ref2, a2, "stream ties")
    check_argmax(idx, y, ref2, a2, orc, "stream ties")
    assert idx[0] == 5


# ---------------------------------------------------------------------------
# 2..8 activation rows, 4-bit, K = 2048, large M: loader waves + matrix cores
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N", [(32768, 8), (151937, 2), (40001, 3), (100001, 4), (70000, 5), (151936, 8), (33000, 7)])
def test_stream_mfma_kernel_random(torch, orc, M, N):
    """Random inputs, with and without the greedy indices and logits; every
    workgroup's run of rows ends in a partial stage at most of these M."""
    K = 2048
    say(f"stream mfma kernel M={M} N={N}")
    rng = synth.rng_for(610, M + N)
    w = synth.draw_weights(synth.U4_G64, M, K, rng)
    x = synth.draw_x(N, K, rng)
    ref, a = orc.qgemv(w.fmt, w.codes, w.scales, w.biases, x, M, K)
    wd = dev(w)
    y, _ = gpu_gemv(torch, wd, x)
    check_bound(y, ref, a, f"stream mfma {M} n{N}")
    y2, idx = gpu_gemv(torch, wd, x, argmax=True)
    assert np.array_equal(y, y2), "logits differ from the plain product"
    check_argmax(idx, y2, ref, a, orc, f"stream mfma {M} n{N}")
    _, idx3 = gpu_greedy(torch, wd, x, logits=False)
    assert np.array_equal(idx, idx3), "greedy indices without logits differ"


@pytest.mark.parametrize("M,N", [(40000, 8), (33001, 2), (65536, 5)])
def test_stream_mfma_kernel_exact(torch, orc, M, N):
    """Exact-arithmetic inputs: bit-exact against the oracle."""
    K = 2048
    say(f"stream mfma kernel exact M={M} N={N}")
    rng = np.random.default_rng([8, M, N])
    w, x = exact_inputs(synth.U4_G64, M, K, N, rng)
    ref, _ = orc.qgemv(w.fmt, w.codes, w.scales, w.biases, x, M, K)
    want = ref.astype(np.float32)
    assert np.array_equal(want.astype(np.float64), ref), "fixture is not exact in float32"
    y, _ = gpu_gemv(torch, dev(w), x)
    assert np.array_equal(y, want), f"not bit-exact: max diff {np.max(np.abs(y - want))}"


def test_stream_mfma_kernel_ties(torch, orc):
    """Per activation row, ties of its maximum across workgroups and within
    a stage (rows duplicated at the first row, mid-stage, at the end of a
    workgroup's run, at the last row); the lowest index wins in every row."""
    M, K, N = 151936, 2048, 8
    say("stream mfma kernel ties")
    rng = synth.rng_for(611, 0)
    w = synth.draw_weights(synth.U4_G64, M, K, rng)
    x = synth.draw_x(N, K, rng)
    ref, _ = orc.qgemv(w.fmt, w.codes, w.scales, w.biases, x, M, K)
    codes, scales, biases = w.codes.copy(), w.scales.copy(), w.biases.copy()
    per_wg = M // 256
    # activation row 3's best row copied to the tie positions
    best = int(np.argmax(ref[3]))
    for dst in (per_wg * 37 - 1, per_wg * 37 + 13, M - 1, 5, 131072, 140000 + 17, best):
        codes[dst], scales[dst], biases[dst] = codes[best], scales[best], biases[best]
    w2 = synth.QWeights(w.fmt, M, K, codes, scales, biases)
    ref2, a2 = orc.qgemv(w2.fmt, w2.codes, w2.scales, w2.biases, x, M, K)
    y, idx = gpu_gemv(torch, dev(w2), x, argmax=True)
    check_bound(y, ref2, a2, "stream mfma ties")
    check_argmax(idx, y, ref2, a2, orc, "stream mfma ties")
    assert idx[3] == 5
