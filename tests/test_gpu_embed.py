"""GPU parity of the embedding gather (qembed, through the C ABI) against the
oracle's row decoder on the same seeded tables and ids.

Bar: bit-exact. Every value the oracle decodes (including -0, binary16
subnormals and infinities) has the same float32 bits on the GPU; NaNs sit in
the same places; a row whose id lies outside the table is all quiet NaN;
guard bands around the output stay untouched; repeated calls give the same
bits.
"""
import numpy as np
import pytest

import gemm_qgemv_amd as q
import oracle
from gemm_qgemv_amd import synth, tensors

pytestmark = pytest.mark.gpu
PAD = 64
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


def gpu_embed(torch, w, ids, dw=None):
    """qembed of ids (numpy int32) from table w; returns float32 [n][K]."""
    dw = dw or tensors.to_device(w)
    n = len(ids)
    idd = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    full = torch.full((n * w.K + 2 * PAD,), CANARY, dtype=torch.float32, device="cuda")
    out = full[PAD:PAD + n * w.K]
    q.qembed(w.fmt, dw.codes, dw.scales, dw.biases, idd, out, w.M, w.K, n)
    torch.cuda.synchronize()
    f = full.cpu().numpy()
    assert np.all(f[:PAD] == CANARY) and np.all(f[-PAD:] == CANARY), "guard band overwritten"
    return f[PAD:PAD + n * w.K].reshape(n, w.K)


def check_same(got, want, ids, M, what):
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    if not np.array_equal(nan_g, nan_w):
        t, k = np.argwhere(nan_g != nan_w)[0]
        raise AssertionError(f"{what}: NaN placement differs first at row {t} (id {ids[t]}) k {k}: "
                             f"gpu {got[t, k]!r} oracle {want[t, k]!r}")
    gb, wb = got.view(np.uint32), want.view(np.uint32)
    bad = (gb != wb) & ~nan_g
    if bad.any():
        t, k = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} values differ; first row {t} (id {ids[t]}) "
                             f"k {k}: gpu {gb[t, k]:#010x} oracle {wb[t, k]:#010x}")
    outside = (ids < 0) | (ids >= M)
    if outside.any():
        rows = got[outside]
        assert np.all(np.isnan(rows)), f"{what}: a row outside the table is not all NaN"
        assert np.all(rows.view(np.uint32) & 0x00400000), f"{what}: NaN rows must be quiet NaNs"


def stress_ids(M, rng, extra=()):
    """Every row once (shuffled), some repeats, and ids outside the table."""
    ids = np.concatenate([rng.permutation(M), rng.integers(0, M, size=M // 4 + 1),
                          np.array([-1, M, M + 7, -(2 ** 31), 2 ** 31 - 1, *extra])])
    return rng.permutation(ids).astype(np.int32)


@pytest.mark.parametrize("M,K", [(2000, 512), (613, 64), (97, 2048), (40, 4096 + 64)])
def test_embed_stress_bit_exact(torch, orc, M, K):
    say(f"embed stress M={M} K={K}")
    rng = synth.rng_for(90, K)
    w = synth.draw_embed_stress(M, K, rng)
    ids = stress_ids(M, rng)
    want = orc.embed(w.codes, w.scales, w.biases, ids, M, K)
    got = gpu_embed(torch, w, ids)
    check_same(got, want, ids, M, f"stress {M}x{K}")
    # the table holds every corner the decode has
    inside = got[(ids >= 0) & (ids < M)]
    fin = inside[np.isfinite(inside)]
    assert np.any((fin == 0) & np.signbit(fin)), "no -0 in the stress table"
    assert np.any((fin != 0) & (np.abs(fin) < 2.0 ** -14)), "no binary16 subnormal"
    assert np.any(np.isinf(inside)), "no overflow"


def test_embed_hand_cases(torch, orc):
    """One group per hand-derived IEEE case (scale, bias, code -> value):
    the tie and near-tie roundings, -0 from a tiny negative sum, +0 from
    -0 + +0, the binary16 overflow, an exactly representable value."""
    cases = [
        (0.5, -1.0, 3, 0.5),
        (1.0, -2.0 ** -30, 0, -0.0),
        (1.0, -3 * 2.0 ** -26, 0, -2.0 ** -24),
        (1.0, -2.0 ** -25, 0, -0.0),
        (8192.0, 0.0, 15, np.inf),
        (1.0, 2.0 ** -11, 1, 1.0),
        (1.0, 3 * 2.0 ** -12, 1, 1.0 + 2.0 ** -10),
        (-0.5, 0.0, 0, 0.0),
        (-0.5, -0.0, 0, -0.0),
        (2.0 ** -10, 2.0 ** -14, 1, 2.0 ** -14 + 2.0 ** -10),
    ]
    G = len(cases)
    K = 64 * G
    sc = np.array([c[0] for c in cases], np.float32)
    bi = np.array([c[1] for c in cases], np.float32)
    sb = (sc.view(np.uint32) >> 16).astype(np.uint16)[None, :]
    bb = (bi.view(np.uint32) >> 16).astype(np.uint16)[None, :]
    nib = np.repeat(np.array([c[2] for c in cases], np.uint8), 64)
    codes = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None, :]
    w = synth.QWeights(q.QG_U4_G64, 1, K, codes, sb, bb)
    ids = np.array([0, 0], np.int32)
    got = gpu_embed(torch, w, ids)
    want = orc.embed(codes, sb, bb, ids, 1, K)
    check_same(got, want, ids, 1, "hand cases")
    for g, (s, b, c, v) in enumerate(cases):
        vals = got[0, 64 * g:64 * (g + 1)]
        assert np.all(vals == v) and np.all(np.signbit(vals) == np.signbit(v)), \
            f"case {g}: ({s}, {b}, {c}) gave {vals[0]!r}, expected {v!r}"


@pytest.mark.parametrize("M,K,n", [(1, 64, 1), (5, 64, 70001), (1000, 192, 333), (3, 128, 5)])
def test_embed_shapes(torch, orc, M, K, n):
    """Single row and single id; more ids than the launch has workgroups
    (the grid-stride loop); K of three groups; ids mostly outside a tiny
    table."""
    say(f"embed shape M={M} K={K} n={n}")
    rng = synth.rng_for(91, n)
    w = synth.draw_weights(q.QG_U4_G64, M, K, rng)
    ids = rng.integers(-2, M + 2, size=n).astype(np.int32)
    want = orc.embed(w.codes, w.scales, w.biases, ids, M, K)
    got = gpu_embed(torch, w, ids)
    check_same(got, want, ids, M, f"shape {M}x{K} n={n}")


def test_embed_prompt_workload(torch, orc):
    """The measured workload at full size: the rows of a 2048-token prompt
    from the 151936 x 2048 head matrix, every value compared; the call
    repeated gives the same bits."""
    case = synth.CASES_BY_NAME["n3_u4_embed_151936x2048_t2048"]
    w, ids = synth.case_inputs(case)
    dw = tensors.to_device(w)
    want = orc.embed(w.codes, w.scales, w.biases, ids, w.M, w.K)
    got = gpu_embed(torch, w, ids, dw)
    check_same(got, want, ids, w.M, case.name)
    again = gpu_embed(torch, w, ids, dw)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), "repeated call differs"
