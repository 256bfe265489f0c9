"""qgemv_argmax_noalloc (the greedy head without a caller workspace, for
callers that cannot allocate) against qgemv_argmax with a workspace, on the
GPU through the C ABI: two calls in a row, the second smaller, each equal
to the workspace call bit for bit and to the oracle within the bound, with
the oracle's argmax."""
import numpy as np
import pytest

import gemm_qgemv_amd as q
import oracle
from gemm_qgemv_amd import synth, tensors

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "these tests need the GPU"
    return t


def run_both(torch, orc, fmt, M, K, N, seed):
    say(f"noalloc fmt={fmt} M={M} K={K} N={N}")
    rng = synth.rng_for(900 + seed, M + N)
    w = synth.draw_weights(fmt, M, K, rng)
    x = synth.draw_x(N, K, rng)
    wd = tensors.to_device(w)
    xd = torch.from_numpy(x).cuda()
    y_a = torch.full((N * M,), float("nan"), device="cuda")
    i_a = torch.full((N,), -7, dtype=torch.int32, device="cuda")
    q.qgemv_argmax_noalloc(fmt, wd.codes, wd.scales, wd.biases, xd, y_a, i_a, M, K, N)
    torch.cuda.synchronize()
    y_b = torch.full((N * M,), float("nan"), device="cuda")
    i_b = torch.full((N,), -7, dtype=torch.int32, device="cuda")
    ws = tensors.workspace(q.QG_OP_GEMV_ARGMAX, fmt, M, K, N)
    q.qgemv_argmax(fmt, wd.codes, wd.scales, wd.biases, xd, y_b, i_b, M, K, N, ws)
    torch.cuda.synchronize()
    ya, yb = y_a.cpu().numpy(), y_b.cpu().numpy()
    ia, ib = i_a.cpu().numpy(), i_b.cpu().numpy()
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), "logits differ from qgemv_argmax"
    assert np.array_equal(ia, ib), "indices differ from qgemv_argmax"
    ref, a = orc.qgemv(fmt, w.codes, w.scales, w.biases, x, M, K)
    err = np.abs(ya.reshape(N, M).astype(np.float64) - ref)
    assert np.all(np.isfinite(ya)) and np.all(err <= 1e-5 * a), "logits outside the bound"
    want, _ = orc.argmax(ref)
    assert np.array_equal(ia, want), "indices differ from the oracle"
    say(f"  idx {ia.tolist()}")


def test_noalloc_matches_workspace_call_twice(torch):
    orc = oracle.get()
    # the 151936 x 2048 4-bit head at batch 8, then a smaller call (batch 1)
    run_both(torch, orc, synth.U4_G64, 151936, 2048, 8, 0)
    run_both(torch, orc, synth.U4_G64, 6144, 2048, 1, 1)


def test_noalloc_other_paths_twice(torch):
    orc = oracle.get()
    # the prefill-shaped head (64 rows, per-tile keys), then the 1-bit
    # lookup kernel with its K chunks combined in the kernel
    run_both(torch, orc, synth.U4_G64, 30000, 2048, 64, 2)
    run_both(torch, orc, synth.B1_G128, 5000, 5120, 1, 3)
