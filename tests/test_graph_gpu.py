"""GPU: every entry point captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed several times, with the program's own eager work and
synchronizations between the replays; each replay must match the eager call
(bitwise for the GEMV and MoE kernels, which use no atomics; within the
oracle's bound for the split-K prefill, whose atomic adds may reorder the
last bits).  The launches record no memset: the prefill's zero fill of a
split-K output is a kernel."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import Q4_0, Q8_0, assert_within, pack_both, qg, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _replays_match(run, out, check):
    """Eager result, then a captured graph of `run` replayed REPLAYS times;
    `check(replay_result, eager_result)` after every replay."""
    torch = torch_cuda()
    run()
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    scratch = torch.empty_like(out)
    for r in range(REPLAYS):
        out.fill_(float("nan"))              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(out.cpu().numpy(), eager, r)
        scratch.copy_(out).mul_(2.0)         # more eager work on the result
        torch.cuda.synchronize()
    del g


@pytest.mark.parametrize("fmt,M,N,K", [(Q4_0, 1, 4096, 4096), (Q4_0, 1, 28672, 4096), (Q4_0, 8, 8192, 2048),
                                       (Q8_0, 2, 6144, 2048), (Q4_0, 3, 2048, 6144)])
def test_gemv_graph_replay_is_bitwise_eager(fmt, M, N, K):
    q = qg()
    w = si.weights(N, K, seed=3)
    x = si.activations(M, K, seed=3)
    pb, _ = pack_both(fmt, w)
    Wd, xd = to_dev(pb), to_dev(x)
    y = torch_cuda().empty((M, N), dtype=torch_cuda().float32, device="cuda")
    f = q.qgemv_q4_0 if fmt == Q4_0 else q.qgemv_q8_0

    def check(rep, eager, r):
        assert np.array_equal(rep.view(np.uint32), eager.view(np.uint32)), f"replay {r} differs from eager"

    _replays_match(lambda: f(Wd, xd, N, K, y), y, check)


def test_moe_graph_replay_is_bitwise_eager():
    q = qg()
    torch = torch_cuda()
    P, E, N, K = 16, 8, 512, 2048
    w = si.weights(P * N, K, seed=5)
    pool = np.concatenate([q.qquantize_q4_0(w[p * N:(p + 1) * N]) for p in range(P)])
    idx = np.random.default_rng(5).choice(P, E, replace=False).astype(np.int32)
    x = si.activations(E, K, seed=5)
    pd, idd, xd = to_dev(pool), to_dev(idx), to_dev(x)
    y = torch.empty((E, N), dtype=torch.float32, device="cuda")

    def check(rep, eager, r):
        assert np.array_equal(rep.view(np.uint32), eager.view(np.uint32)), f"replay {r} differs from eager"

    _replays_match(lambda: q.qmoe_gemv_q4_0(pd, P, idd, xd, N, K, y), y, check)


def test_prefill_split_k_graph_replay_within_bound():
    """2560 x 6144 at 64 tokens splits K (zero-fill kernel, atomic adds)."""
    q = qg()
    torch = torch_cuda()
    M, N, K = 64, 2560, 6144
    w = si.weights(N, K, seed=9)
    X = si.activations(M, K, seed=9)
    pb, po = pack_both(Q4_0, w)
    Wd, Xd = to_dev(pb), to_dev(X)
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y_ref, s = oracle.get().prefill(po, N, K, X)

    def check(rep, eager, r):
        assert np.isfinite(rep).all(), f"replay {r}: non-finite output (zero fill not replayed?)"
        assert_within(rep, y_ref, s, f"prefill graph replay {r}")

    _replays_match(lambda: q.qgemm_q4_0_prefill(Wd, Xd, N, K, Y), Y, check)


@pytest.mark.parametrize("M,N,K", [(1, 6144, 2048), (4, 640, 2560)])
def test_f32in_and_swiglu_graph_replay_is_bitwise_eager(M, N, K):
    q = qg()
    torch = torch_cuda()
    x = to_dev(si.activations32(M, K, seed=7))
    w1 = si.weights(N, K, seed=7)
    w2 = np.concatenate([w1, si.weights(N, K, seed=8)])
    Wd1, Wd2 = to_dev(q.qquantize_q4_0(w1)), to_dev(q.qquantize_q4_0(w2))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def check(rep, eager, r):
        assert np.array_equal(rep.view(np.uint32), eager.view(np.uint32)), f"replay {r} differs from eager"

    _replays_match(lambda: q.qgemv_q4_0_f32in(Wd1, x, N, K, y), y, check)
    _replays_match(lambda: q.qgemv_q4_0_swiglu_f32in(Wd2, x, N, K, y), y, check)
