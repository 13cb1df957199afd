"""GPU parity of the one-launch MoE GEMV (Q4_0) against the oracle: each
expert slot has its own pool matrix and its own token, so a wrong index or a
mixed-up token fails [volta-kernel-bakeoff, "Making it fair"]."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import Q4_0, assert_within, qg, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _pool(P, N, K, seed):
    q = qg()
    o = oracle.get()
    pw = si.expert_pool(P, N, K, seed=seed)
    pb = np.concatenate([q.qquantize_q4_0(pw[j]) for j in range(P)])
    po = np.concatenate([o.quantize(Q4_0, pw[j]) for j in range(P)])
    assert np.array_equal(pb, po)
    return pb, po


def _moe(pool_d, P, idx, x, N, K):
    q = qg()
    y = q.qmoe_gemv_q4_0(pool_d, P, to_dev(idx), to_dev(x), N, K)
    torch_cuda().cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("P,E,N,K", [(12, 10, 640, 2560), (24, 8, 512, 2048), (5, 3, 65, 96), (4, 7, 33, 4096)])
def test_moe_parity(P, E, N, K):
    pb, po = _pool(P, N, K, seed=P)
    g = np.random.default_rng([P, E])
    idx = g.integers(0, P, size=E).astype(np.int32)       # repeats allowed
    x = si.activations(E, K, seed=E)
    y = _moe(to_dev(pb), P, idx, x, N, K)
    y_ref, s = oracle.get().moe(Q4_0, po, P, idx, x, N, K)
    assert_within(y, y_ref, s, f"moe {E} of {P} x {N}x{K}")


@pytest.mark.parametrize("P,E,N,K", [tuple(c) for c in si.MOE_CONFIGS])
def test_moe_full_pool(P, E, N, K):
    """The full pools (10 of 128 experts 640x2560; 8 of 256 experts 512x2048),
    seeded distinct indices, several draws."""
    pb, po = _pool(P, N, K, seed=0)
    pd = to_dev(pb)
    for call in range(3):
        idx = si.expert_indices(P, E, seed=0, call=call)
        x = si.activations(E, K, seed=call)
        y = _moe(pd, P, idx, x, N, K)
        y_ref, s = oracle.get().moe(Q4_0, po, P, idx, x, N, K)
        assert_within(y, y_ref, s, f"moe call {call}")


def test_moe_wrong_index_fails_and_slots_are_independent():
    P, E, N, K = 8, 4, 128, 2560
    pb, po = _pool(P, N, K, seed=3)
    pd = to_dev(pb)
    idx = np.array([6, 1, 4, 1], np.int32)
    x = si.activations(E, K, seed=9)
    y = _moe(pd, P, idx, x, N, K)
    y_ref, s = oracle.get().moe(Q4_0, po, P, idx, x, N, K)
    assert_within(y, y_ref, s, "moe")
    # a different index in slot 2 changes exactly that slot
    idx2 = idx.copy()
    idx2[2] = 5
    y2 = _moe(pd, P, idx2, x, N, K)
    assert np.array_equal(y2[[0, 1, 3]], y[[0, 1, 3]])
    assert not oracle.within_bound(y2[2], y_ref[2], s[2]).all()
    # each slot equals the plain GEMV of its expert
    q = qg()
    stride = q.qpacked_bytes_q4_0(N, K)
    for e in range(E):
        ye = q.qgemv_q4_0(pd[idx[e] * stride:(idx[e] + 1) * stride], to_dev(x[e:e + 1]), N, K)
        torch_cuda().cuda.synchronize()
        assert np.array_equal(ye.cpu().numpy()[0], y[e])
