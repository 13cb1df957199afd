"""GPU parity of the one-launch MoE GEMV (Q4_0) against the oracle: each
expert slot has its own pool matrix and its own token, so a wrong index or a
mixed-up token fails [volta-kernel-bakeoff, "Making it fair"]."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import Q4_0, assert_within, pack_both, qg, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _pool(P, N, K, seed, edit=None):
    """The pool's library bytes and oracle bytes (each expert packed by both
    packers and compared); `edit(pw)` may change the fp32 experts first."""
    pw = si.expert_pool(P, N, K, seed=seed)
    if edit is not None:
        edit(pw)
    both = [pack_both(Q4_0, pw[j]) for j in range(P)]
    return np.concatenate([b[0] for b in both]), np.concatenate([b[1] for b in both])


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


@pytest.mark.parametrize("kind", ["large", "tiny"])
def test_moe_stress_activations(kind):
    """Planted large (+-20000..60000) and tiny (binary16 subnormal) tokens
    [volta-kernel-bakeoff, "Results", the few-tokens bullet on precision]."""
    P, E, N, K = 16, 10, 640, 2560
    pb, po = _pool(P, N, K, seed=21)
    idx = si.expert_indices(P, E, seed=21)
    x = si.stress_activations(E, K, seed=21, kind=kind)
    y = _moe(to_dev(pb), P, idx, x, N, K)
    y_ref, s = oracle.get().moe(Q4_0, po, P, idx, x, N, K)
    assert_within(y, y_ref, s, f"moe stress {kind}")


@pytest.mark.parametrize("K", [32, 96, 2048])
def test_moe_outliers_on_zero_weights(K):
    """Tokens near the binary16 limit on columns whose weights are exactly zero
    in every expert: the exact result is the small remainder."""
    P, E, N = 6, 5, 96
    g = np.random.default_rng([K, 63])
    cols = g.choice(K, 3, replace=False)

    def zero_cols(pw):
        pw[:, :, cols] = 0.0
    pb, po = _pool(P, N, K, seed=K, edit=zero_cols)
    idx = np.array([5, 0, 3, 3, 1], np.int32)
    x = si.activations(E, K, seed=K + 3)
    x[:, cols[0]] = 60000.0
    x[1::2, cols[0]] = -60000.0
    x[:, cols[1]] = -30000.0
    x[:, cols[2]] = 65504.0
    y = _moe(to_dev(pb), P, idx, x, N, K)
    y_ref, s = oracle.get().moe(Q4_0, po, P, idx, x, N, K)
    assert_within(y, y_ref, s, f"moe outliers K={K}")


def test_moe_zero_and_degenerate_blocks():
    """An all-zero expert, all-zero rows and blocks, subnormal binary16 scales
    and a single non-zero weight, and a zero token (exact zeros)."""
    P, E, N, K = 5, 6, 40, 2560

    def degenerate(pw):
        pw[0] = 0.0
        pw[1, 0, :] = 0.0
        pw[1, 1, 32:64] = 0.0
        pw[2] *= np.float32(1e-6)
        pw[3, 3, :] = 0.0
        pw[3, 3, 100] = np.float32(0.5)
    pb, po = _pool(P, N, K, seed=5, edit=degenerate)
    idx = np.array([0, 1, 2, 3, 4, 1], np.int32)
    x = si.activations(E, K, seed=5)
    x[5] = 0.0
    y = _moe(to_dev(pb), P, idx, x, N, K)
    y_ref, s = oracle.get().moe(Q4_0, po, P, idx, x, N, K)
    assert_within(y, y_ref, s, "moe degenerate")
    assert (y[0] == 0).all() and (y[5] == 0).all()


def test_moe_index_outside_pool_gives_nan_slot():
    """A slot whose index lies outside 0..P-1 (negative, P, far beyond) reads
    no weight and returns NaN in every output; the other slots are unchanged
    and correct."""
    P, E, N, K = 4, 5, 300, 2048
    pb, po = _pool(P, N, K, seed=11)
    pd = to_dev(pb)
    x = si.activations(E, K, seed=11)
    good = np.array([2, 0, 3, 1, 2], np.int32)
    y_good = _moe(pd, P, good, x, N, K)
    for bad_slot, bad in ((1, -1), (3, P), (0, 1 << 30), (4, -(1 << 31))):
        idx = good.copy()
        idx[bad_slot] = bad
        y = _moe(pd, P, idx, x, N, K)
        y_ref, s = oracle.get().moe(Q4_0, po, P, idx, x, N, K)
        assert np.isnan(y[bad_slot]).all() and np.isnan(y_ref[bad_slot]).all()
        keep = [e for e in range(E) if e != bad_slot]
        assert np.array_equal(y[keep], y_good[keep])
        assert_within(y[keep], y_ref[keep], s[keep], f"moe slots beside index {bad}")
