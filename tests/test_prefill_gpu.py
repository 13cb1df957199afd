"""GPU parity of the Q4_0 prefill GEMM (fp16 matrix cores, fp32 accumulate)
against the oracle, and of the dense fp16 comparator as a control."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import Q4_0, assert_within, pack_both, qg, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _prefill(Wd, X, N, K):
    Y = qg().qgemm_q4_0_prefill(Wd, to_dev(X), N, K)
    torch_cuda().cuda.synchronize()
    return Y.cpu().numpy()


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (5, 33, 96), (64, 129, 2560), (65, 300, 640), (130, 257, 2048),
                                   (200, 64, 4096), (17, 1000, 32), (3, 4099, 160), (256, 128, 6144)])
def test_prefill_small_parity(M, N, K):
    w = si.weights(N, K, seed=M + N)
    X = si.activations(M, K, seed=K)
    pb, po = pack_both(Q4_0, w)
    Y = _prefill(to_dev(pb), X, N, K)
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    assert_within(Y, Y_ref, S, f"prefill M={M} {N}x{K}")


@pytest.mark.parametrize("N,K", si.PREFILL_SHAPES)
def test_prefill_m64_full(N, K):
    """Every output of the 64-token prefill on the three table shapes."""
    M = 64
    w = si.weights(N, K, seed=0)
    X = si.activations(M, K, seed=0)
    pb, po = pack_both(Q4_0, w)
    Y = _prefill(to_dev(pb), X, N, K)
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    assert_within(Y, Y_ref, S, f"prefill M=64 {N}x{K}")


@pytest.mark.parametrize("N,K", si.PREFILL_SHAPES)
def test_prefill_m512_sampled(N, K):
    """512 tokens: sampled tokens x sampled columns against the oracle, plus
    the whole output against the dense fp16 comparator's bound."""
    M = 512
    torch = torch_cuda()
    w = si.weights(N, K, seed=0)
    X = si.activations(M, K, seed=0)
    pb, po = pack_both(Q4_0, w)
    Wd = to_dev(pb)
    Y = _prefill(Wd, X, N, K)
    g = np.random.default_rng([N, K])
    toks = np.unique(np.concatenate([[0, 1, M - 1], g.choice(M, 29, replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], g.choice(N, 254, replace=False)]))
    sub = np.ascontiguousarray(X[toks])
    y_ref, s = oracle.get().gemv_rows(Q4_0, po, N, K, sub, cols)
    assert_within(Y[np.ix_(toks, cols)], y_ref, s, f"prefill M=512 {N}x{K} sampled")
    assert np.isfinite(Y).all()
    # the comparator path: dequantize to fp16 on the GPU, dense fp16 GEMM
    W16 = qg().qdequant_q4_0(Wd, N, K, fp16=True)
    Yd = torch.matmul(to_dev(X), W16.t().contiguous()).float()
    torch.cuda.synchronize()
    Yd = Yd.cpu().numpy()
    assert_within(Yd[np.ix_(toks, cols)], y_ref, s, "dense fp16 comparator")


def test_prefill_wide_tile_full():
    """The 128 x 192 tile the launcher picks when it gives every CU exactly
    one workgroup (384 tokens x 16000 rows on 256 CUs): every output against
    the oracle, with a ragged last tile along N and an odd block count along
    K (the last K step holds one block)."""
    M, N, K = 384, 16000, 96
    cus = qg().qg_device_cus()
    t128 = -(-N // 128) * 3
    t192 = -(-N // 192) * 3
    if not (t128 > cus and t192 <= cus and t192 * 8 >= cus * 7):
        pytest.skip(f"the wide tile is not chosen on {cus} CUs")
    w = si.weights(N, K, seed=7)
    X = si.activations(M, K, seed=7)
    pb, po = pack_both(Q4_0, w)
    Y = _prefill(to_dev(pb), X, N, K)
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    assert_within(Y, Y_ref, S, f"prefill wide tile M={M} {N}x{K}")


def test_prefill_one_hot_is_the_fp16_dequant_column():
    """X = e_k returns fp16-rounded column k bit-exactly (pins the tile layout
    and the permuted k order)."""
    N, K = 200, 2560
    w = si.weights(N, K, seed=2)
    pb, po = pack_both(Q4_0, w)
    cols = [0, 1, 2, 3, 15, 16, 17, 31, 32, 63, 64, 100, 1279, 2559]
    X = np.zeros((len(cols), K), np.float16)
    for i, k in enumerate(cols):
        X[i, k] = 1.0
    Y = _prefill(to_dev(pb), X, N, K)
    w16 = oracle.get().dequant(Q4_0, po, N, K, "f16").astype(np.float32)
    for i, k in enumerate(cols):
        assert np.array_equal(Y[i], w16[:, k]), f"column {k}"


def test_prefill_sabotage_fails_dense_control_passes():
    torch = torch_cuda()
    M, N, K = 64, 256, 2048
    w = si.weights(N, K, seed=4)
    X = si.activations(M, K, seed=4)
    pb, po = pack_both(Q4_0, w)
    bad = pb.copy()
    nb = N * K // 32
    bad[:nb * 16] ^= 0x11
    bad[nb * 16 + 1:nb * 16 + 2 * nb:2] ^= 0x80
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    Yb = _prefill(to_dev(bad), X, N, K)
    assert not oracle.within_bound(Yb, Y_ref, S).all()
    # control: dense fp16 GEMM on the clean fp16 weights passes
    W16 = torch.from_numpy(oracle.get().dequant(Q4_0, po, N, K, "f16")).cuda()
    Yd = torch.matmul(to_dev(X), W16.t().contiguous()).float()
    torch.cuda.synchronize()
    assert oracle.within_bound(Yd.cpu().numpy(), Y_ref, S).all()


def test_prefill_abi_errors():
    torch = torch_cuda()
    q = qg()
    L = q.lib()
    W = torch.zeros(q.qpacked_bytes_q4_0(64, 256), dtype=torch.uint8, device="cuda")
    X = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    Y = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    s = q._stream()
    assert L.qgemm_q4_0_prefill(None, X.data_ptr(), Y.data_ptr(), 4, 64, 256, s) == 1
    assert L.qgemm_q4_0_prefill(W.data_ptr(), X.data_ptr(), Y.data_ptr(), 0, 64, 256, s) == 2
    assert L.qgemm_q4_0_prefill(W.data_ptr(), X.data_ptr(), Y.data_ptr(), 4, 64, 250, s) == 2
    assert L.qgemm_q4_0_prefill(W.data_ptr() + 8, X.data_ptr(), Y.data_ptr(), 4, 64, 256, s) == 3
