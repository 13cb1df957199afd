"""GPU parity of the Q4_0 prefill GEMM (fp16 matrix cores, fp32 accumulate)
against the oracle, and of the dense fp16 comparator as a control."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import Q4_0, assert_within, check_equal, control_within, pack_both, qg, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _prefill(Wd, X, N, K):
    Y = qg().qgemm_q4_0_prefill(Wd, to_dev(X), N, K)
    torch_cuda().cuda.synchronize()
    return Y.cpu().numpy()


# Launch settings the edge cases run under (persistent workgroups, tile
# configuration): the built-in choice; one workgroup walking every tile
# (whole tiles, plain stores); 3, 7 and 700 workgroups (ranges that cut tiles:
# partial tiles added atomically into a zero-filled Y); every tile
# configuration; the skinny kernel (tile 16, up to 64 tokens) with its
# built-in grid, one workgroup, three, and more workgroups than tiles.
PREFILL_SETTINGS = [(0, 0), (1, 64), (3, 64), (700, 66), (0, 128), (5, 128),
                    (0, 130), (700, 130), (0, 136), (3, 136), (0, 257), (3, 257),
                    (0, 16), (1, 16), (3, 16), (700, 16)]


def _prefill_each_setting(Wd, X, N, K, Y_ref, S, what):
    q = qg()
    try:
        for wgs, tile in PREFILL_SETTINGS:
            if tile == 16 and X.shape[0] > 64:
                continue   # the skinny kernel takes at most 64 tokens
            q.qg_set_prefill_shape(wgs, tile)
            Y = _prefill(Wd, X, N, K)
            assert_within(Y, Y_ref, S, f"{what} workgroups={wgs} tile={tile}")
    finally:
        q.qg_set_prefill_shape(0, 0)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (5, 33, 96), (64, 129, 2560), (65, 300, 640), (130, 257, 2048),
                                   (200, 64, 4096), (17, 1000, 32), (3, 4099, 160), (256, 128, 6144)])
def test_prefill_small_parity(M, N, K):
    """Ragged shapes (tokens, rows and blocks not multiples of a tile or a K
    step) under every launch setting."""
    w = si.weights(N, K, seed=M + N)
    X = si.activations(M, K, seed=K)
    pb, po = pack_both(Q4_0, w)
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    _prefill_each_setting(to_dev(pb), X, N, K, Y_ref, S, f"prefill M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 100, 2048), (7, 17, 32), (16, 4099, 2560), (17, 1000, 2080),
                                   (33, 640, 8192), (48, 257, 6144), (64, 130, 8192), (64, 5000, 96),
                                   (40, 2048, 2560), (64, 31, 16384)])
def test_prefill_skinny_parity(M, N, K):
    """The skinny kernel (up to 64 tokens: activations held in registers,
    weights streamed once) on ragged token, row and block counts, rows of an
    odd number of blocks, and rows long enough to be split over several
    workgroups (parts added atomically into a zero-filled Y), under its
    launch settings; one-hot activations return the fp16-rounded weight
    column exactly."""
    q = qg()
    w = si.weights(N, K, seed=M + K)
    X = si.activations(M, K, seed=N)
    pb, po = pack_both(Q4_0, w)
    Wd = to_dev(pb)
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    try:
        for wgs in (0, 1, 3, 700):
            q.qg_set_prefill_shape(wgs, 16)
            Y = _prefill(Wd, X, N, K)
            assert_within(Y, Y_ref, S, f"skinny M={M} {N}x{K} workgroups={wgs}")
        q.qg_set_prefill_shape(0, 16)
        cols = [0, 31, K // 2, K - 1][:M]
        Xo = np.zeros((len(cols), K), np.float16)
        for i, k in enumerate(cols):
            Xo[i, k] = 1.0
        Yo = _prefill(Wd, Xo, N, K)
        w16 = oracle.get().dequant(Q4_0, po, N, K, "f16").astype(np.float32)
        for i, k in enumerate(cols):
            check_equal(Yo[i], w16[:, k], f"skinny one-hot column {k}", bits=False)
    finally:
        q.qg_set_prefill_shape(0, 0)


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
def test_prefill_m512_full(N, K):
    """512 tokens: every output against the oracle; the GPU's fp16 dequant of
    the same bytes bit-exact; and, as a control that never touches the
    library's packed bytes, the dense fp16 GEMM on the oracle's fp16 weights
    within the same bound."""
    M = 512
    torch = torch_cuda()
    w = si.weights(N, K, seed=0)
    X = si.activations(M, K, seed=0)
    pb, po = pack_both(Q4_0, w)
    del w
    Wd = to_dev(pb)
    Y = _prefill(Wd, X, N, K)
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    assert_within(Y, Y_ref, S, f"prefill M=512 {N}x{K}")
    w16 = oracle.get().dequant(Q4_0, po, N, K, "f16")
    W16 = qg().qdequant_q4_0(Wd, N, K, fp16=True)
    torch.cuda.synchronize()
    check_equal(W16.cpu().numpy(), w16, f"prefill {N}x{K} fp16 dequant")
    Yd = torch.matmul(to_dev(X), to_dev(w16).t().contiguous()).float()
    torch.cuda.synchronize()
    control_within(Yd.cpu().numpy(), Y_ref, S, f"dense fp16 GEMM {N}x{K} M=512")


@pytest.mark.parametrize("N,K,M", [(12288, 2560, 128), (4096, 4096, 512), (14336, 4096, 256)])
def test_prefill_whole_tile_launches_full(N, K, M):
    """Built-in launches whose tile count fills 3/4 to all of the CUs run one
    workgroup per tile, every tile whole (plain stores, no zero fill; on 256
    CUs: 192 tiles of 64 x 128, 256 of 64 x 128, 224 of 128 x 128): every
    output against the oracle, and two calls give the same bits."""
    w = si.weights(N, K, seed=M)
    X = si.activations(M, K, seed=M)
    pb, po = pack_both(Q4_0, w)
    del w
    Wd = to_dev(pb)
    Y = _prefill(Wd, X, N, K)
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    assert_within(Y, Y_ref, S, f"prefill M={M} {N}x{K}")
    Y2 = _prefill(Wd, X, N, K)
    assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32)), f"prefill M={M} {N}x{K}: not bitwise repeatable"


def test_prefill_many_tiles_full():
    """More tiles than workgroup slots (384 tokens x 16000 rows): every output
    against the oracle, with a ragged last tile along N and an odd block
    count along K (the last K step holds one block, the padding steps none)."""
    M, N, K = 384, 16000, 96
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
        check_equal(Y[i], w16[:, k], f"prefill one-hot column {k}", bits=False)


@pytest.mark.parametrize("kind", ["large", "tiny"])
def test_prefill_stress_activations(kind):
    """Planted large (+-20000..60000) and tiny (binary16 subnormal) activations
    [volta-kernel-bakeoff, "Results", the few-tokens bullet on precision];
    fp32 accumulation of the fp16 products must stay inside the bound."""
    M, N, K = 96, 300, 6144
    w = si.weights(N, K, seed=21)
    X = si.stress_activations(M, K, seed=21, kind=kind)
    pb, po = pack_both(Q4_0, w)
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    _prefill_each_setting(to_dev(pb), X, N, K, Y_ref, S, f"prefill stress {kind}")


@pytest.mark.parametrize("K", [32, 96, 640, 4096])
def test_prefill_outliers_on_zero_weights(K):
    """Activations near the binary16 limit (+-60000, -30000, 65504) on columns
    whose weights are exactly zero: the exact result is the small remainder of
    the other columns, and the bound is set by it alone."""
    M, N = 70, 200
    w = si.weights(N, K, seed=K + 3)
    g = np.random.default_rng([K, 62])
    cols = g.choice(K, 3, replace=False)
    w[:, cols] = 0.0
    X = si.activations(M, K, seed=K + 3)
    X[:, cols[0]] = 60000.0
    X[1::2, cols[0]] = -60000.0
    X[:, cols[1]] = -30000.0
    X[:, cols[2]] = 65504.0
    pb, po = pack_both(Q4_0, w)
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    _prefill_each_setting(to_dev(pb), X, N, K, Y_ref, S, f"prefill outliers K={K}")


def test_prefill_zero_and_degenerate_blocks():
    """All-zero rows and blocks (scale 0), subnormal binary16 scales (weights
    that are binary16 subnormals after the fp16 dequant), one non-zero weight
    in a row; and a zero activation matrix gives exact zeros."""
    M, N, K = 80, 160, 2560
    w = si.weights(N, K, seed=5)
    w[0, :] = 0.0
    w[1, 32:64] = 0.0
    w[2, :] *= np.float32(1e-6)
    w[3, :] = 0.0
    w[3, 100] = np.float32(0.5)
    w[150:, :] *= np.float32(1e-6)
    X = si.activations(M, K, seed=5)
    pb, po = pack_both(Q4_0, w)
    Wd = to_dev(pb)
    Y_ref, S = oracle.get().prefill(po, N, K, X)
    _prefill_each_setting(Wd, X, N, K, Y_ref, S, "prefill degenerate")
    Y = _prefill(Wd, X, N, K)
    assert (Y[:, 0] == 0).all()
    Y0 = _prefill(Wd, np.zeros((M, K), np.float16), N, K)
    assert (Y0 == 0).all()


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
