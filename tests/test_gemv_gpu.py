"""GPU parity: the HIP GEMV / dequant kernels against the CPU oracle.

Acceptance per output element: finite and |y - y_ref| <= 1e-3 * s + 1e-6 with
s = sum_k |w_k x_k| (fp32 sums of exact products are far inside this);
dequantized weights bit-exact.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import (Q2W, Q4_0, Q8_0, acts, assert_within, check_equal, pack_both, qg, to_dev,
                      torch_cuda, weights)

pytestmark = pytest.mark.gpu

FMTS = [Q4_0, Q8_0, Q2W]
FNAME = {Q4_0: "q4_0", Q8_0: "q8_0", Q2W: "q2w"}


def _gemv_fn(fmt):
    q = qg()
    return {Q4_0: q.qgemv_q4_0, Q8_0: q.qgemv_q8_0, Q2W: q.qgemv_q2w}[fmt]


def _dequant_fn(fmt):
    q = qg()
    return {Q4_0: q.qdequant_q4_0, Q8_0: q.qdequant_q8_0, Q2W: q.qdequant_q2w}[fmt]


def _gemv(fmt, Wd, xd, N, K):
    q = qg()
    y = _gemv_fn(fmt)(Wd, xd, N, K)
    torch_cuda().cuda.synchronize()
    return y.cpu().numpy()


# Shapes that span several lane/row tiles and ragged tails: K/32 below,
# at and above 64 and not a multiple of 64; N not a multiple of the row group.
SMALL_SHAPES = [(1, 32), (3, 64), (5, 96), (65, 640), (130, 2048), (257, 2560), (33, 4096), (70, 6144),
                (19, 14336), (9, 16384), (11, 4128)]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
@pytest.mark.parametrize("N,K", SMALL_SHAPES)
def test_dequant_bit_exact(fmt, N, K):
    torch = torch_cuda()
    q = qg()
    w = weights(N, K, seed=N + K)
    pb, po = pack_both(fmt, w)
    Wd = to_dev(pb)
    deq = _dequant_fn(fmt)
    f32 = deq(Wd, N, K, fp16=False)
    f16 = deq(Wd, N, K, fp16=True)
    torch.cuda.synchronize()
    o = oracle.get()
    check_equal(f32.cpu().numpy(), o.dequant(fmt, po, N, K, "f32"), f"dequant {FNAME[fmt]} {N}x{K} fp32")
    check_equal(f16.cpu().numpy(), o.dequant(fmt, po, N, K, "f16"), f"dequant {FNAME[fmt]} {N}x{K} fp16")


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", SMALL_SHAPES)
def test_gemv_small_parity(fmt, M, N, K):
    q = qg()
    limit = 16384 * min(8 // M, 4 if fmt == Q8_0 else 7)
    w = weights(N, K, seed=3 * N + K)
    x = acts(M, K, seed=M + K)
    pb, po = pack_both(fmt, w)
    if K > limit:
        with pytest.raises(q.QGError):
            _gemv(fmt, to_dev(pb), to_dev(x), N, K)
        return
    y = _gemv(fmt, to_dev(pb), to_dev(x), N, K)
    y_ref, s = oracle.get().gemv(fmt, po, N, K, x)
    assert_within(y, y_ref, s, f"{FNAME[fmt]} {N}x{K} M={M}")


def test_gemv_q4_0_2048_seed0():
    """Q4_0 GEMV, N=2048 out x K=2048 in, one token, seed 0: every output."""
    N = K = 2048
    w = si.weights(N, K, seed=0)
    x = si.activations(1, K, seed=0)
    pb, po = pack_both(Q4_0, w)
    y = _gemv(Q4_0, to_dev(pb), to_dev(x), N, K)
    y_ref, s = oracle.get().gemv(Q4_0, po, N, K, x)
    assert_within(y, y_ref, s, "2048x2048")


@pytest.mark.parametrize("fmt", [Q4_0, Q2W], ids=lambda f: FNAME[f])
@pytest.mark.parametrize("N,K", si.LLAMA3_8B_SHAPES)
def test_gemv_llama3_8b_full_size(fmt, N, K):
    """Full-size Llama-3-8B projection shapes at one token, in the launch
    configuration the bench times: every output against the oracle."""
    w = si.weights(N, K, seed=0)
    x = si.activations(1, K, seed=0)
    pb, po = pack_both(fmt, w)
    del w
    y = _gemv(fmt, to_dev(pb), to_dev(x), N, K)
    y_ref, s = oracle.get().gemv(fmt, po, N, K, x)
    assert_within(y, y_ref, s, f"{FNAME[fmt]} {N}x{K}")


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
@pytest.mark.parametrize("N,K", si.SMALL_BATCH_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_small_batch_decode(fmt, N, K, M):
    """Small-batch decode shapes, every output against the oracle."""
    w = si.weights(N, K, seed=0)
    x = si.activations(M, K, seed=0)
    pb, po = pack_both(fmt, w)
    y = _gemv(fmt, to_dev(pb), to_dev(x), N, K)
    y_ref, s = oracle.get().gemv(fmt, po, N, K, x)
    assert_within(y, y_ref, s, f"{FNAME[fmt]} {N}x{K} M={M}")


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
def test_one_hot_columns_are_exact(fmt):
    """x = e_k returns column k of the dequantized matrix bit-exactly (pins the
    nibble order and block indexing on the GPU)."""
    N, K = 96, 4096
    w = weights(N, K, seed=12)
    pb, po = pack_both(fmt, w)
    Wd = to_dev(pb)
    cols = [0, 1, 5, 15, 16, 17, 31, 32, 2047, 2048 + 20, 4095]
    x = np.zeros((len(cols), K), np.float16)
    for i, k in enumerate(cols):
        x[i, k] = 1.0
    wh = oracle.get().dequant(fmt, po, N, K, "f32")
    for lo in range(0, len(cols), 8):
        y = _gemv(fmt, Wd, to_dev(x[lo:lo + 8]), N, K)
        for i, k in enumerate(cols[lo:lo + 8]):
            check_equal(y[i], wh[:, k], f"{FNAME[fmt]} one-hot column {k}", bits=False)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
@pytest.mark.parametrize("kind", ["large", "tiny"])
def test_stress_activations(fmt, kind):
    """Planted large (+-20000..60000) and tiny activations, as the pages'
    precision stress; fp32 accumulation must stay inside the bound."""
    N, K = 300, 6144
    w = weights(N, K, seed=21)
    x = si.stress_activations(4, K, seed=21, kind=kind)
    pb, po = pack_both(fmt, w)
    y = _gemv(fmt, to_dev(pb), to_dev(x), N, K)
    y_ref, s = oracle.get().gemv(fmt, po, N, K, x)
    assert_within(y, y_ref, s, f"{FNAME[fmt]} stress {kind}")


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
@pytest.mark.parametrize("K", [32, 96, 640, 4096])
def test_outliers_on_zero_weights(fmt, K):
    """Activations near the binary16 limit (+-60000, -30000) on columns whose
    weights are exactly zero (code 8 / 0), the rest ~N(0, 1): the exact
    result is the small remainder, and the bound is set by it alone.  Short
    rows make that remainder a few units; both engines."""
    q = qg()
    N, M = 64, 4
    w = weights(N, K, seed=K + 3)
    g = np.random.default_rng([K, 61])
    cols = g.choice(K, 3, replace=False)
    w[:, cols] = 0.0
    x = acts(M, K, seed=K + 3)
    x[:, cols[0]] = 60000.0
    x[1::2, cols[0]] = -60000.0
    x[:, cols[1]] = -30000.0
    x[:, cols[2]] = 65504.0
    pb, po = pack_both(fmt, w)
    Wd, xd = to_dev(pb), to_dev(x)
    y_ref, s = oracle.get().gemv(fmt, po, N, K, x)
    try:
        for engine in ((-1, 0) if fmt == Q2W and (K // 32) % 2 else (-1, 0, 1)):
            q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, engine, 0)
            for m in (1, 2, M):
                if engine == 1 and m < 2:
                    continue
                y = _gemv(fmt, Wd, xd[:m], N, K)
                assert_within(y, y_ref[:m], s[:m], f"{FNAME[fmt]} outliers K={K} M={m} engine={engine}")
    finally:
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
def test_zero_and_degenerate_blocks(fmt):
    """All-zero blocks (scale 0), subnormal scales, a single non-zero weight."""
    N, K = 40, 2560
    w = weights(N, K, seed=5)
    w[0, :] = 0.0
    w[1, 32:64] = 0.0
    w[2, :] *= np.float32(1e-6)          # subnormal binary16 scales
    w[3, :] = 0.0
    w[3, 100] = np.float32(0.5)
    x = acts(3, K, seed=5)
    pb, po = pack_both(fmt, w)
    y = _gemv(fmt, to_dev(pb), to_dev(x), N, K)
    y_ref, s = oracle.get().gemv(fmt, po, N, K, x)
    assert_within(y, y_ref, s, "degenerate")
    assert (y[:, 0] == 0).all()
    y0 = _gemv(fmt, to_dev(pb), to_dev(np.zeros((2, K), np.float16)), N, K)
    assert (y0 == 0).all()


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
def test_deterministic_and_copy_invariant(fmt):
    """Same bytes at two addresses, two calls each: bitwise-equal outputs."""
    torch = torch_cuda()
    N, K = 6144, 4096
    w = weights(N, K, seed=8)
    x = acts(2, K, seed=8)
    pb, _ = pack_both(fmt, w)
    A, B = to_dev(pb), to_dev(pb)
    xd = to_dev(x)
    q = qg()
    f = _gemv_fn(fmt)
    ys = [f(A, xd, N, K), f(B, xd, N, K), f(A, xd, N, K)]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])


def test_abi_errors_are_reported_before_launch():
    torch = torch_cuda()
    q = qg()
    L = q.lib()
    N, K = 64, 256
    W = torch.zeros(q.qpacked_bytes_q4_0(N, K) + 256, dtype=torch.uint8, device="cuda")
    x = torch.zeros((9, K), dtype=torch.float16, device="cuda")
    y = torch.zeros((9, N), dtype=torch.float32, device="cuda")
    s = q._stream()
    p = W.data_ptr
    assert L.qgemv_q4_0(None, x.data_ptr(), y.data_ptr(), 1, N, K, s) == 1
    assert L.qgemv_q4_0(p(), x.data_ptr(), y.data_ptr(), 9, N, K, s) == 2        # M > 8
    assert L.qgemv_q4_0(p(), x.data_ptr(), y.data_ptr(), 0, N, K, s) == 2        # M < 1
    assert L.qgemv_q4_0(p(), x.data_ptr(), y.data_ptr(), 1, N, 48, s) == 2       # K % 32
    assert L.qgemv_q4_0(p(), x.data_ptr(), y.data_ptr(), 1, 0, K, s) == 2        # N < 1
    assert L.qgemv_q4_0(p() + 16, x.data_ptr(), y.data_ptr(), 1, N, K, s) == 3   # W alignment
    assert L.qgemv_q4_0(p(), x.data_ptr() + 2, y.data_ptr(), 1, N, K, s) == 3    # x alignment
    assert L.qdequant_q4_0(p(), N, 40, 0, y.data_ptr(), s) == 2
    torch.cuda.synchronize()
    assert (y == 0).all()   # nothing was launched


def test_outputs_stay_in_bounds():
    """Canary elements around y are untouched for ragged shapes."""
    torch = torch_cuda()
    q = qg()
    for fmt in FMTS:
        for (N, K, M) in ((1, 32, 1), (7, 2560, 3), (131, 4096, 8), (4099, 2048, 2)):
            pb, _ = pack_both(fmt, weights(N, K, seed=N))
            x = to_dev(acts(M, K, seed=1))
            buf = torch.full((M * N + 128,), 7.0, dtype=torch.float32, device="cuda")
            y = buf[64:64 + M * N].view(M, N)
            _gemv_fn(fmt)(to_dev(pb), x, N, K, y)
            torch.cuda.synchronize()
            assert (buf[:64] == 7.0).all() and (buf[64 + M * N:] == 7.0).all()


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
@pytest.mark.parametrize("N,K,M", [(257, 4096, 1), (100, 14336, 1), (33, 2560, 1), (70, 6144, 2), (130, 2048, 8),
                                   (5, 512, 1), (3, 1024, 1), (1, 64, 1)])
def test_gemv_every_launch_shape(fmt, N, K, M):
    """Parity for the launch shapes the tuning knob can select (lanes per row,
    blocks per lane, row sets per group, teams, workgroup size, K split,
    LDS-staged activations), including row sets clamped at the matrix tail."""
    q = qg()
    w = weights(N, K, seed=N)
    x = acts(M, K, seed=K)
    pb, po = pack_both(fmt, w)
    Wd, xd = to_dev(pb), to_dev(x)
    y_ref, s = oracle.get().gemv(fmt, po, N, K, x)
    tried = set()
    try:
        for lanes in (0, 16, 32, 64):
            for J in (0, 1, 2, 3, 5, 7):
                for R in (1, 2, 4):
                    for ks in (0, 2):
                        for tpw, teams in ((1, 1), (2, 7), (8, 100000)):
                            for xl in (-1, 0, 1):
                                q.qg_set_gemv_shape(J, R, ks, tpw, teams, xl, 0, lanes)
                                try:
                                    y = _gemv(fmt, Wd, xd, N, K)
                                except q.QGError:
                                    continue
                                tried.add((lanes, J, R, ks, xl))
                                assert_within(y, y_ref, s, f"G{lanes} J{J} R{R} tpw{tpw} teams{teams} ks{ks} xl{xl}")
    finally:
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)
    assert len(tried) >= 10


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
@pytest.mark.parametrize("N,K,M", [(17, 32, 2), (257, 4096, 8), (100, 2560, 3), (33, 6144, 5), (130, 8192, 1),
                                   (64, 96, 8), (4099, 2048, 2), (100, 192, 4), (50, 320, 8), (31, 1472, 6)])
def test_gemv_matrix_core_engine(fmt, N, K, M):
    """The matrix-core few-token kernel, every wave count along K, one or two
    teams per workgroup and a persistent grid of the built-in size, one
    workgroup (it walks every tile) and three (uneven tiles per workgroup),
    against the oracle; one-hot
    columns stay exact on it (exact (q-8) operands, scale applied in fp32)."""
    q = qg()
    w = weights(N, K, seed=N + 1)
    x = acts(M, K, seed=K + 1)
    pb, po = pack_both(fmt, w)
    Wd, xd = to_dev(pb), to_dev(x)
    if fmt == Q2W and (K // 32) % 2:   # q2w on the matrix cores: an even number of blocks per row
        try:
            q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, 1, 0)
            with pytest.raises(q.QGError):
                _gemv(fmt, Wd, xd, N, K)
        finally:
            q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)
        return
    y_ref, s = oracle.get().gemv(fmt, po, N, K, x)
    tried = 0
    try:
        for ks in (0, 1, 2, 3, 4, 6, 7, 8):
            for wgs in (0, 1, 3):
                for tm in (0, 2):   # one team per workgroup, or two sharing the staged activations
                    q.qg_set_gemv_shape(0, 0, ks, tm, wgs, -1, 1, 0)
                    try:
                        y = _gemv(fmt, Wd, xd, N, K)
                    except q.QGError:
                        continue
                    tried += 1
                    assert_within(y, y_ref, s, f"mfma waves={ks} teams={tm} workgroups={wgs}")
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, 1, 0)
        cols = [0, 5, 16, 31, K - 1]
        xo = np.zeros((len(cols), K), np.float16)
        for i, k in enumerate(cols):
            xo[i, k] = 1.0
        y = _gemv(fmt, Wd, to_dev(xo), N, K)
        wh = oracle.get().dequant(fmt, po, N, K, "f32")
        for i, k in enumerate(cols):
            check_equal(y[i], wh[:, k], f"{FNAME[fmt]} mfma one-hot column {k}", bits=False)
    finally:
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)
    assert tried >= 2   # long rows admit only the larger wave counts (<= 32 blocks per wave)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
def test_prepared_call_matches_direct_call(fmt):
    """The pre-validated launch object calls the entry point of its format."""
    q = qg()
    torch = torch_cuda()
    N, K, M = 300, 2560, 2
    pb, po = pack_both(fmt, weights(N, K, seed=8))
    Wd, xd = to_dev(pb), to_dev(acts(M, K, seed=8))
    y1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    q.PreparedGemv(fmt, Wd, xd, y1, N, K)()
    y2 = _gemv_fn(fmt)(Wd, xd, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(y1.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    y_ref, s = oracle.get().gemv(fmt, po, N, K, acts(M, K, seed=8))
    assert_within(y1.cpu().numpy(), y_ref, s, f"prepared {FNAME[fmt]}")
