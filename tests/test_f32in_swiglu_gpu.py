"""GPU parity of the fp32-input Q4_0 GEMV and of the stacked gate + up SwiGLU
kernel against the oracle (fp32 activations rounded to binary16, then the
GEMV definition; silu(g) * u on the halves of the 2N-row table)."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import Q4_0, assert_within, check_equal, check_ok, pack_both, qg, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _x32(M, K, seed, scale=1.0, planted=True):
    """fp32 activations ~N(0, scale^2) with planted large (+-20000..60000),
    tiny (binary16 subnormal range) and exact-tie values."""
    g = np.random.default_rng([seed, M, K, 32])
    x = (g.standard_normal((M, K)) * scale).astype(np.float32)
    if planted and K >= 64:
        for m in range(M):
            cols = g.choice(K, 6, replace=False)
            x[m, cols[0]] = 60000.0 * (1 if m % 2 else -1)
            x[m, cols[1]] = -20000.0
            x[m, cols[2]] = 3e-7
            x[m, cols[3]] = -6e-8
            x[m, cols[4]] = 1.0 + 2.0 ** -11          # a tie: rounds to 1.0
            x[m, cols[5]] = 2049.0                     # a tie at 2048..2050
    return x


def _f32in(Wd, x, N, K):
    y = qg().qgemv_q4_0_f32in(Wd, to_dev(x), N, K)
    torch_cuda().cuda.synchronize()
    return y.cpu().numpy()


def _swiglu(Wd, x, N, K):
    y = qg().qgemv_q4_0_swiglu_f32in(Wd, to_dev(x), N, K)
    torch_cuda().cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("M,N,K", [(1, 17, 32), (1, 4096, 4096), (2, 130, 2048), (3, 4099, 640), (4, 1000, 4096),
                                   (1, 5, 14336), (4, 257, 16384), (2, 64, 32768), (1, 3, 65536)])
def test_f32in_parity(M, N, K):
    w = si.weights(N, K, seed=M + N)
    x = _x32(M, K, seed=K)
    pb, po = pack_both(Q4_0, w)
    y = _f32in(to_dev(pb), x, N, K)
    y_ref, s = oracle.get().gemv_f32in(Q4_0, po, N, K, x)
    assert_within(y, y_ref, s, f"f32in M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K", [(5, 17, 64), (8, 640, 2560), (6, 6144, 2048), (8, 4096, 4096), (7, 257, 8192),
                                   (5, 33, 96), (8, 4099, 1024)])
def test_f32in_five_to_eight_tokens(M, N, K):
    """5-8 tokens of fp32 activations: the matrix-core kernel rounds them to
    binary16 as it stages them; planted large, tiny and tie values."""
    w = si.weights(N, K, seed=M + N + 1)
    x = _x32(M, K, seed=K + M)
    pb, po = pack_both(Q4_0, w)
    y = _f32in(to_dev(pb), x, N, K)
    y_ref, s = oracle.get().gemv_f32in(Q4_0, po, N, K, x)
    assert_within(y, y_ref, s, f"f32in M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K", [(2, 130, 2048), (4, 1000, 4096), (8, 257, 8192), (3, 64, 96)])
def test_f32in_matrix_core_engine_matches_fp16_call(M, N, K):
    """The matrix-core kernel on fp32 activations, every wave count and three
    grid sizes: bitwise equal to the same kernel on the fp16 rounding of x
    (numpy's cast) in the same launch, and within the bound of the oracle."""
    q = qg()
    torch = torch_cuda()
    w = si.weights(N, K, seed=N + 5)
    x = _x32(M, K, seed=K + 5)
    pb, po = pack_both(Q4_0, w)
    Wd = to_dev(pb)
    x16 = to_dev(x.astype(np.float16))
    y_ref, s = oracle.get().gemv_f32in(Q4_0, po, N, K, x)
    tried = 0
    try:
        for ks in (0, 1, 2, 4, 8):
            for wgs in (0, 1, 3):
                for tm in (0, 2):
                    q.qg_set_gemv_shape(0, 0, ks, tm, wgs, -1, 1, 0)
                    try:
                        y = _f32in(Wd, x, N, K)
                    except q.QGError:
                        continue
                    y16 = q.qgemv_q4_0(Wd, x16, N, K)
                    torch.cuda.synchronize()
                    tried += 1
                    assert np.array_equal(y, y16.cpu().numpy()), f"waves={ks} teams={tm} workgroups={wgs}"
                    assert_within(y, y_ref, s, f"f32in mfma M={M} waves={ks} teams={tm} workgroups={wgs}")
    finally:
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)
    assert tried >= 2


def test_f32in_matches_fp16_path_bitwise():
    """Same launch shape as the fp16 kernel (one token, 28672 x 4096): the
    in-kernel conversion gives the fp16 call's bits exactly."""
    q = qg()
    N, K = 28672, 4096
    w = si.weights(N, K, seed=8)
    x = _x32(1, K, seed=8, planted=False)
    pb, po = pack_both(Q4_0, w)
    Wd = to_dev(pb)
    y32 = _f32in(Wd, x, N, K)
    y16 = q.qgemv_q4_0(Wd, to_dev(x.astype(np.float16)), N, K)
    torch_cuda().cuda.synchronize()
    assert np.array_equal(y32.view(np.uint32), y16.cpu().numpy().view(np.uint32))
    y_ref, s = oracle.get().gemv_f32in(Q4_0, po, N, K, x)
    assert_within(y32, y_ref, s, "f32in 28672x4096")


@pytest.mark.parametrize("M,N,K", [(1, 257, 4096), (2, 70, 6144), (3, 33, 2560), (4, 130, 2048), (4, 9, 14336)])
def test_f32in_every_launch_shape(M, N, K):
    """fp32 input through the launch shapes the tuning knob can select, with
    the activations in registers and staged once per workgroup in LDS."""
    q = qg()
    torch = torch_cuda()
    w = si.weights(N, K, seed=N)
    x = _x32(M, K, seed=K)
    pb, po = pack_both(Q4_0, w)
    Wd, xd = to_dev(pb), to_dev(x)
    y_ref, s = oracle.get().gemv_f32in(Q4_0, po, N, K, x)
    buf = torch.full((M * N + 128,), 7.0, dtype=torch.float32, device="cuda")
    yv = buf[64:64 + M * N].view(M, N)
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
                                    q.qgemv_q4_0_f32in(Wd, xd, N, K, yv)
                                except q.QGError:
                                    continue
                                torch.cuda.synchronize()
                                tried.add((lanes, J, R, ks, xl))
                                what = f"f32in M={M} G{lanes} J{J} R{R} ks{ks} tpw{tpw} teams{teams} xl{xl}"
                                assert_within(yv.cpu().numpy(), y_ref, s, what)
                                assert (buf[:64] == 7.0).all() and (buf[64 + M * N:] == 7.0).all(), what
    finally:
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)
    xl_fits = M * (K // 32 + 1) * 64 <= 65536    # the LDS copy of M tokens
    assert len(tried) >= 6 and any(t[4] == 1 for t in tried) == xl_fits


def test_f32in_overflow_is_non_finite_like_the_oracle():
    """|x| > 65504 becomes infinity in binary16: every row with a nonzero
    weight there comes out non-finite, as in the oracle; the rest finite."""
    N, K = 64, 256
    w = si.weights(N, K, seed=4)
    x = _x32(2, K, seed=4, planted=False)
    x[0, 37] = 70000.0
    x[1, 100] = -1e6
    pb, po = pack_both(Q4_0, w)
    y = _f32in(to_dev(pb), x, N, K)
    y_ref, s = oracle.get().gemv_f32in(Q4_0, po, N, K, x)
    fin = np.isfinite(y_ref)
    assert not fin.all()
    check_equal(np.isfinite(y), fin, "f32in overflow: which outputs are finite", bits=False)
    assert_within(y[fin], y_ref[fin], s[fin], "f32in finite rows")


def test_f32in_outliers_on_zero_weights():
    """fp32 activations at and beyond the binary16 limit on columns of zero
    weights, rows of one to twenty blocks: only the small remainder sets the
    bound (65519.99 rounds to 65504, 65520 would overflow)."""
    for K in (32, 96, 640):
        N, M = 40, 4
        w = si.weights(N, K, seed=K + 7)
        cols = np.random.default_rng([K, 62]).choice(K, 2, replace=False)
        w[:, cols] = 0.0
        x = _x32(M, K, seed=K + 7, planted=False)
        x[:, cols[0]] = 65519.99
        x[1::2, cols[0]] = -60000.5
        x[:, cols[1]] = -30000.25
        pb, po = pack_both(Q4_0, w)
        y = _f32in(to_dev(pb), x, N, K)
        y_ref, s = oracle.get().gemv_f32in(Q4_0, po, N, K, x)
        assert_within(y, y_ref, s, f"f32in outliers K={K}")


def _check_swiglu(y, ref, what):
    yr, g, u, sg, su = ref
    check_ok(oracle.swiglu_within_bound(y, yr, g, u, sg, su), f"{what} (SwiGLU bound)")


@pytest.mark.parametrize("M,N,K", [(1, 33, 64), (1, 14336, 4096), (2, 300, 2048), (3, 1000, 640), (4, 4099, 1024),
                                   (1, 7, 14336), (4, 130, 16384), (1, 4096, 4096), (1, 6144, 4096)])
def test_swiglu_parity(M, N, K):
    w = np.concatenate([si.weights(N, K, seed=N + 1), si.weights(N, K, seed=N + 2)])
    x = _x32(M, K, seed=K + 5)
    pb, po = pack_both(Q4_0, w)
    y = _swiglu(to_dev(pb), x, N, K)
    _check_swiglu(y, oracle.get().swiglu(po, N, K, x), f"swiglu M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 2])
def test_swiglu_saturation_and_every_launch_shape(M):
    """Large positive and negative gates (silu -> g and -> 0) with activations
    scaled up, through the launch shapes the tuning knob can select: lanes
    per row, blocks per lane, K split over 1..8 waves, teams and workgroup
    size, with the output guarded on both sides."""
    q = qg()
    torch = torch_cuda()
    N, K = 98, 1024
    w = np.concatenate([si.weights(N, K, seed=31) * 40.0, si.weights(N, K, seed=32)])
    x = _x32(M, K, seed=33, scale=3.0, planted=False)
    pb, po = pack_both(Q4_0, w)
    Wd, xd = to_dev(pb), to_dev(x)
    ref = oracle.get().swiglu(po, N, K, x)
    g = ref[1]
    assert (g > 30).any() and (g < -30).any()
    buf = torch.full((M * N + 128,), 7.0, dtype=torch.float32, device="cuda")
    yv = buf[64:64 + M * N].view(M, N)
    tried = set()
    try:
        for lanes in (0, 16, 32, 64):
            for J in (0, 1, 2, 3):
                for ks in (0, 1, 2, 4, 8):
                    for tpw, teams in ((1, 1), (2, 7), (8, 100000)):
                        for xl in (-1, 1):
                            q.qg_set_gemv_shape(J, 0, ks, tpw, teams, xl, 0, lanes)
                            try:
                                q.qgemv_q4_0_swiglu_f32in(Wd, xd, N, K, yv)
                            except q.QGError:
                                continue
                            torch.cuda.synchronize()
                            tried.add((lanes, J, ks, xl))
                            what = f"swiglu M={M} lanes={lanes} J={J} ks={ks} tpw={tpw} teams={teams} xl={xl}"
                            _check_swiglu(yv.cpu().numpy(), ref, what)
                            assert (buf[:64] == 7.0).all() and (buf[64 + M * N:] == 7.0).all(), what
    finally:
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)
    assert len(tried) >= (8 if M == 1 else 4)
    assert any(t[3] == 1 for t in tried)


@pytest.mark.parametrize("M,N,K", [(5, 17, 64), (8, 640, 2560), (6, 6144, 2048), (8, 1000, 4096), (7, 33, 8192),
                                   (5, 4099, 96)])
def test_swiglu_five_to_eight_tokens(M, N, K):
    """5-8 tokens: the matrix-core kernel pairs each gate tile with its up
    tile N rows below, rounds the fp32 activations as it stages them and
    writes silu(g) * u; row counts that are not multiples of 16 leave gate
    tiles reaching into the up rows, which must not be stored."""
    w = np.concatenate([si.weights(N, K, seed=N + 11), si.weights(N, K, seed=N + 12)])
    x = _x32(M, K, seed=K + 15)
    pb, po = pack_both(Q4_0, w)
    y = _swiglu(to_dev(pb), x, N, K)
    _check_swiglu(y, oracle.get().swiglu(po, N, K, x), f"swiglu M={M} N={N} K={K}")


def test_swiglu_matrix_core_every_wave_count_and_grid():
    """The SwiGLU matrix-core kernel forced at 2-8 tokens, every wave count
    along K and three grid sizes, large positive and negative gates, output
    guarded on both sides."""
    q = qg()
    torch = torch_cuda()
    N, K = 98, 1024
    w = np.concatenate([si.weights(N, K, seed=51) * 40.0, si.weights(N, K, seed=52)])
    pb, po = pack_both(Q4_0, w)
    Wd = to_dev(pb)
    tried = 0
    try:
        for M in (2, 4, 8):
            x = _x32(M, K, seed=53 + M, scale=3.0, planted=False)
            ref = oracle.get().swiglu(po, N, K, x)
            buf = torch.full((M * N + 128,), 7.0, dtype=torch.float32, device="cuda")
            yv = buf[64:64 + M * N].view(M, N)
            for ks in (0, 1, 2, 4, 8):
                for wgs in (0, 1, 3):
                    for tm in (0, 2):
                        q.qg_set_gemv_shape(0, 0, ks, tm, wgs, -1, 1, 0)
                        try:
                            q.qgemv_q4_0_swiglu_f32in(Wd, to_dev(x), N, K, yv)
                        except q.QGError:
                            continue
                        torch.cuda.synchronize()
                        tried += 1
                        _check_swiglu(yv.cpu().numpy(), ref, f"swiglu mfma M={M} waves={ks} teams={tm} workgroups={wgs}")
                        h = buf.cpu().numpy()
                        assert (h[:64] == 7.0).all() and (h[64 + M * N:] == 7.0).all(), "wrote outside y"
    finally:
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)
    assert tried >= 6


def test_swiglu_one_token_narrow_rows():
    """One token, 16 and 32 lanes per row (the built-in choice below 8192
    rows of 65..128 blocks)."""
    q = qg()
    N, K = 512, 4096
    w = np.concatenate([si.weights(N, K, seed=41), si.weights(N, K, seed=42)])
    x = _x32(1, K, seed=43)
    pb, po = pack_both(Q4_0, w)
    Wd = to_dev(pb)
    ref = oracle.get().swiglu(po, N, K, x)
    try:
        for lanes in (0, 16, 32):
            q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, 0, lanes)
            _check_swiglu(_swiglu(Wd, x, N, K), ref, f"swiglu one token lanes={lanes}")
    finally:
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)


def test_f32in_and_swiglu_abi_errors():
    q = qg()
    torch = torch_cuda()
    L = q.lib()
    N, K = 64, 256
    Wd = to_dev(q.qquantize_q4_0(si.weights(2 * N, K, seed=1)))
    x = torch.zeros((8, K), dtype=torch.float32, device="cuda")
    y = torch.zeros((8, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for fn in (L.qgemv_q4_0_f32in, L.qgemv_q4_0_swiglu_f32in):
        assert fn(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), 9, N, K, s) == 2      # > 8 tokens
    xl = torch.zeros((5, 8224), dtype=torch.float32, device="cuda")
    Wl = to_dev(q.qquantize_q4_0(si.weights(N, 8224, seed=1)))
    assert L.qgemv_q4_0_f32in(Wl.data_ptr(), xl.data_ptr(), y.data_ptr(), 5, N, 8224, s) == 2      # 5+ tokens, K > 8192
    x8 = torch.zeros((8, 8192), dtype=torch.float32, device="cuda")
    W8 = to_dev(q.qquantize_q4_0(si.weights(2 * N, 8192, seed=1)))
    assert L.qgemv_q4_0_swiglu_f32in(W8.data_ptr(), x8.data_ptr(), y.data_ptr(), 8, N, 8192, s) == 2  # LDS: K <= 7168
    assert L.qgemv_q4_0_swiglu_f32in(W8.data_ptr(), x8.data_ptr(), y.data_ptr(), 7, N, 8192, s) == 0
    for fn in (L.qgemv_q4_0_f32in, L.qgemv_q4_0_swiglu_f32in):
        assert fn(Wd.data_ptr(), None, y.data_ptr(), 1, N, K, s) == 1              # NULL activations
        assert fn(Wd.data_ptr(), x.data_ptr() + 4, y.data_ptr(), 1, N, K, s) == 3  # misaligned
        assert fn(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), 1, N, 48, s) == 2     # K % 32 != 0
    try:
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, 1, 0)   # matrix-core engine: fp32 GEMV and SwiGLU
        assert L.qgemv_q4_0_f32in(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), 4, N, K, s) == 0
        assert L.qgemv_q4_0_swiglu_f32in(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), 4, N, K, s) == 0
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, 0, 0)   # vector engine: at most 4 fp32 tokens
        for fn in (L.qgemv_q4_0_f32in, L.qgemv_q4_0_swiglu_f32in):
            assert fn(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), 5, N, K, s) == 2
    finally:
        q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)
    torch.cuda.synchronize()
