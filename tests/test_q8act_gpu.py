"""GPU parity of the Q4_0 GEMV on activations quantized to 8-bit blocks
(qgemv_q4_0_q8act) against the oracle's definition: the same per-block
binary32 quantizer, then exact integer block sums times dw * dx."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import Q2W, Q4_0, assert_within, check_equal, check_ok, pack_both, qg, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _q8act(Wd, x16, N, K, y=None, fmt=Q4_0):
    q = qg()
    f = q.qgemv_q4_0_q8act if fmt == Q4_0 else q.qgemv_q2w_q8act
    out = f(Wd, to_dev(x16) if isinstance(x16, np.ndarray) else x16, N, K, y)
    torch_cuda().cuda.synchronize()
    return out.cpu().numpy()


def _acts(M, K, seed, planted=True):
    """fp16 ~N(0, 1) with planted ties at power-of-two scales, large values,
    tiny (subnormal) ones and an all-zero block."""
    g = np.random.default_rng([seed, M, K, 8])
    x = g.standard_normal((M, K))
    if planted and K >= 128:
        for m in range(M):
            x[m, 0:32] = 0.0                                # an all-zero block
            x[m, 32:64] = g.integers(-254, 255, 32) * 0.5   # amax 127 * 2^0 ties
            x[m, 32 + m] = 127.0
            x[m, 64:96] *= 2.0 ** -20                       # binary16 subnormals
            x[m, 96 + (m % 32)] = 60000.0 * (-1) ** m       # one huge value
    return x.astype(np.float16)


@pytest.mark.parametrize("fmt", [Q4_0, Q2W], ids=["q4_0", "q2w"])
@pytest.mark.parametrize("M,N,K", [(1, 17, 32), (1, 4096, 4096), (2, 130, 2048), (3, 4099, 640), (4, 1000, 4096),
                                   (1, 5, 14336), (2, 257, 16384), (4, 64, 8192), (1, 3, 16384)])
def test_q8act_parity(fmt, M, N, K):
    w = si.weights(N, K, seed=M + N + 3)
    x = _acts(M, K, seed=K)
    pb, po = pack_both(fmt, w)
    y = _q8act(to_dev(pb), x, N, K, fmt=fmt)
    y_ref, s = oracle.get().gemv_q8act(po, N, K, x, fmt)
    assert_within(y, y_ref, s, f"q8act fmt={fmt} M={M} {N}x{K}")
    # fp32 sums of exact block integers: far tighter than the bound
    assert (np.abs(y - y_ref) <= 2e-5 * s + 1e-6).all()


@pytest.mark.parametrize("N,K", si.LLAMA3_8B_SHAPES)
def test_q2w_q8act_llama3_8b_full_size(N, K):
    w = si.weights(N, K, seed=0)
    x = si.activations(1, K, seed=0)
    pb, po = pack_both(Q2W, w)
    y = _q8act(to_dev(pb), x, N, K, fmt=Q2W)
    y_ref, s = oracle.get().gemv_q8act(po, N, K, x, Q2W)
    assert_within(y, y_ref, s, f"q2w q8act {N}x{K}")
    assert (np.abs(y - y_ref) <= 2e-5 * s + 1e-6).all()


@pytest.mark.parametrize("N,K", si.LLAMA3_8B_SHAPES)
def test_q8act_llama3_8b_full_size(N, K):
    w = si.weights(N, K, seed=0)
    x = si.activations(1, K, seed=0)
    pb, po = pack_both(Q4_0, w)
    y = _q8act(to_dev(pb), x, N, K)
    y_ref, s = oracle.get().gemv_q8act(po, N, K, x)
    assert_within(y, y_ref, s, f"q8act {N}x{K}")
    # and within the activation rounding of the fp16 GEMV
    y16, s16 = oracle.get().gemv(Q4_0, po, N, K, x)
    _, dx = oracle.get().quantize_act8(x)
    W = np.abs(oracle.get().dequant(Q4_0, po, N, K, "f32").astype(np.float64))
    bound = W @ (0.5 * np.repeat(dx[0].astype(np.float64), 32) * (1 + 1e-5)) + 1e-5 * s16[0]
    assert (np.abs(y[0] - y16[0]) <= bound).all()


def test_q8act_codes_bit_exact():
    """An identity-like table (row k has one weight, on column k) makes
    output k = dw * dx_b * (q - 8) * qx_k: every activation code of every
    block and token shows up alone, ties and extremes included."""
    K = 256
    N = K
    w = np.zeros((N, K), np.float32)
    w[np.arange(N), np.arange(K)] = 0.5
    M = 4
    g = np.random.default_rng(99)
    x = np.zeros((M, K))
    for m in range(M):
        for b in range(K // 32):
            e = int(g.integers(-14, 8))
            blk = g.integers(-254, 255, 32) * 0.5 * 2.0 ** e      # half-integer multiples: ties
            blk[int(g.integers(0, 32))] = 127 * 2.0 ** e * (-1) ** b
            x[m, 32 * b:32 * b + 32] = blk
    x[1, 64:96] = 0.0
    x[2, 96:128] = g.standard_normal(32) * 3e-6          # subnormal binary16 block
    x[3, 128:160] = g.standard_normal(32) * 20000.0
    x16 = x.astype(np.float16)
    pb, po = pack_both(Q4_0, w)
    y = _q8act(to_dev(pb), x16, N, K)
    qx, dx = oracle.get().quantize_act8(x16)
    y_ref, s = oracle.get().gemv_q8act(po, N, K, x16)
    # one term per output: the fp32 result is the exact value rounded twice
    check_ok(np.abs(y - y_ref) <= 2.5e-7 * np.abs(y_ref) + 1e-30, "q8act one term per output")
    # so the codes agree: output k over (dequantized weight k times dx of
    # k's block) is the activation code qx_k
    wk = oracle.get().dequant(Q4_0, po, N, K, "f64")[np.arange(N), np.arange(K)]
    assert (wk != 0).all()
    scale = np.repeat(dx.astype(np.float64), 32, axis=1) * wk[None, :]
    nz = scale != 0
    check_equal(np.rint(y[nz] / scale[nz]), qx.astype(np.float64)[nz], "q8act codes from one-term outputs",
                bits=False)
    assert (y[~nz] == 0).all() and (qx[~nz] == 0).all()


@pytest.mark.parametrize("fmt", [Q4_0, Q2W], ids=["q4_0", "q2w"])
def test_q8act_every_launch_shape(fmt):
    q = qg()
    torch = torch_cuda()
    f = q.qgemv_q4_0_q8act if fmt == Q4_0 else q.qgemv_q2w_q8act
    for (M, N, K) in [(1, 257, 4096), (2, 70, 6144), (3, 33, 2560), (4, 130, 2048)]:
        w = si.weights(N, K, seed=N)
        x = _acts(M, K, seed=K + 1)
        pb, po = pack_both(fmt, w)
        Wd, xd = to_dev(pb), to_dev(x)
        y_ref, s = oracle.get().gemv_q8act(po, N, K, x, fmt)
        buf = torch.full((M * N + 128,), 7.0, dtype=torch.float32, device="cuda")
        yv = buf[64:64 + M * N].view(M, N)
        tried = set()
        try:
            for J in (0, 3, 8):
                for R in (0, 1, 2, 4):
                    for tpw, teams in ((0, 0), (1, 1), (2, 7), (8, 100000)):
                        for xl in (-1, 0, 1):
                            q.qg_set_gemv_shape(J, R, 0, tpw, teams, xl, 0, 0)
                            try:
                                f(Wd, xd, N, K, yv)
                            except q.QGError:
                                assert xl != -1 or J or R, "the built-in choice must launch"
                                continue
                            torch.cuda.synchronize()
                            tried.add((J, R, tpw, xl))
                            what = f"q8act M={M} {N}x{K} J{J} R{R} tpw{tpw} teams{teams} xl{xl}"
                            assert xl != 0, what + ": registers are not an option for 8-bit activations"
                            assert_within(yv.cpu().numpy(), y_ref, s, what)
                            assert (buf[:64] == 7.0).all() and (buf[64 + M * N:] == 7.0).all(), what
        finally:
            q.qg_set_gemv_shape(0, 0, 0, 0, 0, -1, -1, 0)
        assert len(tried) >= 8


def test_q8act_graph_replay_is_bitwise_eager():
    q = qg()
    torch = torch_cuda()
    M, N, K = 2, 6144, 2048
    Wd = to_dev(q.qquantize_q4_0(si.weights(N, K, seed=4)))
    xd = to_dev(si.activations(M, K, seed=4))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    q.qgemv_q4_0_q8act(Wd, xd, N, K, y)
    torch.cuda.synchronize()
    eager = y.cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            q.qgemv_q4_0_q8act(Wd, xd, N, K, y)
    torch.cuda.current_stream().wait_stream(side)
    for r in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), eager.view(np.uint32)), f"replay {r}"
    del g


def test_q8act_abi_errors():
    q = qg()
    torch = torch_cuda()
    L = q.lib()
    N, K = 64, 256
    Wd = to_dev(q.qquantize_q4_0(si.weights(N, 16384, seed=1)))
    x = torch.zeros((8, 16384), dtype=torch.float16, device="cuda")
    y = torch.zeros((8, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    f = L.qgemv_q4_0_q8act
    assert f(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), 5, N, K, s) == 2         # more than 4 tokens
    assert f(Wd.data_ptr(), None, y.data_ptr(), 1, N, K, s) == 1                # NULL activations
    assert f(Wd.data_ptr(), x.data_ptr() + 2, y.data_ptr(), 1, N, K, s) == 3    # misaligned
    assert f(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), 1, N, 48, s) == 2       # K % 32 != 0
    assert f(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), 4, N, 14336, s) == 2    # LDS copy too large
    assert f(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), 1, N, 16384 + 32, s) == 2   # rows too long
    torch.cuda.synchronize()
