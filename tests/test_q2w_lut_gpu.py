"""GPU parity of the times-table GEMV on plain 2-bit weights (qgemv_q2w_lut)
against the oracle's exact q2w GEMV: the fp16 table entries round each pair
sum by at most 2^-11 of |c_a x_a| + |c_b x_b|, inside the 1e-3 sum |w x|
bound."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import Q2W, assert_within, check_equal, check_ok, pack_both, qg, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _lut(Wd, x16, N, K):
    y = qg().qgemv_q2w_lut(Wd, to_dev(x16), N, K)
    torch_cuda().cuda.synchronize()
    return y.cpu().numpy()


# Table widths 32 / 64 / 128 columns (K <= 1024 / 2048 / 4096), odd block
# counts, and row counts on both sides of the one-pass limit (2048 / 8192 /
# 16384 rows for 128 / 64 / 32 columns on 256 CUs).
@pytest.mark.parametrize("N,K", [(1, 32), (3, 64), (17, 96), (130, 640), (257, 2048), (6144, 2048), (33, 2560),
                                 (4099, 4096), (14336, 4096), (8200, 2048), (16400, 1024), (5000, 1056)])
def test_q2w_lut_parity(N, K):
    w = si.weights(N, K, seed=N + K)
    x = si.activations(1, K, seed=K)
    pb, po = pack_both(Q2W, w)
    y = _lut(to_dev(pb), x, N, K)
    y_ref, s = oracle.get().gemv(Q2W, po, N, K, x)
    assert_within(y, y_ref, s, f"q2w lut {N}x{K}")
    # the fp16 entries carry the only rounding beyond fp32 sums (a quarter
    # of slack for those sums)
    assert (np.abs(y - y_ref) <= 2.0 ** -11 * s * 1.25 + 1e-6).all()


def test_q2w_lut_large_and_one_hot_activations():
    """Activations up to +-16000 (entries stay finite), and one-hot inputs:
    a single nonzero activation makes every entry c * x exact, so y is the
    dequantized weight column exactly."""
    N, K = 96, 1024
    w = si.weights(N, K, seed=7)
    pb, po = pack_both(Q2W, w)
    Wd = to_dev(pb)
    g = np.random.default_rng(7)
    x = (g.standard_normal((1, K)) * 3).astype(np.float16)
    x[0, g.choice(K, 20, replace=False)] = (g.uniform(-16000, 16000, 20)).astype(np.float16)
    y = _lut(Wd, x, N, K)
    y_ref, s = oracle.get().gemv(Q2W, po, N, K, x)
    assert_within(y, y_ref, s, "q2w lut large activations")
    wh = oracle.get().dequant(Q2W, po, N, K, "f32")
    for k in (0, 7, 8, 16, 31, 32, 500, K - 1):
        e = np.zeros((1, K), np.float16)
        e[0, k] = 1.0
        yk = _lut(Wd, e, N, K)
        check_equal(yk[0], wh[:, k], f"q2w lut one-hot column {k}", bits=False)


def test_q2w_lut_abi_errors():
    q = qg()
    torch = torch_cuda()
    L = q.lib()
    N = 64
    Wd = to_dev(q.qquantize_q2w(si.weights(N, 8192, seed=2)))
    x = torch.zeros((1, 8192), dtype=torch.float16, device="cuda")
    y = torch.zeros((1, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    f = L.qgemv_q2w_lut
    assert f(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), N, 4096 + 32, s) == 2   # tables beyond 64 KB
    assert f(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), N, 48, s) == 2         # K % 32 != 0
    assert f(Wd.data_ptr(), x.data_ptr(), y.data_ptr(), 0, 256, s) == 2         # no rows
    assert f(Wd.data_ptr(), None, y.data_ptr(), N, 256, s) == 1                 # NULL activations
    assert f(Wd.data_ptr(), x.data_ptr() + 2, y.data_ptr(), N, 256, s) == 3     # misaligned
    torch.cuda.synchronize()


@pytest.mark.parametrize("N,K", [(N, K) for (N, K) in si.LLAMA3_8B_SHAPES if K <= 4096])
def test_q2w_lut_llama3_8b_full_size(N, K):
    """The Llama-3-8B shapes the tables fit (K <= 4096) at full size, in the
    launch the suite times: every output against the oracle."""
    w = si.weights(N, K, seed=0)
    x = si.activations(1, K, seed=0)
    pb, po = pack_both(Q2W, w)
    del w
    y = _lut(to_dev(pb), x, N, K)
    y_ref, s = oracle.get().gemv(Q2W, po, N, K, x)
    assert_within(y, y_ref, s, f"q2w lut {N}x{K}")


def test_q2w_lut_matches_unpacking_kernel_within_bound():
    """Both 2-bit kernels on the same weights agree to the sum of their
    bounds on every output of a 28672 x 4096 table (two passes, 512
    workgroups), against the oracle's s."""
    N, K = 28672, 4096
    w = si.weights(N, K, seed=3)
    x = si.activations(1, K, seed=3)
    pb, po = pack_both(Q2W, w)
    del w
    Wd = to_dev(pb)
    y_lut = _lut(Wd, x, N, K)
    y_unp = qg().qgemv_q2w(Wd, to_dev(x), N, K).cpu().numpy()
    _, s = oracle.get().gemv_rows(Q2W, po, N, K, x, np.arange(N))
    assert (np.abs(y_lut.astype(np.float64) - y_unp) <= 2e-3 * s + 2e-6).all()
    y_ref, _ = oracle.get().gemv(Q2W, po, N, K, x)
    assert_within(y_lut, y_ref, s, "q2w lut 28672x4096")
