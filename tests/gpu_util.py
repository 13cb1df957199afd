"""Helpers shared by the GPU parity tests.

Both sides start from the same seeded fp32 weights: the HIP side packs them
with the library's host quantizer, the oracle side with its own quantizer, and
the two byte strings must be identical before any product is compared.  The
oracle never receives a byte or a value produced by the library.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import seeded_inputs as si

Q4_0, Q8_0, Q2W = 0, 1, 2
REL, ABS = 1e-3, 1e-6


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def qg():
    import quantized_weight_gemv_amd as q
    q.lib()  # fails loudly if the library is not built
    return q


def pack_both(fmt: int, w: np.ndarray):
    """(library bytes, oracle bytes) for the same weights; asserts equality."""
    q = qg()
    pb = {Q4_0: q.qquantize_q4_0, Q8_0: q.qquantize_q8_0, Q2W: q.qquantize_q2w}[fmt](w)
    po = oracle.get().quantize(fmt, w)
    assert pb.size == po.size and np.array_equal(pb, po), "library packer differs from the oracle packer"
    return pb, po


def to_dev(a: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def assert_within(y, y_ref, s, what: str):
    y = np.asarray(y, np.float64)
    ok = oracle.within_bound(y, y_ref, s, REL, ABS)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {bad.shape[0]} of {ok.size} outside |y-ref| <= 1e-3*s + 1e-6; "
                             f"first at {i}: y={y[i]!r} ref={y_ref[i]!r} s={s[i]!r}")


def sample_rows(N: int, count: int = 192, seed: int = 0) -> np.ndarray:
    """First, last and boundary rows plus a seeded uniform sample."""
    g = np.random.default_rng([seed, N, 77])
    fixed = [0, 1, 2, 3, N // 2, N - 4, N - 3, N - 2, N - 1]
    rnd = g.choice(N, size=min(N, count), replace=False)
    return np.unique(np.clip(np.concatenate([fixed, rnd]), 0, N - 1)).astype(np.int64)


def weights(N, K, seed=0):
    return si.weights(N, K, seed)


def acts(M, K, seed=0):
    return si.activations(M, K, seed)
