"""Helpers shared by the GPU parity tests.

Both sides start from the same seeded fp32 weights: the HIP side packs them
with the library's host quantizer, the oracle side with its own quantizer, and
the two byte strings must be identical before any product is compared.  The
oracle never receives a byte or a value produced by the library.

Sabotage switch [volta-kernel-bakeoff, "Making it fair": corrupted packed
weights must fail every check of the packed kernels, while the dense fp16
contender passes as a control].  With QGEMV_SABOTAGE=1 in the environment,
pack_both() hands the tests a corrupted copy of the library's bytes (every
code byte XOR 0x11, which moves each weight by one step of its block's
scale, and every scale's sign bit flipped) while the oracle keeps the clean
bytes.  Every packed-weight check (check_within, check_equal) then records
its outcome instead of raising, and the session ends with the tally: it fails
unless every packed-weight check failed and every control passed.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import seeded_inputs as si

Q4_0, Q8_0, Q2W = 0, 1, 2
REL, ABS = 1e-3, 1e-6
CODE_BYTES = {Q4_0: 16, Q8_0: 32, Q2W: 8}

SABOTAGE = os.environ.get("QGEMV_SABOTAGE", "") == "1"
# packed-weight checks and how many failed; controls and how many passed;
# names of the checks that did not see the corruption
TALLY = {"checks": 0, "failed": 0, "controls": 0, "controls_passed": 0, "unfailed": []}


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def qg():
    import quantized_weight_gemv_amd as q
    q.lib()  # fails loudly if the library is not built
    return q


def corrupt(packed: np.ndarray, fmt: int, N: int, K: int, count: int = 1) -> np.ndarray:
    """A copy of `count` packed N x K matrices laid end to end with every
    code byte XOR 0x11 and every scale's sign bit flipped."""
    bad = packed.copy()
    nb = N * (K // 32)
    cb = CODE_BYTES[fmt]
    s0 = (nb * cb + 255) // 256 * 256
    stride = (s0 + 2 * nb + 255) // 256 * 256
    for m in range(count):
        base = m * stride
        bad[base:base + nb * cb] ^= 0x11
        bad[base + s0 + 1:base + s0 + 2 * nb:2] ^= 0x80
    return bad


def pack_both(fmt: int, w: np.ndarray):
    """(library bytes, oracle bytes) for the same weights; asserts equality.
    Under the sabotage switch the library bytes returned are corrupted."""
    q = qg()
    pb = {Q4_0: q.qquantize_q4_0, Q8_0: q.qquantize_q8_0, Q2W: q.qquantize_q2w}[fmt](w)
    po = oracle.get().quantize(fmt, w)
    assert pb.size == po.size and np.array_equal(pb, po), "library packer differs from the oracle packer"
    if SABOTAGE:
        pb = corrupt(pb, fmt, w.shape[0], w.shape[1])
    return pb, po


def to_dev(a: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _record(ok: bool, what: str, msg: str):
    TALLY["checks"] += 1
    if not ok:
        TALLY["failed"] += 1
    if SABOTAGE:
        if ok:
            TALLY["unfailed"].append(what)
        return
    if not ok:
        raise AssertionError(msg)


def check_within(y, y_ref, s, what: str):
    """A packed-weight check: every element finite and within the bound."""
    y = np.asarray(y, np.float64)
    ok = oracle.within_bound(y, y_ref, s, REL, ABS)
    msg = ""
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        msg = (f"{what}: {bad.shape[0]} of {ok.size} outside |y-ref| <= 1e-3*s + 1e-6; "
               f"first at {i}: y={y[i]!r} ref={y_ref[i]!r} s={s[i]!r}")
    _record(bool(ok.all()), what, msg)


assert_within = check_within


def check_ok(ok, what: str):
    """A packed-weight check given as a boolean array (True = element passes)."""
    ok = np.asarray(ok)
    _record(bool(ok.all()), what, f"{what}: {int((~ok).sum())} of {ok.size} elements fail")


def check_equal(a, b, what: str, bits: bool = True):
    """A packed-weight check that must hold exactly: bit for bit (same dtype;
    -0 and +0 differ), or, with bits=False, as values (np.array_equal; a sum
    can return +0 where the weight itself is -0)."""
    a, b = np.asarray(a), np.asarray(b)
    if bits:
        ok = a.shape == b.shape and a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8))
    else:
        ok = bool(np.array_equal(a, b))
    _record(ok, what, f"{what}: not {'bitwise ' if bits else ''}equal")


def control_within(y, y_ref, s, what: str):
    """A control: computed without the library's packed bytes, it must pass
    with or without sabotage."""
    ok = oracle.within_bound(np.asarray(y, np.float64), y_ref, s, REL, ABS)
    TALLY["controls"] += 1
    TALLY["controls_passed"] += int(ok.all())
    assert ok.all(), f"control {what}: {int((~ok).sum())} of {ok.size} outside the bound"


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
