"""Host-side checks of the HIP library (no GPU): it loads, exports every
symbol include/*.h declares, and its host quantizer writes exactly the
oracle's bytes."""
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import seeded_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _qg():
    import quantized_weight_gemv_amd as q
    if not os.path.exists(q.LIB_PATH):
        pytest.fail("libqgemv.so is not built (run __graft_entry__.build())")
    q.lib()
    return q


def declared_symbols():
    inc = os.path.join(ROOT, "include")
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    q = _qg()
    decl = declared_symbols()
    assert len(decl) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (\S+)", out))
    missing = [s for s in decl if s not in exported]
    assert not missing, missing
    for s in decl:
        getattr(q.lib(), s)
    assert sorted(q.exported_symbols()) == decl


def test_status_strings():
    L = _qg().lib()
    for st in range(8):
        assert L.qg_status_str(st)


def _quantize_fn(q, fmt):
    return {0: q.qquantize_q4_0, 1: q.qquantize_q8_0, 2: q.qquantize_q2w}[fmt]


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (17, 640), (64, 2560), (33, 4096), (8, 14336)])
def test_host_packer_matches_oracle(fmt, N, K):
    q = _qg()
    w = si.weights(N, K, seed=N * K)
    if N > 2:
        w[1, :32] = 0.0                                   # zero block
        w[2, :] *= np.float32(1e-5)                       # subnormal scales
        w[0, :32] = (np.arange(32) - 14).astype(np.float32) * np.float32(2.0 ** -8)   # exact ties
        w[2, 32:64] = -w[0, :32]                          # the extreme weight of either sign
    pb = _quantize_fn(q, fmt)(w)
    po = oracle.get().quantize(fmt, w)
    assert q.packed_bytes(fmt, N, K) == oracle.get().packed_bytes(fmt, N, K) == pb.size
    assert np.array_equal(pb, po)


def test_host_packer_golden_blocks():
    """The library packer reproduces the hand-derived worked blocks."""
    import oracle_pins as pins
    q = _qg()
    for name in ("q4_0_we1.txt", "q8_0_we2.txt", "q4_0_we3_subnormal.txt", "q2w_we6.txt"):
        g = pins.load_golden(name)
        w = pins._golden_weights(g)
        fmt = {"q4_0": 0, "q8_0": 1, "q2w": 2}[g["format"]]
        p = _quantize_fn(q, fmt)(w)
        nb = {0: 16, 1: 32, 2: 8}[fmt]
        assert bytes(p[:nb]) == bytes.fromhex("".join(g["code_bytes"].split())), name
        assert int(p[256]) | (int(p[257]) << 8) == int(g["scale_bits"], 16), name


def test_host_packer_errors():
    q = _qg()
    w = np.zeros((2, 64), np.float32)
    w[1, 5] = np.nan
    with pytest.raises(q.QGError) as e:
        q.qquantize_q4_0(w)
    assert e.value.status == 4
    with pytest.raises(q.QGError):
        q.qquantize_q8_0(np.full((1, 32), 1e9, np.float32))
    with pytest.raises(q.QGError):
        q.qquantize_q4_0(np.zeros((2, 40), np.float32))
    assert q.qpacked_bytes_q4_0(4, 48) == 0 and q.qpacked_bytes_q8_0(0, 64) == 0 and q.qpacked_bytes_q2w(4, 48) == 0
    with pytest.raises(q.QGError) as e:
        q.qquantize_q2w(np.full((1, 32), np.inf, np.float32))
    assert e.value.status == 4
    small = np.empty(10, np.uint8)
    with pytest.raises(ValueError):
        q.qquantize_q4_0(np.zeros((1, 32), np.float32), out=small)
