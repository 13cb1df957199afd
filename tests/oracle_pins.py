"""Pins that tie the CPU oracle to something other than itself.

Each pin takes an ``oracle.Oracle`` and returns a list of failure messages
(empty = pinned).  tests/test_oracle.py runs them on the real oracle and on
builds with planted mistakes, where at least one pin must fail.

What each pin rests on:
  codec        numpy's binary16 conversions (a library routine), all 65536
               patterns and boundary / tie / subnormal doubles.
  golden       hand-derived worked blocks in tests/golden/ (the block rule
               applied by hand; each file shows its derivation).
  nearest      brute force: every code is the nearest grid point
               (code - 8) * scale over all 16 (Q4_0) / 255 (Q8_0) codes,
               ties away from zero; the scale is numpy's
               float16(float32(absmax) / 7 or 127).
  invariants   code range, |w - w_hat| <= scale / 2, absmax -> +-7 / +-127,
               re-quantizing the dequantized weights is the identity.
  exact_gemv   Fraction sums on tiny shapes (exact rational arithmetic).
  special      one-hot input returns a weight column bit-exactly, zero input
               gives zero, linearity, M tokens == M single-token calls.
  moe          reduces to independent GEMVs of the chosen experts.
  prefill      equals a float64 matmul (numpy) on the dequantized weights.
  f32in        fp32 -> binary16 against numpy's float16 cast (a library
               routine) on random, overflow, tie and subnormal values; the
               GEMV on fp32 input equals the GEMV on numpy's cast, bitwise.
  silu         closed forms and published constants: silu(0) = 0,
               silu(ln 3) = (3/4) ln 3, silu(40) = 40 and silu(-40) ~ 0 in
               fp64, the minimum -0.2784645 near -1.2784645, and
               silu(v) - silu(-v) = v.
  swiglu       the stacked table's halves are the separately quantized gate
               and up GEMVs, bitwise; a zero gate gives zero; a large gate
               (silu(g) = g in fp64) gives g * u.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
Q4_0, Q8_0, Q2W = 0, 1, 2


def load_golden(name: str) -> dict:
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = v.strip()
    return d


def _fmt(g):
    return Q4_0 if g["format"] == "q4_0" else Q8_0


# ------------------------------------------------------------------ codec
def pin_codec(orc) -> list:
    fails = []
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for h in range(65536):
        v = orc.half_to_double(h)
        r = ref[h]
        if np.isnan(r):
            if not np.isnan(v):
                fails.append(f"decode {h:#06x}: {v} vs nan")
        elif v != r or np.signbit(v) != np.signbit(r):
            fails.append(f"decode {h:#06x}: {v!r} vs {r!r}")
        if len(fails) > 5:
            return fails
    g = np.random.default_rng(1234)
    vals = [0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e30, -1e30, 2.0**-24, 2.0**-25,
            2.0**-25 * 1.0000001, 3 * 2.0**-26, 2.0**-14, 2.0**-14 - 2.0**-25, 1.0 + 2.0**-11,
            1.0 + 3 * 2.0**-11, 2049.0, 2051.0, -2049.0]
    vals += list(g.standard_normal(20000) * 10.0 ** g.uniform(-9, 5, 20000))
    # exact ties at every binade: (odd multiples of half an ulp)
    for e in range(-24, 16):
        for m in (1, 3, 2045, 2047):
            vals.append(m * 2.0 ** (e - 11))
    for v in vals:
        with np.errstate(over="ignore"):
            want = int(np.array([v], np.float64).astype(np.float16).view(np.uint16)[0])
        got = orc.double_to_half(v)
        if got != want:
            fails.append(f"encode {v!r}: {got:#06x} vs {want:#06x}")
            if len(fails) > 5:
                break
    f32 = g.standard_normal(5000).astype(np.float32) * np.float32(0.02)
    for v in f32:
        want = int(np.array([v], np.float32).astype(np.float16).view(np.uint16)[0])
        if orc.float_to_half(v) != want:
            fails.append(f"encode f32 {v!r}")
            break
    return fails


# ----------------------------------------------------------------- golden
def _golden_weights(g):
    t = np.array([float(v) for v in g["t"].split()], np.float64)
    return (t * 2.0 ** int(g["weight_unit_log2"])).astype(np.float32).reshape(1, 32)


def pin_golden(orc) -> list:
    fails = []
    for name in ("q4_0_we1.txt", "q8_0_we2.txt", "q4_0_we3_subnormal.txt"):
        g = load_golden(name)
        fmt = _fmt(g)
        w = _golden_weights(g)
        p = orc.quantize(fmt, w)
        nb = 16 if fmt == Q4_0 else 32
        code_bytes = bytes.fromhex("".join(g["code_bytes"].split()))
        if bytes(p[:nb]) != code_bytes:
            fails.append(f"{name}: code bytes {bytes(p[:nb]).hex()} vs {code_bytes.hex()}")
        s0 = 256
        sbits = int(p[s0]) | (int(p[s0 + 1]) << 8)
        if sbits != int(g["scale_bits"], 16):
            fails.append(f"{name}: scale {sbits:#06x} vs {g['scale_bits']}")
        codes = np.array([int(c) for c in g["codes"].split()])
        scale = float(np.array([int(g["scale_bits"], 16)], np.uint16).view(np.float16)[0])
        wh = orc.dequant(fmt, p, 1, 32, "f64")[0]
        want = (codes - (8 if fmt == Q4_0 else 0)) * scale
        if not np.array_equal(wh, want):
            fails.append(f"{name}: dequant {wh} vs {want}")
        ones = np.ones((1, 32), np.float16)
        y, _ = orc.gemv(fmt, p, 1, 32, ones)
        if y[0, 0] != float(g["y_ones"]):
            fails.append(f"{name}: y_ones {y[0, 0]!r} vs {g['y_ones']}")
        for key in g:
            if key.startswith("y_e"):
                k = int(key[3:])
                x = np.zeros((1, 32), np.float16)
                x[0, k] = 1.0
                y, _ = orc.gemv(fmt, p, 1, 32, x)
                if y[0, 0] != float(g[key]):
                    fails.append(f"{name}: {key} {y[0, 0]!r} vs {g[key]}")
    # the four-block layout example
    g = load_golden("q4_0_we4_layout.txt")
    w1 = _golden_weights(load_golden("q4_0_we1.txt"))[0]
    N, K = 2, 64
    w = np.zeros((N, K), np.float32)
    for n in range(N):
        for b in range(2):
            w[n, 32 * b:32 * b + 32] = w1 * np.float32(2.0 ** (2 * n + b))
    if orc.packed_bytes(Q4_0, N, K) != int(g["packed_bytes"]):
        fails.append("we4: packed size")
    p = orc.quantize(Q4_0, w)
    we1_bytes = bytes.fromhex("".join(load_golden("q4_0_we1.txt")["code_bytes"].split()))
    for i in range(4):
        if bytes(p[16 * i:16 * i + 16]) != we1_bytes:
            fails.append(f"we4: block {i} codes")
    so = int(g["scale_offset"])
    for i, sb in enumerate(g["scale_bits"].split()):
        got = int(p[so + 2 * i]) | (int(p[so + 2 * i + 1]) << 8)
        if got != int(sb, 16):
            fails.append(f"we4: scale {i} {got:#06x} vs {sb}")
    y, _ = orc.gemv(Q4_0, p, N, K, np.ones((1, K), np.float16))
    if list(y[0]) != [float(v) for v in g["y_ones"].split()]:
        fails.append(f"we4: y_ones {y[0]}")
    x = np.zeros((1, K), np.float16)
    x[0, 37] = 1.0
    y, _ = orc.gemv(Q4_0, p, N, K, x)
    if list(y[0]) != [float(v) for v in g["y_e37"].split()]:
        fails.append(f"we4: y_e37 {y[0]}")
    return fails


# ---------------------------------------------------------------- nearest
def _parse(fmt, p, N, K):
    """Codes (signed multipliers) and scales straight from the documented layout."""
    nb = N * K // 32
    cb = {Q4_0: 16, Q8_0: 32, Q2W: 8}[fmt]
    codes_raw = p[:nb * cb].reshape(nb, cb)
    if fmt == Q4_0:
        q = np.concatenate([codes_raw & 0x0F, codes_raw >> 4], axis=1).astype(np.int64) - 8
    elif fmt == Q2W:
        # element 8 r + j sits in bits 2r..2r+1 of byte j
        q = np.concatenate([(codes_raw >> (2 * r)) & 3 for r in range(4)], axis=1).astype(np.int64) - 2
    else:
        q = codes_raw.view(np.int8).astype(np.int64)
    s0 = (nb * cb + 255) // 256 * 256
    scale = p[s0:s0 + 2 * nb].view(np.uint16).view(np.float16).astype(np.float64)
    return q, scale


def nearest_codes(fmt, w):
    """Brute force: scale = fp16(fl32(absmax)/qmax); each weight's code is the
    nearest multiplier c on the grid c * scale (c in -8..7 / -127..127), ties to
    the larger |c|.  Distances are exact in float64."""
    qmax = 7 if fmt == Q4_0 else 127
    blocks = w.reshape(-1, 32)
    amax = np.abs(blocks).max(axis=1).astype(np.float32)
    d16 = (amax / np.float32(qmax)).astype(np.float16)
    d = d16.astype(np.float64)
    cs = np.arange(-8 if fmt == Q4_0 else -127, qmax + 1, dtype=np.int64)
    best = np.zeros(blocks.shape, np.int64)
    bestd = np.full(blocks.shape, np.inf)
    wv = blocks.astype(np.float64)
    for c in cs:
        dist = np.abs(wv - c * d[:, None])
        better = (dist < bestd) | ((dist == bestd) & (np.abs(c) > np.abs(best)))
        best = np.where(better, c, best)
        bestd = np.where(better, dist, bestd)
    best[d == 0.0] = 0
    return best, d16


def pin_nearest(orc) -> list:
    fails = []
    for fmt, n_w in ((Q4_0, 1 << 20), (Q8_0, 1 << 16)):
        K = 256
        w = si.weights(n_w // K, K, seed=7)
        # plant exact ties and tiny/zero blocks
        w[0, :32] = 0.0
        w[1, :32] = np.float32(1e-9)
        w[1, 0] = np.float32(3e-7)
        w[2, :32] = (np.arange(32) - 14).astype(np.float32) * np.float32(2.0 ** -9)
        p = orc.quantize(fmt, w)
        q, scale = _parse(fmt, p, w.shape[0], K)
        want_q, want_d = nearest_codes(fmt, w)
        if not np.array_equal(scale, want_d.astype(np.float64)):
            fails.append(f"fmt{fmt}: scales differ at {np.flatnonzero(scale != want_d)[:5]}")
        bad = np.flatnonzero((q != want_q).any(axis=1))
        if bad.size:
            fails.append(f"fmt{fmt}: {bad.size} blocks with codes off the nearest grid point")
    return fails


def pin_invariants(orc) -> list:
    fails = []
    for fmt in (Q4_0, Q8_0):
        qmax = 7 if fmt == Q4_0 else 127
        w = si.weights(64, 512, seed=11)
        p = orc.quantize(fmt, w)
        q, scale = _parse(fmt, p, 64, 512)
        wb = w.reshape(-1, 32).astype(np.float64)
        normal = np.abs(scale) >= 2.0 ** -14
        if fmt == Q4_0 and (q[normal] < -7).any():
            fails.append("q4_0: code 0 (multiplier -8) with a normal scale")
        if (np.abs(q) > (8 if fmt == Q4_0 else 127)).any():
            fails.append(f"fmt{fmt}: code out of range")
        wh = orc.dequant(fmt, p, 64, 512, "f64").reshape(-1, 32)
        if not (np.abs(wb - wh) <= scale[:, None] / 2).all():
            fails.append(f"fmt{fmt}: |w - w_hat| > scale/2")
        am = np.abs(wb).argmax(axis=1)
        if not (np.abs(q[np.arange(q.shape[0]), am]) == qmax).all():
            fails.append(f"fmt{fmt}: absmax element not at +-{qmax}")
        p2 = orc.quantize(fmt, orc.dequant(fmt, p, 64, 512, "f32"))
        if not np.array_equal(p, p2):
            fails.append(f"fmt{fmt}: quantize(dequant(.)) is not the identity")
        w16 = orc.dequant(fmt, p, 64, 512, "f16")
        if not np.array_equal(w16, wh.reshape(64, 512).astype(np.float16)):
            fails.append(f"fmt{fmt}: fp16 dequant is not RNE of the exact value")
        f32 = orc.dequant(fmt, p, 64, 512, "f32")
        if not np.array_equal(f32.astype(np.float64), wh.reshape(64, 512)):
            fails.append(f"fmt{fmt}: fp32 dequant not exact")
    return fails


# ------------------------------------------------------------- exact gemv
def pin_exact_gemv(orc) -> list:
    fails = []
    for fmt in (Q4_0, Q8_0, Q2W):
        for (N, K, M) in ((1, 32, 1), (3, 64, 2), (5, 96, 3), (8, 128, 8)):
            w = si.weights(N, K, seed=3)
            x = si.activations(M, K, seed=3)
            p = orc.quantize(fmt, w)
            q, scale = _parse(fmt, p, N, K)
            y, s = orc.gemv(fmt, p, N, K, x)
            xs = [[Fraction(float(v)) for v in row] for row in x]
            for m in range(M):
                for n in range(N):
                    exact = Fraction(0)
                    sab = Fraction(0)
                    for b in range(K // 32):
                        i = n * (K // 32) + b
                        dd = Fraction(float(scale[i]))
                        for k in range(32):
                            t = int(q[i, k]) * dd * xs[m][32 * b + k]
                            exact += t
                            sab += abs(t)
                    err = abs(Fraction(y[m, n]) - exact)
                    if err > Fraction(1, 2 ** 50) * sab or abs(s[m, n] - float(sab)) > 2.0 ** -50 * float(sab):
                        fails.append(f"fmt{fmt} {N}x{K} m{m} n{n}: y {y[m, n]} vs {float(exact)}")
    return fails


def pin_special(orc) -> list:
    fails = []
    for fmt in (Q4_0, Q8_0):
        N, K = 16, 320
        w = si.weights(N, K, seed=5)
        p = orc.quantize(fmt, w)
        wh = orc.dequant(fmt, p, N, K, "f64")
        for k in (0, 5, 16, 31, 32, 47, 319):
            x = np.zeros((1, K), np.float16)
            x[0, k] = 1.0
            y, _ = orc.gemv(fmt, p, N, K, x)
            if not np.array_equal(y[0], wh[:, k]):
                fails.append(f"fmt{fmt}: one-hot e_{k} is not column {k}")
        y, s = orc.gemv(fmt, p, N, K, np.zeros((1, K), np.float16))
        if (y != 0).any() or (s != 0).any():
            fails.append(f"fmt{fmt}: zero input")
        x = np.zeros((1, K), np.float16)
        x[0, 64:96] = 1.0
        y, _ = orc.gemv(fmt, p, N, K, x)
        if not np.array_equal(y[0], wh[:, 64:96].sum(axis=1)):
            fails.append(f"fmt{fmt}: ones on block 2")
        x4 = si.activations(4, K, seed=9)
        y4, _ = orc.gemv(fmt, p, N, K, x4)
        for m in range(4):
            y1, _ = orc.gemv(fmt, p, N, K, x4[m:m + 1])
            if not np.array_equal(y1[0], y4[m]):
                fails.append(f"fmt{fmt}: token {m} of a 4-token call differs from a 1-token call")
        # linearity: x = a + b with a, b on disjoint halves of K
        a = x4[0].copy()
        a[K // 2:] = 0
        b = x4[0].copy()
        b[:K // 2] = 0
        ya, sa = orc.gemv(fmt, p, N, K, a[None])
        yb, sb = orc.gemv(fmt, p, N, K, b[None])
        if not (np.abs(ya + yb - y4[0]) <= 1e-12 * (sa + sb)).all():
            fails.append(f"fmt{fmt}: linearity")
        yr, sr = orc.gemv_rows(fmt, p, N, K, x4, [3, 0, 15])
        if not (np.array_equal(yr, y4[:, [3, 0, 15]])):
            fails.append(f"fmt{fmt}: gemv_rows differs from gemv")
    return fails


def pin_moe(orc) -> list:
    fails = []
    P, E, N, K = 6, 4, 24, 96
    pool_w = si.expert_pool(P, N, K, seed=2)
    stride = orc.packed_bytes(Q4_0, N, K)
    pool = np.concatenate([orc.quantize(Q4_0, pool_w[j]) for j in range(P)])
    x = si.activations(E, K, seed=2)
    for idx in (np.array([5, 0, 3, 1], np.int32), np.array([2, 2, 2, 4], np.int32)):
        y, s = orc.moe(Q4_0, pool, P, idx, x, N, K)
        for e in range(E):
            ye, se = orc.gemv(Q4_0, pool[idx[e] * stride:(idx[e] + 1) * stride], N, K, x[e:e + 1])
            if not (np.array_equal(ye[0], y[e]) and np.array_equal(se[0], s[e])):
                fails.append(f"moe: expert slot {e} (pool {idx[e]}) is not its GEMV")
    perm = np.array([1, 3, 0, 2])
    idx = np.array([5, 0, 3, 1], np.int32)
    y, _ = orc.moe(Q4_0, pool, P, idx, x, N, K)
    yp, _ = orc.moe(Q4_0, pool, P, idx[perm], x[perm], N, K)
    if not np.array_equal(yp, y[perm]):
        fails.append("moe: permuting experts does not permute outputs")
    return fails


def pin_prefill(orc) -> list:
    fails = []
    N, K, M = 40, 192, 24
    w = si.weights(N, K, seed=4)
    X = si.activations(M, K, seed=4)
    p = orc.quantize(Q4_0, w)
    Y, S = orc.prefill(p, N, K, X)
    q, scale = _parse(Q4_0, p, N, K)
    wh = (q * scale[:, None]).reshape(N, K)
    ref = X.astype(np.float64) @ wh.T
    if not (np.abs(Y - ref) <= 1e-12 * S).all():
        fails.append("prefill: differs from float64 matmul")
    sref = np.abs(X.astype(np.float64)) @ np.abs(wh.T)
    if not (np.abs(S - sref) <= 1e-12 * sref).all():
        fails.append("prefill: s differs from |X| @ |W|^T")
    return fails


def pin_f32in(orc) -> list:
    fails = []
    g = np.random.default_rng(11)
    vals = np.concatenate([
        g.standard_normal(4096).astype(np.float32) * np.float32(3),
        np.array([0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 70000.0, -1e6, 1e-7, 5.96e-8, 2.98e-8,
                  2.9802322e-08, 6.1035156e-05, 6.1e-05, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, -(1.0 + 2 ** -11),
                  2048.0 + 1.0, 2048.0 + 3.0, 1e-10, -3e-8], np.float32),
        (g.standard_normal(512) * 30000).astype(np.float32),
        (g.standard_normal(512) * 1e-6).astype(np.float32)])
    ours = orc.floats_to_half(vals)
    with np.errstate(over="ignore"):                 # 70000 and -1e6 overflow on purpose
        ref = vals.astype(np.float16).view(np.uint16)
    bad = np.flatnonzero(ours != ref)
    if bad.size:
        i = bad[0]
        fails.append(f"f32 -> f16 of {vals[i]!r}: {ours[i]:#06x} vs numpy {ref[i]:#06x} ({bad.size} differ)")
    nan = orc.floats_to_half(np.array([np.nan], np.float32))[0]
    if not ((nan & 0x7c00) == 0x7c00 and (nan & 0x3ff)):
        fails.append("f32 -> f16 of NaN is not a NaN")
    for fmt in (Q4_0, Q8_0):
        N, K, M = 12, 128, 3
        p = orc.quantize(fmt, si.weights(N, K, seed=6))
        x32 = (g.standard_normal((M, K)) * 4).astype(np.float32)
        y, s_ = orc.gemv_f32in(fmt, p, N, K, x32)
        y2, s2 = orc.gemv(fmt, p, N, K, x32.astype(np.float16))
        if not (np.array_equal(y, y2) and np.array_equal(s_, s2)):
            fails.append(f"fmt{fmt}: GEMV on fp32 input differs from the GEMV on numpy's float16 cast")
    return fails


def pin_silu(orc) -> list:
    fails = []
    ln3 = float(np.log(3.0))
    checks = [(0.0, 0.0, 0.0), (ln3, 0.75 * ln3, 1e-15), (40.0, 40.0, 1e-15)]
    for v, want, rel in checks:
        got = orc.silu(v)
        if abs(got - want) > rel * abs(want):
            fails.append(f"silu({v}) = {got!r}, want {want!r}")
    if abs(orc.silu(-40.0)) > 1e-15:
        fails.append(f"silu(-40) = {orc.silu(-40.0)!r} is not ~0")
    vmin = orc.silu(-1.2784645)
    if abs(vmin + 0.2784645) > 1e-7:
        fails.append(f"silu at its minimum -1.2784645 is {vmin!r}, not -0.2784645")
    if orc.silu(-1.2784645 - 0.01) < vmin or orc.silu(-1.2784645 + 0.01) < vmin:
        fails.append("silu's minimum is not near -1.2784645")
    for v in np.random.default_rng(12).standard_normal(64) * 5:
        d = orc.silu(v) - orc.silu(-v)
        if abs(d - v) > 1e-14 * abs(v):
            fails.append(f"silu({v}) - silu({-v}) = {d!r} is not {v!r}")
            break
    return fails


def pin_swiglu(orc) -> list:
    fails = []
    N, K, M = 10, 96, 2
    wg = si.weights(N, K, seed=21)
    wu = si.weights(N, K, seed=22)
    stacked = orc.quantize(Q4_0, np.concatenate([wg, wu]))
    x32 = (np.random.default_rng(23).standard_normal((M, K)) * 2).astype(np.float32)
    y, g, u, sg, su = orc.swiglu(stacked, N, K, x32)
    g1, sg1 = orc.gemv_f32in(Q4_0, orc.quantize(Q4_0, wg), N, K, x32)
    u1, su1 = orc.gemv_f32in(Q4_0, orc.quantize(Q4_0, wu), N, K, x32)
    if not (np.array_equal(g, g1) and np.array_equal(sg, sg1)):
        fails.append("swiglu: gate half is not the gate table's GEMV")
    if not (np.array_equal(u, u1) and np.array_equal(su, su1)):
        fails.append("swiglu: up half is not the up table's GEMV")
    # a zero gate table: silu(0) = 0 whatever the up rows give
    yz, gz, uz, _, _ = orc.swiglu(orc.quantize(Q4_0, np.concatenate([np.zeros_like(wg), wu])), N, K, x32)
    if (yz != 0).any() or (uz == 0).all():
        fails.append("swiglu: a zero gate table does not give zero")
    # a large gate (every gate weight 0.875, activations 2: g = 56, silu(g) = g
    # in fp64) gives g * u
    big = np.full((N, K), 0.875, np.float32)
    xb = np.full((M, K), 2.0, np.float32)
    yb, gb, ub, _, _ = orc.swiglu(orc.quantize(Q4_0, np.concatenate([big, wu])), N, K, xb)
    if not (gb == 0.875 * 2.0 * K).all():
        fails.append(f"swiglu: gate of constant rows is {gb[0, 0]!r}, not {0.875 * 2.0 * K}")
    if not (np.abs(yb - gb * ub) <= 1e-12 * np.abs(gb * ub)).all():
        fails.append("swiglu: a large gate does not give gate * up")
    return fails


def pin_act8(orc) -> list:
    """8-bit activation quantizer and the GEMV on its codes."""
    fails = []
    # hand-derived worked example (ties to even, the all-zero block, fl32(1/127))
    g = load_golden("act8_we5.txt")
    K = int(g["K"])
    x = np.concatenate([np.array([float(v) for v in g[f"x{b}"].split()]) for b in range(K // 32)])
    x16 = x.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x), "WE5 inputs must be exact binary16 values"
    qx, dx = orc.quantize_act8(x16[None, :])
    want_q = np.concatenate([np.array([int(v) for v in g[f"q{b}"].split()]) for b in range(K // 32)])
    if not np.array_equal(qx[0].astype(np.int64), want_q):
        i = int(np.flatnonzero(qx[0] != want_q)[0])
        fails.append(f"act8 WE5: code {i} of x = {x[i]} is {qx[0, i]}, want {want_q[i]}")
    want_d = np.array([int(v, 16) for v in g["dx_bits"].split()], np.uint32)
    if not np.array_equal(dx[0].view(np.uint32), want_d):
        fails.append(f"act8 WE5: scales {[hex(v) for v in dx[0].view(np.uint32)]} vs {list(g['dx_bits'].split())}")
    # blocks whose amax is 127 * 2^e: dx = 2^e, inv = 2^-e exactly, so the
    # codes are numpy's round-half-even of x / 2^e (an exact division)
    rng = np.random.default_rng(31)
    for e in (-12, -3, 0, 2, 7):
        xb = (rng.uniform(-1, 1, (3, 64)) * 127 * 2.0 ** e).astype(np.float16)
        xb[:, 5] = 127 * 2.0 ** e
        xb[:, 40] = -127 * 2.0 ** e
        xb[1, 7] = 2.5 * 2.0 ** e                     # ties
        xb[2, 50] = -0.5 * 2.0 ** e
        q, d = orc.quantize_act8(xb)
        if not (d == np.float32(2.0 ** e)).all():
            fails.append(f"act8: amax 127*2^{e} gives scales {np.unique(d)}")
        want = np.rint(xb.astype(np.float64) / 2.0 ** e)
        if not np.array_equal(q.astype(np.float64), want):
            fails.append(f"act8: amax 127*2^{e}: codes differ from round-half-even of x / 2^{e}")
    # invariants on wide-range data: |q| <= 127, the block's largest |x| maps
    # to +-127, reconstruction within half a step
    xr = (rng.standard_normal((4, 512)) * np.exp(rng.uniform(-8, 8, (4, 1)))).astype(np.float16)
    xr[0, :32] = 0
    xr[1, 32:64] = np.float16(3e4) * np.sign(rng.standard_normal(32)).astype(np.float16)
    q, d = orc.quantize_act8(xr)
    xf = xr.astype(np.float64).reshape(4, -1, 32)
    qb = q.astype(np.float64).reshape(4, -1, 32)
    if (np.abs(qb) > 127).any():
        fails.append("act8: a code beyond +-127")
    amax_at = np.abs(xf).argmax(axis=2)
    top = np.take_along_axis(qb, amax_at[..., None], axis=2)[..., 0]
    nz = np.abs(xf).max(axis=2) > 0
    if not (np.abs(top[nz]) == 127).all():
        fails.append("act8: the largest |x| of a block does not map to +-127")
    if (qb[~nz] != 0).any() or (d[~nz] != 0).any():
        fails.append("act8: an all-zero block does not give codes 0 and scale 0")
    err = np.abs(xf - qb * d.astype(np.float64)[..., None])
    if (err > 0.5 * d.astype(np.float64)[..., None] * (1 + 1e-5)).any():
        fails.append("act8: reconstruction error above half a step")
    # the GEMV on the codes equals numpy's fp64 matmul of the exactly
    # dequantized weights (Q4_0 and q2w) with the dequantized activations
    N, K, M = 9, 160, 3
    xa = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    q, d = orc.quantize_act8(xa)
    A = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    for fmt in (Q4_0, Q2W):
        p = orc.quantize(fmt, si.weights(N, K, seed=41))
        y, s_ = orc.gemv_q8act_codes(p, N, K, q, d, fmt)
        W = orc.dequant(fmt, p, N, K, "f64")
        yr = A @ W.T
        sr = np.abs(A) @ np.abs(W).T
        if not (np.abs(y - yr) <= 1e-12 * sr).all():
            fails.append(f"act8 GEMV (fmt {fmt}) differs from the matmul of dequantized weights and activations")
        if not (np.abs(s_ - sr) <= 1e-12 * sr).all():
            fails.append(f"act8 GEMV (fmt {fmt}): sum |w x| differs from the matmul of the absolute values")
        y2, _ = orc.gemv_q8act(p, N, K, xa, fmt)
        if not np.array_equal(y, y2):
            fails.append("act8: gemv_q8act is not quantize_act8 then the GEMV on the codes")
    p = orc.quantize(Q4_0, si.weights(N, K, seed=41))
    y, _ = orc.gemv_q8act(p, N, K, xa)
    W = orc.dequant(Q4_0, p, N, K, "f64")
    # within the activation rounding of the exact fp16 GEMV
    ye, _ = orc.gemv(Q4_0, p, N, K, xa)
    bound = np.abs(W) @ (0.5 * np.repeat(d.astype(np.float64), 32, axis=1) * (1 + 1e-5)).T
    if not (np.abs(y - ye) <= bound.T + 1e-12).all():
        fails.append("act8 GEMV further from the fp16 GEMV than the activation rounding allows")
    return fails


def pin_q2w(orc) -> list:
    """Plain 2-bit blocks: the hand-derived block, the scale rule, nearest
    codes by brute force, invariants, and the GEMV against numpy's matmul."""
    fails = []
    g = load_golden("q2w_we6.txt")
    w = _golden_weights(g)
    p = orc.quantize(Q2W, w)
    if p.size != orc.packed_bytes(Q2W, 1, 32) or p.size != 512:
        fails.append(f"q2w: packed size {p.size} for one block, want 512 (8 code bytes and a scale, 256-aligned)")
    want = bytes.fromhex("".join(g["code_bytes"].split()))
    if bytes(p[:8]) != want:
        fails.append(f"q2w WE6: code bytes {bytes(p[:8]).hex()} vs {want.hex()}")
    sbits = int(p[256]) | (int(p[257]) << 8)
    if sbits != int(g["scale_bits"], 16):
        fails.append(f"q2w WE6: scale {sbits:#06x} vs {g['scale_bits']}")
    q, scale = _parse(Q2W, p, 1, 32)
    codes = np.array([int(c) for c in g["codes"].split()])
    if not np.array_equal(q[0], codes):
        fails.append(f"q2w WE6: parsed codes {q[0]} vs {codes}")
    if not np.array_equal(orc.dequant(Q2W, p, 1, 32, "f64")[0], codes * scale[0]):
        fails.append("q2w WE6: dequant is not code * scale")
    y, _ = orc.gemv(Q2W, p, 1, 32, np.ones((1, 32), np.float16))
    if y[0, 0] != float(g["y_ones"]):
        fails.append(f"q2w WE6: y_ones {y[0, 0]!r} vs {g['y_ones']}")
    for key in ("y_e3", "y_e8"):
        x = np.zeros((1, 32), np.float16)
        x[0, int(key[3:])] = 1.0
        y, _ = orc.gemv(Q2W, p, 1, 32, x)
        if y[0, 0] != float(g[key]):
            fails.append(f"q2w WE6: {key} {y[0, 0]!r} vs {g[key]}")
    # scale rule and nearest codes by brute force on many blocks, with ties,
    # both signs of the extreme weight, zero and tiny blocks
    N, K = 256, 256
    w = si.weights(N, K, seed=17)
    w[0, :32] = 0.0
    w[1, :32] = np.float32(1e-9)
    w[2, :32] = (np.arange(32) - 14).astype(np.float32) * np.float32(2.0 ** -6)
    w[3, :32] = -w[2, :32]
    w[4, 32:64] = np.float32(0.25) * ((np.arange(32) % 5) - 2).astype(np.float32)
    p = orc.quantize(Q2W, w)
    q, scale = _parse(Q2W, p, N, K)
    blocks = w.reshape(-1, 32)
    first = np.abs(blocks).argmax(axis=1)                 # numpy: the first maximum
    m = blocks[np.arange(blocks.shape[0]), first]
    d16 = (m / np.float32(-2.0)).astype(np.float16)
    if not np.array_equal(scale, d16.astype(np.float64)):
        fails.append(f"q2w: scales differ from fp16(m / -2) at {np.flatnonzero(scale != d16)[:5]}")
    d = d16.astype(np.float64)
    best = np.zeros(blocks.shape, np.int64)
    bestd = np.full(blocks.shape, np.inf)
    for c in (-2, -1, 0, 1):
        dist = np.abs(blocks.astype(np.float64) - c * d[:, None])
        better = (dist < bestd) | ((dist == bestd) & (abs(c) > np.abs(best)))
        best = np.where(better, c, best)
        bestd = np.where(better, dist, bestd)
    best[d == 0.0] = 0
    bad = np.flatnonzero((q != best).any(axis=1))
    if bad.size:
        fails.append(f"q2w: {bad.size} blocks with codes off the nearest grid point (first {bad[0]})")
    normal = np.abs(d) >= 2.0 ** -14
    if not (q[np.arange(q.shape[0]), first][normal] == -2).all():
        fails.append("q2w: the largest-magnitude weight is not at code -2")
    p2 = orc.quantize(Q2W, orc.dequant(Q2W, p, N, K, "f32"))
    if not np.array_equal(p, p2):
        fails.append("q2w: quantize(dequant(.)) is not the identity")
    # the GEMV against numpy's fp64 matmul of the dequantized weights
    x = si.activations(3, K, seed=17)
    y, s_ = orc.gemv(Q2W, p, N, K, x)
    W = (q * scale[:, None]).reshape(N, K)
    yr = x.astype(np.float64) @ W.T
    sr = np.abs(x.astype(np.float64)) @ np.abs(W).T
    if not (np.abs(y - yr) <= 1e-12 * sr).all():
        fails.append("q2w GEMV differs from the matmul of the parsed weights")
    return fails


ALL_PINS = [pin_codec, pin_golden, pin_nearest, pin_invariants, pin_exact_gemv, pin_special, pin_moe,
            pin_prefill, pin_f32in, pin_silu, pin_swiglu, pin_act8, pin_q2w]
