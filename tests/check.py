#!/usr/bin/env python3
"""Standalone correctness run with an exit status [volta-kernel-bakeoff,
"Run it": a check mode that exits non-zero on any failure; "Making it fair":
corrupted packed weights must fail every packed-kernel check while the dense
fp16 contender passes as a control].

    python tests/check.py              exit 0 iff every check passes
    python tests/check.py --sabotage   exit 0 iff every packed-weight check
                                       fails on corrupted bytes and the dense
                                       fp16 control passes
    --quick                            only one case per entry point

Checks, each against the oracle on seeded inputs:
  * the headline workload: qgemv_q4_0 at one token on the six Llama-3-8B
    shapes, every output;
  * qgemm_q4_0_prefill on the three prefill tables at 64 and 512 tokens,
    every output;
  * qmoe_gemv_q4_0 on both expert pools;
  * one case per entry point (the GPU sabotage test's list: every format of
    the GEMV on both engines, fp32 input, SwiGLU, 8-bit activations, the
    times-table GEMV, the prefill and the dequant);
  * the control: the dense fp16 GEMM (PyTorch) on the oracle's fp16 weights,
    which never reads the library's packed bytes.
With --sabotage every packed matrix the library receives is a corrupted copy
(every code byte XOR 0x11, every scale's sign flipped) while the oracle keeps
the clean bytes.

Test infrastructure: this script calls the oracle (it lives beside the tests
for that reason); the library itself never does.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path[:0] = [ROOT, HERE]

import numpy as np  # noqa: E402


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--sabotage", action="store_true",
                    help="corrupt every packed matrix the library receives; pass iff every packed check fails")
    ap.add_argument("--quick", action="store_true", help="skip the full-size headline, prefill and MoE workloads")
    a = ap.parse_args()

    import torch
    if not torch.cuda.is_available():
        print("check: no GPU visible", flush=True)
        return 2
    import oracle
    import seeded_inputs as si
    from gpu_util import Q2W, Q4_0, Q8_0, corrupt, qg, to_dev
    from test_sabotage_gpu import _cases, _within

    q = qg()
    o = oracle.get()
    cus = q.qg_device_cus()
    quant = {Q4_0: q.qquantize_q4_0, Q8_0: q.qquantize_q8_0, Q2W: q.qquantize_q2w}

    cases = []
    if not a.quick:
        for (N, K) in si.LLAMA3_8B_SHAPES:
            x = si.activations(1, K, seed=0)
            cases.append((f"headline qgemv_q4_0 {N}x{K} M=1, every output", Q4_0, N, K, N,
                          lambda Wd, x=x, N=N, K=K: q.qgemv_q4_0(Wd, to_dev(x), N, K),
                          lambda po, x=x, N=N, K=K: (lambda y: _within(y, o.gemv(Q4_0, po, N, K, x)))))
        for (N, K) in si.PREFILL_SHAPES:
            for M in si.PREFILL_TOKENS:
                X = si.activations(M, K, seed=0)
                cases.append((f"qgemm_q4_0_prefill M={M} {N}x{K}, every output", Q4_0, N, K, N,
                              lambda Wd, X=X, N=N, K=K: q.qgemm_q4_0_prefill(Wd, to_dev(X), N, K),
                              lambda po, X=X, N=N, K=K: (lambda y: _within(y, o.prefill(po, N, K, X)))))
    cases += _cases(q, o, cus)

    results = []   # (name, passed)
    t0 = time.time()
    for name, fmt, N, K, rows, run, mk in cases:
        w = si.weights(rows, K, seed=rows + K)
        pb = quant[fmt](w)
        po = o.quantize(fmt, w)
        del w
        if not np.array_equal(pb, po):
            print(f"FAIL  {name}: the library's packed bytes differ from the oracle's", flush=True)
            results.append((name, False))
            continue
        passes = mk(po)
        y = run(to_dev(corrupt(pb, fmt, rows, K) if a.sabotage else pb))
        torch.cuda.synchronize()
        ok = passes(y.cpu().numpy())
        results.append((name, ok))
        print(f"{'PASS' if ok else 'FAIL'}  {name}", flush=True)
        del y, pb, po

    moe = si.MOE_CONFIGS if not a.quick else [si.MOE_CONFIGS[0]]
    for (P, E, N, K) in moe:
        pw = si.expert_pool(P, N, K, seed=0)
        pb = np.concatenate([q.qquantize_q4_0(pw[j]) for j in range(P)])
        po = np.concatenate([o.quantize(Q4_0, pw[j]) for j in range(P)])
        del pw
        name = f"qmoe_gemv_q4_0 {E} of {P} experts {N}x{K}"
        if not np.array_equal(pb, po):
            print(f"FAIL  {name}: the library's packed bytes differ from the oracle's", flush=True)
            results.append((name, False))
            continue
        idx = si.expert_indices(P, E, seed=0)
        x = si.activations(E, K, seed=0)
        y = q.qmoe_gemv_q4_0(to_dev(corrupt(pb, Q4_0, N, K, count=P) if a.sabotage else pb), P, to_dev(idx),
                             to_dev(x), N, K)
        torch.cuda.synchronize()
        ok = _within(y.cpu().numpy(), o.moe(Q4_0, po, P, idx, x, N, K))
        results.append((name, ok))
        print(f"{'PASS' if ok else 'FAIL'}  {name}", flush=True)

    # control: the dense fp16 GEMM on the oracle's clean fp16 weights
    M, N, K = 64, 384, 2048
    po = o.quantize(Q4_0, si.weights(N, K, seed=N + K))
    X = si.activations(M, K, seed=M)
    Yd = torch.matmul(to_dev(X), to_dev(o.dequant(Q4_0, po, N, K, "f16")).t().contiguous()).float()
    torch.cuda.synchronize()
    control = _within(Yd.cpu().numpy(), o.prefill(po, N, K, X))
    print(f"{'PASS' if control else 'FAIL'}  control: dense fp16 GEMM {M}x{N}x{K} on the oracle's weights",
          flush=True)

    passed = sum(ok for _, ok in results)
    n = len(results)
    secs = time.time() - t0
    if a.sabotage:
        good = passed == 0 and control
        print(f"check --sabotage: {n - passed} of {n} packed-weight checks failed on corrupted bytes; "
              f"control {'passed' if control else 'FAILED'} ({secs:.0f} s): {'OK' if good else 'NOT OK'}",
              flush=True)
    else:
        good = passed == n and control
        print(f"check: {passed} of {n} packed-weight checks passed; control {'passed' if control else 'FAILED'} "
              f"({secs:.0f} s): {'OK' if good else 'NOT OK'}", flush=True)
    return 0 if good else 1


if __name__ == "__main__":
    sys.exit(main())
