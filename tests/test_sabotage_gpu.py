"""Sabotage sweep over every entry point that reads packed weights
[volta-kernel-bakeoff, "Making it fair": corrupted packed weights must fail
every check of the packed kernels, while the dense fp16 contender, which
never reads them, passes as a control].

Each case runs twice on the same inputs: on the library's bytes as packed
(the check must pass) and on a corrupted copy (every code byte XOR 0x11, so
each weight moves by one step of its block's scale, and every scale's sign
flipped; the check must fail).  The oracle always keeps the clean bytes.
The tally (failures == checks, controls passed) is asserted and printed in
the session summary.  The suite-wide switch QGEMV_SABOTAGE=1 applies the
same corruption to every packed-weight check of the other GPU tests.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import Q2W, Q4_0, Q8_0, REL, ABS, SABOTAGE, TALLY, corrupt, qg, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _within(y, ref):
    y_ref, s = ref
    return bool(oracle.within_bound(np.asarray(y, np.float64), y_ref, s, REL, ABS).all())


def _cases(q, o, cus):
    """(name, fmt, N, K, rows of the packed table, run(Wd) -> output, passes(output) -> bool)."""
    cases = []
    big = 16 * cus   # rows for which the matrix-core kernel takes several tokens

    def gemv(fmt, N, K, M, seed):
        x = si.activations(M, K, seed=seed)
        fn = {Q4_0: q.qgemv_q4_0, Q8_0: q.qgemv_q8_0, Q2W: q.qgemv_q2w}[fmt]
        return (lambda Wd: fn(Wd, to_dev(x), N, K),
                lambda po: (lambda y: _within(y, o.gemv(fmt, po, N, K, x))))

    for fmt, name in ((Q4_0, "qgemv_q4_0"), (Q8_0, "qgemv_q8_0"), (Q2W, "qgemv_q2w")):
        for (N, K, M) in ((300, 2560, 1), (130, 6144, 3), (big, 2048, 8)):
            run, mk = gemv(fmt, N, K, M, seed=N + M)
            cases.append((f"{name} {N}x{K} M={M}", fmt, N, K, N, run, mk))
    for (N, K, M) in ((257, 4096, 1), (640, 2560, 4), (big, 2048, 6)):
        x32 = si.activations32(M, K, seed=M)
        cases.append((f"qgemv_q4_0_f32in {N}x{K} M={M}", Q4_0, N, K, N,
                      lambda Wd, x32=x32, N=N, K=K: q.qgemv_q4_0_f32in(Wd, to_dev(x32), N, K),
                      lambda po, x32=x32, N=N, K=K: (lambda y: _within(y, o.gemv_f32in(Q4_0, po, N, K, x32)))))
        def sw_ok(po, x32=x32, N=N, K=K):
            yr, g, u, sg, su = o.swiglu(po, N, K, x32)
            return lambda y: bool(oracle.swiglu_within_bound(y, yr, g, u, sg, su).all())
        cases.append((f"qgemv_q4_0_swiglu_f32in 2x{N}x{K} M={M}", Q4_0, N, K, 2 * N,
                      lambda Wd, x32=x32, N=N, K=K: q.qgemv_q4_0_swiglu_f32in(Wd, to_dev(x32), N, K), sw_ok))
    for fmt, name, fn in ((Q4_0, "qgemv_q4_0_q8act", q.qgemv_q4_0_q8act), (Q2W, "qgemv_q2w_q8act", q.qgemv_q2w_q8act)):
        for (N, K, M) in ((300, 4096, 1), (1000, 2048, 4)):
            x = si.activations(M, K, seed=K + M)
            cases.append((f"{name} {N}x{K} M={M}", fmt, N, K, N,
                          lambda Wd, fn=fn, x=x, N=N, K=K: fn(Wd, to_dev(x), N, K),
                          lambda po, fmt=fmt, x=x, N=N, K=K: (lambda y: _within(y, o.gemv_q8act(po, N, K, x, fmt=fmt)))))
    x = si.activations(1, 2048, seed=9)
    cases.append(("qgemv_q2w_lut 500x2048", Q2W, 500, 2048, 500,
                  lambda Wd: q.qgemv_q2w_lut(Wd, to_dev(x), 500, 2048),
                  lambda po: (lambda y: _within(y, o.gemv(Q2W, po, 500, 2048, x)))))
    for (M, N, K) in ((64, 384, 2048), (300, 256, 2560)):
        X = si.activations(M, K, seed=M)
        cases.append((f"qgemm_q4_0_prefill M={M} {N}x{K}", Q4_0, N, K, N,
                      lambda Wd, X=X, N=N, K=K: q.qgemm_q4_0_prefill(Wd, to_dev(X), N, K),
                      lambda po, X=X, N=N, K=K: (lambda y: _within(y, o.prefill(po, N, K, X)))))
    for fmt, name, fn in ((Q4_0, "qdequant_q4_0", q.qdequant_q4_0), (Q8_0, "qdequant_q8_0", q.qdequant_q8_0),
                          (Q2W, "qdequant_q2w", q.qdequant_q2w)):
        for f16 in (False, True):
            N, K = 70, 640
            cases.append((f"{name} {'fp16' if f16 else 'fp32'}", fmt, N, K, N,
                          lambda Wd, fn=fn, f16=f16, N=N, K=K: fn(Wd, N, K, fp16=f16),
                          lambda po, fmt=fmt, f16=f16, N=N, K=K: (
                              lambda y: np.array_equal(y.view(np.uint16 if f16 else np.uint32),
                                                       o.dequant(fmt, po, N, K, "f16" if f16 else "f32")
                                                       .view(np.uint16 if f16 else np.uint32)))))
    return cases


def test_sabotage_fails_every_packed_weight_check():
    if SABOTAGE:
        pytest.skip("the suite-wide sabotage switch is on: this sweep's clean runs would read corrupted bytes")
    torch = torch_cuda()
    q = qg()
    o = oracle.get()
    cus = q.qg_device_cus()
    checks = failed = clean_ok = 0
    names = []
    for name, fmt, N, K, rows, run, mk in _cases(q, o, cus):
        w = si.weights(rows, K, seed=rows + K)
        pb = {Q4_0: q.qquantize_q4_0, Q8_0: q.qquantize_q8_0, Q2W: q.qquantize_q2w}[fmt](w)
        po = o.quantize(fmt, w)
        assert np.array_equal(pb, po)
        passes = mk(po)
        y = run(to_dev(pb))
        torch.cuda.synchronize()
        assert passes(y.cpu().numpy()), f"{name}: the clean run fails"
        clean_ok += 1
        yb = run(to_dev(corrupt(pb, fmt, rows, K)))
        torch.cuda.synchronize()
        checks += 1
        if passes(yb.cpu().numpy()):
            names.append(name)
        else:
            failed += 1
    # MoE: every expert of the pool corrupted
    P, E, N, K = 12, 10, 640, 2560
    pw = si.expert_pool(P, N, K, seed=1)
    pb = np.concatenate([q.qquantize_q4_0(pw[j]) for j in range(P)])
    po = np.concatenate([o.quantize(Q4_0, pw[j]) for j in range(P)])
    assert np.array_equal(pb, po)
    idx = si.expert_indices(P, E, seed=1)
    x = si.activations(E, K, seed=1)
    ref = o.moe(Q4_0, po, P, idx, x, N, K)
    for bytes_, clean in ((pb, True), (corrupt(pb, Q4_0, N, K, count=P), False)):
        y = q.qmoe_gemv_q4_0(to_dev(bytes_), P, to_dev(idx), to_dev(x), N, K)
        torch.cuda.synchronize()
        ok = _within(y.cpu().numpy(), ref)
        if clean:
            assert ok, "qmoe_gemv_q4_0: the clean run fails"
            clean_ok += 1
        else:
            checks += 1
            failed += int(not ok)
            if ok:
                names.append("qmoe_gemv_q4_0")
    # control: the dense fp16 GEMM on the oracle's clean fp16 weights
    M, N, K = 64, 384, 2048
    w = si.weights(N, K, seed=N + K)
    po = o.quantize(Q4_0, w)
    X = si.activations(M, K, seed=M)
    Yd = torch.matmul(to_dev(X), to_dev(o.dequant(Q4_0, po, N, K, "f16")).t().contiguous()).float()
    torch.cuda.synchronize()
    control = _within(Yd.cpu().numpy(), o.prefill(po, N, K, X))
    TALLY["sweep"] = (failed, checks, int(control))
    print(f"sabotage sweep: {failed} of {checks} packed-weight checks failed on corrupted bytes "
          f"({clean_ok} clean runs passed); dense fp16 control {'passed' if control else 'FAILED'}")
    assert not names, f"checks that did not see the corruption: {names}"
    assert failed == checks and checks >= 29
    assert control
