"""GPU parity of speculative decoding: output-only verify of T drafts, rollback by pointer move
with the commit-time flush, and the per-draft snapshot baseline, against the float64 oracle.

Truth: from the committed state, the drafts run one by one through the stepwise recurrence; all T
outputs are compared (rejected ones included); after rollback the committed state is the state
after the accepted prefix. Pointers are compared bit-exactly with the oracle's pointer machine for
every sequence.
"""
import numpy as np
import pytest
import torch

import hybrid_mamba_decode_amd as rs
import oracle
import workload
from gpu_harness import PREC_CODE, Case, dev, host, log, rel

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5


def _pointer_machine(Bt, L, Tmax):
    """The oracle's replay machine with 1x1x1 heads: only its pointers are used."""
    z = np.zeros((Bt, 1, 1, 1), np.float32)
    return oracle.Replay(z, np.array([-1.0], np.float32), np.zeros(1, np.float32), 1, L, Tmax)


def _run_spec(case, T, iters, sample, read_prec="fp32", tol=TOL_F32, accept=None, snapshot=False,
              interleave_steps=False):
    log(f"[spec] Bt={case.Bt} H={case.H} P={case.P} N={case.N} G={case.G} L={case.L} T={T} "
        f"iters={iters} prec={read_prec} sample={list(sample)} snapshot={snapshot}")
    lay = case.layer(read_prec, Tmax=T)
    sample = np.asarray(sample)
    S = case.S0[sample].astype(np.float64)
    ptr = _pointer_machine(case.Bt, case.L, T)
    # replay form with the same read copy: until a sampled sequence first flushes, its copy is the
    # oracle's encoding bit for bit, so the verify outputs must match this model to fp32 rounding
    dual = oracle.Replay(case.S0[sample], case.A, case.D, case.G, case.L, T, PREC_CODE[read_prec])
    zeros_tok = [np.zeros((case.Bt, T, 1, 1), np.float32), np.zeros((case.Bt, T, 1, 1), np.float32),
                 np.zeros((case.Bt, T, 1, 1), np.float32), np.zeros((case.Bt, T, 1), np.float32)]
    cfg = rs.make_config(case.Bt, case.H, case.P, case.N, case.G)
    if snapshot:
        slots = torch.zeros(case.Bt, T + 1, case.H, case.P, case.N, device="cuda")
        slots[:, 0] = dev(case.S0)
        cur = torch.zeros(case.Bt, dtype=torch.int32, device="cuda")
        cur_ref = np.zeros(case.Bt, np.int64)
    A, D = dev(case.A), dev(case.D)
    worst = 0.0
    for it in range(iters):
        x, B, C, dt = case.draft_inputs(it, T)
        acc = accept(it) if accept else workload.accepted_counts(case.seed, it, case.Bt, T)
        y = lay.spec_verify(dev(x), dev(B), dev(C), dev(dt))
        lay.rollback(dev(acc))
        S_before = S.copy()
        y_ref = oracle.spec_stepwise(S, T, x[sample], B[sample], C[sample], dt[sample], case.A, case.D,
                                     acc[sample])
        e = rel(host(y)[sample], y_ref)
        worst = max(worst, e)
        assert e <= tol, f"verify {it}: output error {e:.3e}"
        never_flushed = not dual.pointers()[1].any()
        y_dual = dual.verify(T, x[sample], B[sample], C[sample], dt[sample])
        dual.rollback(acc[sample])
        if never_flushed or read_prec == "fp32":
            e_dual = rel(host(y)[sample], y_dual)
            assert e_dual <= TOL_F32, f"verify {it}: error vs the dual-precision model {e_dual:.3e}"
        ptr.verify(T, *zeros_tok)
        ptr.rollback(acc)
        pos, ck = lay.get_pointers()
        opos, ock = ptr.pointers()
        assert pos == list(opos) and ck == list(ock), f"verify {it}: pointers differ"
        if snapshot:
            ys = torch.empty_like(y)
            rs.snapshot_spec_verify(cfg, slots, cur, T, dev(x), dev(B), dev(C), dev(dt), A, D, ys)
            rs.snapshot_commit(cfg, cur, dev(acc), T)
            ref_snap = oracle.spec_stepwise(S_before.copy(), T, x[sample], B[sample], C[sample], dt[sample],
                                            case.A, case.D, acc[sample])
            assert rel(host(ys)[sample], ref_snap) <= TOL_F32
            cur_ref = (cur_ref + acc) % (T + 1)
            assert np.array_equal(host(cur), cur_ref)
        if interleave_steps and it % 3 == 2:
            xs, Bs, Cs, dts = workload.step_inputs(case.seed + 1, it, case.Bt, case.H, case.P, case.N, case.G)
            ys1 = lay.step(dev(xs), dev(Bs), dev(Cs), dev(dts))
            y1_ref = oracle.step(S, xs[sample], Bs[sample], Cs[sample], dts[sample], case.A, case.D)
            dual.step(xs[sample], Bs[sample], Cs[sample], dts[sample])
            assert rel(host(ys1)[sample], y1_ref) <= tol
            one = [np.zeros((case.Bt, 1, 1), np.float32)] * 3 + [np.zeros((case.Bt, 1), np.float32)]
            ptr.step(*one)
            pos, ck = lay.get_pointers()
            opos, ock = ptr.pointers()
            assert pos == list(opos) and ck == list(ock)
    st = host(lay.materialize_state())[sample]
    assert rel(st, S) <= TOL_F32, f"committed state error {rel(st, S):.3e}"
    if snapshot:
        cur_h = host(cur)
        for i, b in enumerate(sample):
            assert rel(host(slots[b, int(cur_h[b])]), S[i]) <= TOL_F32
    assert lay.check() == rs.RSSM_OK
    return worst


def test_spec_serving_batch512_T4():
    """Spec decode on the serving layer: batch 512, T = 4 drafts, accepted prefix uniform in
    {0..4}, 128 verify steps; per-draft snapshot baseline alongside."""
    c = workload.SPEC
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(3), Tmax=c["T"])
    worst = _run_spec(case, c["T"], c["steps"], [1, 300, 511], snapshot=True)
    log(f"spec serving: worst verify-output error {worst:.2e}")


@pytest.mark.parametrize("T,L", [(1, 4), (3, 7), (8, 16), (4, 4)])
def test_spec_small(T, L):
    case = Case(3, 4, 16, 32, 2, L, 17 + T, Tmax=T)
    _run_spec(case, T, 30, range(3), snapshot=True)


def test_spec_maximum_sizes():
    """T 8 with L 64, P 256 (four row splits) and N 256: the largest supported verify window."""
    case = Case(2, 2, 256, 256, 1, 64, 61, Tmax=8)
    _run_spec(case, 8, 20, range(2), snapshot=True)


def test_spec_accept_extremes_and_interleaved_steps():
    case = Case(4, 8, 32, 64, 2, 8, 29, Tmax=3)
    pattern = [np.array([0, 3, 0, 3], np.int32), np.array([3, 3, 3, 3], np.int32),
               np.array([0, 0, 0, 0], np.int32)]
    _run_spec(case, 3, 24, range(4), accept=lambda it: pattern[it % 3], interleave_steps=True)


@pytest.mark.parametrize("prec,tol", [("bf16", 2e-2), ("fp8", 6e-2), ("mxfp4", 0.25)])
def test_spec_dual_precision(prec, tol):
    case = Case(2, 8, 64, 128, 2, 16, 41, Tmax=4)
    _run_spec(case, 4, 40, range(2), read_prec=prec, tol=tol)


def test_rollback_flags_bad_accept_count():
    """An accepted count above T sets the device flag; that sequence is left unchanged."""
    case = Case(2, 4, 16, 16, 1, 8, 3, Tmax=2)
    lay = case.layer(Tmax=2)
    x, B, C, dt = case.draft_inputs(0, 2)
    lay.spec_verify(dev(x), dev(B), dev(C), dev(dt))
    lay.rollback(dev(np.array([1, 3], np.int32)))
    assert lay.check() == rs.RSSM_E_STATE
    lay.load_state(dev(case.S0))
    assert lay.check() == rs.RSSM_OK
