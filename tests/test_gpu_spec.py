"""GPU parity of speculative decoding: output-only verify of T drafts, rollback by pointer move
with the commit-time flush, and the per-draft snapshot baseline, against the float64 oracle.

Truth: from the committed state, the drafts run one by one through the stepwise recurrence; all T
outputs are compared (rejected ones included); after rollback the committed state is the state
after the accepted prefix. Pointers are compared bit-exactly with the oracle's pointer machine for
every sequence. Every verify output is also compared at 1e-5 with the oracle's replay-form model
reading the same copy; whenever a sequence flushes, its GPU master must equal the committed truth
(1e-5), its read copy must be the oracle's encoding of that master bit for bit, and the model
continues from that master.
"""
import numpy as np
import pytest
import torch

import hybrid_mamba_decode_amd as rs
import oracle
import workload
from gpu_harness import PREC_CODE, Case, assert_copy_encodes, dev, host, log, rel

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5


def _pointer_machine(Bt, L, Tmax):
    """The oracle's replay machine with 1x1x1 heads: only its pointers are used."""
    z = np.zeros((Bt, 1, 1, 1), np.float32)
    return oracle.Replay(z, np.array([-1.0], np.float32), np.zeros(1, np.float32), 1, L, Tmax)


def _reseed_flushed(lay, dual, sample, ck_prev, ck, S, read_prec, what):
    """Sequences of the sample whose checkpoint moved were just flushed: their GPU master must
    equal the committed truth, their read copy must be the oracle's encoding of that master, and
    the same-copy model continues from it (O6). Returns the number reseeded."""
    flushed = [i for i, b in enumerate(sample) if ck[b] != ck_prev[b]]
    if not flushed:
        return 0
    rows = np.asarray(sample)[flushed]
    m = host(lay.master()[torch.as_tensor(rows, device="cuda")])
    e = rel(m, S[flushed])
    assert e <= TOL_F32, f"{what}: post-flush checkpoint error {e:.3e}"
    if read_prec != "fp32":
        assert_copy_encodes(lay, read_prec, m, rows, what)
    dual.set_checkpoint(m, flushed)
    return len(flushed)


def _run_spec(case, T, iters, sample, read_prec="fp32", tol=TOL_F32, accept=None, snapshot=False,
              interleave_steps=False):
    log(f"[spec] Bt={case.Bt} H={case.H} P={case.P} N={case.N} G={case.G} L={case.L} T={T} "
        f"iters={iters} prec={read_prec} sample={len(sample)} seqs snapshot={snapshot}")
    lay = case.layer(read_prec, Tmax=T)
    sample = np.asarray(sample)
    S = case.S0[sample].astype(np.float64)
    ptr = _pointer_machine(case.Bt, case.L, T)
    # replay form with the same read copy; after each flush it continues from the GPU's master
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
    worst = worst_dual = 0.0
    reseeded = 0
    ck_prev = [0] * case.Bt
    for it in range(iters):
        x, B, C, dt = case.draft_inputs(it, T)
        acc = accept(it) if accept else workload.accepted_counts(case.seed, it, case.Bt, T)
        y = lay.spec_verify(dev(x), dev(B), dev(C), dev(dt))
        lay.rollback(dev(acc))
        if snapshot:
            ys = torch.empty_like(y)
            rs.snapshot_spec_verify(cfg, slots, cur, T, dev(x), dev(B), dev(C), dev(dt), A, D, ys)
            rs.snapshot_commit(cfg, cur, dev(acc), T)
        y_ref = oracle.spec_stepwise(S, T, x[sample], B[sample], C[sample], dt[sample], case.A, case.D,
                                     acc[sample])
        yh = host(y)[sample]
        e = rel(yh, y_ref)
        worst = max(worst, e)
        assert e <= tol, f"verify {it}: output error {e:.3e}"
        y_dual = dual.verify(T, x[sample], B[sample], C[sample], dt[sample])
        dual.rollback(acc[sample])
        e_dual = rel(yh, y_dual)
        worst_dual = max(worst_dual, e_dual)
        assert e_dual <= TOL_F32, f"verify {it}: error vs the same-copy model {e_dual:.3e}"
        ptr.verify(T, *zeros_tok)
        ptr.rollback(acc)
        pos, ck = lay.get_pointers()
        opos, ock = ptr.pointers()
        assert pos == list(opos) and ck == list(ock), f"verify {it}: pointers differ"
        reseeded += _reseed_flushed(lay, dual, sample, ck_prev, ck, S, read_prec, f"verify {it}")
        ck_prev = ck
        if snapshot:
            # same starting state and drafts as the truth above: the per-draft snapshots must
            # give the same outputs, and the committed slot moves by the accepted count
            assert rel(host(ys)[sample], y_ref) <= TOL_F32, f"verify {it}: snapshot outputs"
            cur_ref = (cur_ref + acc) % (T + 1)
            assert np.array_equal(host(cur), cur_ref)
        if interleave_steps and it % 3 == 2:
            xs, Bs, Cs, dts = workload.step_inputs(case.seed + 1, it, case.Bt, case.H, case.P, case.N, case.G)
            ys1 = host(lay.step(dev(xs), dev(Bs), dev(Cs), dev(dts)))[sample]
            y1_ref = oracle.step(S, xs[sample], Bs[sample], Cs[sample], dts[sample], case.A, case.D)
            y1_dual = dual.step(xs[sample], Bs[sample], Cs[sample], dts[sample])
            assert rel(ys1, y1_ref) <= tol
            assert rel(ys1, y1_dual) <= TOL_F32
            one = [np.zeros((case.Bt, 1, 1), np.float32)] * 3 + [np.zeros((case.Bt, 1), np.float32)]
            ptr.step(*one)
            pos, ck = lay.get_pointers()
            opos, ock = ptr.pointers()
            assert pos == list(opos) and ck == list(ock)
            reseeded += _reseed_flushed(lay, dual, sample, ck_prev, ck, S, read_prec, f"step after verify {it}")
            ck_prev = ck
    st = host(lay.materialize_state())[sample]
    assert rel(st, S) <= TOL_F32, f"committed state error {rel(st, S):.3e}"
    if snapshot:
        cur_h = host(cur)
        for i, b in enumerate(sample):
            assert rel(host(slots[b, int(cur_h[b])]), S[i]) <= TOL_F32
    assert lay.check() == rs.RSSM_OK
    log(f"  worst vs truth {worst:.2e}, vs same-copy model {worst_dual:.2e}; {reseeded} post-flush reseeds")
    return worst


def test_spec_serving_batch512_T4():
    """Spec decode on the serving layer: batch 512, T = 4 drafts, accepted prefix uniform in
    {0..4}, 128 verify steps, every sequence compared; per-draft snapshot baseline alongside."""
    c = workload.SPEC
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(3), Tmax=c["T"])
    worst = _run_spec(case, c["T"], c["steps"], range(c["Bt"]), snapshot=True)
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


def test_spec_fp8_blocks_of_64_rows():
    """Spec verify and rollback through an fp8 copy with P = 128 (two scale blocks per head)."""
    case = Case(2, 4, 128, 64, 2, 8, 43, Tmax=3)
    _run_spec(case, 3, 30, range(2), read_prec="fp8", tol=6e-2)


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


def test_snapshot_spec_step_one_call():
    """The one-call snapshot baseline at the speculative-decoding shape (batch 512, the serving
    heads, T = 4, accepted prefix uniform in {0..4}): all T outputs of every sequence against the
    per-draft truth at 1e-5, cur bit-exact, and the committed slot equal to the truth's state."""
    c = workload.SPEC
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(3), Tmax=c["T"])
    T = c["T"]
    log(f"[snapshot_spec_step] Bt={case.Bt} T={T}")
    cfg = rs.make_config(case.Bt, case.H, case.P, case.N, case.G)
    slots = torch.zeros(case.Bt, T + 1, case.H, case.P, case.N, device="cuda")
    slots[:, 0] = dev(case.S0)
    cur = torch.zeros(case.Bt, dtype=torch.int32, device="cuda")
    cur_ref = np.zeros(case.Bt, np.int64)
    S = case.S0.astype(np.float64)
    A, D = dev(case.A), dev(case.D)
    for it in range(6):
        x, B, C, dt = case.draft_inputs(it, T)
        acc = workload.accepted_counts(case.seed, it, case.Bt, T)
        y = torch.empty(case.Bt, T, case.H, case.P, device="cuda")
        rs.snapshot_spec_step(cfg, slots, cur, T, dev(x), dev(B), dev(C), dev(dt), A, D, y, dev(acc))
        y_ref = oracle.spec_stepwise(S, T, x, B, C, dt, case.A, case.D, acc)
        assert rel(host(y), y_ref) <= TOL_F32, f"iteration {it}"
        cur_ref = (cur_ref + acc) % (T + 1)
        assert np.array_equal(host(cur), cur_ref), f"iteration {it}: cur"
    cur_h = host(cur)
    committed = torch.stack([slots[b, int(cur_h[b])] for b in range(case.Bt)])
    assert rel(host(committed), S) <= TOL_F32
