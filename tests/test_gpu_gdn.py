"""GPU parity of the Gated DeltaNet ReplaySSM path (gdnreplay.h) against the float64 oracle.

Bars: pointers and flush schedule bit-exact with the oracle's pointer machine; outputs, flushed
checkpoints and materialized states within 1e-5 normwise relative error of the stepwise
recurrence (O1g); spec-decode outputs of all T drafts and committed states within 1e-5 of the
per-draft definition (O5g); an exactly representable case bit-identical. Full-size workloads run
the whole batch on the GPU and compare sampled sequences.
"""
import numpy as np
import pytest
import torch

import hybrid_mamba_decode_amd as rs
import oracle
import workload
from gpu_harness import dev, host, log, rel

pytestmark = pytest.mark.gpu

TOL = 1e-5


class GCase:
    def __init__(self, Bt, H, G, Dv, Dk, L, seed, Tmax=1):
        self.Bt, self.H, self.G, self.Dv, self.Dk, self.L, self.Tmax = Bt, H, G, Dv, Dk, L, Tmax
        self.seed = seed
        self.S0 = workload.gdn_initial_state(seed, Bt, H, Dv, Dk)

    def step_inputs(self, t):
        return workload.gdn_step_inputs(self.seed, t, self.Bt, self.H, self.G, self.Dv, self.Dk)

    def draft_inputs(self, t, T):
        return workload.gdn_draft_inputs(self.seed, t, self.Bt, T, self.H, self.G, self.Dv, self.Dk)

    def layer(self, Tmax=None, lockstep=True):
        lay = rs.GDNReplay(self.Bt, self.H, self.G, self.Dv, self.Dk, buffer_len=self.L,
                           max_draft=Tmax or self.Tmax)
        lay.set_lockstep(lockstep)
        lay.load_state(dev(self.S0))
        return lay


def _run(case, steps, sample, check_state_every=1, lockstep=True):
    log(f"[gdn replay] Bt={case.Bt} H={case.H} G={case.G} Dv={case.Dv} Dk={case.Dk} L={case.L} "
        f"Tmax={case.Tmax} steps={steps} sample={list(sample)} lockstep={lockstep}")
    lay = case.layer(lockstep=lockstep)
    sample = np.asarray(sample)
    S = case.S0[sample].astype(np.float64)
    rep = oracle.GDNReplay(case.S0[sample], case.G, case.L, case.Tmax)
    period = case.L - case.Tmax + 1
    worst = 0.0
    for t in range(steps):
        ins = case.step_inputs(t)
        o = lay.step(*(dev(a) for a in ins))
        sub = [a[sample] for a in ins]
        o_ref = oracle.gdn_step(S, *sub)
        o_rep = rep.step(*sub)
        e = rel(host(o)[sample], o_ref)
        worst = max(worst, e)
        assert e <= TOL, f"step {t}: output error {e:.3e}"
        assert rel(host(o)[sample], o_rep) <= TOL
        pos, ck = lay.get_pointers()
        opos, ock = rep.pointers()
        assert pos == [t + 1] * case.Bt and list(opos) == [t + 1] * len(sample)
        assert ck == [int(ock[0])] * case.Bt and (t + 1 - ck[0]) == (t + 1) % period
        if check_state_every and (t % check_state_every == 0 or (t + 1) % period == 0):
            assert rel(host(lay.materialize_state())[sample], S) <= TOL, f"step {t}: state"
        if (t + 1) % period == 0:
            assert rel(host(lay.master())[sample], S) <= TOL, f"step {t}: post-flush checkpoint"
    assert lay.check() == rs.RSSM_OK
    return worst


@pytest.mark.parametrize("lockstep", [True, False])
def test_gdn_tiny(lockstep):
    c = workload.GDN_TINY
    _run(GCase(c["Bt"], c["H"], c["G"], c["Dv"], c["Dk"], c["L"], workload.config_seed(5)), c["steps"], range(c["Bt"]),
         lockstep=lockstep)


def test_gdn_serving():
    """Serving-size GDN layer: batch 256, 32 value heads and 16 key heads of 128, L = 16, 64 steps
    (4 flushes); sequences 0, 97, 255 against the oracle, pointers of all 256."""
    c = workload.GDN_SERVING
    worst = _run(GCase(c["Bt"], c["H"], c["G"], c["Dv"], c["Dk"], c["L"], workload.config_seed(6)), c["steps"],
                 [0, 97, 255], check_state_every=8)
    log(f"gdn serving: worst output error {worst:.2e}")


@pytest.mark.parametrize("shape", [
    dict(Bt=1, H=6, G=3, Dv=20, Dk=16, L=5),      # smallest Dk, ragged rows
    dict(Bt=3, H=4, G=2, Dv=100, Dk=32, L=7),     # Dv split over 2 work-groups, ragged tail
    dict(Bt=2, H=4, G=4, Dv=64, Dk=64, L=32),     # window bucket 32
    dict(Bt=2, H=2, G=1, Dv=32, Dk=256, L=20),    # largest Dk
    dict(Bt=2, H=4, G=2, Dv=16, Dk=32, L=64),     # window bucket 64
    dict(Bt=4, H=4, G=2, Dv=64, Dk=128, L=1),     # every step flushes
    dict(Bt=1, H=32, G=16, Dv=128, Dk=128, L=16), # batch 1 at the serving head shape
])
def test_gdn_shapes(shape):
    case = GCase(shape["Bt"], shape["H"], shape["G"], shape["Dv"], shape["Dk"], shape["L"], 131)
    _run(case, 2 * shape["L"] + 3, range(shape["Bt"]), check_state_every=4)


def test_gdn_exact_arithmetic_bit_identical():
    """alpha in {1, 1/2}, beta in {1/2, 1}, small integers (unnormalized k, q in {-1, 0, 1}):
    every fp32 intermediate is exact, so replay outputs, flushed checkpoints and the conventional
    step equal the oracle bit for bit."""
    Bt, H, G, Dv, Dk, L = 2, 4, 2, 8, 16, 4
    rng = np.random.default_rng(99)
    S0 = rng.integers(-2, 3, (Bt, H, Dv, Dk)).astype(np.float32)
    lay = rs.GDNReplay(Bt, H, G, Dv, Dk, buffer_len=L)
    lay.load_state(dev(S0))
    conv = dev(S0.copy())
    cfg = rs.make_gdn_config(Bt, H, G, Dv, Dk)
    S = S0.astype(np.float64)
    for t in range(10):
        q = rng.integers(-1, 2, (Bt, G, Dk)).astype(np.float32)
        k = np.zeros((Bt, G, Dk), np.float32)
        for b in range(Bt):                      # one or two nonzeros per key keeps values small
            for g in range(G):
                k[b, g, rng.integers(Dk, size=2)] = rng.choice([-1.0, 1.0], 2)
        v = rng.integers(-2, 3, (Bt, H, Dv)).astype(np.float32)
        a = rng.choice([1.0, 0.5], (Bt, H)).astype(np.float32)
        be = rng.choice([0.5, 1.0], (Bt, H)).astype(np.float32)
        ins = (q, k, v, a, be)
        o = lay.step(*(dev(x) for x in ins))
        oc = torch.empty_like(o)
        rs.gdn_conventional_step(cfg, conv, *(dev(x) for x in ins), oc)
        o_ref = oracle.gdn_step(S, *ins)
        assert np.array_equal(host(o).astype(np.float64), o_ref), f"step {t}"
        assert np.array_equal(host(oc).astype(np.float64), o_ref), f"conventional step {t}"
        if (t + 1) % L == 0:
            assert np.array_equal(host(lay.master()).astype(np.float64), S)
    assert np.array_equal(host(conv).astype(np.float64), S)


@pytest.mark.parametrize("which", ["tiny", "serving"])
def test_gdn_conventional_step(which):
    c = workload.GDN_TINY if which == "tiny" else workload.GDN_SERVING
    case = GCase(c["Bt"], c["H"], c["G"], c["Dv"], c["Dk"], c["L"], workload.config_seed(5))
    sample = list(range(c["Bt"])) if which == "tiny" else [3, 128, 254]
    cfg = rs.make_gdn_config(case.Bt, case.H, case.G, case.Dv, case.Dk)
    state = dev(case.S0)
    S = case.S0[sample].astype(np.float64)
    for t in range(16 if which == "serving" else c["steps"]):
        ins = case.step_inputs(t)
        o = torch.empty(case.Bt, case.H, case.Dv, device="cuda")
        rs.gdn_conventional_step(cfg, state, *(dev(a) for a in ins), o)
        assert rel(host(o)[sample], oracle.gdn_step(S, *[a[sample] for a in ins])) <= TOL
    assert rel(host(state)[sample], S) <= TOL


def test_gdn_masked_flush_and_materialize():
    case = GCase(4, 4, 2, 32, 64, 16, 55)
    lay = case.layer()
    S = case.S0.astype(np.float64)
    for t in range(6):
        ins = case.step_inputs(t)
        lay.step(*(dev(a) for a in ins))
        oracle.gdn_step(S, *ins)
    assert rel(host(lay.materialize_state()), S) <= TOL
    lay.flush(dev(np.array([1, 0, 1, 0], np.int32)))
    pos, ck = lay.get_pointers()
    assert pos == [6] * 4 and ck == [6, 0, 6, 0]
    m = host(lay.master())
    assert rel(m[[0, 2]], S[[0, 2]]) <= TOL and np.array_equal(m[[1, 3]], case.S0[[1, 3]])
    for t in range(6, 30):
        ins = case.step_inputs(t)
        o = lay.step(*(dev(a) for a in ins))
        assert rel(host(o), oracle.gdn_step(S, *ins)) <= TOL
    lay.flush()
    pos, ck = lay.get_pointers()
    assert pos == ck == [30] * 4
    assert rel(host(lay.master()), S) <= TOL


@pytest.mark.parametrize("lockstep", [True, False])
def test_gdn_corrupted_pointers_flag(lockstep):
    case = GCase(2, 4, 2, 16, 32, 4, 11)
    lay = case.layer(lockstep=lockstep)
    ins = [dev(a) for a in case.step_inputs(0)]
    lay.step(*ins)
    pos, ck = lay.pointer_arrays()
    ck[1] = 5
    torch.cuda.synchronize()
    lay.step(*ins)
    assert lay.check() == rs.RSSM_E_STATE
    with pytest.raises(rs.ReplaySSMError):
        lay.step(*ins)
    lay.load_state(dev(case.S0))
    assert lay.check() == rs.RSSM_OK and lay.get_pointers() == ([0, 0], [0, 0])


def _run_spec(case, T, iters, sample, snapshot=False, accept=None, interleave=False):
    log(f"[gdn spec] Bt={case.Bt} H={case.H} G={case.G} Dv={case.Dv} Dk={case.Dk} L={case.L} T={T} "
        f"iters={iters} sample={list(sample)} snapshot={snapshot}")
    lay = case.layer(Tmax=T)
    sample = np.asarray(sample)
    S = case.S0[sample].astype(np.float64)
    ptr = oracle.GDNReplay(np.zeros((case.Bt, 1, 1, 1), np.float32), 1, case.L, T)
    z = lambda lead: [np.zeros(lead + (1, 1), np.float32)] * 3 + [np.zeros(lead + (1,), np.float32)] * 2
    cfg = rs.make_gdn_config(case.Bt, case.H, case.G, case.Dv, case.Dk)
    if snapshot:
        slots = torch.zeros(case.Bt, T + 1, case.H, case.Dv, case.Dk, device="cuda")
        slots[:, 0] = dev(case.S0)
        cur = torch.zeros(case.Bt, dtype=torch.int32, device="cuda")
        cur_ref = np.zeros(case.Bt, np.int64)
    rng = np.random.default_rng(case.seed)
    worst = 0.0
    for it in range(iters):
        drafts = case.draft_inputs(it, T)
        acc = accept(it) if accept else rng.integers(0, T + 1, case.Bt).astype(np.int32)
        o = lay.spec_verify(*(dev(a) for a in drafts))
        lay.rollback(dev(acc))
        S_before = S.copy()
        o_ref = oracle.gdn_spec_stepwise(S, T, *[a[sample] for a in drafts], acc[sample])
        e = rel(host(o)[sample], o_ref)
        worst = max(worst, e)
        assert e <= TOL, f"verify {it}: output error {e:.3e}"
        ptr.verify(T, *z((case.Bt, T)))
        ptr.rollback(acc)
        pos, ck = lay.get_pointers()
        opos, ock = ptr.pointers()
        assert pos == list(opos) and ck == list(ock), f"verify {it}: pointers"
        if snapshot:
            os_ = torch.empty_like(o)
            rs.gdn_snapshot_spec_verify(cfg, slots, cur, T, *(dev(a) for a in drafts), os_)
            rs.snapshot_commit(rs.make_config(case.Bt, case.H, 4, 16, 1), cur, dev(acc), T)
            ref_snap = oracle.gdn_spec_stepwise(S_before.copy(), T, *[a[sample] for a in drafts], acc[sample])
            assert rel(host(os_)[sample], ref_snap) <= TOL
            cur_ref = (cur_ref + acc) % (T + 1)
            assert np.array_equal(host(cur), cur_ref)
        if interleave and it % 3 == 2:
            ins = workload.gdn_step_inputs(case.seed + 1, it, case.Bt, case.H, case.G, case.Dv, case.Dk)
            o1 = lay.step(*(dev(a) for a in ins))
            assert rel(host(o1)[sample], oracle.gdn_step(S, *[a[sample] for a in ins])) <= TOL
            ptr.step(*z((case.Bt,)))
    assert rel(host(lay.materialize_state())[sample], S) <= TOL
    if snapshot:
        cur_h = host(cur)
        for i, b in enumerate(sample):
            assert rel(host(slots[b, int(cur_h[b])]), S[i]) <= TOL
    assert lay.check() == rs.RSSM_OK
    return worst


def test_gdn_spec_serving_batch512_T4():
    c = workload.GDN_SPEC
    case = GCase(c["Bt"], c["H"], c["G"], c["Dv"], c["Dk"], c["L"], workload.config_seed(7), Tmax=c["T"])
    worst = _run_spec(case, c["T"], 32, [1, 300, 511], snapshot=True)
    log(f"gdn spec serving: worst verify-output error {worst:.2e}")


@pytest.mark.parametrize("T,L", [(1, 4), (3, 7), (8, 16), (4, 4)])
def test_gdn_spec_small(T, L):
    case = GCase(3, 4, 2, 16, 32, L, 17 + T, Tmax=T)
    _run_spec(case, T, 30, range(3), snapshot=True)


def test_gdn_maximum_sizes():
    """Dv 256 (four row splits), Dk 256, L 64: standard steps across a flush, then T 8 verifies."""
    case = GCase(2, 2, 1, 256, 256, 64, 63)
    _run(case, 70, range(2), check_state_every=16)
    spec = GCase(2, 2, 1, 256, 256, 64, 64, Tmax=8)
    _run_spec(spec, 8, 12, range(2), snapshot=True)


def test_gdn_spec_accept_extremes_and_interleaved_steps():
    case = GCase(4, 4, 2, 32, 64, 8, 29, Tmax=3)
    pattern = [np.array([0, 3, 0, 3], np.int32), np.array([3, 3, 3, 3], np.int32), np.array([0, 0, 0, 0], np.int32)]
    _run_spec(case, 3, 24, range(4), accept=lambda it: pattern[it % 3], interleave=True)


@pytest.mark.parametrize("lockstep", [True, False])
def test_gdn_graph_replay_of_whole_windows(lockstep):
    """A captured graph of one whole window replays correctly, with the lockstep arguments (they
    repeat every window) or the device pointers (updated in place); each replay matches the
    oracle; eager steps continue afterwards."""
    Bt, H, G, Dv, Dk, L = 4, 4, 2, 64, 128, 4
    case = GCase(Bt, H, G, Dv, Dk, L, 91)
    lay = case.layer(lockstep=lockstep)
    bufs = [tuple(dev(a) for a in case.step_inputs(t)) for t in range(L)]
    outs = [torch.empty(Bt, H, Dv, device="cuda") for _ in range(L)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(L):
            lay.step(*bufs[i], outs[i])
    S = case.S0.astype(np.float64)
    for r in range(3):
        for i in range(L):
            for d, src in zip(bufs[i], case.step_inputs(r * L + i)):
                d.copy_(dev(src))
        g.replay()
        torch.cuda.synchronize()
        for i in range(L):
            o_ref = oracle.gdn_step(S, *case.step_inputs(r * L + i))
            assert rel(host(outs[i]), o_ref) <= TOL, f"replay {r} step {i}"
        assert lay.get_pointers() == ([(r + 1) * L] * Bt, [(r + 1) * L] * Bt)
        _ = torch.ones(1 << 20, device="cuda").sum().item()
    for t in range(3 * L, 4 * L + 2):
        ins = case.step_inputs(t)
        assert rel(host(lay.step(*(dev(a) for a in ins))), oracle.gdn_step(S, *ins)) <= TOL
    assert lay.check() == rs.RSSM_OK
