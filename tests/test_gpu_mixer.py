"""GPU parity of the mixer-edge step (replayssm_mixer_step) and its conventional baseline against
the oracle's mixer models (oracle_mixer.c + O1 / the replay form).

Bars: pointers bit-exact; the conv history read back (replayssm_materialize_conv_state) equal to
the oracle's raw history bit for bit (raw inputs are copied, never rounded); fp32 outputs,
checkpoint and materialized state within 1e-5 of the float64 truth (the edge adds a K-term fp32
conv, fp32 expf / log1pf in SiLU and softplus: a few fp32 roundings of O(1) values, below the
step's own 1e-5 budget). Every output within 1e-5 of the oracle's replay-form mixer with the same
read copy or master: after each flush the model continues from the GPU's own master, whose
encoding must then be the GPU's read copy bit for bit. Against the truth, a read copy's error is
bounded on the SSM output y before the gate (bf16 2e-2, fp8 6e-2, MXFP4 0.25 of max |y|); the gate
multiplies each value by silu(z), so the test holds max |o - o_true| to that gate times
max |y_true| * max |silu(z)|. fp16 and fp8 masters at the bars of their own tests (fp8 on the
gated scale).
"""
import numpy as np
import pytest
import torch

import hybrid_mamba_decode_amd as rs
import oracle
import workload
from gpu_harness import (MASTER_CODE, PREC_CODE, assert_copy_encodes, check_fp8_flush, dev, host, log, master_values,
                         rel, reseed)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5


class MixCase:
    def __init__(self, Bt, H, P, N, G, L, K, seed, Tmax=1):
        self.Bt, self.H, self.P, self.N, self.G, self.L, self.K, self.seed, self.Tmax = Bt, H, P, N, G, L, K, seed, Tmax
        self.CD = workload.mixer_conv_dim(H, P, G, N)
        self.A, self.D = workload.layer_params(seed, H)
        self.w, self.b, self.bias = workload.mixer_params(seed, H, P, G, N, K)
        self.S0 = workload.initial_state(seed, Bt, H, P, N)
        self.h0 = workload.mixer_history(seed, Bt, K, self.CD)

    def inputs(self, t):
        return workload.mixer_step_inputs(self.seed, t, self.Bt, self.H, self.P, self.G, self.N)

    def layer(self, read_prec="fp32", master_prec="fp32", lockstep=True, history=True, sr_seed=0):
        lay = rs.ReplaySSM(self.Bt, self.H, self.P, self.N, self.G, dev(self.A), dev(self.D), buffer_len=self.L,
                           max_draft=self.Tmax, read_prec=read_prec, master_prec=master_prec, sr_seed=sr_seed,
                           d_conv=self.K)
        lay.set_lockstep(lockstep)
        lay.set_mixer(dev(self.w), dev(self.b), dev(self.bias))
        lay.load_state(dev(self.S0))
        if history:
            lay.load_conv_state(dev(self.h0))
        return lay


def gated_err(o, o_true, y_true, z):
    """max |o - o_true| / (max |y_true| * max |silu(z)|): the error of the gated output on the
    scale of the SSM output before the gate (silu from the oracle's gate applied to ones)."""
    s = oracle.mixer_gate(np.ones(z.shape), z)
    den = float(np.max(np.abs(y_true))) * float(np.max(np.abs(s)))
    return float(np.max(np.abs(np.asarray(o, np.float64) - o_true))) / max(den, 1e-30)


def _run(case, steps, sample, read_prec="fp32", master_prec="fp32", lockstep=True, tol_nonflush=TOL_F32,
         check_every=4):
    log(f"[mixer] Bt={case.Bt} H={case.H} P={case.P} N={case.N} G={case.G} L={case.L} K={case.K} "
        f"read={read_prec} master={master_prec} lockstep={lockstep} steps={steps} sample={len(sample)} seqs")
    lay = case.layer(read_prec, master_prec, lockstep, sr_seed=3)
    sample = np.asarray(sample)
    truth = oracle.MixerStepwise(case.S0[sample], case.h0[sample], case.A, case.D, case.w, case.b, case.bias, case.G)
    model = oracle.MixerReplay(case.S0[sample], case.h0[sample], case.A, case.D, case.w, case.b, case.bias, case.G,
                               case.L, 1, PREC_CODE[read_prec], MASTER_CODE[master_prec], 3, seq_ids=sample)
    assert np.array_equal(host(lay.materialize_conv_state())[sample], case.h0[sample])
    worst_model = worst_gated = 0.0
    for t in range(steps):
        xbc, z, dt_raw = case.inputs(t)
        o = host(lay.mixer_step(dev(xbc), dev(z), dev(dt_raw)))[sample]
        sub = (xbc[sample], z[sample], dt_raw[sample])
        y_true, o_true = truth.step(*sub, with_y=True)
        o_model = model.step(*sub)
        flushes = (t + 1) // case.L
        flush_step = (t + 1) % case.L == 0
        fp8 = master_prec in ("fp8", "fp8_sr")
        lowp_flush = master_prec != "fp32" and flush_step
        if lowp_flush:
            # a low-precision flush rounds the fold, where the GPU's fp32 fold and the oracle's
            # float64 fold may straddle a rounding point: the output is checked against the stored
            # master
            x_e, B_e, C_e, _ = truth.last_edge
            y_m = oracle.step(master_values(lay, master_prec, sample), x_e, B_e, C_e,
                              np.zeros_like(truth.last_edge[3]), case.A, case.D)
            e_model = rel(o, oracle.mixer_gate(y_m, sub[1]))
        else:
            e_model = rel(o, o_model)
        worst_model = max(worst_model, e_model)
        assert e_model <= TOL_F32, f"step {t}: vs the same-copy replay model {e_model:.2e}"
        if master_prec == "fp32":
            if read_prec == "fp32" or flush_step:
                assert rel(o, o_true) <= TOL_F32, f"step {t}: vs truth {rel(o, o_true):.2e}"
            else:
                e_g = gated_err(o, o_true, y_true, sub[1])
                worst_gated = max(worst_gated, e_g)
                assert e_g <= tol_nonflush, f"step {t}: vs truth {e_g:.2e} > {tol_nonflush:.2e}"
        elif fp8:
            # reading R9's bound on the state (load 1/28, each flush 1/28 or 1/14 of the head's
            # largest value), on the SSM output's scale before the gate
            bound = (1 + flushes * (1 if master_prec == "fp8" else 2)) / 28
            e_g = gated_err(o, o_true, y_true, sub[1])
            worst_gated = max(worst_gated, e_g)
            assert e_g <= bound, f"step {t}: vs truth {e_g:.2e} > {bound:.2e}"
        else:
            assert rel(o, o_true) <= (flushes + 1) * 2.0 ** -10, f"step {t}: vs truth {rel(o, o_true):.2e}"
        pos, ck = lay.get_pointers()
        assert pos == [t + 1] * case.Bt and ck == [flushes * case.L] * case.Bt
        if t % check_every == 0 or flush_step:
            assert np.array_equal(host(lay.materialize_conv_state())[sample], truth.hist), f"step {t}: conv history"
            bound = TOL_F32 if master_prec == "fp32" else (
                (1 + flushes * (1 if master_prec == "fp8" else 2)) / 28 if fp8 else (flushes + 1) * 2.0 ** -10)
            assert rel(host(lay.materialize_state())[sample], truth.S) <= bound
        if flush_step and fp8:
            check_fp8_flush(lay, model.rep, sample, f"step {t}")
            reseed(model.rep, lay, master_prec, sample)
        elif flush_step:
            m = host(lay.master())[sample].astype(np.float32)
            if master_prec != "fp32":
                diff = m.astype(np.float64) != model.checkpoint()
                assert float(np.mean(diff)) <= 1e-3, f"step {t}: fp16 master vs model"
            if read_prec != "fp32":
                assert_copy_encodes(lay, read_prec, m, sample, f"step {t}")
            model.set_checkpoint(m)
    assert lay.check() == rs.RSSM_OK
    log(f"  worst vs the same-copy model {worst_model:.2e}; worst gated error vs truth {worst_gated:.2e}")
    return lay


def test_tiny_mixer_fp32():
    c = workload.MIXER_TINY
    case = MixCase(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], c["K"], 31)
    _run(case, c["steps"], range(c["Bt"]), check_every=1)


@pytest.mark.parametrize("lockstep", [True, False])
def test_serving_mixer_fp32(lockstep):
    """The serving layer with the edges: batch 256, 128 heads, P 64, N 128, 8 groups, L 16, K 4;
    48 steps (3 flushes), every sequence against the oracle."""
    c = workload.MIXER
    case = MixCase(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], c["K"], 32)
    _run(case, 48, range(c["Bt"]), lockstep=lockstep, check_every=16)


@pytest.mark.parametrize("read_prec,tol", [("bf16", 2e-2), ("fp8", 6e-2), ("mxfp4", 0.25)])
def test_mixer_with_read_copy(read_prec, tol):
    case = MixCase(3, 8, 32, 64, 2, 6, 4, 33)
    _run(case, 20, range(3), read_prec=read_prec, tol_nonflush=tol)


@pytest.mark.parametrize("master_prec", ["fp16", "fp16_sr", "fp8", "fp8_sr"])
def test_mixer_with_lowp_master(master_prec):
    case = MixCase(3, 8, 32, 64, 2, 6, 4, 34)
    _run(case, 20, range(3), master_prec=master_prec)


@pytest.mark.parametrize("shape", [
    (2, 6, 100, 32, 3, 5, 3),     # P over two row splits, ragged; K = 3
    (3, 4, 20, 16, 4, 1, 2),      # one head per group, L = 1 (every step flushes), K = 2
    (2, 4, 64, 256, 2, 32, 4),    # N = 256 (two B/C channels per thread), L bucket 32
])
def test_mixer_shapes(shape):
    Bt, H, P, N, G, L, K = shape
    case = MixCase(Bt, H, P, N, G, L, K, 35)
    _run(case, 2 * L + 3, range(Bt), check_every=3)


def test_fresh_history_is_zero():
    """load_state alone starts every sequence with a zero conv history."""
    case = MixCase(2, 4, 16, 32, 2, 4, 4, 36)
    lay = case.layer(history=False)
    assert not host(lay.materialize_conv_state()).any()
    truth = oracle.MixerStepwise(case.S0, np.zeros_like(case.h0), case.A, case.D, case.w, case.b, case.bias, case.G)
    for t in range(6):
        xbc, z, dt_raw = case.inputs(t)
        o = host(lay.mixer_step(dev(xbc), dev(z), dev(dt_raw)))
        assert rel(o, truth.step(xbc, z, dt_raw)) <= TOL_F32


def test_conventional_mixer_step():
    """The baseline with the same edges, against the stepwise mixer truth; its ring of K slots
    ([Bt, K, CD]) holds position q at slot q mod K (the initial history at positions -3..-1)."""
    c = workload.MIXER_TINY
    case = MixCase(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], c["K"], 37)
    K = case.K
    cfg = rs.make_config(case.Bt, case.H, case.P, case.N, case.G, d_conv=K)
    ring = np.zeros((case.Bt, K, case.CD), np.float32)
    for i in range(K - 1):
        ring[:, (i - (K - 1)) % K] = case.h0[:, i]
    ring_d, state = dev(ring), dev(case.S0)
    truth = oracle.MixerStepwise(case.S0, case.h0, case.A, case.D, case.w, case.b, case.bias, case.G)
    args = [dev(a) for a in (case.A, case.D, case.w, case.b, case.bias)]
    for t in range(12):
        xbc, z, dt_raw = case.inputs(t)
        o = torch.empty(case.Bt, case.H, case.P, device="cuda")
        rs.conventional_mixer_step(cfg, state, ring_d, t, dev(xbc), dev(z), dev(dt_raw), *args, o)
        assert rel(host(o), truth.step(xbc, z, dt_raw)) <= TOL_F32, t
    assert rel(host(state), truth.S) <= TOL_F32


def test_mixer_graph_replay_of_whole_windows():
    """Lockstep arguments (window slots and the conv ring slot pos mod R) repeat every
    lcm(L, R) steps: a captured window of L = 8 steps with R = 4 replays correctly, inputs copied
    into the captured buffers, eager work in between."""
    case = MixCase(4, 8, 64, 128, 2, 8, 4, 38)
    lay = case.layer()
    bufs = [tuple(dev(a) for a in case.inputs(i)) for i in range(case.L)]
    outs = [torch.empty(case.Bt, case.H, case.P, device="cuda") for _ in range(case.L)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(case.L):
            lay.mixer_step(*bufs[i], outs[i])
    truth = oracle.MixerStepwise(case.S0, case.h0, case.A, case.D, case.w, case.b, case.bias, case.G)
    for r in range(3):
        for i in range(case.L):
            for d, src in zip(bufs[i], case.inputs(r * case.L + i)):
                d.copy_(dev(src))
        g.replay()
        torch.cuda.synchronize()
        for i in range(case.L):
            o_ref = truth.step(*case.inputs(r * case.L + i))
            assert rel(host(outs[i]), o_ref) <= TOL_F32, f"replay {r} step {i}"
        assert np.array_equal(host(lay.materialize_conv_state()), truth.hist)
        _ = torch.ones(1 << 20, device="cuda").sum().item()
    assert lay.check() == rs.RSSM_OK


def test_mixer_graph_replay_flags_a_ring_slot_mismatch():
    """A captured window whose length is not a multiple of the conv ring's R slots (L = 4, K = 3,
    R = 3): the first replay starts where the capture did and is correct; the second replays the
    captured ring slots at positions where pos mod R differs, and the lockstep check raises the
    device flag instead of reading a stale history silently."""
    case = MixCase(2, 4, 32, 64, 2, 4, 3, 39)
    lay = case.layer()
    bufs = [tuple(dev(a) for a in case.inputs(i)) for i in range(case.L)]
    outs = [torch.empty(case.Bt, case.H, case.P, device="cuda") for _ in range(case.L)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(case.L):
            lay.mixer_step(*bufs[i], outs[i])
    truth = oracle.MixerStepwise(case.S0, case.h0, case.A, case.D, case.w, case.b, case.bias, case.G)
    g.replay()
    torch.cuda.synchronize()
    for i in range(case.L):
        assert rel(host(outs[i]), truth.step(*case.inputs(i))) <= TOL_F32, f"first replay step {i}"
    assert lay.check() == rs.RSSM_OK
    g.replay()
    torch.cuda.synchronize()
    assert lay.check() == rs.RSSM_E_STATE


def _spec_case(case, iters, sample, interleave=True):
    log(f"[mixer spec] Bt={case.Bt} H={case.H} P={case.P} N={case.N} G={case.G} L={case.L} K={case.K} "
        f"T={case.Tmax} iters={iters} sample={list(sample)}")
    T = case.Tmax
    lay = case.layer()
    sample = np.asarray(sample)
    truth = oracle.MixerStepwise(case.S0[sample], case.h0[sample], case.A, case.D, case.w, case.b, case.bias, case.G)
    model = oracle.MixerReplay(case.S0[sample], case.h0[sample], case.A, case.D, case.w, case.b, case.bias, case.G,
                               case.L, T, seq_ids=sample)
    ptr = oracle.MixerReplay(np.zeros((case.Bt, 1, 1, 1), np.float32), np.zeros((case.Bt, case.K - 1, 3), np.float32),
                             np.array([-1.0], np.float32), np.zeros(1, np.float32), np.zeros((3, case.K), np.float32),
                             np.zeros(3, np.float32), np.zeros(1, np.float32), 1, case.L, T)   # pointer machine
    for it in range(iters):
        if interleave and it % 3 == 2:
            xbc, z, dt_raw = case.inputs(1000 + it)
            o = host(lay.mixer_step(dev(xbc), dev(z), dev(dt_raw)))[sample]
            sub = (xbc[sample], z[sample], dt_raw[sample])
            assert rel(o, truth.step(*sub)) <= TOL_F32 and rel(o, model.step(*sub)) <= TOL_F32, f"step {it}"
            ptr.step(np.zeros((case.Bt, 3), np.float32), np.zeros((case.Bt, 1, 1), np.float32), np.zeros((case.Bt, 1), np.float32))
        else:
            xbc, z, dt_raw = workload.mixer_draft_inputs(case.seed, it, case.Bt, T, case.H, case.P, case.G, case.N)
            acc = workload.accepted_counts(case.seed, it, case.Bt, T)
            acc[it % case.Bt] = T if it % 2 else 0
            o = host(lay.mixer_spec_verify(dev(xbc), dev(z), dev(dt_raw)))[sample]
            lay.rollback(dev(acc))
            sub = (xbc[sample], z[sample], dt_raw[sample])
            o_true = truth.spec(T, *sub, acc[sample])
            o_model = model.verify(T, *sub)
            model.rollback(acc[sample])
            assert rel(o, o_true) <= TOL_F32, f"verify {it}: vs truth {rel(o, o_true):.2e}"
            assert rel(o, o_model) <= TOL_F32, f"verify {it}: vs replay model {rel(o, o_model):.2e}"
            ptr.verify(T, np.zeros((case.Bt, T, 3), np.float32), np.zeros((case.Bt, T, 1, 1), np.float32),
                       np.zeros((case.Bt, T, 1), np.float32))
            ptr.rollback(acc)
        pos, ck = lay.get_pointers()
        opos, ock = ptr.pointers()
        assert pos == list(opos) and ck == list(ock), f"iteration {it}: pointers"
        assert np.array_equal(host(lay.materialize_conv_state())[sample], truth.hist), f"iteration {it}: conv history"
        assert rel(host(lay.materialize_state())[sample], truth.S) <= TOL_F32
    assert lay.check() == rs.RSSM_OK


@pytest.mark.parametrize("T,L,K", [(1, 4, 4), (3, 7, 4), (4, 16, 3), (8, 16, 4)])
def test_mixer_spec_verify_rollback(T, L, K):
    """Verify T drafts through the edges (each draft's conv over the committed history and the
    drafts before it), roll back by accepted counts 0..T, standard mixer steps interleaved: all
    T outputs vs the per-draft truth and the replay model, the conv history after each rollback
    is the accepted prefix's (bit for bit), pointers bit-exact."""
    case = MixCase(3, 6, 32, 64, 2, L, K, 40 + T, Tmax=T)
    _spec_case(case, 18, range(3))


def test_mixer_maximum_sizes():
    """P 256 (four row splits), N 256, L 32 (the mixer's largest bucket), K 4, T 8."""
    case = MixCase(2, 2, 256, 256, 1, 32, 4, 65, Tmax=8)
    _spec_case(case, 10, range(2))


def test_mixer_spec_serving_batch512_T4():
    """Batch 512 of the serving layer with the edges, T = 4, L = 16: sequences 7 and 400."""
    c = workload.MIXER
    case = MixCase(512, c["H"], c["P"], c["N"], c["G"], c["L"], c["K"], 41, Tmax=4)
    _spec_case(case, 12, [7, 400])
