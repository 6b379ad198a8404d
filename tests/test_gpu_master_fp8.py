"""GPU parity of the fp8 master recurrence (master_prec fp8 / fp8_sr: E4M3FN codes with one scale
per sequence and head, the fp8 read copy's format; reading R9 of oracle.c) against the oracle.

Bars:
* pointers bit-exact; after load the codes and scales equal the oracle's bit for bit;
* every non-flush output within 1e-5 of the oracle's fp8-master replay model, which after each
  flush continues from the GPU's own codes and scales;
* each flush, from that shared checkpoint and the same records: scales within 2^-20 relative of
  the model's, at most 1e-3 of the codes differ and each differing code is a neighbour of the
  model's on the E4M3 grid (the GPU's fp32 fold and the oracle's float64 fold straddled one
  rounding point; the stochastic rule uses the same Philox field on both sides); the flush step's
  output is read from the stored master, so it must equal (code * scale) . C_t + D x_t within
  1e-5;
* against the stepwise float64 truth, with k flushes done: checkpoint and materialized state
  within U8 + k * u, U8 = 1/28 (the load's nearest-even rounding: half of the top binade's
  spacing of 32, relative to the largest value 448 that the scale maps each head's amax to) and
  u = 1/28 (nearest even) or 1/14 (stochastic: up to one spacing); outputs within the same bound;
* an exactly representable case (every head's largest value held at 7, so the scale is 2^-6;
  A = 0, dyadic inputs): every code and scale bit-identical after every flush, for both roundings.
"""
import numpy as np
import pytest
import torch

import hybrid_mamba_decode_amd as rs
import oracle
import workload
from gpu_harness import (MASTER_CODE, PREC_CODE, Case, check_fp8_flush, dev, fp8_master, host, log, master_values,
                         reseed, rel)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
U8 = 1.0 / 28
STEP = {"fp8": 1.0 / 28, "fp8_sr": 1.0 / 14}


def _bound(master, flushes):
    return U8 + flushes * STEP[master]


def _run(case, steps, sample, master, seed=5, check_state_every=8):
    log(f"[fp8 master] Bt={case.Bt} H={case.H} P={case.P} N={case.N} G={case.G} L={case.L} master={master} "
        f"steps={steps} sample={len(sample)} seqs")
    lay = case.layer(master_prec=master, sr_seed=seed)
    sample = np.asarray(sample)
    S = case.S0[sample].astype(np.float64)
    rep = oracle.Replay(case.S0[sample], case.A, case.D, case.G, case.L, 1, oracle.READ_FP32, MASTER_CODE[master],
                        seed, seq_ids=sample)
    codes, scales = fp8_master(lay, sample)
    mc, ms = rep.fp8_master()
    assert np.array_equal(codes, mc) and np.array_equal(scales, ms), "load: codes or scales differ"
    growth, worst_flips = [], 0.0
    for t in range(steps):
        x, B, C, dt = case.step_inputs(t)
        y = host(lay.step(dev(x), dev(B), dev(C), dev(dt)))[sample]
        sub = (x[sample], B[sample], C[sample], dt[sample])
        y_true = oracle.step(S, *sub, case.A, case.D)
        y_rep = rep.step(*sub)
        flushes = (t + 1) // case.L
        flush_step = (t + 1) % case.L == 0
        bound = _bound(master, flushes)
        if not flush_step:
            e_model = rel(y, y_rep)
            assert e_model <= TOL_F32, f"step {t}: vs fp8 model {e_model:.2e}"
        e = rel(y, y_true)
        assert e <= bound, f"step {t}: vs truth {e:.2e} > {bound:.2e}"
        pos, ck = lay.get_pointers()
        assert pos == [t + 1] * case.Bt and ck == [flushes * case.L] * case.Bt
        if flush_step:
            worst_flips = max(worst_flips, check_fp8_flush(lay, rep, sample, f"step {t}"))
            m = master_values(lay, master, sample)
            y_m = oracle.step(m, *sub[:3], np.zeros_like(sub[3]), case.A, case.D)
            assert rel(y, y_m) <= TOL_F32, f"step {t}: flush output vs the stored master {rel(y, y_m):.2e}"
            e_ck = rel(m, S)
            assert e_ck <= bound, f"step {t}: checkpoint vs truth {e_ck:.2e} > {bound:.2e}"
            growth.append((flushes, e_ck, e))
            reseed(rep, lay, master, sample)
        if t % check_state_every == 0 or flush_step:
            assert rel(host(lay.materialize_state())[sample], S) <= bound
    assert lay.check() == rs.RSSM_OK
    log(f"  worst fraction of flipped fp8 codes {worst_flips:.1e}; flushes / checkpoint error / output "
        "error vs truth: " + "  ".join(f"{k}:{a:.1e}/{b:.1e}" for k, a, b in growth))
    return growth


@pytest.mark.parametrize("master", ["fp8", "fp8_sr"])
def test_tiny_fp8_master(master):
    c = workload.TINY
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(0))
    _run(case, 24, range(c["Bt"]), master, check_state_every=1)


@pytest.mark.parametrize("master", ["fp8", "fp8_sr"])
def test_serving_fp8_master(master):
    """Serving layer (batch 256, 128 heads, P 64, N 128, L 16), 64 steps (4 flushes), every
    sequence against the oracle."""
    c = workload.DUAL_PRECISION
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(2))
    _run(case, 64, range(c["Bt"]), master, check_state_every=32)


@pytest.mark.parametrize("shape", [(3, 6, 24, 64, 2, 6), (2, 4, 64, 256, 1, 5), (5, 2, 40, 32, 2, 1),
                                   (2, 3, 100, 64, 1, 5)])
def test_fp8_master_shapes(shape):
    """Ragged P (24, 40: rows past the tile's end), N = 256 and 32, L = 1 (every step flushes),
    P = 100 (two scale blocks per head, the per-row flush path)."""
    case = Case(*shape, 77)
    _run(case, 12, range(shape[0]), "fp8_sr", check_state_every=3)


def _exact_case(rng, Bt, H, P, N):
    """State: multiples of 2^-15 in [-4, 4] (E4M3 values times 2^-6 after load) and one anchor
    7.0 = 448 * 2^-6 per head in row 0, which no input changes (x = 0 there): the scale stays
    2^-6 exactly and every value code * 2^-6 is exact in fp32."""
    S0 = (rng.integers(-(1 << 17), (1 << 17) + 1, (Bt, H, P, N)) * 2.0 ** -15).astype(np.float32)
    S0[:, :, 0, :] = 0.0
    S0[:, :, 0, 0] = 7.0
    return S0


@pytest.mark.parametrize("master", ["fp8", "fp8_sr"])
def test_fp8_master_exact_codes(master):
    """A = 0 (decay 1, weights dt), dt in {1/2, 1}, x in -3..3 (0 on row 0), B multiples of 2^-8
    up to 3/256 and the anchored state: every fold is exact in fp32 and float64 and a = v * 64
    exactly, so the codes -- nearest even, or stochastic with Philox -- and the scales must be
    identical on both sides after every flush; outputs within 1e-6 (their sums of up to N
    products may round in fp32)."""
    Bt, H, P, N, G, L = 2, 8, 64, 128, 2, 4
    rng = np.random.default_rng(2026)
    S0 = _exact_case(rng, Bt, H, P, N)
    A = np.zeros(H, np.float32)
    D = rng.integers(-2, 3, H).astype(np.float32)
    lay = rs.ReplaySSM(Bt, H, P, N, G, dev(A), dev(D), buffer_len=L, master_prec=master, sr_seed=99)
    lay.load_state(dev(S0))
    rep = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, MASTER_CODE[master], 99)
    sample = np.arange(Bt)
    for t in range(4 * L):
        x = rng.integers(-3, 4, (Bt, H, P)).astype(np.float32)
        x[:, :, 0] = 0.0
        B = (rng.integers(-3, 4, (Bt, G, N)) * 2.0 ** -8).astype(np.float32)
        C = rng.integers(-2, 3, (Bt, G, N)).astype(np.float32)
        dt = rng.choice([0.5, 1.0], (Bt, H)).astype(np.float32)
        y = host(lay.step(dev(x), dev(B), dev(C), dev(dt))).astype(np.float64)
        y_rep = rep.step(x, B, C, dt)
        assert rel(y, y_rep) <= 1e-6, f"step {t}"
        if (t + 1) % L == 0:
            codes, scales = fp8_master(lay, sample)
            mc, ms = rep.fp8_master()
            assert np.all(scales == 2.0 ** -6) and np.all(ms == 2.0 ** -6)
            assert np.array_equal(codes, mc), f"flush at step {t}: {np.mean(codes != mc):.2e} of the codes differ"
    assert lay.check() == rs.RSSM_OK


def test_fp8_sr_differs_from_nearest_and_depends_on_seed():
    """Stochastic rounding is actually stochastic: two seeds give different codes after a flush,
    both differing from nearest even, each at most one E4M3 step from it."""
    case = Case(2, 4, 16, 32, 1, 4, 8)
    lays = {k: case.layer(master_prec=m, sr_seed=s) for k, (m, s) in
            {"rne": ("fp8", 0), "s1": ("fp8_sr", 1), "s2": ("fp8_sr", 2)}.items()}
    for t in range(4):
        ins = [dev(a) for a in case.step_inputs(t)]
        for lay in lays.values():
            lay.step(*ins)
    codes = {k: fp8_master(l, range(case.Bt))[0].astype(np.int64) for k, l in lays.items()}
    order = {k: np.where(c & 0x80, -(c & 0x7F), c & 0x7F) for k, c in codes.items()}
    assert not np.array_equal(codes["s1"], codes["s2"]) and not np.array_equal(codes["s1"], codes["rne"])
    for k in ("s1", "s2"):
        assert int(np.abs(order[k] - order["rne"]).max()) <= 1


@pytest.mark.parametrize("master", ["fp8", "fp8_sr"])
def test_fp8_master_spec_verify_rollback(master):
    """Verify T = 3 drafts and roll back (commit-time flushes fold into the fp8 master) against
    the oracle's fp8-master replay: every verify output within 1e-5 of the model (continued from
    the GPU's codes and scales after each commit-time flush), within the flush-count bound of the
    per-draft truth; each flush's codes as in standard decode; pointers bit-exact."""
    T, L = 3, 7
    case = Case(4, 6, 32, 64, 2, L, 404)
    lay = case.layer(Tmax=T, master_prec=master, sr_seed=13)
    sample = np.arange(case.Bt)
    log(f"[fp8 master spec] {master} T={T} L={L} batch={case.Bt}")
    S = case.S0[sample].astype(np.float64)
    dual = oracle.Replay(case.S0[sample], case.A, case.D, case.G, L, T, oracle.READ_FP32, MASTER_CODE[master], 13,
                         seq_ids=sample)
    flushes = np.zeros(case.Bt, np.int64)
    for it in range(24):
        x, B, C, dt = case.draft_inputs(it, T)
        acc = workload.accepted_counts(case.seed, it, case.Bt, T)
        y = host(lay.spec_verify(dev(x), dev(B), dev(C), dev(dt)))[sample]
        lay.rollback(dev(acc))
        sub = (x[sample], B[sample], C[sample], dt[sample])
        ck_before = dual.pointers()[1].copy()
        y_dual = dual.verify(T, *sub)
        dual.rollback(acc[sample])
        y_ref = oracle.spec_stepwise(S, T, *sub, case.A, case.D, acc[sample])
        e_model = rel(y, y_dual)
        assert e_model <= TOL_F32, f"verify {it}: vs fp8 model {e_model:.2e}"
        bound = _bound(master, int(flushes.max()))
        assert rel(y, y_ref) <= bound, f"verify {it}: vs truth {rel(y, y_ref):.2e}"
        pos, ck = lay.get_pointers()
        opos, ock = dual.pointers()
        assert [pos[b] for b in sample] == list(opos) and [ck[b] for b in sample] == list(ock)
        moved = np.nonzero(ock != ck_before)[0]
        if moved.size:
            flushes[moved] += 1
            check_fp8_flush(lay, dual, sample, f"verify {it}", rows=moved)
            reseed(dual, lay, master, sample, rows=moved)
        assert rel(host(lay.materialize_state())[sample], S) <= _bound(master, int(flushes.max()))
    assert flushes.min() >= 4
    assert lay.check() == rs.RSSM_OK


def test_fp8_sr_master_graph_replay_matches_eager():
    """Stochastic rounding draws its fields from the device's own flush position, so a captured
    window replayed several times (eager work in between) gives, bit for bit, the outputs, codes
    and scales of the same steps run eagerly on a second layer with the same seed."""
    Bt, H, P, N, G, L = 4, 8, 64, 128, 2, 4
    case = Case(Bt, H, P, N, G, L, 93)
    gl = case.layer(master_prec="fp8_sr", sr_seed=3)
    el = case.layer(master_prec="fp8_sr", sr_seed=3)
    bufs = [tuple(dev(a) for a in case.step_inputs(t)) for t in range(L)]
    ys = [torch.empty(Bt, H, P, device="cuda") for _ in range(L)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(L):
            gl.step(*bufs[i], ys[i])
    for r in range(3):
        for i in range(L):
            for d, src in zip(bufs[i], case.step_inputs(r * L + i)):
                d.copy_(dev(src))
        g.replay()
        torch.cuda.synchronize()
        for i in range(L):
            y = el.step(*(dev(a) for a in case.step_inputs(r * L + i)))
            assert torch.equal(ys[i], y), f"replay {r} step {i}"
        assert torch.equal(gl.master(), el.master()), f"replay {r}: master codes differ"
        assert torch.equal(gl.scales(), el.scales()), f"replay {r}: master scales differ"
        assert gl.get_pointers() == ([(r + 1) * L] * Bt, [(r + 1) * L] * Bt)
        _ = torch.ones(1 << 20, device="cuda").sum().item()
    assert gl.check() == rs.RSSM_OK and el.check() == rs.RSSM_OK


def test_fp8_sr_master_avoids_stagnation():
    """workload.stagnation_case with the body at 0.4375 and row p = 0 at 0.875 = 448 * 2^-9 (x = 0
    there), so the scale stays 2^-9 and the body sits on the E4M3 value 224 (spacing 16): each
    flush adds 2^-14, a thirty-second of a scaled unit, exactly. Nearest even keeps the body
    where it is; the stochastic codes equal the oracle's bit for bit after every flush, and the
    body's mean moves up."""
    (Bt, H, P, N, G, L), S0, A, D, (x, B, C, dt) = workload.stagnation_case()
    S0 = np.full_like(S0, 0.4375)
    S0[:, :, 0, :] = 0.875
    x = x.copy()
    x[:, :, 0] = 0.0
    tok = (x, B, C, dt)
    lays = {m: rs.ReplaySSM(Bt, H, P, N, G, dev(A), dev(D), buffer_len=L, master_prec=m, sr_seed=9)
            for m in ("fp8", "fp8_sr")}
    for lay in lays.values():
        lay.load_state(dev(S0))
    sr = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP8_SR, seed=9)
    toks = tuple(dev(a) for a in tok)
    sample = np.arange(Bt)
    for t in range(32 * L):
        for lay in lays.values():
            lay.step(*toks)
        sr.step(*tok)
        if (t + 1) % L == 0:
            codes, scales = fp8_master(lays["fp8_sr"], sample)
            mc, ms = sr.fp8_master()
            assert np.array_equal(codes, mc) and np.array_equal(scales, ms), f"flush at {t}"
    rne = master_values(lays["fp8"], "fp8", sample)
    assert np.all(rne[:, :, 1:, :] == 0.4375) and np.all(rne[:, :, 0, :] == 0.875)
    m = master_values(lays["fp8_sr"], "fp8_sr", sample)[:, :, 1:, :]
    assert float(m.mean()) > 0.4375 + 16 * 2.0 ** -14


@pytest.mark.parametrize("master", ["fp8", "fp8_sr"])
def test_fp8_master_staggered_flushes(master):
    """Speculative rounds with random accepted counts leave the sequences at different window
    positions; the standard steps that follow then flush some sequences and not others in one
    launch (the per-sequence flush path). Per step and sequence: outputs of sequences that did
    not flush within 1e-5 of the model; those that flushed have their codes checked as in
    standard decode and their output read from the stored master; pointers bit-exact."""
    T, L = 3, 7
    case = Case(5, 6, 48, 64, 2, L, 505)
    lay = case.layer(Tmax=T, master_prec=master, sr_seed=21)
    sample = np.arange(case.Bt)
    model = oracle.Replay(case.S0, case.A, case.D, case.G, L, T, oracle.READ_FP32, MASTER_CODE[master], 21,
                          seq_ids=sample)
    for it in range(5):
        x, B, C, dt = case.draft_inputs(it, T)
        acc = workload.accepted_counts(case.seed, it, case.Bt, T)
        lay.spec_verify(dev(x), dev(B), dev(C), dev(dt))
        lay.rollback(dev(acc))
        ck_before = model.pointers()[1].copy()
        model.verify(T, x, B, C, dt)
        model.rollback(acc)
        moved = np.nonzero(model.pointers()[1] != ck_before)[0]
        if moved.size:
            check_fp8_flush(lay, model, sample, f"round {it}", rows=moved)
            reseed(model, lay, master, sample, rows=moved)
    pos0 = model.pointers()[0]
    assert len(set((pos0 - model.pointers()[1]).tolist())) > 1, "rounds left every sequence at one position"
    mixed = 0
    for t in range(2 * L):
        x, B, C, dt = case.step_inputs(100 + t)
        y = host(lay.step(dev(x), dev(B), dev(C), dev(dt)))
        ck_before = model.pointers()[1].copy()
        y_model = model.step(x, B, C, dt)
        pos, ck = lay.get_pointers()
        opos, ock = model.pointers()
        assert pos == list(opos) and ck == list(ock), f"step {t}: pointers"
        fl = ock != ck_before
        mixed += bool(fl.any() and not fl.all())
        if (~fl).any():
            assert rel(y[~fl], y_model[~fl]) <= TOL_F32, f"step {t}: non-flushing sequences vs model"
        if fl.any():
            rows = np.nonzero(fl)[0]
            check_fp8_flush(lay, model, sample, f"step {t}", rows=rows)
            m = master_values(lay, master, rows)
            y_m = oracle.step(m, x[rows], B[rows], C[rows], np.zeros_like(dt[rows]), case.A, case.D)
            assert rel(y[rows], y_m) <= TOL_F32, f"step {t}: flushed sequences vs the stored master"
            reseed(model, lay, master, sample, rows=rows)
    assert mixed >= 2, "no step flushed some sequences and not others"
    assert lay.check() == rs.RSSM_OK
