"""GPU parity of the fp16 master recurrence (master_prec fp16 / fp16_sr) against the oracle.

Bars:
* pointers bit-exact;
* every non-flush output within 1e-5 of the oracle's fp16-master replay model: both sides start
  from the same nearest-even fp16 checkpoint, and after each flush the model continues from the
  GPU's own fp16 master (with a read copy, that master's encoding must be the GPU's copy, bit for
  bit);
* each flush, from that shared checkpoint and the same records: the GPU's fp16 codes equal the
  model's except for at most 1e-3 of the values, and every code that differs is a neighbour of the
  model's (the GPU's fp32 fold and the oracle's float64 fold straddled one rounding point; the
  stochastic rule uses the same Philox word on both sides); the flush step's output is read from
  the stored master, so it must equal S_master . C_t + D x_t within 1e-5;
* against the stepwise float64 truth, with k flushes done: outputs, checkpoint and materialized
  state within (k + 1) * 2^-10 -- one rounding per flush plus the load, each at most half a
  spacing (nearest even) or one spacing (stochastic) of fp16, 2^-11 / 2^-10 relative;
* an exactly representable case (A = 0, dyadic inputs) with every fp16 code bit-identical after
  every flush, for nearest-even and for stochastic rounding (Philox on both sides).
"""
import numpy as np
import pytest
import torch

import hybrid_mamba_decode_amd as rs
import oracle
import workload
from gpu_harness import MASTER_CODE, PREC_CODE, Case, assert_copy_encodes, dev, host, log, rel

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
U16 = 2.0 ** -10
READ_TOL = {"fp32": 0.0, "bf16": 2e-2, "mxfp4": 0.25}


def _f16_order(v):
    """Integer position of fp16 values on the number line (neighbouring codes differ by 1)."""
    bits = np.asarray(v, np.float16).view(np.uint16).astype(np.int64)
    mag = bits & 0x7FFF
    return np.where(bits & 0x8000, -mag, mag)


def _check_flush_codes(m, ck_model, what):
    """GPU fp16 master m vs the model's fold of the same checkpoint and records: at most 1e-3 of
    the values differ, and each differing code is a neighbour of the model's."""
    diff = m.astype(np.float64) != ck_model
    flips = float(np.mean(diff))
    assert flips <= 1e-3, f"{what}: {flips:.2e} of the fp16 master differs from the model's"
    if diff.any():
        gap = np.abs(_f16_order(m[diff]) - _f16_order(ck_model[diff]))
        assert int(gap.max()) == 1, f"{what}: fp16 codes {int(gap.max())} apart"
    return flips


def _run(case, steps, sample, master, read="fp32", seed=5, check_state_every=8):
    log(f"[master] Bt={case.Bt} H={case.H} P={case.P} N={case.N} G={case.G} L={case.L} master={master} "
        f"read={read} steps={steps} sample={len(sample)} seqs")
    lay = case.layer(read, master_prec=master, sr_seed=seed)
    sample = np.asarray(sample)
    S = case.S0[sample].astype(np.float64)
    rep = oracle.Replay(case.S0[sample], case.A, case.D, case.G, case.L, 1, PREC_CODE[read], MASTER_CODE[master], seed,
                        seq_ids=sample)
    assert np.array_equal(host(lay.master())[sample].astype(np.float64), rep.checkpoint())
    growth, worst_flips = [], 0.0
    for t in range(steps):
        x, B, C, dt = case.step_inputs(t)
        y = host(lay.step(dev(x), dev(B), dev(C), dev(dt)))[sample]
        sub = (x[sample], B[sample], C[sample], dt[sample])
        y_true = oracle.step(S, *sub, case.A, case.D)
        y_rep = rep.step(*sub)
        flushes = (t + 1) // case.L
        flush_step = (t + 1) % case.L == 0
        bound = (flushes + 1) * U16
        if not flush_step:
            e_model = rel(y, y_rep)
            assert e_model <= TOL_F32, f"step {t}: vs fp16 model {e_model:.2e}"
        e = rel(y, y_true)
        read_tol = 0.0 if flush_step else READ_TOL[read]
        assert e <= bound + read_tol, f"step {t}: vs truth {e:.2e} > {bound + read_tol:.2e}"
        pos, ck = lay.get_pointers()
        assert pos == [t + 1] * case.Bt and ck == [flushes * case.L] * case.Bt
        if flush_step:
            m = host(lay.master())[sample].astype(np.float32)
            worst_flips = max(worst_flips, _check_flush_codes(m, rep.checkpoint(), f"step {t}"))
            # the flush step's output comes from the stored master: O1 with dt = 0 reads it as is
            y_m = oracle.step(m.astype(np.float64), *sub[:3], np.zeros_like(sub[3]), case.A, case.D)
            assert rel(y, y_m) <= TOL_F32, f"step {t}: flush output vs the stored master {rel(y, y_m):.2e}"
            e_ck = rel(m, S)
            assert e_ck <= bound, f"step {t}: checkpoint vs truth {e_ck:.2e} > {bound:.2e}"
            growth.append((flushes, e_ck, e))
            if read != "fp32":
                assert_copy_encodes(lay, read, m, sample, f"step {t}")
            rep.set_checkpoint(m)
        if t % check_state_every == 0 or flush_step:
            assert rel(host(lay.materialize_state())[sample], S) <= bound
    assert lay.check() == rs.RSSM_OK
    log(f"  worst fraction of flipped fp16 codes {worst_flips:.1e}; flushes / checkpoint error / output "
        "error vs truth: " + "  ".join(f"{k}:{a:.1e}/{b:.1e}" for k, a, b in growth))
    return growth


@pytest.mark.parametrize("master", ["fp16", "fp16_sr"])
def test_tiny_fp16_master(master):
    c = workload.TINY
    case = Case(c["Bt"], c["H"], c["P"], 32, c["G"], c["L"], workload.config_seed(0))
    _run(case, c["steps"], range(c["Bt"]), master, check_state_every=1)


@pytest.mark.parametrize("master", ["fp16", "fp16_sr"])
def test_serving_fp16_master(master):
    """Serving layer (batch 256, 128 heads, P 64, N 128, L 16), 128 steps (8 flushes), every
    sequence against the oracle."""
    c = workload.DUAL_PRECISION
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(2))
    _run(case, 128, range(c["Bt"]), master, check_state_every=64)


@pytest.mark.parametrize("master,read", [("fp16_sr", "bf16"), ("fp16", "mxfp4")])
def test_fp16_master_with_read_copy(master, read):
    case = Case(3, 6, 24, 64, 2, 6, 321)
    _run(case, 20, range(3), master, read, check_state_every=4)


@pytest.mark.parametrize("master", ["fp16", "fp16_sr"])
def test_fp16_master_exact_codes(master):
    """A = 0 (decay 1, weights dt), dt in {1/2, 1}, small-integer x, B, C, and a state of
    multiples of 2^-12 (mostly not fp16-representable): every fold is exact in fp32 and float64,
    so the rounded fp16 codes -- nearest even, or stochastic with Philox -- must be identical on
    both sides after every flush, and the outputs bit-identical."""
    Bt, H, P, N, G, L = 2, 8, 64, 128, 2, 4
    rng = np.random.default_rng(2025)
    S0 = (rng.integers(-8192, 8193, (Bt, H, P, N)) / 4096.0).astype(np.float32)
    A = np.zeros(H, np.float32)
    D = rng.integers(-2, 3, H).astype(np.float32)
    lay = rs.ReplaySSM(Bt, H, P, N, G, dev(A), dev(D), buffer_len=L, master_prec=master, sr_seed=99)
    lay.load_state(dev(S0))
    rep = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, MASTER_CODE[master], 99)
    for t in range(4 * L):
        x = rng.integers(-3, 4, (Bt, H, P)).astype(np.float32)
        B = rng.integers(-3, 4, (Bt, G, N)).astype(np.float32)
        C = rng.integers(-2, 3, (Bt, G, N)).astype(np.float32)
        dt = rng.choice([0.5, 1.0], (Bt, H)).astype(np.float32)
        y = host(lay.step(dev(x), dev(B), dev(C), dev(dt))).astype(np.float64)
        y_rep = rep.step(x, B, C, dt)
        assert np.array_equal(y, y_rep), f"step {t}"
        if (t + 1) % L == 0:
            assert np.array_equal(host(lay.master()).astype(np.float64), rep.checkpoint()), f"flush at step {t}"
    assert lay.check() == rs.RSSM_OK


def test_fp16_sr_differs_from_nearest_and_depends_on_seed():
    """Stochastic rounding is actually stochastic: two seeds give different checkpoints after a
    flush, both differing from nearest-even rounding, each within one fp16 spacing of it."""
    case = Case(2, 4, 16, 32, 1, 4, 8)
    lays = {k: case.layer(master_prec=m, sr_seed=s) for k, (m, s) in
            {"rne": ("fp16", 0), "s1": ("fp16_sr", 1), "s2": ("fp16_sr", 2)}.items()}
    for t in range(4):
        ins = [dev(a) for a in case.step_inputs(t)]
        for lay in lays.values():
            lay.step(*ins)
    m = {k: host(l.master()).astype(np.float64) for k, l in lays.items()}
    assert not np.array_equal(m["s1"], m["s2"]) and not np.array_equal(m["s1"], m["rne"])
    mag = np.abs(m["rne"]).astype(np.float16)
    spacing = np.nextafter(mag, np.float16(np.inf)).astype(np.float64) - mag.astype(np.float64)
    for k in ("s1", "s2"):
        assert np.all(np.abs(m[k] - m["rne"]) <= spacing * 1.0000001)


@pytest.mark.parametrize("master", ["fp16", "fp16_sr"])
def test_fp16_master_spec_verify_rollback(master):
    """Verify T = 3 drafts and roll back (commit-time flushes fold into the fp16 master) against
    the oracle's fp16-master replay: every verify output within 1e-5 of the model (which continues
    from the GPU's master after each commit-time flush), within (k + 1) 2^-10 of the per-draft
    truth; each flush's codes as in standard decode; pointers bit-exact."""
    T, L = 3, 7
    case = Case(4, 6, 32, 64, 2, L, 404)
    lay = case.layer(Tmax=T, master_prec=master, sr_seed=13)
    sample = np.arange(case.Bt)
    log(f"[master spec] {master} T={T} L={L} batch={case.Bt}")
    S = case.S0[sample].astype(np.float64)
    dual = oracle.Replay(case.S0[sample], case.A, case.D, case.G, L, T, oracle.READ_FP32, MASTER_CODE[master], 13,
                         seq_ids=sample)
    flushes = 0
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
        assert e_model <= TOL_F32, f"verify {it}: vs fp16 model {e_model:.2e}"
        assert rel(y, y_ref) <= (flushes + 1) * U16, f"verify {it}: vs truth {rel(y, y_ref):.2e}"
        pos, ck = lay.get_pointers()
        opos, ock = dual.pointers()
        assert [pos[b] for b in sample] == list(opos) and [ck[b] for b in sample] == list(ock)
        moved = np.nonzero(ock != ck_before)[0]
        if moved.size:
            flushes += 1
            m = host(lay.master())[sample[moved]].astype(np.float32)
            _check_flush_codes(m, dual.checkpoint()[moved], f"verify {it}")
            dual.set_checkpoint(m, moved)
        assert rel(host(lay.materialize_state())[sample], S) <= (flushes + 1) * U16
    assert flushes >= 4
    assert lay.check() == rs.RSSM_OK


def test_fp16_sr_master_graph_replay_matches_eager():
    """Stochastic rounding draws its words from the device's own flush position, so a captured
    window replayed several times (eager work in between) gives, bit for bit, the outputs and
    fp16 master codes of the same steps run eagerly on a second layer with the same seed."""
    Bt, H, P, N, G, L = 4, 8, 64, 128, 2, 4
    case = Case(Bt, H, P, N, G, L, 92)
    gl = case.layer(master_prec="fp16_sr", sr_seed=3)
    el = case.layer(master_prec="fp16_sr", sr_seed=3)
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
        assert gl.get_pointers() == ([(r + 1) * L] * Bt, [(r + 1) * L] * Bt)
        _ = torch.ones(1 << 20, device="cuda").sum().item()
    assert gl.check() == rs.RSSM_OK and el.check() == rs.RSSM_OK


def test_fp16_sr_master_avoids_stagnation():
    """Increments of a sixteenth of a spacing per flush (decay 1, exact arithmetic; the oracle
    test of the same case pins the statistics): the nearest-even master stays exactly 1.0 and the
    stochastic one equals the oracle's codes bit for bit after every flush."""
    (Bt, H, P, N, G, L), S0, A, D, tok = workload.stagnation_case()
    lays = {m: rs.ReplaySSM(Bt, H, P, N, G, dev(A), dev(D), buffer_len=L, master_prec=m, sr_seed=9)
            for m in ("fp16", "fp16_sr")}
    for lay in lays.values():
        lay.load_state(dev(S0))
    sr = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP16_SR, seed=9)
    toks = tuple(dev(a) for a in tok)
    for t in range(32 * L):
        for lay in lays.values():
            lay.step(*toks)
        sr.step(*tok)
        if (t + 1) % L == 0:
            assert np.array_equal(host(lays["fp16_sr"].master()).astype(np.float64), sr.checkpoint()), f"flush at {t}"
    assert bool((lays["fp16"].master() == 1.0).all())
    assert float(host(lays["fp16_sr"].master()).astype(np.float64).mean()) > 1.0 + 16 * 2.0 ** -14


@pytest.mark.parametrize("master", ["fp16", "fp16_sr"])
def test_fp16_master_subnormal_codes(master):
    """The whole state inside fp16's subnormal range (|v| < 2^-14, spacing 2^-24), where the
    stochastic rule takes its general path: A = 0, dt in {1/2, 1}, small-integer x, C, B and S0
    as multiples of 2^-30, so every fold is exact in fp32 and float64 and the fp16 codes after
    every flush must equal the oracle's bit for bit."""
    Bt, H, P, N, G, L = 2, 4, 64, 64, 2, 4
    rng = np.random.default_rng(4242)
    S0 = (rng.integers(-(1 << 12), (1 << 12) + 1, (Bt, H, P, N)) * 2.0 ** -30).astype(np.float32)
    A = np.zeros(H, np.float32)
    D = np.zeros(H, np.float32)
    lay = rs.ReplaySSM(Bt, H, P, N, G, dev(A), dev(D), buffer_len=L, master_prec=master, sr_seed=123)
    lay.load_state(dev(S0))
    rep = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, MASTER_CODE[master], 123)
    assert np.array_equal(host(lay.master()).astype(np.float64), rep.checkpoint())
    for t in range(4 * L):
        x = rng.integers(-3, 4, (Bt, H, P)).astype(np.float32)
        B = (rng.integers(-64, 65, (Bt, G, N)) * 2.0 ** -30).astype(np.float32)
        C = rng.integers(-2, 3, (Bt, G, N)).astype(np.float32)
        dt = rng.choice([0.5, 1.0], (Bt, H)).astype(np.float32)
        lay.step(dev(x), dev(B), dev(C), dev(dt))
        rep.step(x, B, C, dt)
        if (t + 1) % L == 0:
            m = host(lay.master()).astype(np.float64)
            assert np.max(np.abs(m)) < 2.0 ** -14
            assert np.array_equal(m, rep.checkpoint()), f"flush at step {t}"
    assert lay.check() == rs.RSSM_OK
