"""Pins for the replay-form oracle (O3) and its pointer/flush machine (O4).

The replay form is an algebraic rewrite of the recurrence, so it must reproduce the stepwise
oracle (itself pinned in test_oracle_recurrence.py) at every step; the checkpoint after a flush
must equal the stepwise state; with L = 1 it must collapse to the conventional step bit for bit;
rollback to an accepted prefix must equal recomputing from that prefix; the flush schedule must
follow the closed form of "a flush every L steps".
"""
import numpy as np
import pytest

import oracle
from oracle import brute
import workload


def _rel(a, ref):
    return float(np.max(np.abs(a - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _setup(seed, Bt, H, P, N, G):
    A, D = workload.layer_params(seed, H)
    S0 = workload.initial_state(seed, Bt, H, P, N)
    return S0, A, D


@pytest.mark.parametrize("L,Tmax", [(4, 1), (16, 1), (5, 2), (8, 3)])
def test_replay_equals_stepwise_every_step(L, Tmax):
    """Tiny layer (batch 2, 4 heads, P=N=16), 64 steps: replay outputs, the materialized state
    and, right after each flush, the checkpoint itself all equal the stepwise float64 state."""
    cfg = workload.TINY
    Bt, H, P, N, G = cfg["Bt"], cfg["H"], cfg["P"], cfg["N"], cfg["G"]
    seed = workload.config_seed(0)
    S0, A, D = _setup(seed, Bt, H, P, N, G)
    rep = oracle.Replay(S0, A, D, G, L, Tmax)
    S = S0.astype(np.float64)
    period = L - Tmax + 1
    flushes = 0
    for t in range(cfg["steps"]):
        x, B, C, dt = workload.step_inputs(seed, t, Bt, H, P, N, G)
        y_ref = oracle.step(S, x, B, C, dt, A, D)
        y = rep.step(x, B, C, dt)
        assert _rel(y, y_ref) <= 1e-12
        assert _rel(rep.materialize(), S) <= 1e-12
        pos, ck = rep.pointers()
        assert np.all(pos == t + 1)
        assert np.all(pos - ck == (t + 1) % period)   # closed form of the lockstep schedule
        if (t + 1) % period == 0:
            flushes += 1
            assert np.all(ck == pos)
            assert _rel(rep.checkpoint(), S) <= 1e-12
    assert flushes == cfg["steps"] // period


def test_serving_schedule_matches_golden():
    """Buffer length 16, 64 steps: flushes on the steps whose append fills the buffer,
    4 in total (the stored golden schedule)."""
    import json, os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "schedule.json")))
    case = gold["serving_L16_64_steps"]
    S0 = np.zeros((1, 1, 1, 1), np.float32)
    rep = oracle.Replay(S0, np.array([-1.0], np.float32), np.zeros(1, np.float32), 1, case["L"], 1)
    flush_steps = []
    for t in range(case["steps"]):
        one = np.ones((1, 1, 1), np.float32)
        rep.step(one, np.ones((1, 1, 1), np.float32), one, np.full((1, 1), 0.01, np.float32))
        pos, ck = rep.pointers()
        if ck[0] == pos[0]:
            flush_steps.append(t)
    assert flush_steps == case["flush_steps"]
    assert len(flush_steps) == case["flushes"]


def test_never_flushing_window_equals_dual_form():
    """With L larger than the run, no flush happens: the replay output is the pure unrolled
    window over all tokens, i.e. the brute-force dual form."""
    Bt, H, P, N, G, steps = 1, 2, 3, 4, 1, 7
    seed = 17
    S0, A, D = _setup(seed, Bt, H, P, N, G)
    rep = oracle.Replay(S0, A, D, G, 8, 1)
    toks = [workload.step_inputs(seed, t, Bt, H, P, N, G) for t in range(steps)]
    toks = [(x, B, C, (dt * 20).astype(np.float32)) for x, B, C, dt in toks]
    ref = brute.dual_form(S0.tolist(), [t[0].tolist() for t in toks], [t[1].tolist() for t in toks],
                          [t[2].tolist() for t in toks], [t[3].tolist() for t in toks],
                          A.tolist(), D.tolist())
    for t in range(steps):
        y = rep.step(*toks[t])
        assert _rel(y, np.array(ref[t])) <= 1e-12
    pos, ck = rep.pointers()
    assert pos[0] == steps and ck[0] == 0


def test_L1_is_conventional_bit_exact():
    """L = 1: every step appends one record and folds it at once. The fold then performs exactly
    the conventional update (decay exp(dt*A), weight dt), so outputs and state are bit-identical."""
    cfg = workload.TINY
    Bt, H, P, N, G = cfg["Bt"], cfg["H"], cfg["P"], cfg["N"], cfg["G"]
    seed = 23
    S0, A, D = _setup(seed, Bt, H, P, N, G)
    rep = oracle.Replay(S0, A, D, G, 1, 1)
    S = S0.astype(np.float64)
    for t in range(20):
        x, B, C, dt = workload.step_inputs(seed, t, Bt, H, P, N, G)
        y_ref = oracle.step(S, x, B, C, dt, A, D)
        y = rep.step(x, B, C, dt)
        assert np.array_equal(y, y_ref)
        assert np.array_equal(rep.checkpoint(), S)


@pytest.mark.parametrize("L,T", [(16, 4), (6, 3), (4, 4)])
def test_rollback_equals_recompute_from_prefix(L, T):
    """Verify T drafts, accept a random prefix per sequence, repeat. The draft outputs equal the
    per-draft definition (O5, all T of them); after rollback the committed state equals a fresh
    stepwise run fed only the accepted tokens; decoding continues correctly from there."""
    Bt, H, P, N, G = 4, 4, 8, 8, 2
    seed = 31
    S0, A, D = _setup(seed, Bt, H, P, N, G)
    rep = oracle.Replay(S0, A, D, G, L, T)
    S_spec = S0.astype(np.float64)          # O5 committed state
    # independent recompute: plain stepwise over only the accepted tokens, per sequence
    S_plain = S0.astype(np.float64)
    for it in range(12):
        x, B, C, dt = workload.draft_inputs(seed, it, Bt, T, H, P, N, G)
        acc = workload.accepted_counts(seed, it, Bt, T)
        if it == 0:
            acc[:] = [0, T, 1, 0]
        y = rep.verify(T, x, B, C, dt)
        y_ref = oracle.spec_stepwise(S_spec, T, x, B, C, dt, A, D, acc)
        assert _rel(y, y_ref) <= 1e-12
        rep.rollback(acc)
        for b in range(Bt):
            for i in range(acc[b]):
                sl = slice(b, b + 1)
                oracle.step(S_plain[sl], x[sl, i], B[sl, i], C[sl, i], dt[sl, i], A, D)
        assert _rel(rep.materialize(), S_plain) <= 1e-12
        assert _rel(S_spec, S_plain) <= 1e-12
        # interleave a committed standard step every third iteration
        if it % 3 == 2:
            xs, Bs, Cs, dts = workload.step_inputs(seed + 1, it, Bt, H, P, N, G)
            y1 = rep.step(xs, Bs, Cs, dts)
            y1_ref = oracle.step(S_plain, xs, Bs, Cs, dts, A, D)
            S_spec = S_plain.copy()
            assert _rel(y1, y1_ref) <= 1e-12


def test_spec_pointer_machine_properties():
    """Random accept streams over many verify/rollback rounds: pos moves by exactly the accepted
    count; ckpt_pos only changes by jumping to pos, and only when more than L - T records are
    pending; T drafts always fit after every commit (count + T <= L)."""
    Bt, H, P, N, G, L, T = 64, 1, 1, 1, 1, 16, 4
    seed = 41
    rep = oracle.Replay(np.zeros((Bt, H, P, N), np.float32), np.array([-1.0], np.float32),
                        np.zeros(1, np.float32), G, L, T)
    pos_prev, ck_prev = rep.pointers()
    flushes = 0
    for it in range(200):
        x, B, C, dt = workload.draft_inputs(seed, it, Bt, T, H, P, N, G)
        rep.verify(T, x, B, C, dt)
        p_mid, c_mid = rep.pointers()
        assert np.array_equal(p_mid, pos_prev) and np.array_equal(c_mid, ck_prev)
        acc = workload.accepted_counts(seed, it, Bt, T)
        rep.rollback(acc)
        pos, ck = rep.pointers()
        assert np.array_equal(pos, pos_prev + acc)
        pending = pos - ck_prev
        flushed = ck != ck_prev
        assert np.array_equal(flushed, pending > L - T)
        assert np.all(ck[flushed] == pos[flushed])
        assert np.all(pos - ck + T <= L)
        flushes += int(flushed.sum())
        pos_prev, ck_prev = pos, ck
    assert flushes > 0


def test_state_machine_rejects_misuse():
    S0 = np.zeros((1, 1, 2, 2), np.float32)
    A = np.array([-1.0], np.float32)
    D = np.zeros(1, np.float32)
    rep = oracle.Replay(S0, A, D, 1, 4, 2)
    x, B, C, dt = workload.draft_inputs(1, 0, 1, 2, 1, 2, 2, 1)
    with pytest.raises(RuntimeError):
        rep.rollback(np.zeros(1, np.int32))            # rollback without verify
    with pytest.raises(RuntimeError):
        rep.verify(3, *workload.draft_inputs(1, 0, 1, 3, 1, 2, 2, 1))   # T > Tmax
    rep.verify(2, x, B, C, dt)
    with pytest.raises(RuntimeError):
        rep.verify(2, x, B, C, dt)                     # verify twice
    xs, Bs, Cs, dts = workload.step_inputs(1, 0, 1, 1, 2, 2, 1)
    with pytest.raises(RuntimeError):
        rep.step(xs, Bs, Cs, dts)                      # step while a verify is pending
    with pytest.raises(RuntimeError):
        rep.rollback(np.array([3], np.int32))          # accepted > T
    rep.rollback(np.array([2], np.int32))
    with pytest.raises(ValueError):
        oracle.Replay(S0, A, D, 1, 2, 3)               # Tmax > L


def test_explicit_flush_and_mask():
    """An explicit flush folds only the selected sequences; unselected ones keep their records,
    and the materialized state is unchanged by flushing."""
    cfg = workload.TINY
    Bt, H, P, N, G = 3, cfg["H"], cfg["P"], cfg["N"], cfg["G"]
    seed = 51
    S0, A, D = _setup(seed, Bt, H, P, N, G)
    rep = oracle.Replay(S0, A, D, G, 8, 1)
    for t in range(5):
        rep.step(*workload.step_inputs(seed, t, Bt, H, P, N, G))
    before = rep.materialize()
    rep.flush(np.array([1, 0, 1], np.int32))
    pos, ck = rep.pointers()
    assert list(ck) == [5, 0, 5] and list(pos) == [5, 5, 5]
    assert _rel(rep.materialize(), before) <= 1e-13
    assert _rel(rep.checkpoint()[0], before[0]) <= 1e-13
    assert np.array_equal(rep.checkpoint()[1], S0[1].astype(np.float64))


@pytest.mark.parametrize("read_prec", [oracle.READ_BF16, oracle.READ_FP8])
def test_dual_precision_model(read_prec):
    """Read copy = decoded (encoded fp32 master). Flush-step outputs come from the fresh master,
    so they match the stepwise truth to float64 rounding; non-flush outputs carry only the read
    copy's rounding (bounded well inside the workload gates), and the copy is refreshed at every
    flush from the master, never otherwise."""
    cfg = workload.TINY
    Bt, H, P, N, G, L = cfg["Bt"], cfg["H"], cfg["P"], cfg["N"], cfg["G"], cfg["L"]
    seed = 61
    S0, A, D = _setup(seed, Bt, H, P, N, G)
    rep = oracle.Replay(S0, A, D, G, L, 1, read_prec)
    S = S0.astype(np.float64)
    copy0 = rep.read_copy()
    if read_prec == oracle.READ_BF16:
        exp0 = oracle.bf16_decode(oracle.bf16_encode(S0)).astype(np.float64)
    else:
        codes, scales = oracle.e4m3_encode_tiles(S0, P * N)
        table = oracle.e4m3_decode_table().astype(np.float64)
        exp0 = (table[codes].reshape(Bt * H, P * N) * scales[:, None]).reshape(S0.shape)
    assert np.array_equal(copy0, exp0)
    gate = 2e-2 if read_prec == oracle.READ_BF16 else 6e-2
    for t in range(32):
        x, B, C, dt = workload.step_inputs(seed, t, Bt, H, P, N, G)
        y_ref = oracle.step(S, x, B, C, dt, A, D)
        y = rep.step(x, B, C, dt)
        if (t + 1) % L == 0:
            assert _rel(y, y_ref) <= 1e-12
        else:
            assert 0 < _rel(y, y_ref) <= gate
            if t % L == 0 and t > 0:
                assert not np.array_equal(rep.read_copy(), copy0)
        if t == L - 2:
            assert np.array_equal(rep.read_copy(), copy0)


@pytest.mark.parametrize("read_prec", [oracle.READ_FP32, oracle.READ_BF16, oracle.READ_FP8, oracle.READ_MXFP4])
def test_set_checkpoint_restarts_the_model(read_prec):
    """Continuing the replay model from a given fp32 checkpoint after a flush is the same as a
    fresh model loaded with that state: outputs and decoded read copies equal bit for bit (the
    read copy is re-encoded from the given values, the records and pointers are kept)."""
    Bt, H, P, N, G, L = 2, 4, 16, 32, 2, 4
    seed = 404
    S0, A, D = _setup(seed, Bt, H, P, N, G)
    a = oracle.Replay(S0, A, D, G, L, 1, read_prec)
    for t in range(L):
        a.step(*workload.step_inputs(seed, t, Bt, H, P, N, G))
    assert np.all(a.pointers()[1] == L)
    # a checkpoint that is not the model's own: the fold rounded to fp32, one value nudged
    S1 = a.checkpoint().astype(np.float32)
    S1[1, 2, 3, 4] = np.float32(S1[1, 2, 3, 4] * 1.5 + 0.25)
    a.set_checkpoint(S1)
    assert np.array_equal(a.checkpoint(), S1.astype(np.float64))
    b = oracle.Replay(S1, A, D, G, L, 1, read_prec)
    assert np.array_equal(a.read_copy(), b.read_copy())
    for t in range(L, 2 * L - 1):
        ins = workload.step_inputs(seed, t, Bt, H, P, N, G)
        assert np.array_equal(a.step(*ins), b.step(*ins)), f"step {t}"


def test_set_checkpoint_changes_outputs_by_the_decayed_term():
    """Closed form: after a flush (empty window), replacing one checkpoint value S[b,h,p,n] by
    S + d changes the next replayed output only at (b, h, p), by exp(A_h dt_t) * d * C_t[b,g,n];
    every other output is unchanged."""
    Bt, H, P, N, G, L = 2, 4, 8, 16, 2, 3
    seed = 405
    S0, A, D = _setup(seed, Bt, H, P, N, G)
    ref = oracle.Replay(S0, A, D, G, L, 1)
    mod = oracle.Replay(S0, A, D, G, L, 1)
    for t in range(L):
        ins = workload.step_inputs(seed, t, Bt, H, P, N, G)
        ref.step(*ins)
        mod.step(*ins)
    S1 = ref.checkpoint().astype(np.float32)
    ref.set_checkpoint(S1)
    b, h, p, n, d = 1, 3, 5, 7, 0.75
    S2 = S1.copy()
    S2[b, h, p, n] += np.float32(d)
    d = float(S2[b, h, p, n]) - float(S1[b, h, p, n])
    mod.set_checkpoint(S2)
    x, B, C, dt = workload.step_inputs(seed, L, Bt, H, P, N, G)
    y0, y1 = ref.step(x, B, C, dt), mod.step(x, B, C, dt)
    g = h // (H // G)
    expect = np.exp(float(A[h]) * float(dt[b, h])) * d * float(C[b, g, n])
    diff = y1 - y0
    assert abs(diff[b, h, p] - expect) <= 1e-12 * max(1.0, abs(expect))
    diff[b, h, p] = 0.0
    assert np.all(diff == 0.0)


def test_set_checkpoint_of_selected_rows():
    """Setting the checkpoints of listed sequences leaves the others exactly as they were."""
    Bt, H, P, N, G, L = 3, 2, 8, 32, 1, 4
    seed = 406
    S0, A, D = _setup(seed, Bt, H, P, N, G)
    a = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP8)
    before_ck, before_copy = a.checkpoint(), a.read_copy()
    S1 = (S0[[2, 0]] * np.float32(0.5)).astype(np.float32)
    a.set_checkpoint(S1, [2, 0])
    ck, cp = a.checkpoint(), a.read_copy()
    assert np.array_equal(ck[[2, 0]], S1.astype(np.float64))
    assert np.array_equal(ck[1], before_ck[1]) and np.array_equal(cp[1], before_copy[1])
    assert np.array_equal(cp[[2, 0]], oracle.Replay(S1, A, D, G, L, 1, oracle.READ_FP8).read_copy())
    with pytest.raises(RuntimeError):
        a.set_checkpoint(S1, [2, 3])


def test_fp8_copy_scales_per_64_row_block():
    """Reading R6 for P > 64: the fp8 copy of a head with P = 100 rows takes one scale per block
    of 64 rows (rows 0..63 and 64..99), each amax / 448 of its block; codes against PyTorch's
    float8_e4m3fn of the block divided by its scale (a library rounding), both blocks. A state
    whose two blocks differ in magnitude by 2^10 keeps the small block at full fp8 resolution
    (a per-head scale would flush most of it to zero)."""
    import torch
    Bt, H, P, N, G, L = 2, 3, 100, 32, 1, 4
    seed = 71
    S0, A, D = _setup(seed, Bt, H, P, N, G)
    S0[:, :, 64:, :] *= 2.0 ** -10
    rep = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP8)
    got = rep.read_copy()
    for kb, (p0, p1) in enumerate([(0, 64), (64, 100)]):
        blk = S0[:, :, p0:p1, :]
        amax = np.abs(blk).max(axis=(2, 3), keepdims=True)
        scale = (amax / np.float32(448.0)).astype(np.float32)
        a = np.clip(blk * (np.float32(1.0) / scale), -448.0, 448.0).astype(np.float32)
        q = torch.from_numpy(a).to(torch.float8_e4m3fn).double().numpy()
        assert np.array_equal(got[:, :, p0:p1, :], q * scale.astype(np.float64)), f"block {kb}"
    small = got[:, :, 64:, :]
    assert np.mean(small == 0) < 0.01
    codes, scales = oracle.e4m3_encode_rows(S0)
    assert scales.shape == (Bt, H, 2)
    table = oracle.e4m3_decode_table().astype(np.float64)
    assert np.array_equal(table[codes] * np.repeat(scales, 64, axis=-1)[..., :P, None], got)
