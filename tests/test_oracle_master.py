"""Pins for the oracle's low-precision master (reading R8 of oracle.c): the Philox4x32-10 stream,
fp16 rounding to nearest even, stochastic rounding, and the dual model that keeps the checkpoint
in fp16.

Independent references: the generator's published known-answer vectors
(tests/golden/philox_kat.json), numpy's float16 conversion (a library routine), fp16 neighbours
and thresholds computed with numpy.nextafter and exact fractions, and an fp32-master replay whose
flushed checkpoint numpy rounds to fp16.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox_kat.json")


def test_philox_known_answers():
    for vec in json.load(open(GOLDEN))["vectors"]:
        ctr = [int(x, 16) for x in vec["ctr"]]
        key = [int(x, 16) for x in vec["key"]]
        want = [int(x, 16) for x in vec["out"]]
        assert list(oracle.philox4x32_10(ctr, key)) == want


def test_f16_nearest_even_vs_numpy():
    """Every fp32 pattern with exponent field in [80, 143] (|v| from 2^-47 to 65536, subnormals of
    fp16 included) on a mantissa stride of 97, plus fp16 midpoints and their neighbours."""
    mant = np.arange(0, 1 << 23, 97, dtype=np.uint32)
    vals = []
    for e in range(80, 143):
        bits = (np.uint32(e) << np.uint32(23)) | mant
        vals.append(bits.view(np.float32))
    h = np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[:-1] + h[1:]) / 2).astype(np.float32)
    vals += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))]
    v = np.concatenate(vals).astype(np.float32)
    v = v[np.abs(v) <= 65504]
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.f16_encode(v), v.astype(np.float16).view(np.uint16))


def test_f16_decode_vs_numpy():
    codes = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (codes & 0x7C00) != 0x7C00
    got = oracle.f16_decode(codes[finite])
    assert np.array_equal(got, codes[finite].view(np.float16).astype(np.float32))


def _threshold(v):
    """Round-up threshold of stochastic rounding: (|v| - q) / ulp * 2^16 as an exact Fraction,
    with q = the fp16 magnitude toward zero (numpy) and ulp the gap to the next one."""
    a = abs(float(np.float32(v)))
    q16 = np.float16(a)
    if float(q16) > a:
        q16 = np.nextafter(q16, np.float16(0))
    nxt = np.nextafter(q16, np.float16(np.inf))
    q, up = Fraction(float(q16)), Fraction(float(nxt))
    return (Fraction(a) - q) / (up - q) * 2 ** 16, float(q16), float(nxt)


def test_stochastic_rounding_threshold_and_unbiasedness():
    """The magnitude rounds up iff r16 < T (T exact). In fp16's normal range an fp32 value has
    13 bits below the fp16 spacing, so T is a multiple of 8 and the mean over all 2^16 values of
    r16 is exactly v -- the same distribution a wider random integer would give. T is an integer
    except deep in the subnormal range (|v| < 2^-17, where fp32 keeps finer bits than 2^-16 of
    the spacing 2^-24); there the mean is within 2^-16 of a spacing of v. Representable values
    never change."""
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(400) * np.exp2(rng.integers(-30, 14, 400))).astype(np.float32)
    v = np.concatenate([v, np.float16(rng.standard_normal(50)).astype(np.float32)])
    n_int = n_normal = 0
    for x in v:
        T, q, nxt = _threshold(x)
        assert 0 <= T < 2 ** 16
        c = -(-T.numerator // T.denominator)              # ceil(T): the number of r16 that round up
        sign = -1.0 if x < 0 else 1.0
        rs = np.array(sorted({0, max(c - 1, 0), min(c, 2 ** 16 - 1), min(c + 1, 2 ** 16 - 1), 2 ** 16 - 1}), np.uint32)
        got = oracle.f16_decode(oracle.f16_encode(np.full(len(rs), x, np.float32), rs)).astype(np.float64)
        want = [sign * (nxt if Fraction(int(r)) < T else q) for r in rs]
        assert np.array_equal(got, np.array(want)), (x, T)
        mean = Fraction(c) * Fraction(nxt) + Fraction(2 ** 16 - c) * Fraction(q)   # times 2^16
        err = abs(mean - Fraction(abs(float(x))) * 2 ** 16)
        assert err <= Fraction(nxt) - Fraction(q)
        if abs(float(x)) >= 2.0 ** -14:
            assert T.denominator == 1 and T.numerator % 8 == 0, (x, T)
            n_normal += 1
        if abs(float(x)) >= 2.0 ** -17:
            assert T.denominator == 1, (x, T)
        if T.denominator == 1:
            assert err == 0
            n_int += 1
    assert n_int > 300 and n_normal > 200


def test_fp16_master_dual_model():
    """Checkpoint after load = numpy's fp16 of S0; after the first flush = numpy's fp16 (nearest
    even) of an fp32-master replay's checkpoint started from that fp16 state; with stochastic
    rounding, the code of each value is its toward-zero or next fp16 value, chosen by the
    Philox word of its element; outputs stay within 1e-3 of the stepwise truth (2 u of fp16)."""
    Bt, H, P, N, G, L = 2, 4, 16, 32, 2, 4
    seed = 19
    S0 = workload.initial_state(seed, Bt, H, P, N)
    A, D = workload.layer_params(seed, H)
    S16 = S0.astype(np.float16).astype(np.float32)
    rne = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP16)
    sr = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP16_SR, seed=77)
    ref = oracle.Replay(S16, A, D, G, L, 1)            # fp32 master from the fp16 state
    assert np.array_equal(rne.checkpoint(), S16.astype(np.float64))
    assert np.array_equal(sr.checkpoint(), S16.astype(np.float64))
    S = S0.astype(np.float64)
    for t in range(L):
        ins = workload.step_inputs(seed, t, Bt, H, P, N, G)
        y_true = oracle.step(S, *ins, A, D)
        for r in (rne, sr):
            y = r.step(*ins)
            assert np.abs(y - y_true).max() / np.abs(y_true).max() <= 1e-3
        ref.step(*ins)
    v32 = ref.checkpoint().astype(np.float32)           # fp32 fold of the same records
    assert np.array_equal(rne.checkpoint(), v32.astype(np.float16).astype(np.float64))
    flat = v32.reshape(Bt, -1)
    r16 = np.empty_like(flat, dtype=np.uint32)
    for b in range(Bt):
        for g in range(flat.shape[1] // 8):
            w = oracle.philox4x32_10([g, b, L, 0], [77, 0])
            # element 8g + i: the low half of word i // 2 for even i, the high half for odd i
            r16[b, 8 * g:8 * g + 8] = [(int(w[i // 2]) >> (16 * (i % 2))) & 0xFFFF for i in range(8)]
    want = oracle.f16_decode(oracle.f16_encode(flat, r16)).astype(np.float64).reshape(S0.shape)
    assert np.array_equal(sr.checkpoint(), want)
    assert not np.array_equal(sr.checkpoint(), rne.checkpoint())


def test_sampled_rows_round_as_in_the_full_batch():
    """A replay over rows [2, 0] of a batch, told their batch indices, rounds stochastically
    exactly as those rows of the full-batch replay; without the indices it does not."""
    Bt, H, P, N, G, L = 3, 2, 8, 16, 1, 3
    seed = 23
    S0 = workload.initial_state(seed, Bt, H, P, N)
    A, D = workload.layer_params(seed, H)
    rows = np.array([2, 0])
    full = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP16_SR, seed=5)
    part = oracle.Replay(S0[rows], A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP16_SR, seed=5, seq_ids=rows)
    blind = oracle.Replay(S0[rows], A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP16_SR, seed=5)
    for t in range(2 * L):
        x, B, C, dt = workload.step_inputs(seed, t, Bt, H, P, N, G)
        y = full.step(x, B, C, dt)
        assert np.array_equal(part.step(x[rows], B[rows], C[rows], dt[rows]), y[rows])
        blind.step(x[rows], B[rows], C[rows], dt[rows])
    assert np.array_equal(part.checkpoint(), full.checkpoint()[rows])
    assert not np.array_equal(blind.checkpoint(), full.checkpoint()[rows])


def test_stochastic_rounding_avoids_stagnation():
    """workload.stagnation_case: increments of a sixteenth of fp16's spacing per flush (exact in
    float32 and float64). Nearest even loses every one (the checkpoint stays 1.0),
    stochastic rounding keeps them in expectation -- after 64 flushes the mean checkpoint is
    within 10 standard deviations (binomial, p = 1/16 per flush and value) of 1 + 64 * 2^-14."""
    (Bt, H, P, N, G, L), S0, A, D, tok = workload.stagnation_case()
    rne = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP16)
    sr = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP16_SR, seed=9)
    flushes = 64
    for _ in range(flushes * L):
        rne.step(*tok)
        sr.step(*tok)
    assert np.all(rne.checkpoint() == 1.0)
    truth = 1.0 + flushes * 2.0 ** -14
    m = sr.checkpoint()
    assert set(np.unique(m)) <= {1.0 + i * 2.0 ** -10 for i in range(flushes + 1)}
    sd = 2.0 ** -10 * np.sqrt(flushes * (1 / 16) * (15 / 16) / m.size)
    assert abs(float(m.mean()) - truth) <= 10 * sd


@pytest.mark.parametrize("master", [oracle.MASTER_FP16, oracle.MASTER_FP16_SR])
def test_rounding_at_flushes_only_compounds_less(master):
    """[Clarity] "Why it matters": when the state is stored less often, its rounding is fed back
    into the recurrence less often. With the same fp16 state, the replay form at L = 1 rounds
    on every step (the conventional step) and at L = 16 on every 16th: over 128 steps its rms
    state and output errors against float64 must be well below (here < 0.6x; measured 0.25-0.39x
    over seeds) those of rounding every step."""
    Bt, H, P, N, G = 2, 4, 16, 32, 2
    seed = 4
    A, D = workload.layer_params(seed, H)
    S0 = workload.initial_state(seed, Bt, H, P, N)

    def rms(a, ref):
        return float(np.sqrt(np.mean((a - ref) ** 2)) / np.sqrt(np.mean(ref ** 2)))

    res = {}
    for L in (1, 16):
        r = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, master, seed=5)
        S = S0.astype(np.float64)
        errs = []
        for t in range(128):
            ins = workload.step_inputs(seed, t, Bt, H, P, N, G)
            y_true = oracle.step(S, *ins, A, D)
            errs.append(rms(r.step(*ins), y_true))
        res[L] = (rms(r.materialize(), S), float(np.mean(errs)))
    assert res[16][0] < 0.6 * res[1][0] and res[16][1] < 0.6 * res[1][1], res
