"""Pins for the oracle's low-precision master (readings R8 and R9 of oracle.c): the Philox4x32-10
stream, fp16 and E4M3 rounding to nearest even and stochastically, and the dual models that keep
the checkpoint in fp16 or in fp8.

Independent references: the generator's published known-answer vectors
(tests/golden/philox_kat.json), numpy's float16 and PyTorch's float8_e4m3fn conversions (library
routines), neighbours and thresholds computed with numpy.nextafter, the library's E4M3 code table
and exact fractions, and an fp32-master replay whose flushed checkpoint the libraries round.
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


def _e4m3_values():
    """Non-negative finite E4M3FN values, ascending, from PyTorch's float8_e4m3fn (a library
    conversion, independent of the oracle's codec)."""
    import torch
    t = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    return t.astype(np.float64)


def test_e4m3_stochastic_rounding_threshold():
    """Reading R9 of oracle.c: the magnitude rounds up to the next E4M3 value iff r16 < T,
    T = (|a| - q) / (next - q) * 2^16 exactly (q the E4M3 value toward zero, from the library's code table);
    values beyond +-448 clamp to 448; representable values never change. An fp32 value keeps 20
    bits below E4M3's spacing, so T is a multiple of 1/16 in the normal range and the mean over
    all 2^16 values of r16 is within 2^-16 of a spacing of the value (exact where T is an
    integer)."""
    vals = _e4m3_values()
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(600) * np.exp2(rng.integers(-12, 10, 600))).astype(np.float32)
    a = np.concatenate([a, vals[rng.integers(0, len(vals), 40)].astype(np.float32),
                        np.float32([448.0, 500.0, -1e6, 2.0 ** -9, 2.0 ** -10, 0.0])])
    table = oracle.e4m3_decode_table().astype(np.float64)
    n_frac = 0
    for x in a:
        m = min(abs(float(x)), 448.0)
        k = int(np.searchsorted(vals, m, side="right")) - 1
        q = vals[k]
        sign = -1.0 if (x < 0 or (x == 0 and np.signbit(x))) else 1.0
        if q == m:
            rs = np.array([0, 1, 32768, 65535], np.uint32)
            got = table[oracle.e4m3_encode_sr(np.full(4, x, np.float32), rs)]
            assert np.all(got == sign * q), x
            continue
        nxt = vals[k + 1]
        T = (Fraction(m) - Fraction(q)) / (Fraction(nxt) - Fraction(q)) * 2 ** 16
        assert 0 < T < 2 ** 16
        if m >= 2.0 ** -6:
            assert (T * 16).denominator == 1, (x, T)
        c = -(-T.numerator // T.denominator)
        rs = np.array(sorted({0, max(c - 1, 0), min(c, 2 ** 16 - 1), min(c + 1, 2 ** 16 - 1), 2 ** 16 - 1}), np.uint32)
        got = table[oracle.e4m3_encode_sr(np.full(len(rs), x, np.float32), rs)]
        want = [sign * (nxt if Fraction(int(r)) < T else q) for r in rs]
        assert np.array_equal(got, np.array(want)), (x, T)
        mean = Fraction(c) * Fraction(nxt) + Fraction(2 ** 16 - c) * Fraction(q)    # times 2^16
        err = abs(mean - Fraction(m) * 2 ** 16)
        assert err < Fraction(nxt) - Fraction(q)
        if T.denominator == 1:
            assert err == 0
        else:
            n_frac += 1
    assert n_frac > 100


def _e4m3_nearest_per_head(S):
    """S [Bt,H,P,N] rounded to E4M3FN per (sequence, head) by the fp8 read copy's recipe, with
    PyTorch's float8_e4m3fn conversion for the rounding: scale = amax / 448 in fp32 (1 if 0)."""
    import torch
    S = np.asarray(S, np.float32)
    amax = np.abs(S).max(axis=(2, 3), keepdims=True)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    a = np.clip(S * (np.float32(1.0) / scale), -448.0, 448.0).astype(np.float32)
    q = torch.from_numpy(a).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    return q * scale.astype(np.float64), scale, a


def test_fp8_master_dual_model():
    """Reading R9 of oracle.c: after load the checkpoint is the nearest-even E4M3 of S0 with
    the per-head scale; after the first flush, the nearest-even E4M3 of an fp32-master replay's checkpoint
    started from that state; with stochastic rounding each value is its E4M3 neighbour toward
    zero or away, chosen by the Philox field of its element as for the fp16 master. The outputs
    stay within 0.07 of the stepwise truth's largest value (fp8's half step is 2^-4)."""
    Bt, H, P, N, G, L = 2, 4, 16, 32, 2, 4
    seed = 21
    S0 = workload.initial_state(seed, Bt, H, P, N)
    A, D = workload.layer_params(seed, H)
    S8, _, _ = _e4m3_nearest_per_head(S0)
    rne = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP8)
    sr = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP8_SR, seed=77)
    ref = oracle.Replay(S8.astype(np.float32), A, D, G, L, 1)
    assert np.array_equal(rne.checkpoint(), S8)
    assert np.array_equal(sr.checkpoint(), S8)
    S = S0.astype(np.float64)
    for t in range(L):
        ins = workload.step_inputs(seed, t, Bt, H, P, N, G)
        y_true = oracle.step(S, *ins, A, D)
        for r in (rne, sr):
            y = r.step(*ins)
            assert np.abs(y - y_true).max() / np.abs(y_true).max() <= 0.07
        ref.step(*ins)
    v32 = ref.checkpoint().astype(np.float32)
    want_rne, scale, a = _e4m3_nearest_per_head(v32)
    assert np.array_equal(rne.checkpoint(), want_rne)
    vals = _e4m3_values()
    flat_a = a.reshape(Bt, -1)
    got = (sr.checkpoint() / scale.astype(np.float64)).reshape(Bt, -1)
    ups = 0
    for b in range(Bt):
        for g in range(flat_a.shape[1] // 8):
            w = oracle.philox4x32_10([g, b, L, 0], [77, 0])
            for i in range(8):
                e = 8 * g + i
                r16 = (int(w[i // 2]) >> (16 * (i % 2))) & 0xFFFF
                m = abs(float(flat_a[b, e]))
                k = int(np.searchsorted(vals, m, side="right")) - 1
                q = vals[k]
                if q == m:
                    want = q
                else:
                    T = (Fraction(m) - Fraction(q)) / (Fraction(vals[k + 1]) - Fraction(q)) * 2 ** 16
                    want = vals[k + 1] if Fraction(r16) < T else q
                    ups += want != q
                assert abs(got[b, e]) == want and (got[b, e] == 0 or np.sign(got[b, e]) == np.sign(flat_a[b, e])), (b, e)
    assert ups > 100
    assert not np.array_equal(sr.checkpoint(), rne.checkpoint())


def test_fp8_master_stochastic_rounding_avoids_stagnation():
    """Reading R9 of oracle.c on workload.stagnation_case with the state at 0.5 and row p = 0
    fixed (x = 0 there) holding the anchor 1.0, so the per-head scale stays amax / 448 = 1/448 and the body
    sits on the E4M3 value 224 (spacing 16, i.e. 1/28 of state). Each flush adds 2^-14 = 0.027
    of a scaled unit: nearest even loses every increment, stochastic rounding keeps them in
    expectation -- after 64 flushes the body's mean is within 10 standard deviations (binomial,
    p = 0.027 / 16 per flush and value) of 0.5 + 64 * 2^-14."""
    (Bt, H, P, N, G, L), S0, A, D, (x, B, C, dt) = workload.stagnation_case()
    S0 = np.full_like(S0, 0.5)
    S0[:, :, 0, :] = 1.0
    x = x.copy()
    x[:, :, 0] = 0.0
    tok = (x, B, C, dt)
    rne = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP8)
    sr = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP8_SR, seed=9)
    flushes = 64
    for _ in range(flushes * L):
        rne.step(*tok)
        sr.step(*tok)
    scale = float(np.float32(1.0) / np.float32(448.0))
    assert np.all(rne.checkpoint()[:, :, 0, :] == 448 * scale)
    assert np.all(rne.checkpoint()[:, :, 1:, :] == 224 * scale)
    m = sr.checkpoint()[:, :, 1:, :]
    truth = 0.5 + flushes * 2.0 ** -14
    p = (2.0 ** -14 * 448) / 16
    sd = 16 * scale * np.sqrt(flushes * p * (1 - p) / m.size)
    assert abs(float(m.mean()) - truth) <= 10 * sd, (float(m.mean()), truth, sd)


def test_fp8_master_export_and_import():
    """Reading R9's state as codes and scales: the exported codes times the scales are the
    checkpoint exactly (decoded with the library's E4M3 table); importing a row's codes and scales
    into a second replay at the same position reproduces that row, and both replays then flush
    identically."""
    Bt, H, P, N, G, L = 3, 2, 8, 32, 1, 4
    seed = 31
    S0 = workload.initial_state(seed, Bt, H, P, N)
    A, D = workload.layer_params(seed, H)
    a = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP8_SR, seed=6)
    b = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP8_SR, seed=6)
    import torch
    table = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for t in range(L + 1):
        ins = workload.step_inputs(seed, t, Bt, H, P, N, G)
        a.step(*ins)
        if t < L - 1:
            b.step(*ins)
    codes, scales = a.fp8_master()
    assert scales.shape == (Bt, H, 1)
    assert np.array_equal(table[codes] * scales[:, :, :, None].astype(np.float64), a.checkpoint())
    with pytest.raises(RuntimeError):
        oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP16).fp8_master()
    # b is one token short of a's flush; it takes a's post-flush state for rows 2 and 0 after
    # stepping through the same flush itself, then both continue in lockstep
    b.step(*workload.step_inputs(seed, L - 1, Bt, H, P, N, G))
    b.step(*workload.step_inputs(seed, L, Bt, H, P, N, G))
    b.set_master_fp8(codes[[2, 0]], scales[[2, 0]], [2, 0])
    assert np.array_equal(b.checkpoint(), a.checkpoint())
    for t in range(L + 1, 2 * L + 2):
        ins = workload.step_inputs(seed, t, Bt, H, P, N, G)
        assert np.array_equal(a.step(*ins), b.step(*ins))
    assert np.array_equal(b.checkpoint(), a.checkpoint())


def test_fp8_master_blocks_of_64_rows():
    """Reading R9 with P = 100: the fp8 master's load takes the fp8 copy's per-block scales (rows
    0..63 and 64..99), codes against PyTorch's float8_e4m3fn of each block over its amax / 448."""
    import torch
    Bt, H, P, N, G, L = 2, 2, 100, 32, 1, 4
    seed = 73
    S0 = workload.initial_state(seed, Bt, H, P, N)
    A, D = workload.layer_params(seed, H)
    r = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_FP32, oracle.MASTER_FP8)
    codes, scales = r.fp8_master()
    assert scales.shape == (Bt, H, 2)
    for kb, (p0, p1) in enumerate([(0, 64), (64, 100)]):
        blk = S0[:, :, p0:p1, :]
        scale = (np.abs(blk).max(axis=(2, 3)) / np.float32(448.0)).astype(np.float32)
        assert np.array_equal(scales[:, :, kb], scale)
        a = np.clip(blk * (np.float32(1.0) / scale[:, :, None, None]), -448.0, 448.0).astype(np.float32)
        want = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes[:, :, p0:p1, :], want), f"block {kb}"
