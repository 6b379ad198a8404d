"""Pins for the oracle's MXFP4 read-copy codec (reading R7 of the oracle).

No library in this environment converts to FP4 E2M1, so the codec is pinned by values derived by
hand from the OCP MX v1.0 definitions (tests/golden/mxfp4_codes.json), by a closed form for the
block scale computed from integer exponents (not from the oracle's frexp), and by properties any
correct encoder has: representable values round-trip exactly, the error is at most half the code
spacing below the clamp, the encode is monotone, and the dual-precision replay carries only the
copy's rounding.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "mxfp4_codes.json")
MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_e2m1_table():
    g = _golden()
    for code, want in enumerate(g["e2m1_values"]):
        got = oracle.e2m1_decode(code)
        assert got == want and np.signbit(got) == np.signbit(want), (code, got, want)


def test_element_codes_hand_derived():
    g = _golden()
    vals = np.array([float(v) for v, _ in g["element_codes_at_scale_1"]])
    want = np.array([c for _, c in g["element_codes_at_scale_1"]], np.uint8)
    assert np.array_equal(oracle.e2m1_encode_scaled(vals), want)


def test_scale_codes_hand_derived():
    g = _golden()
    for v, want in g["scale_codes"]:
        blk = np.zeros(32, np.float32)
        blk[7] = np.float32(float(v))
        blk[3] = -blk[7] * np.float32(0.5)
        assert oracle.mx_scale_code(blk) == want, v


def test_scale_closed_form_every_exponent():
    """amax = m * 2^k for every fp32 exponent k: code = clamp(k - 2 + 127, 0, 254), from integer
    k; the sign and the other elements of the block do not matter."""
    rng = np.random.default_rng(5)
    for k in range(-149, 128):
        for m in ((1.0,) if k < -126 else (1.0, 1.25, 1.9999999)):
            amax = np.float32(np.ldexp(m, k))
            blk = (rng.uniform(-1, 1, 32) * float(amax)).astype(np.float32)
            blk[rng.integers(32)] = -amax if k % 2 else amax
            want = min(max(k - 2 + 127, 0), 254)
            assert oracle.mx_scale_code(blk) == want, (k, m)


def test_packed_blocks_hand_derived():
    g = _golden()
    for blk in g["blocks"]:
        a = np.zeros(32, np.float32)
        a[:len(blk["lead"])] = [float(v) for v in blk["lead"]]
        codes, scales = oracle.mxfp4_encode(a[None, :])
        assert scales[0, 0] == blk["scale"]
        lead = blk["lead_bytes"]
        assert list(codes[0, :len(lead)]) == lead
        assert not codes[0, len(lead):].any()


def test_representable_values_round_trip():
    """Blocks made only of representable values at scale 2^s (with a 4 or 6 present, so the scale
    is exactly 2^s) decode to themselves, for scales across the whole E8M0 range fp32 reaches."""
    rng = np.random.default_rng(9)
    signed = np.concatenate([MAGS, -MAGS[1:]])
    for s in range(-125, 126, 3):
        vals = rng.choice(signed, size=(16, 32))
        vals[:, 0] = rng.choice([4.0, 6.0, -4.0, -6.0], size=16)
        a = np.ldexp(vals, s).astype(np.float32)
        codes, scales = oracle.mxfp4_encode(a)
        assert np.all(scales == s + 127)
        assert np.array_equal(oracle.mxfp4_decode(codes, scales), a.astype(np.float64))


def test_error_bound_and_monotone():
    """Random blocks over many magnitudes: below the clamp (|v| <= 6X) the error is at most half
    the code spacing at |v| (0.5X under 2X, X under 4X, 2X above); above it the value decodes
    to +-6X. Within a block the encode is monotone in the value."""
    rng = np.random.default_rng(13)
    a = (rng.standard_normal((4000, 32)) * np.exp2(rng.integers(-60, 60, size=(4000, 1)))).astype(np.float32)
    a[::7, 5] = 0.0
    codes, scales = oracle.mxfp4_encode(a)
    d = oracle.mxfp4_decode(codes, scales)
    X = np.exp2(scales.astype(np.float64) - 127)          # [4000, 1]
    r = np.abs(a.astype(np.float64)) / X
    half = np.where(r < 2, 0.25, np.where(r < 4, 0.5, 1.0)) * X
    inside = r <= 6
    assert np.all(np.abs(d - a)[inside] <= half[inside])
    assert np.all(np.abs(d)[~inside] == (6 * X * np.ones_like(d))[~inside])
    assert np.all(r < 8)                                   # the scale rule never lets a block overflow
    order = np.argsort(a, axis=1)
    ds = np.take_along_axis(d, order, axis=1)
    assert np.all(np.diff(ds, axis=1) >= 0)


def test_dual_precision_model_mxfp4():
    """Read copy = MXFP4 of the fp32 master (decoded in float64). Flush-step outputs come from the
    fresh master and match the stepwise truth to float64 rounding; non-flush outputs carry the
    copy's rounding only, inside the MXFP4 output gate (0.25: about 2.2x the format's 0.115 rms
    relative error on Gaussian blocks); the copy changes only at flushes."""
    cfg = workload.TINY
    Bt, H, P, N, G, L = cfg["Bt"], cfg["H"], cfg["P"], 32, cfg["G"], cfg["L"]
    seed = 71
    S0 = workload.initial_state(seed, Bt, H, P, N)
    A, D = workload.layer_params(seed, H)
    rep = oracle.Replay(S0, A, D, G, L, 1, oracle.READ_MXFP4)
    codes, scales = oracle.mxfp4_encode(S0)
    copy0 = rep.read_copy()
    assert np.array_equal(copy0, oracle.mxfp4_decode(codes, scales))
    S = S0.astype(np.float64)
    for t in range(32):
        x, B, C, dt = workload.step_inputs(seed, t, Bt, H, P, N, G)
        y_ref = oracle.step(S, x, B, C, dt, A, D)
        y = rep.step(x, B, C, dt)
        e = np.abs(y - y_ref).max() / np.abs(y_ref).max()
        if (t + 1) % L == 0:
            assert e <= 1e-12
        else:
            assert 0 < e <= 0.25
        if t == L - 2:
            assert np.array_equal(rep.read_copy(), copy0)
    assert not np.array_equal(rep.read_copy(), copy0)


def test_mxfp4_requires_blocks_of_32():
    S0 = np.zeros((1, 1, 4, 16), np.float32)
    with pytest.raises(ValueError):
        oracle.Replay(S0, np.full(1, -1.0, np.float32), np.zeros(1, np.float32), 1, 4, 1, oracle.READ_MXFP4)
