"""Pins for the oracle's read-copy quantizers (O7).

bf16 and OCP fp8 E4M3FN encoders are checked against the format definitions (a hand-checked code
table, a brute-force nearest-code search with ties to even) and against an independent library
routine (PyTorch's CPU float8_e4m3fn / bfloat16 conversions): bf16 over all 2^32 fp32 bit
patterns, e4m3 over every non-negative pattern the clamp does not decide plus a strided sweep of
the rest.
"""
import numpy as np
import pytest
import torch

import oracle


def _patterns(first_chunk, end_chunk, chunk_bits=24):
    """fp32 values of bit patterns [first_chunk << chunk_bits, end_chunk << chunk_bits), one chunk
    at a time, with a NaN mask computed on the integer bits."""
    base = np.arange(1 << chunk_bits, dtype=np.uint32)
    buf = np.empty_like(base)
    for hi in range(first_chunk, end_chunk):
        np.add(base, np.uint32(hi << chunk_bits), out=buf)
        yield buf.view(np.float32), (buf & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)


def test_e4m3_code_table():
    """Hand-checked codes of OCP E4M3FN: bias 7, subnormal step 2^-9, max finite 448, NaN only
    at S.1111.111, no infinities; the library decode agrees on all 256 codes."""
    t = oracle.e4m3_decode_table()
    assert t[0x00] == 0.0 and t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9
    assert t[0x08] == 2.0 ** -6 and t[0x38] == 1.0 and t[0x39] == 1.125
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0 and t[0x77] == 240.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert int(np.isfinite(t).sum()) == 254
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                     # codes 0..126 strictly increasing
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    same = (lib == t) | (np.isnan(lib) & np.isnan(t))
    assert same.all()


def test_e4m3_encode_vs_nearest_code_search():
    """Brute force: for every value, the code is the nearest of the 127 non-negative finite
    magnitudes (after clamping to 448), ties to the even code. Inputs include every midpoint
    between adjacent codes and its fp32 neighbours, plus a dense random sample."""
    t = oracle.e4m3_decode_table().astype(np.float64)
    mags = t[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2
    base = np.concatenate([mags, mids, mids * 1.0000001, mids * 0.9999999,
                           np.random.default_rng(0).uniform(0, 500, 200000),
                           np.random.default_rng(1).uniform(0, 2.0 ** -5, 100000),
                           [449.0, 464.0, 470.0, 479.0, 480.0, 1e6, 3.4e38]]).astype(np.float32)
    vals = np.concatenate([base, -base])
    codes = oracle.e4m3_encode_at(vals, 1.0)
    v = np.minimum(np.abs(vals.astype(np.float64)), 448.0)
    dist = np.abs(v[:, None] - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among the tied nearest codes pick the even one
    idx = np.where(cand.sum(1) == 1, dist.argmin(1),
                   np.argmax(cand & (np.arange(0x7F)[None, :] % 2 == 0), axis=1))
    expect = idx.astype(np.uint8) | np.where(np.signbit(vals), 0x80, 0).astype(np.uint8)
    assert np.array_equal(codes, expect)


@pytest.mark.slow
def test_e4m3_encode_exhaustive_vs_library():
    """Every non-negative fp32 pattern up to 480 (the last value the clamp does not decide) and
    a strided sweep of all other patterns, both signs: the oracle encoder at scale 1 equals
    PyTorch's float8_e4m3fn conversion of the value clamped to +-448 (the library rounds to
    nearest even but does not saturate, hence the clamp). NaN patterns are skipped."""
    end = (0x43F00000 >> 24) + 1
    chunks = list(range(0, end)) + list(range(end, 256, 5))
    for hi in chunks:
        for v, nan in _patterns(hi, hi + 1):
            mine = oracle.e4m3_encode_at(v, 1.0)
            ref = torch.from_numpy(np.clip(v, -448.0, 448.0)).to(torch.float8_e4m3fn).view(
                torch.uint8).numpy()
            assert np.all((mine == ref) | nan)


@pytest.mark.slow
def test_bf16_encode_exhaustive_vs_library():
    """All 2^32 fp32 patterns (NaN skipped): round-to-nearest-even to bf16 equals PyTorch's
    bfloat16 conversion, including overflow to infinity."""
    for v, nan in _patterns(0, 256):
        mine = oracle.bf16_encode(v)
        ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.all((mine == ref) | nan)


def test_bf16_ties_and_carries():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  np.finfo(np.float32).max, -2.0 ** -133], np.float32)
    enc = oracle.bf16_encode(f)
    dec = oracle.bf16_decode(enc)
    assert dec[0] == 1.0
    assert dec[1] == 1.0                          # tie -> even (down)
    assert dec[2] == 1.0 + 4 * 2 ** -8            # tie -> even (up)
    assert dec[3] == 1.0 + 2 * 2 ** -8            # above the tie -> up
    assert np.isinf(dec[4])                       # rounds past the largest bf16 -> inf
    assert dec[5] == -2.0 ** -133                 # subnormal kept exactly


def test_e4m3_tile_scale():
    """Per-tile scale = amax/448 (fp32), 1 for an all-zero tile; the amax element encodes to
    +-448 and decode(code) * scale reproduces each value within half a code step."""
    rng = np.random.default_rng(3)
    tiles = rng.standard_normal((5, 1024)).astype(np.float32)
    tiles[1] *= 1e-3
    tiles[2] = 0.0
    tiles[3, 17] = -9.5
    codes, scales = oracle.e4m3_encode_tiles(tiles, 1024)
    amax = np.abs(tiles).max(1)
    exp_scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(scales, exp_scale)
    codes = codes.reshape(5, 1024)
    assert np.all(codes[2] == 0) and scales[2] == 1.0
    assert codes[3, 17] == 0xFE
    t = oracle.e4m3_decode_table().astype(np.float64)
    dec = t[codes] * scales[:, None]
    # relative step of e4m3 normals is 2^-3; half of it bounds the rounding error
    big = np.abs(tiles) >= scales[:, None] * 2.0 ** -6
    err = np.abs(dec - tiles)[big] / np.abs(tiles)[big]
    assert err.max() <= 2.0 ** -4 * (1 + 1e-6)
