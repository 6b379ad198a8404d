"""Pins for the oracle's Gated DeltaNet part (oracle_gdn.c): the stepwise recurrence (O1g), its
replay form by the backward sweep (O3g) with the pointer machine, and per-draft spec decoding
(O5g).

Each pin is independent of the code it checks: explicit d_k x d_k matrices in numpy, exact
rational arithmetic, closed-form special cases of the delta rule, and the unrolled window written
as products of explicit matrices.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workload


def _rel(a, ref):
    return float(np.max(np.abs(np.asarray(a) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _inputs(seed, Bt, H, G, Dv, Dk, t):
    return workload.gdn_step_inputs(seed, t, Bt, H, G, Dv, Dk)


def _numpy_step(S, q, k, v, alpha, beta):
    """S_t = alpha S (I - beta k k^T) + beta v k^T, o = S_t q, with explicit matrices."""
    Bt, H, Dv, Dk = S.shape
    G = q.shape[1]
    o = np.empty((Bt, H, Dv))
    for b in range(Bt):
        for h in range(H):
            g = h // (H // G)
            kk = k[b, g].astype(np.float64)
            M = np.eye(Dk) - float(beta[b, h]) * np.outer(kk, kk)
            S[b, h] = float(alpha[b, h]) * S[b, h] @ M + float(beta[b, h]) * np.outer(v[b, h].astype(np.float64), kk)
            o[b, h] = S[b, h] @ q[b, g].astype(np.float64)
    return o


@pytest.mark.parametrize("shape", [(2, 4, 2, 8, 16), (1, 6, 3, 5, 7), (3, 2, 1, 16, 32)])
def test_one_step_vs_explicit_matrices(shape):
    Bt, H, G, Dv, Dk = shape
    S0 = workload.gdn_initial_state(3, Bt, H, Dv, Dk).astype(np.float64)
    S_ref = S0.copy()
    S = S0.copy()
    for t in range(3):
        q, k, v, a, b = _inputs(3, Bt, H, G, Dv, Dk, t)
        o = oracle.gdn_step(S, q, k, v, a, b)
        o_ref = _numpy_step(S_ref, q, k, v, a, b)
        assert _rel(o, o_ref) <= 1e-13 and _rel(S, S_ref) <= 1e-13


def test_exact_rationals_bit_equal():
    """Small integers with alpha in {1, 1/2}, beta in {1/2, 1}: every value is a dyadic rational of
    modest size, so float64 is exact and must equal the Fraction recurrence bit for bit."""
    rng = np.random.default_rng(11)
    Bt, H, G, Dv, Dk = 1, 2, 1, 3, 4
    S = rng.integers(-2, 3, (Bt, H, Dv, Dk)).astype(np.float64)
    F = [[[[Fraction(int(S[0, h, p, n])) for n in range(Dk)] for p in range(Dv)] for h in range(H)]]
    for t in range(6):
        q = rng.integers(-1, 2, (Bt, G, Dk)).astype(np.float32)
        k = rng.integers(-1, 2, (Bt, G, Dk)).astype(np.float32)
        v = rng.integers(-2, 3, (Bt, H, Dv)).astype(np.float32)
        a = rng.choice([1.0, 0.5], (Bt, H)).astype(np.float32)
        b = rng.choice([0.5, 1.0], (Bt, H)).astype(np.float32)
        o = oracle.gdn_step(S, q, k, v, a, b)
        for h in range(H):
            A, Bv = Fraction(float(a[0, h])), Fraction(float(b[0, h]))
            kk = [Fraction(int(x)) for x in k[0, 0]]
            for p in range(Dv):
                row = F[0][h][p]
                sk = sum(row[n] * kk[n] for n in range(Dk))
                F[0][h][p] = [A * (row[n] - Bv * sk * kk[n]) + Bv * int(v[0, h, p]) * kk[n] for n in range(Dk)]
                want = sum(F[0][h][p][n] * int(q[0, 0, n]) for n in range(Dk))
                assert o[0, h, p] == float(want)
        assert np.array_equal(S, np.array([[[[float(x) for x in r] for r in hh] for hh in F[0]]]))


def test_special_cases_of_the_delta_rule():
    """beta = 0: pure decay, S_t = alpha S. k = e_i, alpha = beta = 1: column i of S becomes v
    and the other columns are untouched."""
    Bt, H, G, Dv, Dk = 1, 2, 1, 4, 6
    S0 = workload.gdn_initial_state(5, Bt, H, Dv, Dk).astype(np.float64)
    q, k, v, a, _ = _inputs(5, Bt, H, G, Dv, Dk, 0)
    S = S0.copy()
    o = oracle.gdn_step(S, q, k, v, a, np.zeros((Bt, H), np.float32))
    for h in range(H):
        assert np.array_equal(S[0, h], float(a[0, h]) * S0[0, h])
    assert _rel(o[0], np.einsum("hpn,n->hp", S[0], q[0, 0].astype(np.float64))) <= 1e-15
    i = 3
    e = np.zeros((Bt, G, Dk), np.float32)
    e[0, 0, i] = 1.0
    S = S0.copy()
    oracle.gdn_step(S, q, e, v, np.ones((Bt, H), np.float32), np.ones((Bt, H), np.float32))
    for h in range(H):
        assert np.array_equal(S[0, h][:, i], v[0, h].astype(np.float64))
        keep = [n for n in range(Dk) if n != i]
        assert np.array_equal(S[0, h][:, keep], S0[0, h][:, keep])


@pytest.mark.parametrize("L,Tmax", [(4, 1), (16, 1), (5, 2), (1, 1)])
def test_replay_matches_stepwise(L, Tmax):
    """Replay outputs equal O1g at every step; after each flush the checkpoint equals the O1g state;
    materialize equals it always. L = 1 (every step flushes) is the stepwise form itself."""
    cfg = workload.GDN_TINY
    Bt, H, G, Dv, Dk = cfg["Bt"], cfg["H"], cfg["G"], cfg["Dv"], cfg["Dk"]
    seed = 21
    S0 = workload.gdn_initial_state(seed, Bt, H, Dv, Dk)
    rep = oracle.GDNReplay(S0, G, L, Tmax)
    S = S0.astype(np.float64)
    period = L - Tmax + 1
    for t in range(40):
        ins = _inputs(seed, Bt, H, G, Dv, Dk, t)
        o_ref = oracle.gdn_step(S, *ins)
        o = rep.step(*ins)
        if L == 1:
            assert np.array_equal(o, o_ref)
        assert _rel(o, o_ref) <= 1e-12, t
        pos, ck = rep.pointers()
        assert list(pos) == [t + 1] * Bt and list(ck) == [(t + 1) // period * period] * Bt
        assert _rel(rep.materialize(), S) <= 1e-12
        if (t + 1) % period == 0:
            assert _rel(rep.checkpoint(), S) <= 1e-12


def test_replay_window_vs_explicit_products():
    """A window that never flushes, against S_t = S_c A_0..A_t + sum_j beta_j v_j k_j^T A_{j+1}..A_t
    with A_j = alpha_j (I - beta_j k_j k_j^T) built as explicit matrices, o_t = S_t q_t."""
    Bt, H, G, Dv, Dk, steps = 2, 4, 2, 6, 8, 12
    seed = 33
    S0 = workload.gdn_initial_state(seed, Bt, H, Dv, Dk)
    rep = oracle.GDNReplay(S0, G, 16, 1)
    toks = [_inputs(seed, Bt, H, G, Dv, Dk, t) for t in range(steps)]
    for t in range(steps):
        o = rep.step(*toks[t])
        for b in range(Bt):
            for h in range(H):
                g = h // (H // G)
                A = []
                for j in range(t + 1):
                    kk = toks[j][1][b, g].astype(np.float64)
                    A.append(float(toks[j][3][b, h]) * (np.eye(Dk) - float(toks[j][4][b, h]) * np.outer(kk, kk)))
                P = np.eye(Dk)
                for j in range(t + 1):
                    P = P @ A[j]
                St = S0[b, h].astype(np.float64) @ P
                for j in range(t + 1):
                    tail = np.eye(Dk)
                    for i in range(j + 1, t + 1):
                        tail = tail @ A[i]
                    kk = toks[j][1][b, g].astype(np.float64)
                    St = St + float(toks[j][4][b, h]) * np.outer(toks[j][2][b, h].astype(np.float64), kk) @ tail
                o_ref = St @ toks[t][0][b, g].astype(np.float64)
                assert _rel(o[b, h], o_ref) <= 1e-12


@pytest.mark.parametrize("T,L", [(4, 16), (3, 7), (1, 4)])
def test_spec_verify_rollback_vs_per_draft(T, L):
    """Verify outputs of all T drafts and the committed state after each rollback equal the
    per-draft definition (O5g), with standard steps interleaved; accepted counts include 0 and T."""
    Bt, H, G, Dv, Dk = 3, 4, 2, 8, 16
    seed = 45
    S0 = workload.gdn_initial_state(seed, Bt, H, Dv, Dk)
    rep = oracle.GDNReplay(S0, G, L, T)
    S = S0.astype(np.float64)
    rng = np.random.default_rng(seed)
    for it in range(24):
        drafts = workload.gdn_draft_inputs(seed, it, Bt, T, H, G, Dv, Dk)
        acc = rng.integers(0, T + 1, Bt).astype(np.int32)
        acc[it % Bt] = T if it % 2 else 0
        o = rep.verify(T, *drafts)
        o_ref = oracle.gdn_spec_stepwise(S, T, *drafts, acc)
        assert _rel(o, o_ref) <= 1e-12, it
        rep.rollback(acc)
        pos, ck = rep.pointers()
        assert np.all(pos - ck <= L - T) and np.all(pos - ck >= 0)
        assert _rel(rep.materialize(), S) <= 1e-12
        if it % 3 == 2:
            ins = _inputs(seed + 1, Bt, H, G, Dv, Dk, it)
            assert _rel(rep.step(*ins), oracle.gdn_step(S, *ins)) <= 1e-12


def test_state_machine_rejections():
    S0 = np.zeros((1, 1, 2, 4), np.float32)
    rep = oracle.GDNReplay(S0, 1, 4, 2)
    z = workload.gdn_draft_inputs(1, 0, 1, 2, 1, 1, 2, 4)
    with pytest.raises(RuntimeError):
        rep.rollback(np.zeros(1, np.int32))              # no verify pending
    rep.verify(2, *z)
    with pytest.raises(RuntimeError):
        rep.verify(2, *z)                                # verify twice
    with pytest.raises(RuntimeError):
        rep.rollback(np.array([3], np.int32))            # accepted > T
    rep.rollback(np.array([2], np.int32))
    with pytest.raises(ValueError):
        oracle.GDNReplay(S0, 1, 4, 5)                    # Tmax > L


def test_bf16_read_copy_model():
    """Reading G4 (bf16 read copy): before the first flush every output equals, bit for bit, the
    fp32-checkpoint replay started from torch's bfloat16 rounding of S0 (a library routine); flush
    steps read the folded checkpoint, so they equal the fp32-checkpoint replay from S0 itself;
    after a flush the copy is torch's bfloat16 of the float32-rounded checkpoint; outputs stay
    within 2e-2 of O1g (bf16's 2^-9 relative rounding over a normwise product)."""
    import torch
    cfg = workload.GDN_TINY
    Bt, H, G, Dv, Dk, L = cfg["Bt"], cfg["H"], cfg["G"], cfg["Dv"], cfg["Dk"], cfg["L"]
    seed = 27
    S0 = workload.gdn_initial_state(seed, Bt, H, Dv, Dk)
    S0_bf = torch.from_numpy(S0).bfloat16().float().numpy()
    cp = oracle.GDNReplay(S0, G, L, 1, oracle.READ_BF16)
    from_bf = oracle.GDNReplay(S0_bf, G, L, 1)
    full = oracle.GDNReplay(S0, G, L, 1)
    S = S0.astype(np.float64)
    assert np.array_equal(cp.read_copy(), S0_bf.astype(np.float64))
    for t in range(3 * L):
        ins = _inputs(seed, Bt, H, G, Dv, Dk, t)
        o, o_bf, o_full = cp.step(*ins), from_bf.step(*ins), full.step(*ins)
        o_true = oracle.gdn_step(S, *ins)
        if t < L - 1:
            assert np.array_equal(o, o_bf), t
        if (t + 1) % L == 0:
            assert _rel(o, o_full) <= 1e-12, t
            ck = cp.checkpoint()
            assert _rel(ck, full.checkpoint()) <= 1e-12
            want = torch.from_numpy(ck.astype(np.float32)).bfloat16().float().numpy().astype(np.float64)
            assert np.array_equal(cp.read_copy(), want), t
        assert _rel(o, o_true) <= 2e-2, t
    assert _rel(cp.materialize(), S) <= 1e-12


def test_set_checkpoint_restarts_the_model():
    """Continuing the GDN replay model from a given fp32 checkpoint after a flush equals a fresh
    model loaded with it (bf16 copy re-encoded from the given values): outputs equal bit for bit;
    and torch's bfloat16 of the given checkpoint is the new copy."""
    import torch
    Bt, H, G, Dv, Dk, L = 2, 4, 2, 16, 32, 4
    seed = 31
    S0 = workload.gdn_initial_state(seed, Bt, H, Dv, Dk)
    a = oracle.GDNReplay(S0, G, L, 1, oracle.READ_BF16)
    for t in range(L):
        a.step(*_inputs(seed, Bt, H, G, Dv, Dk, t))
    S1 = a.checkpoint().astype(np.float32)
    S1[0, 1, 2, 3] = np.float32(-2.5)
    a.set_checkpoint(S1)
    want = torch.from_numpy(S1).bfloat16().float().numpy().astype(np.float64)
    assert np.array_equal(a.read_copy(), want)
    b = oracle.GDNReplay(S1, G, L, 1, oracle.READ_BF16)
    for t in range(L, 2 * L - 1):
        ins = _inputs(seed, Bt, H, G, Dv, Dk, t)
        assert np.array_equal(a.step(*ins), b.step(*ins)), t


_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _mxfp4_round_trip(S):
    """OCP MX v1.0 FP4 by its definition, in numpy: blocks of 32 consecutive values of the last
    axis, scale 2^(E - 2) with E the unbiased exponent of the block's amax read from its fp32
    bits (an all-zero block takes the smallest scale), each value / scale to the nearest E2M1
    magnitude with ties to the even code, clamped to 6, sign kept."""
    S = np.asarray(S, np.float32)
    blk = S.reshape(-1, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=1).astype(np.float32)
    ebits = ((amax.view(np.uint32) >> 23) & 0xFF).astype(np.int64)
    code = np.maximum(ebits - 2, 0)
    scale = np.exp2((code - 127).astype(np.float64))[:, None]
    a = np.minimum(np.abs(blk) / scale, 6.0)
    d = np.abs(a[..., None] - _E2M1)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    ties_even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    idx = np.where(ties_even < 99, ties_even, cand.min(axis=-1))
    return (np.sign(blk) * _E2M1[idx] * scale).reshape(S.shape)


def _fp8_round_trip(S):
    """The fp8 copy by its recipe with PyTorch's float8_e4m3fn conversion: one scale amax / 448
    per block of 64 value rows of each (sequence, value head)."""
    import torch
    S = np.asarray(S, np.float32)
    out = np.empty(S.shape, np.float64)
    for p0 in range(0, S.shape[2], 64):
        blk = S[:, :, p0:p0 + 64, :]
        amax = np.abs(blk).max(axis=(2, 3), keepdims=True)
        scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        a = np.clip(blk * (np.float32(1.0) / scale), -448.0, 448.0).astype(np.float32)
        out[:, :, p0:p0 + 64, :] = torch.from_numpy(a).to(torch.float8_e4m3fn).double().numpy() * scale
    return out


@pytest.mark.parametrize("read_prec,gate", [(oracle.READ_FP8, 6e-2), (oracle.READ_MXFP4, 0.25)])
def test_narrow_read_copy_models(read_prec, gate):
    """Reading G4 with the fp8 and MXFP4 copies (Dv = 80: two fp8 scale blocks, one partial; Dk =
    64: two MX blocks per row): the copy equals the format's definition applied to S0 (fp8 per
    64 value rows with PyTorch's e4m3 conversion; MXFP4 by the OCP rule in numpy); before the
    first flush every output equals the fp32-checkpoint replay started from that decoded copy --
    bit for bit for MXFP4, within 1e-6 for fp8, whose decoded values fp32 rounds; flush steps
    read the folded checkpoint (= the fp32 replay from S0); after a
    flush the copy is the definition applied to the float32-rounded checkpoint; outputs stay
    within the copy's gate of O1g."""
    Bt, H, G, Dv, Dk, L = 2, 4, 2, 80, 64, 4
    seed = 29
    S0 = workload.gdn_initial_state(seed, Bt, H, Dv, Dk)
    enc = _fp8_round_trip if read_prec == oracle.READ_FP8 else _mxfp4_round_trip
    S0_c = enc(S0)
    cp = oracle.GDNReplay(S0, G, L, 1, read_prec)
    from_c = oracle.GDNReplay(S0_c.astype(np.float32), G, L, 1)
    full = oracle.GDNReplay(S0, G, L, 1)
    # MXFP4 values (E2M1 times a power of two) are fp32 numbers, so the fp32 replay from the copy
    # is the same model bit for bit; an fp8 value code * scale carries up to 28 significant bits,
    # which the fp32 start state rounds (2^-24 relative)
    exact = bool(np.array_equal(S0_c.astype(np.float32).astype(np.float64), S0_c))
    assert exact == (read_prec == oracle.READ_MXFP4)
    S = S0.astype(np.float64)
    assert np.array_equal(cp.read_copy(), S0_c)
    for t in range(3 * L):
        ins = _inputs(seed, Bt, H, G, Dv, Dk, t)
        o, o_c, o_full = cp.step(*ins), from_c.step(*ins), full.step(*ins)
        o_true = oracle.gdn_step(S, *ins)
        if t < L - 1:
            assert np.array_equal(o, o_c) if exact else _rel(o, o_c) <= 1e-6, t
        if (t + 1) % L == 0:
            assert _rel(o, o_full) <= 1e-12, t
            assert np.array_equal(cp.read_copy(), enc(cp.checkpoint().astype(np.float32))), t
        assert _rel(o, o_true) <= gate, t
    with pytest.raises(ValueError):
        oracle.GDNReplay(workload.gdn_initial_state(seed, 1, 2, 16, 16), 1, 4, 1, oracle.READ_MXFP4)
