"""Pins for the oracle's Mamba-2 mixer edges (oracle_mixer.c, reading M1): SiLU and softplus
against their closed forms and library routines, the causal conv1d against numpy.convolve over the
whole token sequence, the channel split, the streaming history, a whole mixer step against an
independent numpy composition, and the replay-form mixer (with rollback of the conv history)
against the stepwise one.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import workload


def _rel(a, ref):
    return float(np.max(np.abs(np.asarray(a, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def test_silu_softplus_closed_forms():
    v = np.concatenate([np.linspace(-50, 50, 2001), [-800.0, -40.0, 0.0, 1e-12, 40.0, 800.0]])
    silu = np.array([oracle.silu(x) for x in v])
    assert np.allclose(silu, v * expit(v), rtol=1e-15, atol=1e-300)
    assert oracle.silu(0.0) == 0.0 and oracle.silu(800.0) == 800.0 and oracle.silu(-800.0) == 0.0
    sp = np.array([oracle.softplus(x) for x in v])
    assert np.allclose(sp, np.logaddexp(0.0, v), rtol=1e-15, atol=1e-300)
    assert oracle.softplus(0.0) == np.log(2.0) and oracle.softplus(800.0) == 800.0


def _conv_reference(hist0, raw, w, b):
    """u_t over a whole sequence by numpy.convolve per channel: the history rows precede the
    tokens; u_t[c] = b[c] + sum_i w[c,i] seq[t+i][c] over the K-window ending at token t."""
    K = w.shape[1]
    seq = np.concatenate([hist0, raw], axis=0).astype(np.float64)     # [(K-1)+T, CD]
    T = raw.shape[0]
    u = np.empty((T, seq.shape[1]))
    for c in range(seq.shape[1]):
        full = np.convolve(seq[:, c], w[c, ::-1].astype(np.float64))  # full[m] = sum_i w[i] seq[m-K+1+i]
        u[:, c] = full[np.arange(T) + K - 1] + float(b[c])
    return u


@pytest.mark.parametrize("K", [2, 3, 4])
def test_conv_matches_numpy_convolve_and_streams(K):
    """Token by token through the oracle's history equals one convolution over the concatenated
    sequence (history first), then SiLU and the x / B / C split; dt is softplus(dt_raw + bias)."""
    H, P, G, N, T, seed = 3, 4, 1, 8, 9, 5
    CD = workload.mixer_conv_dim(H, P, G, N)
    w, b, bias = workload.mixer_params(seed, H, P, G, N, K)
    hist = workload.mixer_history(seed, 1, K, CD)
    h0 = hist[0].copy()
    raws, outs = [], []
    for t in range(T):
        xbc, _, dt_raw = workload.mixer_step_inputs(seed, t, 1, H, P, G, N)
        x, B, C, dt = oracle.mixer_edge(hist, xbc, dt_raw, w, b, bias, H, P, G, N)
        raws.append(xbc[0])
        outs.append(np.concatenate([x.reshape(-1), B.reshape(-1), C.reshape(-1)]))
        want_dt = np.logaddexp(0.0, dt_raw[0].astype(np.float64) + bias)
        assert np.allclose(dt[0], want_dt, rtol=2 ** -23, atol=0)
    u = _conv_reference(h0, np.array(raws), w, b)
    ref = u * expit(u)
    got = np.array(outs, np.float64)
    assert np.allclose(got, ref, rtol=2 ** -23, atol=1e-30)     # one fp32 rounding (reading M2)
    # the history now holds the last K-1 raw tokens, oldest first
    assert np.array_equal(hist[0], np.array(raws[-(K - 1):]))


def test_channel_split_and_tap_order():
    """Identity conv (weight 1 on the newest tap) gives silu of this token's channels, split as
    x (head-major), B, C; weight 1 on the oldest tap reads the token K-1 back."""
    H, P, G, N, K = 2, 3, 2, 4, 4
    CD = workload.mixer_conv_dim(H, P, G, N)
    raw = np.arange(CD, dtype=np.float32)[None] / CD - 0.5
    hist = np.stack([np.full((1, CD), float(i + 1), np.float32) for i in range(K - 1)], axis=1)   # oldest = 1
    for tap, expect in ((K - 1, raw[0].astype(np.float64)), (0, np.full(CD, 1.0))):
        w = np.zeros((CD, K), np.float32)
        w[:, tap] = 1.0
        h = hist.copy()
        x, B, C, _ = oracle.mixer_edge(h, raw, np.zeros((1, H), np.float32), w, np.zeros(CD, np.float32),
                                       np.zeros(H, np.float32), H, P, G, N)
        s = (expect * expit(expect)).astype(np.float32)
        assert np.array_equal(x[0].reshape(-1), s[:H * P])
        assert np.array_equal(B[0].reshape(-1), s[H * P:H * P + G * N])
        assert np.array_equal(C[0].reshape(-1), s[H * P + G * N:])


def _numpy_mixer_step(S, hist, xbc, z, dt_raw, A, D, w, b, bias, H, P, G, N):
    """Independent composition: conv window as an explicit product, SSM by numpy outer products,
    gate by expit. S float64 and hist float64 updated in place."""
    K = w.shape[1]
    win = np.concatenate([hist, xbc[:, None, :].astype(np.float64)], axis=1)   # [Bt, K, CD]
    u = np.einsum("bkc,ck->bc", win, w.astype(np.float64)) + b
    v = u * expit(u)
    hist[:] = win[:, 1:]
    Bt = S.shape[0]
    x = v[:, :H * P].reshape(Bt, H, P)
    Bm = v[:, H * P:H * P + G * N].reshape(Bt, G, N)
    Cm = v[:, H * P + G * N:].reshape(Bt, G, N)
    dt = np.logaddexp(0.0, dt_raw.astype(np.float64) + bias)
    y = np.empty((Bt, H, P))
    for bb in range(Bt):
        for h in range(H):
            g = h // (H // G)
            a = np.exp(dt[bb, h] * float(A[h]))
            S[bb, h] = a * S[bb, h] + dt[bb, h] * np.outer(x[bb, h], Bm[bb, g])
            y[bb, h] = S[bb, h] @ Cm[bb, g] + float(D[h]) * x[bb, h]
    return y * z * expit(z.astype(np.float64))


def test_mixer_step_vs_numpy_composition():
    c = workload.MIXER_TINY
    Bt, H, P, N, G, K = c["Bt"], c["H"], c["P"], c["N"], c["G"], c["K"]
    seed = 7
    CD = workload.mixer_conv_dim(H, P, G, N)
    A, D = workload.layer_params(seed, H)
    w, b, bias = workload.mixer_params(seed, H, P, G, N, K)
    S0 = workload.initial_state(seed, Bt, H, P, N)
    h0 = workload.mixer_history(seed, Bt, K, CD)
    mix = oracle.MixerStepwise(S0, h0, A, D, w, b, bias, G)
    S, hist = S0.astype(np.float64), h0.astype(np.float64)
    for t in range(12):
        xbc, z, dt_raw = workload.mixer_step_inputs(seed, t, Bt, H, P, G, N)
        o = mix.step(xbc, z, dt_raw)
        o_ref = _numpy_mixer_step(S, hist, xbc, z, dt_raw, A, D, w, b, bias, H, P, G, N)
        # the oracle hands the SSM fp32 edge values (reading M2): a few fp32 roundings apart
        assert _rel(o, o_ref) <= 1e-6, t
    assert _rel(mix.S, S) <= 1e-6


@pytest.mark.parametrize("T,L", [(1, 4), (3, 7)])
def test_mixer_replay_vs_stepwise_with_rollback(T, L):
    """Replay-form mixer equals the stepwise mixer: standard steps, and verify + rollback where
    the conv history is cut back with the records (accepted counts 0..T)."""
    c = workload.MIXER_TINY
    Bt, H, P, N, G, K = c["Bt"], c["H"], c["P"], c["N"], c["G"], c["K"]
    seed = 9
    CD = workload.mixer_conv_dim(H, P, G, N)
    A, D = workload.layer_params(seed, H)
    w, b, bias = workload.mixer_params(seed, H, P, G, N, K)
    S0 = workload.initial_state(seed, Bt, H, P, N)
    h0 = workload.mixer_history(seed, Bt, K, CD)
    rep = oracle.MixerReplay(S0, h0, A, D, w, b, bias, G, L, T)
    ref = oracle.MixerStepwise(S0, h0, A, D, w, b, bias, G)
    for it in range(16):
        if T > 1 and it % 2:
            xbc, z, dt_raw = workload.mixer_draft_inputs(seed, it, Bt, T, H, P, G, N)
            acc = workload.accepted_counts(seed, it, Bt, T)
            o = rep.verify(T, xbc, z, dt_raw)
            rep.rollback(acc)
            o_ref = ref.spec(T, xbc, z, dt_raw, acc)
        else:
            xbc, z, dt_raw = workload.mixer_step_inputs(seed, it, Bt, H, P, G, N)
            o, o_ref = rep.step(xbc, z, dt_raw), ref.step(xbc, z, dt_raw)
        assert _rel(o, o_ref) <= 1e-12, it
        assert np.array_equal(rep.hist, ref.hist)
        assert _rel(rep.materialize(), ref.S) <= 1e-12


def test_rollback_history_equals_fresh_run_on_accepted_tokens():
    """After verify + rollback(acc) the conv history is that of a fresh run over the committed
    tokens only: the drafts beyond the accepted prefix leave no trace."""
    c = workload.MIXER_TINY
    Bt, H, P, N, G, K = c["Bt"], c["H"], c["P"], c["N"], c["G"], c["K"]
    seed, T = 11, 4
    CD = workload.mixer_conv_dim(H, P, G, N)
    A, D = workload.layer_params(seed, H)
    w, b, bias = workload.mixer_params(seed, H, P, G, N, K)
    S0 = workload.initial_state(seed, Bt, H, P, N)
    h0 = workload.mixer_history(seed, Bt, K, CD)
    rep = oracle.MixerReplay(S0, h0, A, D, w, b, bias, G, 16, T)
    xbc, z, dt_raw = workload.mixer_draft_inputs(seed, 0, Bt, T, H, P, G, N)
    acc = np.array([1, 3], np.int32)
    rep.verify(T, xbc, z, dt_raw)
    rep.rollback(acc)
    for bb in range(Bt):
        seq = np.concatenate([h0[bb], xbc[bb, :acc[bb]]], axis=0)
        assert np.array_equal(rep.hist[bb], seq[-(K - 1):])
