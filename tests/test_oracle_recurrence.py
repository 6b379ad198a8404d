"""Pins for the stepwise float64 oracle (O1) and the per-draft spec definition (O5).

Each test checks the oracle against something other than itself: numpy's outer product and
matrix-vector product, exact rational arithmetic, a closed-form special case, and the brute-force
dual form of the recurrence written in pure Python.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
import workload


def _rand_layer(rng, Bt, H, P, N, G):
    S = rng.standard_normal((Bt, H, P, N)).astype(np.float32)
    x = rng.standard_normal((Bt, H, P)).astype(np.float32)
    B = (rng.standard_normal((Bt, G, N)) / np.sqrt(N)).astype(np.float32)
    C = (rng.standard_normal((Bt, G, N)) / np.sqrt(N)).astype(np.float32)
    dt = np.logaddexp(0, rng.standard_normal((Bt, H)) - 1.0).astype(np.float32)
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    return S, x, B, C, dt, A, D


@pytest.mark.parametrize("shape", [(2, 4, 16, 16, 1), (3, 6, 5, 7, 3), (1, 8, 4, 12, 2)])
def test_single_step_matches_numpy_outer_and_matvec(shape):
    """One token of O1 equals numpy: S' = a*S + dt*outer(x, B); y = S' @ C + D*x, per head,
    with head h using group h // (H/G)."""
    Bt, H, P, N, G = shape
    rng = np.random.default_rng(11)
    S, x, B, C, dt, A, D = _rand_layer(rng, Bt, H, P, N, G)
    S64 = S.astype(np.float64)
    y = oracle.step(S64, x, B, C, dt, A, D)
    hpg = H // G
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            a = np.exp(np.float64(dt[b, h]) * np.float64(A[h]))
            ref_S = a * S[b, h].astype(np.float64) + np.float64(dt[b, h]) * np.outer(
                x[b, h].astype(np.float64), B[b, g].astype(np.float64))
            ref_y = ref_S @ C[b, g].astype(np.float64) + np.float64(D[h]) * x[b, h]
            np.testing.assert_allclose(S64[b, h], ref_S, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(y[b, h], ref_y, rtol=1e-12, atol=1e-12)


def test_exact_arithmetic_A0_matches_rationals():
    """With A = 0 (decay exactly 1), dt in {0.5, 1} and small integers, every value is exact:
    the oracle must equal exact rational arithmetic bit for bit."""
    rng = np.random.default_rng(5)
    Bt, H, P, N, G, steps = 2, 4, 3, 5, 2, 6
    S0 = rng.integers(-4, 5, (Bt, H, P, N)).astype(np.float32)
    xs = [rng.integers(-4, 5, (Bt, H, P)).astype(np.float32) for _ in range(steps)]
    Bs = [rng.integers(-4, 5, (Bt, G, N)).astype(np.float32) for _ in range(steps)]
    Cs = [rng.integers(-4, 5, (Bt, G, N)).astype(np.float32) for _ in range(steps)]
    dts = [rng.choice([0.5, 1.0], (Bt, H)).astype(np.float32) for _ in range(steps)]
    A = np.zeros(H, np.float32)
    D = rng.integers(-3, 4, H).astype(np.float32)
    exact_y, exact_S = brute.exact_stepwise_A0(S0.tolist(), [v.tolist() for v in xs],
                                               [v.tolist() for v in Bs], [v.tolist() for v in Cs],
                                               [v.tolist() for v in dts], D.tolist())
    S = S0.astype(np.float64)
    for t in range(steps):
        y = oracle.step(S, xs[t], Bs[t], Cs[t], dts[t], A, D)
        assert np.array_equal(y, np.array(exact_y[t], dtype=np.float64))
    assert np.array_equal(S, np.array(exact_S, dtype=np.float64))


def test_dt_zero_leaves_state_and_reads_it():
    """dt = 0: the decay is exp(0) = 1 and the input term vanishes, so the state is unchanged
    and y = S @ C + D*x exactly as numpy computes it from the untouched state."""
    rng = np.random.default_rng(7)
    S, x, B, C, dt, A, D = _rand_layer(rng, 2, 4, 8, 8, 2)
    dt[:] = 0.0
    S64 = S.astype(np.float64)
    y = oracle.step(S64, x, B, C, dt, A, D)
    assert np.array_equal(S64, S.astype(np.float64))
    for b in range(2):
        for h in range(4):
            ref = S[b, h].astype(np.float64) @ C[b, h // 2].astype(np.float64) + np.float64(
                D[h]) * x[b, h]
            np.testing.assert_allclose(y[b, h], ref, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("G", [1, 2])
def test_stepwise_matches_brute_force_dual_form(G):
    """O1 run for 10 tokens equals the stateless dual form evaluated in pure Python with fsum."""
    Bt, H, P, N, steps = 2, 4, 3, 4, 10
    seed = 99
    A, D = workload.layer_params(seed, H)
    S0 = workload.initial_state(seed, Bt, H, P, N)
    toks = [workload.step_inputs(seed, t, Bt, H, P, N, G) for t in range(steps)]
    # larger dt than the workload so that the decay terms matter
    toks = [(x, B, C, (dt * 20).astype(np.float32)) for x, B, C, dt in toks]
    ref = brute.dual_form(S0.tolist(), [t[0].tolist() for t in toks], [t[1].tolist() for t in toks],
                          [t[2].tolist() for t in toks], [t[3].tolist() for t in toks],
                          A.tolist(), D.tolist())
    S = S0.astype(np.float64)
    for t in range(steps):
        y = oracle.step(S, *toks[t], A, D)
        r = np.array(ref[t])
        assert np.max(np.abs(y - r)) <= 1e-12 * max(1.0, np.max(np.abs(r)))


def test_spec_stepwise_is_prefix_of_plain_steps():
    """O5: the T draft outputs equal T plain O1 steps, and the committed state equals the state
    after the accepted prefix (accepted = 0 leaves it unchanged)."""
    Bt, H, P, N, G, T = 3, 4, 8, 8, 2, 4
    seed = 3
    A, D = workload.layer_params(seed, H)
    S0 = workload.initial_state(seed, Bt, H, P, N).astype(np.float64)
    x, B, C, dt = workload.draft_inputs(seed, 0, Bt, T, H, P, N, G)
    acc = np.array([0, 2, 4], np.int32)
    S = S0.copy()
    y = oracle.spec_stepwise(S, T, x, B, C, dt, A, D, acc)
    for b in range(Bt):
        w = S0[b:b + 1].copy()
        for i in range(T):
            yi = oracle.step(w, x[b:b + 1, i], B[b:b + 1, i], C[b:b + 1, i], dt[b:b + 1, i], A, D)
            assert np.array_equal(yi[0], y[b, i])
            if i + 1 == acc[b]:
                assert np.array_equal(w[0], S[b])
        if acc[b] == 0:
            assert np.array_equal(S[b], S0[b])
    with pytest.raises(ValueError):
        oracle.spec_stepwise(S0.copy(), T, x, B, C, dt, A, D, np.array([0, 5, 1], np.int32))


def test_decay_sign_matters():
    """A plausible slip -- exp(-dt*A) instead of exp(dt*A) -- would grow the state; with
    A < 0, dt > 0 and x = 0 the state must shrink by exactly exp(dt*A) per element."""
    S = np.ones((1, 1, 2, 2), np.float64)
    x = np.zeros((1, 1, 2), np.float32)
    B = np.ones((1, 1, 2), np.float32)
    C = np.ones((1, 1, 2), np.float32)
    dt = np.array([[0.5]], np.float32)
    A = np.array([-2.0], np.float32)
    D = np.zeros(1, np.float32)
    y = oracle.step(S, x, B, C, dt, A, D)
    assert np.allclose(S, math.exp(-1.0), rtol=1e-15)
    assert np.allclose(y, 2 * math.exp(-1.0), rtol=1e-15)
