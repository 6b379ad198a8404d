"""Brute-force forms of the Mamba-2 decode recurrence for tiny shapes -- TEST INFRASTRUCTURE ONLY.

Pure Python loops, no numpy arithmetic, so these serve as pins for the float64 oracle:

* ``dual_form``: the recurrence unrolled from the initial state with no state at all. For token t
  of head h (group g), with every product and sum taken over all earlier tokens:
      y_t[p] = exp(A_h * sum_{i<=t} dt_i) * (S0[p,:] . C_t)
             + sum_{j<=t} dt_j * exp(A_h * sum_{j<i<=t} dt_i) * (B_j . C_t) * x_j[p]
             + D_h * x_t[p]
  This is what unrolling the update-then-read recurrence over a window gives ([AT Pulse]
  "Technical analysis" and [Clarity] claim ledger [17]: the recurrence expanded across a window).
  Sums use math.fsum (exactly rounded), exponentials math.exp.
* ``exact_stepwise_A0``: the stepwise recurrence in exact rational arithmetic for A = 0, where
  the decay is exactly 1 and every value is a small dyadic rational.

Pages: [AT Pulse] "NVIDIA and Princeton's ReplaySSM stores a checkpoint and recent inputs instead
of full SSM state to speed up hybrid-model decoding"; [Clarity] "NVIDIA and Princeton cache SSM
inputs in place of state to speed hybrid-model decoding".
"""
import math
from fractions import Fraction


def dual_form(S0, xs, Bs, Cs, dts, A, D):
    """S0[b][h][p][n]; xs[t][b][h][p]; Bs/Cs[t][b][g][n]; dts[t][b][h]; A[h]; D[h] (floats).
    Returns ys[t][b][h][p] as Python floats."""
    steps = len(xs)
    Bt, H, P, N = len(S0), len(S0[0]), len(S0[0][0]), len(S0[0][0][0])
    G = len(Bs[0][0])
    hpg = H // G
    ys = []
    for t in range(steps):
        yt = []
        for b in range(Bt):
            yb = []
            for h in range(H):
                g = h // hpg
                a = float(A[h])
                total = math.fsum(float(dts[i][b][h]) for i in range(t + 1))
                decay = math.exp(a * total)
                Ct = [float(v) for v in Cs[t][b][g]]
                weights = []
                for j in range(t + 1):
                    after = math.fsum(float(dts[i][b][h]) for i in range(j + 1, t + 1))
                    wj = float(dts[j][b][h]) * math.exp(a * after)
                    score = math.fsum(float(Bs[j][b][g][n]) * Ct[n] for n in range(N))
                    weights.append(wj * score)
                yh = []
                for p in range(P):
                    u = math.fsum(float(S0[b][h][p][n]) * Ct[n] for n in range(N))
                    terms = [decay * u]
                    terms += [weights[j] * float(xs[j][b][h][p]) for j in range(t + 1)]
                    terms.append(float(D[h]) * float(xs[t][b][h][p]))
                    yh.append(math.fsum(terms))
                yb.append(yh)
            yt.append(yb)
        ys.append(yt)
    return ys


def exact_stepwise_A0(S0, xs, Bs, Cs, dts, D):
    """Stepwise recurrence with A = 0 (decay exactly 1) in exact rationals.
    Returns (ys[t][b][h][p], final state) as Fractions."""
    Bt, H, P, N = len(S0), len(S0[0]), len(S0[0][0]), len(S0[0][0][0])
    G = len(Bs[0][0])
    hpg = H // G
    S = [[[[Fraction(float(S0[b][h][p][n])) for n in range(N)] for p in range(P)]
          for h in range(H)] for b in range(Bt)]
    ys = []
    for t in range(len(xs)):
        yt = []
        for b in range(Bt):
            yb = []
            for h in range(H):
                g = h // hpg
                dt = Fraction(float(dts[t][b][h]))
                yh = []
                for p in range(P):
                    xp = Fraction(float(xs[t][b][h][p]))
                    acc = Fraction(0)
                    for n in range(N):
                        S[b][h][p][n] = S[b][h][p][n] + dt * xp * Fraction(float(Bs[t][b][g][n]))
                        acc += S[b][h][p][n] * Fraction(float(Cs[t][b][g][n]))
                    yh.append(acc + Fraction(float(D[h])) * xp)
                yb.append(yh)
            yt.append(yb)
        ys.append(yt)
    return ys, S
