"""GPU parity at the sweep workload's shapes: the serving head shape (128 heads, P 64, N 128,
8 groups) across buffer lengths 4, 8 and 32 and batches 8, 64 and 512, and a stack of independent
layers stepped token by token as the sweep benchmark runs them.

Bars as for the standard path: pointers and flush schedule bit-exact, fp32 outputs and
checkpoints within 1e-5 normwise relative error of the float64 oracle, which computes a sample of
sequences one by one (sequences and layers are independent).
"""
import numpy as np
import pytest

import hybrid_mamba_decode_amd as rs
import oracle
import workload
from gpu_harness import Case, dev, host, log, rel
from test_gpu_replay import TOL_F32, _run_replay

pytestmark = pytest.mark.gpu

SW = workload.SWEEP


@pytest.mark.parametrize("Bt,L", [(8, 4), (8, 8), (8, 32), (64, 16), (512, 4)])
def test_sweep_shapes(Bt, L):
    """Two whole windows plus three steps; sequences 0 and Bt-1 against the oracle."""
    case = Case(Bt, SW["H"], SW["P"], SW["N"], SW["G"], L, workload.config_seed(4) + L)
    _run_replay(case, 2 * L + 3, [0, Bt - 1], check_state_every=L)


def test_stacked_layers_are_independent():
    """Three layers (distinct parameters, states and inputs) stepped in turn for each token, as in
    the sweep's stack: every layer's outputs, pointers and post-flush checkpoint match its own
    oracle run."""
    Bt, L, steps, sample = 8, 8, 19, [1, 6]
    cases = [Case(Bt, SW["H"], SW["P"], SW["N"], SW["G"], L, workload.config_seed(4) + 100 + i)
             for i in range(3)]
    lays = [c.layer("fp32", True, 1) for c in cases]
    truth = [c.S0[sample].astype(np.float64) for c in cases]
    log(f"[stack] Bt={Bt} L={L} layers={len(cases)} steps={steps}")
    for t in range(steps):
        for i, (c, lay) in enumerate(zip(cases, lays)):
            x, B, C, dt = c.step_inputs(t)
            y = lay.step(dev(x), dev(B), dev(C), dev(dt))
            y_ref = oracle.step(truth[i], x[sample], B[sample], C[sample], dt[sample], c.A, c.D)
            e = rel(host(y)[sample], y_ref)
            assert e <= TOL_F32, f"layer {i} step {t}: output error {e:.3e}"
            pos, ck = lay.get_pointers()
            assert pos == [t + 1] * Bt and ck == [(t + 1) // L * L] * Bt
            if (t + 1) % L == 0:
                m = host(lay.master())[sample]
                assert rel(m, truth[i]) <= TOL_F32, f"layer {i} step {t}: checkpoint error"
    for lay in lays:
        assert lay.check() == rs.RSSM_OK
