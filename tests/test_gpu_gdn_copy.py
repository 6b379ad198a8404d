"""GPU parity of the Gated DeltaNet path with a read copy (gdnreplay.h, read_prec bf16 / fp8 /
MXFP4) against the oracle's replay model with the same copy (reading G4) and the stepwise truth.

Bars: the copy after load equal, bit for bit, to the format's encoding of the initial state (bf16:
torch's bfloat16 rounding; fp8: the oracle's per-64-row encoder, scales included; MXFP4: the
oracle's MX encoder, scale bytes included); every replayed output within 1e-5 of the oracle's copy
model: after each flush the model continues from the GPU's own fp32 checkpoint, whose encoding must
be the GPU's copy bit for bit; flush steps (read from the folded fp32 checkpoint) and checkpoints
within 1e-5 of the truth; replayed outputs within a fixed gate of the truth (bf16 2e-2, fp8 6e-2,
MXFP4 0.3 -- the float64 model with the same copy itself reaches 0.26 on the tiny layer, whose
rows are a single MX block); pointers bit-exact. The serving shape compares every sequence.
"""
import numpy as np
import pytest
import torch

import hybrid_mamba_decode_amd as rs
import oracle
import workload
from gpu_harness import PREC_CODE, dev, host, log, rel

pytestmark = pytest.mark.gpu

TOL = 1e-5
GATE = {"bf16": 2e-2, "fp8": 6e-2, "mxfp4": 0.3}
PRECS = ["bf16", "fp8", "mxfp4"]


def _bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).bfloat16().view(torch.int16).numpy()


def _assert_copy(lay, prec, m, rows, what):
    """The GPU's copy of the sequences in rows is, bit for bit, the format's encoding of the fp32
    checkpoint values m[rows] (scales too)."""
    rows = np.asarray(rows)
    idx = torch.as_tensor(rows, device="cuda")
    got = host(lay.read_copy()[idx])
    mm = np.ascontiguousarray(m[rows], np.float32)
    if prec == "bf16":
        assert np.array_equal(got, _bf16_bits(mm)), f"{what}: bf16 copy"
        return
    if prec == "fp8":
        codes, scales = oracle.e4m3_encode_rows(mm)
    else:
        codes, scales = oracle.mxfp4_encode(mm)
    assert np.array_equal(host(lay.scales()[idx]), scales), f"{what}: {prec} scales"
    assert np.array_equal(got, codes), f"{what}: {prec} codes"


def _check_outputs(o, o_model, o_true, flush_step, prec, what):
    if flush_step:
        assert rel(o, o_true) <= TOL, f"{what}: flush step vs truth {rel(o, o_true):.2e}"
        return
    e_model = rel(o, o_model)
    assert e_model <= TOL, f"{what}: vs copy model {e_model:.2e}"
    assert rel(o, o_true) <= GATE[prec], f"{what}: vs truth {rel(o, o_true):.2e} > {GATE[prec]:.2e}"


def _run(prec, Bt, H, G, Dv, Dk, L, seed, steps, sample, lockstep=True):
    log(f"[gdn {prec}] Bt={Bt} H={H} G={G} Dv={Dv} Dk={Dk} L={L} steps={steps} sample={len(sample)} seqs "
        f"lockstep={lockstep}")
    S0 = workload.gdn_initial_state(seed, Bt, H, Dv, Dk)
    lay = rs.GDNReplay(Bt, H, G, Dv, Dk, buffer_len=L, read_prec=prec)
    lay.set_lockstep(lockstep)
    lay.load_state(dev(S0))
    _assert_copy(lay, prec, S0, range(Bt), "load")
    sample = np.asarray(sample)
    model = oracle.GDNReplay(S0[sample], G, L, 1, PREC_CODE[prec])
    S = S0[sample].astype(np.float64)
    for t in range(steps):
        ins = workload.gdn_step_inputs(seed, t, Bt, H, G, Dv, Dk)
        o = host(lay.step(*(dev(a) for a in ins)))[sample]
        sub = [a[sample] for a in ins]
        o_true = oracle.gdn_step(S, *sub)
        o_model = model.step(*sub)
        flush_step = (t + 1) % L == 0
        _check_outputs(o, o_model, o_true, flush_step, prec, f"step {t}")
        pos, ck = lay.get_pointers()
        assert pos == [t + 1] * Bt and ck == [(t + 1) // L * L] * Bt
        if flush_step:
            m = host(lay.master())
            assert rel(m[sample], S) <= TOL, f"step {t}: checkpoint"
            _assert_copy(lay, prec, m, range(Bt), f"step {t}: copy of the checkpoint")
            model.set_checkpoint(m[sample])
    assert rel(host(lay.materialize_state())[sample], S) <= TOL
    assert lay.check() == rs.RSSM_OK


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("lockstep", [True, False])
def test_gdn_copy_tiny(prec, lockstep):
    c = workload.GDN_TINY
    _run(prec, c["Bt"], c["H"], c["G"], c["Dv"], c["Dk"], c["L"], workload.config_seed(5), 40, range(c["Bt"]),
         lockstep)


@pytest.mark.parametrize("prec", PRECS)
def test_gdn_copy_serving(prec):
    """Serving GDN layer (batch 256, 32 x 16 heads of 128, L 16): 48 steps, every sequence."""
    c = workload.GDN_SERVING
    _run(prec, c["Bt"], c["H"], c["G"], c["Dv"], c["Dk"], c["L"], workload.config_seed(6), 48, range(c["Bt"]))


@pytest.mark.parametrize("shape", [
    (3, 4, 2, 100, 32, 7, True),     # one ragged 128-row tile
    (2, 2, 1, 32, 256, 5, True),     # Dk 256: 64-row tiles
    (2, 4, 2, 64, 128, 1, True),     # L 1: every step flushes
    (3, 4, 2, 200, 64, 20, False),   # two 128-row tiles (128 + 72), L 32 bucket, device pointers
    (2, 2, 2, 256, 16, 9, True),     # Dk 16, two full 128-row tiles
    (2, 2, 1, 128, 128, 40, False),  # L 64 bucket: 64-row tiles
])
@pytest.mark.parametrize("prec", PRECS)
def test_gdn_copy_shapes(prec, shape):
    """Replayed steps with 128-row copy tiles (Dk <= 128, L <= 32) and with 64-row tiles."""
    Bt, H, G, Dv, Dk, L, lockstep = shape
    if prec == "mxfp4" and Dk < 32:
        pytest.skip("MXFP4 blocks are 32 key columns: Dk 16 is rejected (tested on the CPU)")
    _run(prec, Bt, H, G, Dv, Dk, L, 141, 2 * L + 3, range(Bt), lockstep)


@pytest.mark.parametrize("T,L,Dv,Dk", [
    (3, 7, 32, 64),      # one ragged 128-row tile
    (4, 16, 32, 64),
    (8, 16, 200, 128),   # two 128-row tiles (128 + 72), the widest draft bucket
    (2, 32, 128, 32),    # L 32 bucket
    (4, 40, 64, 128),    # L 64 bucket: 64-row tiles
])
@pytest.mark.parametrize("prec", PRECS)
def test_gdn_copy_spec(prec, T, L, Dv, Dk):
    """Verify + rollback through the copy (128-row tiles for Dk <= 128 and L <= 32, 64-row tiles
    otherwise); the commit-time flushes refresh it."""
    Bt, H, G, seed = 3, 4, 2, 151
    S0 = workload.gdn_initial_state(seed, Bt, H, Dv, Dk)
    lay = rs.GDNReplay(Bt, H, G, Dv, Dk, buffer_len=L, max_draft=T, read_prec=prec)
    lay.load_state(dev(S0))
    model = oracle.GDNReplay(S0, G, L, T, PREC_CODE[prec])
    S = S0.astype(np.float64)
    rng = np.random.default_rng(seed)
    flushed = False
    for it in range(24 if L <= 16 else 2 * L + 8):  # long enough for a commit-time flush
        drafts = workload.gdn_draft_inputs(seed, it, Bt, T, H, G, Dv, Dk)
        acc = rng.integers(0, T + 1, Bt).astype(np.int32)
        o = host(lay.spec_verify(*(dev(a) for a in drafts)))
        lay.rollback(dev(acc))
        ck_before = model.pointers()[1].copy()
        o_model = model.verify(T, *drafts)
        model.rollback(acc)
        o_true = oracle.gdn_spec_stepwise(S, T, *drafts, acc)
        _check_outputs(o, o_model, o_true, False, prec, f"verify {it}")
        pos, ck = lay.get_pointers()
        assert pos == list(model.pointers()[0]) and ck == list(model.pointers()[1])
        moved = np.nonzero(model.pointers()[1] != ck_before)[0]
        if moved.size:
            flushed = True
            m = host(lay.master())
            assert rel(m[moved], S[moved]) <= TOL, f"verify {it}: committed checkpoint"
            _assert_copy(lay, prec, m, moved, f"verify {it}: copy")
            model.set_checkpoint(m)
        assert rel(host(lay.materialize_state()), S) <= TOL
    assert flushed
    _assert_copy(lay, prec, host(lay.master()), range(Bt), "end")
    assert lay.check() == rs.RSSM_OK
