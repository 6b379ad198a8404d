"""GPU parity of the standard decode path (replay + append, fused flush, explicit flush,
materialize, the conventional baseline) against the float64 oracle.

Bars:
* pointers and flush schedule bit-exact for every sequence after every step;
* fp32 outputs, post-flush checkpoints and materialized states within 1e-5 normwise relative
  error (max |diff| / max |ref| over the compared tensor) of the stepwise float64 truth;
* every output, of every step, within 1e-5 of the oracle's replay-form model with the same read
  copy. At load both sides encode the same fp32 state. After each flush the model continues from
  the GPU's own fp32 master, and the GPU's read copy (and its scales) must then be, bit for bit,
  the oracle's encoder applied to that master: the copy the layer reads is exactly the one the
  format definition gives, and the replayed outputs are exactly what that copy implies;
* against the stepwise truth the bf16 read copy within 2e-2, fp8 e4m3 within 6e-2 and MXFP4
  within 0.25 on non-flush outputs (each about 2.2x the format's rms relative rounding error);
  flush-step outputs, read from the fresh fp32 state, within 1e-5 in every mode;
* read-copy bytes at load bit-exact with the oracle's encoder, including crafted tiles.
The serving-size tests compare the whole batch; the oracle runs every sequence.
"""
import numpy as np
import pytest
import torch

import hybrid_mamba_decode_amd as rs
import oracle
import workload
from gpu_harness import PREC_CODE, Case, assert_copy_encodes, dev, host, log, rel

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TOL_FP8 = 6e-2
TOL_FP4 = 0.25


def _run_replay(case, steps, sample, read_prec="fp32", store_C=True, Tmax=1, check_state_every=1,
                tol=TOL_F32):
    """Run `steps` standard decode steps on the GPU (whole batch) and the oracle (the sequences in
    `sample`); compare outputs, pointers, checkpoints, read copies and the materialized state.
    Returns the output-error curves against the truth (non-flush steps, flush steps) and the
    largest error against the same-copy model."""
    log(f"[replay] Bt={case.Bt} H={case.H} P={case.P} N={case.N} G={case.G} L={case.L} "
        f"Tmax={Tmax} prec={read_prec} steps={steps} sample={len(sample)} seqs")
    lay = case.layer(read_prec, store_C, Tmax)
    sample = np.asarray(sample)
    S = case.S0[sample].astype(np.float64)                 # O1 truth
    # the replay form with the same read copy: pointer machine and dual-precision model (O3, O4)
    rep = oracle.Replay(case.S0[sample], case.A, case.D, case.G, case.L, Tmax, PREC_CODE[read_prec])
    period = case.L - Tmax + 1
    errs, flush_errs, worst_dual = [], [], 0.0
    for t in range(steps):
        x, B, C, dt = case.step_inputs(t)
        y = lay.step(dev(x), dev(B), dev(C), dev(dt))
        y_ref = oracle.step(S, x[sample], B[sample], C[sample], dt[sample], case.A, case.D)
        y_rep = rep.step(x[sample], B[sample], C[sample], dt[sample])
        yh = host(y)[sample]
        e = rel(yh, y_ref)
        e_dual = rel(yh, y_rep)
        worst_dual = max(worst_dual, e_dual)
        assert e_dual <= TOL_F32, f"step {t}: error vs the same-copy replay model {e_dual:.3e}"
        flush_step = (t + 1) % period == 0
        (flush_errs if flush_step else errs).append(e)
        bound = TOL_F32 if flush_step else tol
        assert e <= bound, f"step {t}: output error {e:.3e} > {bound}"
        pos, ck = lay.get_pointers()
        opos, ock = rep.pointers()
        assert pos == [t + 1] * case.Bt
        assert ck == [int(ock[0])] * case.Bt and list(opos) == [t + 1] * len(sample)
        assert (t + 1 - ck[0]) == (t + 1) % period
        if check_state_every and (t % check_state_every == 0 or flush_step):
            st = host(lay.materialize_state())[sample]
            assert rel(st, S) <= TOL_F32, f"step {t}: state error {rel(st, S):.3e}"
        if flush_step:
            m = host(lay.master())[sample]
            assert rel(m, S) <= TOL_F32, f"step {t}: post-flush checkpoint error {rel(m, S):.3e}"
            if read_prec != "fp32":
                assert_copy_encodes(lay, read_prec, m, sample, f"step {t}")
            rep.set_checkpoint(m)
    assert lay.check() == rs.RSSM_OK
    log(f"  worst error vs the same-copy model {worst_dual:.2e}")
    return errs, flush_errs


def test_tiny_layer_fp32():
    """Tiny layer: batch 2, 4 heads, P=N=16, 1 group, L=4, 64 steps (16 flushes)."""
    c = workload.TINY
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(0))
    _run_replay(case, c["steps"], range(c["Bt"]))


@pytest.mark.parametrize("prec,tol,N", [("bf16", TOL_BF16, 16), ("fp8", TOL_FP8, 16), ("mxfp4", TOL_FP4, 32)])
def test_tiny_layer_dual_precision(prec, tol, N):
    """Tiny layer with each read copy (MXFP4 blocks need N >= 32)."""
    c = workload.TINY
    case = Case(c["Bt"], c["H"], c["P"], N, c["G"], c["L"], workload.config_seed(0))
    _run_replay(case, c["steps"], range(c["Bt"]), read_prec=prec, tol=tol)


def test_serving_layer_fp32():
    """Serving-size layer: batch 256, 128 heads, P=64, N=128, 8 groups, L=16, 64 steps
    (4 flushes), in the launch configuration the benchmark times; every sequence compared."""
    c = workload.SERVING
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(1))
    errs, ferrs = _run_replay(case, c["steps"], range(c["Bt"]), check_state_every=16)
    log(f"serving fp32: max non-flush err {max(errs):.2e}, max flush-step err {max(ferrs):.2e}")
    assert len(ferrs) == 4


@pytest.mark.parametrize("prec,tol", [("bf16", TOL_BF16), ("fp8", TOL_FP8), ("mxfp4", TOL_FP4)])
def test_serving_dual_precision(prec, tol):
    """Dual-precision checkpoint at serving size, 256 steps (16 flushes), every sequence: outputs
    within 1e-5 of the same-copy model continued from the GPU's master after each flush, the copy
    bit-exact after each flush, non-flush outputs within the read-copy gate of the truth and
    flush-step outputs (read from the fresh fp32 state) within the fp32 bar."""
    c = workload.DUAL_PRECISION
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(2))
    errs, ferrs = _run_replay(case, c["steps"], range(c["Bt"]), read_prec=prec, tol=tol, check_state_every=64)
    log(f"serving {prec}: max non-flush err {max(errs):.3e} (first window {max(errs[:15]):.3e}, "
        f"last {max(errs[-15:]):.3e}); max flush-step err {max(ferrs):.2e}")
    assert len(ferrs) == 16


@pytest.mark.parametrize("prec", ["bf16", "fp8", "mxfp4"])
def test_read_copy_bytes_bit_exact(prec):
    """The read copy written at load is bit-identical to the oracle's encoder applied to the same
    fp32 state, over the whole serving-size batch; fp8 scales too. A second state sweeps values
    across many binades, zero tiles, ties and saturation."""
    c = workload.SERVING
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(2))
    lay = case.layer(prec)
    got = host(lay.read_copy())
    if prec == "bf16":
        exp = oracle.bf16_encode(case.S0).view(np.int16)
        assert np.array_equal(got, exp)
    elif prec == "fp8":
        codes, scales = oracle.e4m3_encode_rows(case.S0)
        assert np.array_equal(got, codes)
        assert np.array_equal(host(lay.scales()), scales)
    else:
        codes, scales = oracle.mxfp4_encode(case.S0)
        assert np.array_equal(got, codes)
        assert np.array_equal(host(lay.scales()), scales)
    # crafted values: per-tile amax spread over 2^-40 .. 2^40, random fp32 mantissas, exact ties
    rng = np.random.default_rng(77)
    Bt, H, P, N = 8, c["H"], c["P"], c["N"]
    mant = rng.integers(0, 1 << 23, size=(Bt, H, P, N), dtype=np.uint32)
    expo = rng.integers(87, 168, size=(Bt, H, P, N), dtype=np.uint32)
    sign = rng.integers(0, 2, size=(Bt, H, P, N), dtype=np.uint32)
    S = ((sign << 31) | (expo << 23) | mant).view(np.float32).copy()
    S[0, 0] = 0.0                                  # all-zero tile: scale 1
    S[0, 1, :, :] = np.float32(1.0 + 2 ** -8)      # bf16 tie -> even
    S[0, 2] *= np.float32(1e-30)                   # tiny tile
    S[1, 3, 0, 0] = np.float32(448.0)              # scale exactly 1 where it is the amax
    S[1, 3, 1:] = np.linspace(-448, 448, (P - 1) * N, dtype=np.float32).reshape(P - 1, N)
    if prec == "mxfp4":
        # blocks of 32 along n: denormal-range blocks, a block holding one denormal next to
        # normal values, ties of the element rounding at scale 1, saturation, signed zeros
        S[2, 0, 0, :32] = np.ldexp(np.arange(1, 33, dtype=np.float64), -140).astype(np.float32)
        S[2, 0, 1, :32] = np.float32(2.0 ** -127)
        S[2, 0, 2, :32] = 0.0
        S[2, 0, 2, 5] = np.float32(-1e-45)
        S[2, 0, 3, :32] = np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 7.99, -0.25,
                                    -0.75, -5.0, -0.1, -0.0, 0.0] * 2, np.float32)
        S[2, 0, 4, :32] = np.float32(2.0 ** 127) * np.linspace(-1.9, 1.9, 32).astype(np.float32)
        S[2, 0, 5, :32] = np.float32(2.0 ** -126) * np.linspace(-1, 1, 32).astype(np.float32)
    small = Case(Bt, H, P, N, c["G"], c["L"], 5)
    small.S0 = S
    lay2 = small.layer(prec)
    got = host(lay2.read_copy())
    if prec == "bf16":
        assert np.array_equal(got, oracle.bf16_encode(S).view(np.int16))
    elif prec == "mxfp4":
        codes, scales = oracle.mxfp4_encode(S)
        assert np.array_equal(host(lay2.scales()), scales)
        assert np.array_equal(got, codes)
    else:
        codes, scales = oracle.e4m3_encode_rows(S)
        assert np.array_equal(host(lay2.scales()), scales)
        assert np.array_equal(got, codes)


@pytest.mark.parametrize("shape", [
    dict(Bt=1, H=6, P=20, N=32, G=3, L=5),      # ragged rows in one work-group, 6 blocks
    dict(Bt=3, H=5, P=100, N=64, G=1, L=7),     # P split over 2 work-groups, ragged tail
    dict(Bt=2, H=4, P=64, N=256, G=2, L=32),    # largest N, window bucket 32
    dict(Bt=2, H=8, P=8, N=16, G=4, L=64),      # window bucket 64
    dict(Bt=4, H=16, P=64, N=128, G=2, L=1),    # every step flushes
    dict(Bt=1, H=128, P=64, N=128, G=8, L=16),  # batch 1 at the serving head shape
    dict(Bt=2, H=2, P=256, N=256, G=1, L=64),   # maximum sizes: P 256 (4 row splits), N 256, L 64
])
def test_shapes_fp32(shape):
    case = Case(shape["Bt"], shape["H"], shape["P"], shape["N"], shape["G"], shape["L"], 123)
    _run_replay(case, 2 * shape["L"] + 3, range(shape["Bt"]), check_state_every=4)


@pytest.mark.parametrize("prec,tol", [("bf16", TOL_BF16), ("fp8", TOL_FP8), ("mxfp4", TOL_FP4)])
def test_shapes_dual_precision(prec, tol):
    case = Case(3, 6, 24, 64, 2, 6, 321)
    _run_replay(case, 20, range(3), read_prec=prec, tol=tol)


@pytest.mark.parametrize("shape", [
    dict(Bt=2, H=4, P=100, N=32, G=2, L=5),     # P split over 2 work-groups (no per-head scale)
    dict(Bt=2, H=8, P=64, N=256, G=2, L=32),    # largest N: 8 blocks per row, window bucket 32
    dict(Bt=1, H=4, P=12, N=128, G=1, L=64),    # ragged rows, window bucket 64
])
def test_shapes_mxfp4(shape):
    case = Case(shape["Bt"], shape["H"], shape["P"], shape["N"], shape["G"], shape["L"], 77)
    _run_replay(case, shape["L"] + 4, range(shape["Bt"]), read_prec="mxfp4", tol=TOL_FP4)


@pytest.mark.parametrize("shape", [
    dict(Bt=3, H=5, P=100, N=64, G=1, L=7),     # two scale blocks, the second ragged (36 rows)
    dict(Bt=2, H=4, P=128, N=128, G=2, L=16),   # two full blocks
    dict(Bt=2, H=2, P=256, N=32, G=1, L=5),     # four blocks
])
def test_shapes_fp8_blocks_of_64_rows(shape):
    """fp8 copies with P > 64 (one scale per 64-row block): the copy written at load bit-exact
    with the oracle's per-block encoder, scales [Bt,H,ceil(P/64)] included; then the replay run,
    whose same-copy checks re-encode the GPU's master after every flush."""
    case = Case(shape["Bt"], shape["H"], shape["P"], shape["N"], shape["G"], shape["L"], 88)
    lay = case.layer("fp8")
    assert tuple(lay.scales().shape) == (case.Bt, case.H, (case.P + 63) // 64)
    assert_copy_encodes(lay, "fp8", case.S0, range(case.Bt), "load")
    _run_replay(case, 2 * shape["L"] + 3, range(shape["Bt"]), read_prec="fp8", tol=TOL_FP8, check_state_every=4)


def test_spec_handle_standard_steps_and_no_C():
    """A handle with max_draft 3 flushes when more than L - 3 records are pending; records
    without C behave identically."""
    case = Case(2, 4, 16, 32, 2, 8, 9)
    _run_replay(case, 20, range(2), Tmax=3, store_C=False)


def test_exact_arithmetic_bit_identical():
    """A = 0, dt in {0.5, 1}, small-integer state and inputs: every intermediate is exact in
    fp32, so replay outputs, flushed checkpoints and the conventional step equal the oracle
    bit for bit, at the serving head shape."""
    Bt, H, P, N, G, L = 2, 16, 64, 128, 2, 16
    rng = np.random.default_rng(2024)
    S0 = rng.integers(-4, 5, (Bt, H, P, N)).astype(np.float32)
    A = np.zeros(H, np.float32)
    D = rng.integers(-3, 4, H).astype(np.float32)
    lay = rs.ReplaySSM(Bt, H, P, N, G, dev(A), dev(D), buffer_len=L)
    lay.load_state(dev(S0))
    conv_state = dev(S0.copy())
    cfg = rs.make_config(Bt, H, P, N, G)
    S = S0.astype(np.float64)
    for t in range(40):
        x = rng.integers(-4, 5, (Bt, H, P)).astype(np.float32)
        B = rng.integers(-4, 5, (Bt, G, N)).astype(np.float32)
        C = rng.integers(-4, 5, (Bt, G, N)).astype(np.float32)
        dt = rng.choice([0.5, 1.0], (Bt, H)).astype(np.float32)
        y = lay.step(dev(x), dev(B), dev(C), dev(dt))
        yc = torch.empty_like(y)
        rs.conventional_step(cfg, conv_state, dev(x), dev(B), dev(C), dev(dt), dev(A), dev(D), yc)
        y_ref = oracle.step(S, x, B, C, dt, A, D)
        assert np.array_equal(host(y).astype(np.float64), y_ref), f"step {t}"
        assert np.array_equal(host(yc).astype(np.float64), y_ref), f"conventional step {t}"
        if (t + 1) % L == 0:
            assert np.array_equal(host(lay.master()).astype(np.float64), S)
    assert np.array_equal(host(conv_state).astype(np.float64), S)


@pytest.mark.parametrize("which", ["tiny", "serving"])
def test_conventional_step(which):
    c = workload.TINY if which == "tiny" else workload.SERVING
    case = Case(c["Bt"], c["H"], c["P"], c["N"], c["G"], c["L"], workload.config_seed(0 if which == "tiny" else 1))
    sample = list(range(c["Bt"])) if which == "tiny" else [3, 128, 254]
    cfg = rs.make_config(case.Bt, case.H, case.P, case.N, case.G)
    state = dev(case.S0)
    S = case.S0[sample].astype(np.float64)
    A, D = dev(case.A), dev(case.D)
    steps = c["steps"] if which == "tiny" else 16
    for t in range(steps):
        x, B, C, dt = case.step_inputs(t)
        y = torch.empty(case.Bt, case.H, case.P, device="cuda")
        rs.conventional_step(cfg, state, dev(x), dev(B), dev(C), dev(dt), A, D, y)
        y_ref = oracle.step(S, x[sample], B[sample], C[sample], dt[sample], case.A, case.D)
        assert rel(host(y)[sample], y_ref) <= TOL_F32
    assert rel(host(state)[sample], S) <= TOL_F32


def test_explicit_flush_with_mask_and_materialize():
    case = Case(4, 8, 32, 64, 2, 16, 55)
    lay = case.layer()
    S = case.S0.astype(np.float64)
    for t in range(6):
        x, B, C, dt = case.step_inputs(t)
        lay.step(dev(x), dev(B), dev(C), dev(dt))
        oracle.step(S, x, B, C, dt, case.A, case.D)
    before = host(lay.materialize_state())
    assert rel(before, S) <= TOL_F32
    mask = dev(np.array([1, 0, 1, 0], np.int32))
    lay.flush(mask)
    pos, ck = lay.get_pointers()
    assert pos == [6] * 4 and ck == [6, 0, 6, 0]
    m = host(lay.master())
    assert rel(m[[0, 2]], S[[0, 2]]) <= TOL_F32
    assert np.array_equal(m[[1, 3]], case.S0[[1, 3]])
    assert rel(host(lay.materialize_state()), S) <= TOL_F32
    # decoding continues across the mixed state; an all-sequence flush empties every buffer
    for t in range(6, 30):
        x, B, C, dt = case.step_inputs(t)
        y = lay.step(dev(x), dev(B), dev(C), dev(dt))
        assert rel(host(y), oracle.step(S, x, B, C, dt, case.A, case.D)) <= TOL_F32
    lay.flush()
    pos, ck = lay.get_pointers()
    assert pos == ck == [30] * 4
    assert rel(host(lay.master()), S) <= TOL_F32


def test_batch_zero_is_a_no_op():
    A = torch.zeros(4, device="cuda")
    lay = rs.ReplaySSM(0, 4, 16, 16, 1, A, A, buffer_len=4)
    lay.load_state(torch.zeros(0, 4, 16, 16, device="cuda"))
    x = torch.zeros(0, 4, 16, device="cuda")
    BC = torch.zeros(0, 1, 16, device="cuda")
    y = lay.step(x, BC, BC, torch.zeros(0, 4, device="cuda"))
    assert y.shape == (0, 4, 16)
    assert lay.get_pointers() == ([], [])


@pytest.mark.parametrize("prec,lockstep", [("fp32", True), ("fp32", False), ("fp8", True), ("fp8", False),
                                           ("mxfp4", False)])
def test_device_flag_on_corrupted_pointers(prec, lockstep):
    """Pointers corrupted by the caller (ckpt_pos > pos): kernels detect the breach, skip the
    sequence and set the device flag; the handle then refuses work until the next load. Covers
    the lane-along-N and the one-row-per-lane step kernels, in lockstep and device-pointer mode."""
    case = Case(2, 4, 16, 32, 1, 4, 11)
    lay = case.layer(prec)
    lay.set_lockstep(lockstep)
    x, B, C, dt = case.step_inputs(0)
    lay.step(dev(x), dev(B), dev(C), dev(dt))
    pos, ck = lay.pointer_arrays()
    ck[1] = 5                                    # > pos
    torch.cuda.synchronize()
    y = lay.step(dev(x), dev(B), dev(C), dev(dt))
    assert lay.check() == rs.RSSM_E_STATE
    with pytest.raises(rs.ReplaySSMError):
        lay.step(dev(x), dev(B), dev(C), dev(dt), y)
    with pytest.raises(rs.ReplaySSMError):
        lay.get_pointers()
    lay.load_state(dev(case.S0))
    assert lay.check() == rs.RSSM_OK
    assert lay.get_pointers() == ([0, 0], [0, 0])


@pytest.mark.parametrize("prec,tol,lockstep", [("fp32", TOL_F32, True), ("fp32", TOL_F32, False),
                                               ("fp8", TOL_FP8, True), ("bf16", TOL_BF16, False),
                                               ("mxfp4", TOL_FP4, True)])
def test_graph_replay_of_whole_windows(prec, tol, lockstep):
    """A captured HIP graph of one whole window (L steps, from a window boundary) replays
    correctly with the lockstep fast path on (its arguments repeat every window) and off (device
    pointers in place): each replay, with new inputs copied into the captured buffers and eager
    work and synchronizations in between, matches the oracle, and the pointers advance by L per
    replay; eager steps afterwards continue from the replayed state."""
    Bt, H, P, N, G, L = 4, 8, 64, 128, 2, 4
    case = Case(Bt, H, P, N, G, L, 91)
    lay = case.layer(prec)
    lay.set_lockstep(lockstep)
    lay.load_state(dev(case.S0))
    toks = [case.step_inputs(t) for t in range(L)]
    bufs = [tuple(dev(a) for a in tk) for tk in toks]
    ys = [torch.empty(Bt, H, P, device="cuda") for _ in range(L)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(L):
            lay.step(*bufs[i], ys[i])
    S = case.S0.astype(np.float64)
    for r in range(4):
        for i in range(L):
            x, B, C, dt = case.step_inputs(r * L + i)
            for d, src in zip(bufs[i], (x, B, C, dt)):
                d.copy_(dev(src))
        g.replay()
        torch.cuda.synchronize()
        for i in range(L):
            x, B, C, dt = case.step_inputs(r * L + i)
            y_ref = oracle.step(S, x, B, C, dt, case.A, case.D)
            bound = TOL_F32 if i == L - 1 else tol
            assert rel(host(ys[i]), y_ref) <= bound, f"replay {r} step {i}"
        pos, ck = lay.get_pointers()
        assert pos == [(r + 1) * L] * Bt and ck == [(r + 1) * L] * Bt
        _ = torch.ones(1 << 20, device="cuda").sum().item()   # eager work between replays
    assert rel(host(lay.master()), S) <= TOL_F32
    for t in range(4 * L, 6 * L + 1):
        x, B, C, dt = case.step_inputs(t)
        y = lay.step(dev(x), dev(B), dev(C), dev(dt))
        bound = TOL_F32 if (t + 1) % L == 0 else tol
        assert rel(host(y), oracle.step(S, x, B, C, dt, case.A, case.D)) <= bound, f"eager step {t}"
    assert lay.check() == rs.RSSM_OK
