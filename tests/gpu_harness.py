"""Shared helpers of the GPU parity tests: device transfer, the normwise error metric, and a
helper that runs the HIP layer and the float64 oracle side by side on the same seeded inputs."""
import numpy as np
import torch

import oracle
import workload

PREC_CODE = {"fp32": oracle.READ_FP32, "bf16": oracle.READ_BF16, "fp8": oracle.READ_FP8,
             "mxfp4": oracle.READ_MXFP4}
MASTER_CODE = {"fp32": oracle.MASTER_FP32, "fp16": oracle.MASTER_FP16, "fp16_sr": oracle.MASTER_FP16_SR,
               "fp8": oracle.MASTER_FP8, "fp8_sr": oracle.MASTER_FP8_SR}


def row_scales(scales, P):
    """Per-block fp8 scales [..., ceil(P/64)] as float64 per row [..., P, 1] (block = 64 rows)."""
    return np.repeat(np.asarray(scales, np.float64), 64, axis=-1)[..., :P, None]


def fp8_master(lay, sample):
    """An fp8 master's E4M3FN codes [n,H,P,N] and per-head scales [n,H] of the sampled rows."""
    idx = torch.as_tensor(np.asarray(sample), device="cuda")
    return host(lay.master()[idx]), host(lay.scales()[idx])


def master_values(lay, master, sample):
    """The sampled rows of the stored checkpoint as float64 values (fp8: code * scale, exact)."""
    if master in ("fp8", "fp8_sr"):
        codes, scales = fp8_master(lay, sample)
        return oracle.e4m3_decode_table().astype(np.float64)[codes] * row_scales(scales, codes.shape[2])
    idx = torch.as_tensor(np.asarray(sample), device="cuda")
    return host(lay.master()[idx]).astype(np.float64)


def reseed(rep, lay, master, sample, rows=None):
    """Continue the oracle's replay model rep from the GPU's own stored checkpoint: every sampled
    row, or the model rows `rows` (indices into sample)."""
    sel = np.asarray(sample) if rows is None else np.asarray(sample)[rows]
    if master in ("fp8", "fp8_sr"):
        codes, scales = fp8_master(lay, sel)
        rep.set_master_fp8(codes, scales, rows)
    else:
        idx = torch.as_tensor(sel, device="cuda")
        rep.set_checkpoint(host(lay.master()[idx]).astype(np.float32), rows)


def _e4m3_order(codes):
    c = np.asarray(codes, np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def check_fp8_flush(lay, rep, sample, what, rows=None):
    """An fp8 master after a flush vs the model's fold of the same checkpoint and records: scales
    within 2^-20 relative (the two folds of a head's largest value may differ in their last
    bits), at most 1e-3 of the codes differ, each by one step of the E4M3 grid. Returns the
    fraction of differing codes."""
    sel = np.asarray(sample) if rows is None else np.asarray(sample)[rows]
    codes, scales = fp8_master(lay, sel)
    mc, ms = rep.fp8_master()
    if rows is not None:
        mc, ms = mc[rows], ms[rows]
    assert np.all(np.abs(scales.astype(np.float64) / ms - 1.0) <= 2.0 ** -20), f"{what}: fp8 master scales"
    diff = codes != mc
    flips = float(np.mean(diff))
    assert flips <= 1e-3, f"{what}: {flips:.2e} of the fp8 master codes differ from the model's"
    if diff.any():
        gap = np.abs(_e4m3_order(codes[diff]) - _e4m3_order(mc[diff]))
        assert int(gap.max()) <= 1, f"{what}: fp8 codes {int(gap.max())} steps apart"
    return flips

def assert_copy_encodes(lay, prec, m, sample, what=""):
    """The layer's read copy of the sampled sequences is, bit for bit, the oracle's encoder (O7)
    applied to the fp32 checkpoint values m [len(sample),H,P,N] -- normally the GPU's own master
    right after a flush; fp8 per-head scales and MXFP4 scale codes too."""
    idx = torch.as_tensor(np.asarray(sample), device="cuda")
    got = host(lay.read_copy()[idx])
    m = np.ascontiguousarray(m, np.float32)
    if prec == "bf16":
        ok = np.array_equal(got, oracle.bf16_encode(m).view(np.int16))
        assert ok, f"{what}: bf16 copy differs from the encoded master"
    elif prec == "fp8":
        codes, scales = oracle.e4m3_encode_rows(m)
        assert np.array_equal(host(lay.scales()[idx]), scales), f"{what}: fp8 scales differ"
        assert np.array_equal(got, codes), f"{what}: fp8 codes differ from the encoded master"
    elif prec == "mxfp4":
        codes, scales = oracle.mxfp4_encode(m)
        assert np.array_equal(host(lay.scales()[idx]), scales), f"{what}: MXFP4 scale codes differ"
        assert np.array_equal(got, codes), f"{what}: MXFP4 codes differ from the encoded master"
    else:
        raise ValueError(prec)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    return t.detach().cpu().numpy()


def rel(a, ref):
    """Normwise relative error: max |a - ref| / max |ref| over the whole tensor."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 1.0
    return float(np.max(np.abs(a - ref))) / max(den, 1e-30) if ref.size else 0.0


def log(msg):
    print(msg, flush=True)


class Case:
    """A layer workload: shapes, seed, layer params and the initial state (fp32 arrays)."""

    def __init__(self, Bt, H, P, N, G, L, seed, Tmax=1):
        self.Bt, self.H, self.P, self.N, self.G, self.L, self.Tmax = Bt, H, P, N, G, L, Tmax
        self.seed = seed
        self.A, self.D = workload.layer_params(seed, H)
        self.S0 = workload.initial_state(seed, Bt, H, P, N)

    def step_inputs(self, t):
        return workload.step_inputs(self.seed, t, self.Bt, self.H, self.P, self.N, self.G)

    def draft_inputs(self, t, T):
        return workload.draft_inputs(self.seed, t, self.Bt, T, self.H, self.P, self.N, self.G)

    def layer(self, read_prec="fp32", store_C=True, Tmax=None, master_prec="fp32", sr_seed=0):
        import hybrid_mamba_decode_amd as rs
        lay = rs.ReplaySSM(self.Bt, self.H, self.P, self.N, self.G, dev(self.A), dev(self.D),
                           buffer_len=self.L, max_draft=Tmax or self.Tmax, read_prec=read_prec,
                           store_C=store_C, master_prec=master_prec, sr_seed=sr_seed)
        lay.load_state(dev(self.S0))
        return lay
