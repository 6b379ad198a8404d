"""Shared helpers of the GPU parity tests: device transfer, the normwise error metric, and a
helper that runs the HIP layer and the float64 oracle side by side on the same seeded inputs."""
import numpy as np
import torch

import oracle
import workload

PREC_CODE = {"fp32": oracle.READ_FP32, "bf16": oracle.READ_BF16, "fp8": oracle.READ_FP8,
             "mxfp4": oracle.READ_MXFP4}
MASTER_CODE = {"fp32": oracle.MASTER_FP32, "fp16": oracle.MASTER_FP16, "fp16_sr": oracle.MASTER_FP16_SR}

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
        codes, scales = oracle.e4m3_encode_tiles(m, m.shape[2] * m.shape[3])
        assert np.array_equal(host(lay.scales()[idx]).reshape(-1), scales), f"{what}: fp8 scales differ"
        assert np.array_equal(got.reshape(-1), codes), f"{what}: fp8 codes differ from the encoded master"
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
