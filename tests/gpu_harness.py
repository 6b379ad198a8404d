"""Shared helpers of the GPU parity tests: device transfer, the normwise error metric, and a
helper that runs the HIP layer and the float64 oracle side by side on the same seeded inputs."""
import json
import os

import numpy as np
import torch

import oracle
import workload

PREC_CODE = {"fp32": oracle.READ_FP32, "bf16": oracle.READ_BF16, "fp8": oracle.READ_FP8,
             "mxfp4": oracle.READ_MXFP4}
MASTER_CODE = {"fp32": oracle.MASTER_FP32, "fp16": oracle.MASTER_FP16, "fp16_sr": oracle.MASTER_FP16_SR}

_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "mxfp4_codes.json")
with open(_GOLDEN) as _f:
    _E2M1 = np.array(json.load(_f)["e2m1_values"], np.float64)   # hand-derived code table


def decode_copy(lay, prec, sample):
    """Values of the layer's read copy for the sampled sequences, float64, decoded without the
    oracle: bf16 by bit shift, fp8 by PyTorch's float8_e4m3fn, MXFP4 by the hand-derived E2M1
    table times 2^(scale code - 127)."""
    idx = torch.as_tensor(np.asarray(sample), device="cuda")
    if prec == "bf16":
        c = host(lay.read_copy()[idx]).view(np.uint16).astype(np.uint32) << 16
        return c.view(np.float32).astype(np.float64)
    if prec == "fp8":
        v = host(lay.read_copy()[idx].view(torch.float8_e4m3fn).float()).astype(np.float64)
        return v * host(lay.scales()[idx]).astype(np.float64)[:, :, None, None]
    if prec == "mxfp4":
        b = host(lay.read_copy()[idx])
        codes = np.stack([b & 15, b >> 4], axis=-1).reshape(b.shape[:-1] + (b.shape[-1] * 2,))
        sc = host(lay.scales()[idx]).astype(np.int64) - 127
        return np.ldexp(_E2M1[codes], np.repeat(sc, 32, axis=-1))
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
