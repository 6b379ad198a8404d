"""Shared helpers of the GPU parity tests: device transfer, the normwise error metric, and a
driver that runs the HIP layer and the float64 oracle side by side on the same seeded inputs."""
import numpy as np
import torch

import oracle
import workload


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

    def layer(self, read_prec="fp32", store_C=True, Tmax=None):
        import hybrid_mamba_decode_amd as rs
        lay = rs.ReplaySSM(self.Bt, self.H, self.P, self.N, self.G, dev(self.A), dev(self.D),
                           buffer_len=self.L, max_draft=Tmax or self.Tmax, read_prec=read_prec,
                           store_C=store_C)
        lay.load_state(dev(self.S0))
        return lay
