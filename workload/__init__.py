"""Seeded synthetic inputs for the Mamba-2 decode layer.

This module holds no arithmetic of the method: it only draws random inputs. Both the GPU path's
tests/benchmark and the float64 oracle are fed the same fp32 arrays from here.

Value distributions (per the workload definitions for the layer; the pages themselves measure on
served models whose weights are not available, so these synthetic inputs stand in for them):
  initial state S0 ~ N(0, 1)
  x ~ N(0, 1);  B, C ~ N(0, 1/N)
  dt = softplus(z - 4), z ~ N(0, 1), fresh per (sequence, head, token)   (already positive)
  A_h = -exp(u), u ~ U(0, ln 16), so A_h in [-16, -1];  D_h ~ N(0, 1)
Everything is drawn in float64 with numpy's PCG64 and rounded once to float32.

Streams are keyed by (seed, stream id, index) through numpy's SeedSequence, so the inputs of step
k do not depend on how many other steps were drawn or in what order.
"""
import numpy as np

STREAM_PARAMS, STREAM_STATE, STREAM_STEP, STREAM_ACCEPT, STREAM_DRAFT = 0, 1, 2, 3, 4
STREAM_GDN_PARAMS, STREAM_GDN_STATE, STREAM_GDN_STEP, STREAM_GDN_DRAFT = 10, 11, 12, 14
STREAM_MIX_PARAMS, STREAM_MIX_HIST, STREAM_MIX_STEP, STREAM_MIX_DRAFT = 20, 21, 22, 24


def rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, index])))


def softplus(z):
    """log(1 + e^z), evaluated stably in float64 (input generation only)."""
    return np.logaddexp(0.0, z)


def layer_params(seed: int, H: int):
    """(A, D) float32 [H]."""
    g = rng(seed, STREAM_PARAMS)
    A = -np.exp(g.uniform(0.0, np.log(16.0), size=H))
    D = g.standard_normal(H)
    return A.astype(np.float32), D.astype(np.float32)


def initial_state(seed: int, Bt: int, H: int, P: int, N: int):
    """S0 float32 [Bt,H,P,N] ~ N(0,1)."""
    return rng(seed, STREAM_STATE).standard_normal((Bt, H, P, N), dtype=np.float64).astype(np.float32)


def token_inputs(seed: int, index: int, lead: tuple, H: int, P: int, N: int, G: int,
                 stream: int = STREAM_STEP):
    """One token's (x [*lead,H,P], B [*lead,G,N], C [*lead,G,N], dt [*lead,H]) as float32."""
    g = rng(seed, stream, index)
    x = g.standard_normal(lead + (H, P))
    B = g.standard_normal(lead + (G, N)) / np.sqrt(N)
    C = g.standard_normal(lead + (G, N)) / np.sqrt(N)
    dt = softplus(g.standard_normal(lead + (H,)) - 4.0)
    return (x.astype(np.float32), B.astype(np.float32), C.astype(np.float32),
            dt.astype(np.float32))


def step_inputs(seed: int, step: int, Bt: int, H: int, P: int, N: int, G: int):
    """Inputs of decode step `step` for the whole batch: x [Bt,H,P], B/C [Bt,G,N], dt [Bt,H]."""
    return token_inputs(seed, step, (Bt,), H, P, N, G, STREAM_STEP)


def draft_inputs(seed: int, step: int, Bt: int, T: int, H: int, P: int, N: int, G: int):
    """T draft tokens per sequence: x [Bt,T,H,P], B/C [Bt,T,G,N], dt [Bt,T,H]."""
    return token_inputs(seed, step, (Bt, T), H, P, N, G, STREAM_DRAFT)


def accepted_counts(seed: int, step: int, Bt: int, T: int):
    """Accepted-prefix length per sequence, uniform in {0..T}, int32 [Bt]."""
    return rng(seed, STREAM_ACCEPT, step).integers(0, T + 1, size=Bt).astype(np.int32)


def config_seed(config_index: int) -> int:
    """Seed of a numbered workload configuration (1000 * index + 7)."""
    return 1000 * config_index + 7


# --------------------------------------------------------------------------------------------
# Gated DeltaNet layer inputs: H value heads of Dv, G key heads of Dk (value head h reads key head
# h / (H/G)). q, k ~ N(0, 1) per key head, scaled to unit L2 norm (the layer normalizes them before
# the recurrence); v ~ N(0, 1); gate alpha = exp(a_h * softplus(z - 4)), z ~ N(0, 1), with per-head
# rates a_h = -exp(u), u ~ U(0, ln 16) (so alpha in (0, 1), mostly 0.6-0.99); write strength
# beta = sigmoid(N(0, 1)); S0 ~ N(0, 1). float64 draws rounded once to float32.
# --------------------------------------------------------------------------------------------
def gdn_gate_rates(seed: int, H: int):
    """a_h float64 [H] (negative)."""
    return -np.exp(rng(seed, STREAM_GDN_PARAMS).uniform(0.0, np.log(16.0), size=H))


def gdn_initial_state(seed: int, Bt: int, H: int, Dv: int, Dk: int):
    return rng(seed, STREAM_GDN_STATE).standard_normal((Bt, H, Dv, Dk), dtype=np.float64).astype(np.float32)


def gdn_token_inputs(seed: int, index: int, lead: tuple, H: int, G: int, Dv: int, Dk: int,
                     stream: int = STREAM_GDN_STEP):
    """One token's (q [*lead,G,Dk], k [*lead,G,Dk], v [*lead,H,Dv], alpha [*lead,H],
    beta [*lead,H]) as float32."""
    g = rng(seed, stream, index)
    q = g.standard_normal(lead + (G, Dk))
    k = g.standard_normal(lead + (G, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal(lead + (H, Dv))
    alpha = np.exp(gdn_gate_rates(seed, H) * softplus(g.standard_normal(lead + (H,)) - 4.0))
    beta = 1.0 / (1.0 + np.exp(-g.standard_normal(lead + (H,))))
    return tuple(a.astype(np.float32) for a in (q, k, v, alpha, beta))


def gdn_step_inputs(seed: int, step: int, Bt: int, H: int, G: int, Dv: int, Dk: int):
    return gdn_token_inputs(seed, step, (Bt,), H, G, Dv, Dk, STREAM_GDN_STEP)


def gdn_draft_inputs(seed: int, step: int, Bt: int, T: int, H: int, G: int, Dv: int, Dk: int):
    return gdn_token_inputs(seed, step, (Bt, T), H, G, Dv, Dk, STREAM_GDN_DRAFT)


# Named workloads (shapes from the layer definitions): (Bt, H, P, N, G, L, steps)
TINY = dict(Bt=2, H=4, P=16, N=16, G=1, L=4, steps=64)
SERVING = dict(Bt=256, H=128, P=64, N=128, G=8, L=16, steps=64)
DUAL_PRECISION = dict(Bt=256, H=128, P=64, N=128, G=8, L=16, steps=256)
SPEC = dict(Bt=512, H=128, P=64, N=128, G=8, L=16, T=4, steps=128)
SWEEP = dict(H=128, P=64, N=128, G=8, batches=(1, 8, 64, 256, 512), Ls=(4, 8, 16, 32),
             layers=10, steps=64)
# Gated DeltaNet: H value heads of Dv, G key heads of Dk (the pages give no GDN shape; this is a
# common GDN layer shape: 32 value heads and 16 key heads of 128), 2 MiB fp32 state per sequence.
MIXER_TINY = dict(Bt=2, H=4, P=16, N=32, G=2, L=4, K=4, steps=40)
MIXER = dict(Bt=256, H=128, P=64, N=128, G=8, L=16, K=4, steps=64)
GDN_TINY = dict(Bt=2, H=4, G=2, Dv=16, Dk=32, L=4, steps=64)
GDN_SERVING = dict(Bt=256, H=32, G=16, Dv=128, Dk=128, L=16, steps=64)
GDN_SPEC = dict(Bt=512, H=32, G=16, Dv=128, Dk=128, L=16, T=4, steps=64)


def stagnation_case():
    """Constant inputs for the master-precision stagnation case: decay 1 (A = 0, D = 0), every
    state value 1.0, and every token adds dt * x * B = 2^-16 to every value (dt = 1, x = 1,
    B = 2^-16, C = 1), so a flush of L = 4 tokens adds 2^-14. Returns ((Bt, H, P, N, G, L), S0, A,
    D, (x, B, C, dt))."""
    Bt, H, P, N, G, L = 2, 2, 64, 128, 1, 4
    S0 = np.ones((Bt, H, P, N), np.float32)
    A = np.zeros(H, np.float32)
    D = np.zeros(H, np.float32)
    x = np.ones((Bt, H, P), np.float32)
    B = np.full((Bt, G, N), 2.0 ** -16, np.float32)
    C = np.ones((Bt, G, N), np.float32)
    dt = np.ones((Bt, H), np.float32)
    return (Bt, H, P, N, G, L), S0, A, D, (x, B, C, dt)


# ---- Mamba-2 mixer edges: in-projection outputs and edge parameters ------------------------------
# Recipe: conv weights and bias ~ U(-1/sqrt(K), 1/sqrt(K)) (a depthwise conv's default init,
# fan-in K); dt_bias = the inverse softplus of dt0, dt0 log-uniform in [1e-3, 1e-1] (Mamba-2's
# dt init); in-projection outputs xBC, z, dt_raw ~ N(0, 1); the initial conv history (raw xBC of
# the K-1 tokens before the first) ~ N(0, 1).
def mixer_conv_dim(H: int, P: int, G: int, N: int) -> int:
    return H * P + 2 * G * N


def mixer_params(seed: int, H: int, P: int, G: int, N: int, K: int):
    """conv_w [CD, K], conv_b [CD], dt_bias [H] (float32)."""
    r = rng(seed, STREAM_MIX_PARAMS)
    CD = mixer_conv_dim(H, P, G, N)
    bound = 1.0 / np.sqrt(K)
    conv_w = r.uniform(-bound, bound, (CD, K)).astype(np.float32)
    conv_b = r.uniform(-bound, bound, CD).astype(np.float32)
    dt0 = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), H))
    dt_bias = (dt0 + np.log(-np.expm1(-dt0))).astype(np.float32)
    return conv_w, conv_b, dt_bias


def mixer_history(seed: int, Bt: int, K: int, CD: int):
    """Raw xBC of the K-1 tokens before the first, oldest first: float32 [Bt, K-1, CD]."""
    return rng(seed, STREAM_MIX_HIST).standard_normal((Bt, K - 1, CD)).astype(np.float32)


def mixer_token_inputs(seed: int, index: int, lead: tuple, H: int, P: int, G: int, N: int,
                       stream: int = STREAM_MIX_STEP):
    """xbc lead+(CD,), z lead+(H, P), dt_raw lead+(H,) (float32)."""
    r = rng(seed, stream, index)
    CD = mixer_conv_dim(H, P, G, N)
    xbc = r.standard_normal(lead + (CD,)).astype(np.float32)
    z = r.standard_normal(lead + (H, P)).astype(np.float32)
    dt_raw = r.standard_normal(lead + (H,)).astype(np.float32)
    return xbc, z, dt_raw


def mixer_step_inputs(seed: int, step: int, Bt: int, H: int, P: int, G: int, N: int):
    return mixer_token_inputs(seed, step, (Bt,), H, P, G, N)


def mixer_draft_inputs(seed: int, step: int, Bt: int, T: int, H: int, P: int, G: int, N: int):
    """Draft inputs with the draft index second: xbc [Bt,T,CD], z [Bt,T,H,P], dt_raw [Bt,T,H]."""
    return mixer_token_inputs(seed, step, (Bt, T), H, P, G, N, STREAM_MIX_DRAFT)
