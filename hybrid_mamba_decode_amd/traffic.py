"""Algorithmic HBM bytes of each kernel class, per sequence and step (the roofline's numerator).

Counted once per byte the method must move: each state/copy element read or written once, every
input read once, every record written once and every stored record the window needs read once
(B of a group counted once per sequence, as it is shared by the group's heads). Indices, pointers
and the per-head fp8 scales of a read are tiny and are counted where they are part of the format.

Shapes: H heads, P headdim, N state, G groups; `k` = records in the window including the current
token (1..L). `prec` is the precision reads come from (the read copy's, or the master's when reads
use no copy) and `master` the checkpoint's own ("fp32", "fp16", or "fp8": E4M3 codes with their
per-head scales, which reads then use directly).
"""

F32 = 4
ELEM = {"fp32": 4, "fp16": 2, "bf16": 2, "fp8": 1, "mxfp4": 0.5}


def read_source(read_prec, master="fp32"):
    """Precision a replay reads the state in: the copy's, or the master's when there is no copy."""
    return master if read_prec == "fp32" else read_prec


def state_bytes(H, P, N, prec="fp32"):
    """One state (or read copy) of H heads: fp8 adds its fp32 scales (one per 64 rows of a head),
    MXFP4 its E8M0 byte per block of 32 values."""
    b = int(H * P * N * ELEM[prec])
    if prec == "fp8":
        b += H * ((P + 63) // 64) * F32
    elif prec == "mxfp4":
        b += H * P * N // 32
    return b


def token_input_bytes(H, P, N, G):
    """x, B, C, dt of one token (read by every call that consumes a token)."""
    return F32 * (H * P + 2 * G * N + H)


def record_write_bytes(H, P, N, G, store_C=True):
    return F32 * (H * P + (2 if store_C else 1) * G * N + H)


def record_read_bytes(H, P, N, G):
    """A stored record as replay and flush read it: x, B, dt (C of past tokens is never read)."""
    return F32 * (H * P + G * N + H)


def output_bytes(H, P):
    return F32 * H * P


def replay_nonflush(H, P, N, G, k, prec="fp32", store_C=True):
    return (state_bytes(H, P, N, prec) + token_input_bytes(H, P, N, G) +
            record_write_bytes(H, P, N, G, store_C) + output_bytes(H, P) +
            (k - 1) * record_read_bytes(H, P, N, G))


def replay_flush_step(H, P, N, G, L, prec="fp32", master="fp32"):
    """Fused flush step: read the master, write it and the read copy (`prec` here is the copy's
    precision, "fp32" for none); read the L-1 stored records and this token's inputs; write y.
    The token's record is folded, not stored."""
    copy = 0 if prec == "fp32" else state_bytes(H, P, N, prec)
    return (2 * state_bytes(H, P, N, master) + copy + token_input_bytes(H, P, N, G) +
            output_bytes(H, P) + (L - 1) * record_read_bytes(H, P, N, G))


def replay_window_amortized(H, P, N, G, L, prec="fp32", store_C=True, master="fp32"):
    """Mean bytes per step over one window of L steps (L-1 non-flush steps + 1 flush step)."""
    src = read_source(prec, master)
    tot = sum(replay_nonflush(H, P, N, G, k, src, store_C) for k in range(1, L))
    return (tot + replay_flush_step(H, P, N, G, L, prec, master)) / L


def conventional(H, P, N, G):
    return 2 * state_bytes(H, P, N) + token_input_bytes(H, P, N, G) + output_bytes(H, P)


def verify(H, P, N, G, T, k_old, prec="fp32", store_C=True):
    """Spec verify: one read of the checkpoint copy for T queries, T token inputs, T record
    writes, T outputs, and the k_old committed records."""
    return (state_bytes(H, P, N, prec) + T * (token_input_bytes(H, P, N, G) +
            record_write_bytes(H, P, N, G, store_C) + output_bytes(H, P)) +
            k_old * record_read_bytes(H, P, N, G))


def rollback_flush(H, P, N, G, count, prec="fp32", master="fp32"):
    """Commit-time flush of `count` records (master read + write, read copy write)."""
    copy = 0 if prec == "fp32" else state_bytes(H, P, N, prec)
    return 2 * state_bytes(H, P, N, master) + copy + count * record_read_bytes(H, P, N, G)


def snapshot_verify(H, P, N, G, T):
    """Per-draft snapshot baseline: one state read and T state writes, plus T tokens of I/O."""
    return (1 + T) * state_bytes(H, P, N) + T * (token_input_bytes(H, P, N, G) + output_bytes(H, P))


# ---- Gated DeltaNet (H value heads of Dv, G key heads of Dk) -------------------------------------
def gdn_state_bytes(H, Dv, Dk, prec="fp32"):
    """One GDN state or read copy (value rows of Dk key columns), scales included as for Mamba-2."""
    return state_bytes(H, Dv, Dk, prec)


def gdn_token_input_bytes(H, G, Dv, Dk):
    """q, k, v, alpha, beta of one token."""
    return F32 * (2 * G * Dk + H * Dv + 2 * H)


def gdn_record_bytes(H, G, Dv, Dk):
    """A stored record (k, v, alpha, beta), written once and read once per window use."""
    return F32 * (G * Dk + H * Dv + 2 * H)


def gdn_replay_nonflush(H, G, Dv, Dk, k, prec="fp32"):
    """prec: the precision the checkpoint product reads (the fp32 checkpoint or its copy)."""
    return (gdn_state_bytes(H, Dv, Dk, prec) + gdn_token_input_bytes(H, G, Dv, Dk) + gdn_record_bytes(H, G, Dv, Dk)
            + F32 * H * Dv + (k - 1) * gdn_record_bytes(H, G, Dv, Dk))


def gdn_replay_flush_step(H, G, Dv, Dk, L, prec="fp32"):
    """Read and write the fp32 checkpoint, plus the copy's write with a read copy."""
    copy = 0 if prec == "fp32" else gdn_state_bytes(H, Dv, Dk, prec)
    return (2 * gdn_state_bytes(H, Dv, Dk) + copy + gdn_token_input_bytes(H, G, Dv, Dk) + F32 * H * Dv
            + (L - 1) * gdn_record_bytes(H, G, Dv, Dk))


def gdn_conventional(H, G, Dv, Dk):
    return 2 * gdn_state_bytes(H, Dv, Dk) + gdn_token_input_bytes(H, G, Dv, Dk) + F32 * H * Dv


def gdn_verify(H, G, Dv, Dk, T, k_old, prec="fp32"):
    return (gdn_state_bytes(H, Dv, Dk, prec) + T * (gdn_token_input_bytes(H, G, Dv, Dk) + gdn_record_bytes(H, G, Dv, Dk)
            + F32 * H * Dv) + k_old * gdn_record_bytes(H, G, Dv, Dk))


def gdn_snapshot_verify(H, G, Dv, Dk, T):
    return (1 + T) * gdn_state_bytes(H, Dv, Dk) + T * (gdn_token_input_bytes(H, G, Dv, Dk) + F32 * H * Dv)


# ---- Mamba-2 mixer edges (causal conv of width K over CD = H*P + 2*G*N channels; gate z) --------
def conv_dim(H, P, N, G):
    return H * P + 2 * G * N


def mixer_edge_bytes(H, P, N, G, K):
    """Per sequence and token, what the edges add to a step: the raw xBC read, its K-1 history
    taps read and its write into the conv ring, and z read. dt_raw replaces dt and the gated
    output replaces y, so they are counted where the step counts dt and y."""
    CD = conv_dim(H, P, N, G)
    return F32 * (CD + (K - 1) * CD + CD + H * P)


def mixer_param_bytes(H, P, N, G, K):
    """Per launch: conv weights and bias, dt_bias (shared by every sequence)."""
    CD = conv_dim(H, P, N, G)
    return F32 * (CD * K + CD + H)


def _edge_delta(H, P, N, G, K):
    # x, B, C are formed in the launch instead of read
    return mixer_edge_bytes(H, P, N, G, K) - F32 * (H * P + 2 * G * N)


def replay_mixer_nonflush(H, P, N, G, k, K, prec="fp32", store_C=True):
    return replay_nonflush(H, P, N, G, k, prec, store_C) + _edge_delta(H, P, N, G, K)


def replay_mixer_flush_step(H, P, N, G, L, K, prec="fp32", master="fp32"):
    return replay_flush_step(H, P, N, G, L, prec, master) + _edge_delta(H, P, N, G, K)


def conventional_mixer(H, P, N, G, K):
    return conventional(H, P, N, G) + _edge_delta(H, P, N, G, K)


def unfused_mixer_nonflush(H, P, N, G, k, K, prec="fp32", store_C=True):
    """The same token through three launches: an edge kernel (raw xBC, taps and ring write as
    above, dt_raw read; x, B, C, dt written), the plain replay step, and a gate kernel (y and z
    read, o written)."""
    CD = conv_dim(H, P, N, G)
    edge = F32 * (CD + (K - 1) * CD + CD + H + (H * P + 2 * G * N + H))
    gate = F32 * 3 * H * P
    return edge + replay_nonflush(H, P, N, G, k, prec, store_C) + gate
