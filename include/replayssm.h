/*
 * replayssm.h -- C ABI of the ReplaySSM Mamba-2 decode-step library for AMD MI355X (gfx950).
 *
 * The method (described in prose by three web pages; cited by page and section):
 *   [AT Pulse]   "NVIDIA and Princeton's ReplaySSM stores a checkpoint and recent inputs instead of
 *                full SSM state to speed up hybrid-model decoding" (at-pulse.com, story 2558)
 *   [Clarity]    "NVIDIA and Princeton cache SSM inputs in place of state to speed hybrid-model
 *                decoding" (theclarity.today)
 *   [WittyWires] "ReplaySSM cuts memory traffic to speed up hybrid-model decoding"
 *
 * A Mamba-2 layer's per-sequence state S[h,p,n] is kept as a checkpoint S_c (all tokens before
 * ckpt_pos folded in) plus a buffer of per-token records (x, B, C, dt) for the tokens since. A
 * decode step forms its output from the checkpoint and the records and stores only its own record;
 * when the buffer fills, a flush folds it into the checkpoint. With a = exp(dt*A_h), the layer
 * computes exactly the Mamba-2 recurrence S <- a*S + dt * x (outer) B, y = S.C + D*x (update,
 * then read), unrolled over the window of records since the checkpoint:
 *     y_t[p] = decay_t * (S_c[p,:] . C_t) + sum_{j=c..t} w_j * (B_j . C_t) * x_j[p] + D_h * x_t[p]
 *     decay_t = exp(A_h * sum_{i=c..t} dt_i),   w_j = dt_j * exp(A_h * sum_{i=j+1..t} dt_i)
 *     flush:  S_c <- decay_t * S_c + sum_j w_j * x_j (outer) B_j
 *
 * Shapes: batch Bt sequences, H heads of headdim P, state size N, G groups (head h reads group
 * h / (H/G) of B and C), buffer length L. All arrays are row-major, last index fastest:
 *     x [Bt,H,P]  B, C [Bt,G,N]  dt [Bt,H] (positive: softplus already applied)  A, D [H]
 *     state [Bt,H,P,N]  y [Bt,H,P]
 *     spec-decode inputs: x [Bt,T,H,P]  B, C [Bt,T,G,N]  dt [Bt,T,H]  y [Bt,T,H,P]
 * All float arrays are fp32. Supported: N in {16, 32, 64, 128, 256}; P a multiple of 4, at most
 * 256; 1 <= L <= 64; 1 <= max_draft <= min(L, 8); H a multiple of G. The fp8 read copy needs
 * P <= 64 (one work-group owns a whole head tile, so the per-head scale is exact); the MXFP4 read
 * copy needs N >= 32 (its scale blocks are 32 consecutive n of one row).
 *
 * Memory. The caller owns every device buffer: inputs, outputs, A, D and the workspace (from
 * PyTorch or hipMalloc). The library allocates no device memory. The handle is host memory.
 * Device float arrays must be 16-byte aligned, int32 arrays 4-byte aligned, the workspace
 * 256-byte aligned. With batch 0 the (empty) batch arrays may be NULL.
 *
 * Streams. `stream` is a hipStream_t (NULL = the null stream). Every call only enqueues work on
 * it, except replayssm_get_pointers / replayssm_check / replayssm_materialize_state's status, which
 * synchronize it. Inputs must stay valid until the stream reaches the call.
 *
 * Errors. Every call returns rssm_status; nothing aborts and nothing throws across the ABI.
 * Argument, shape and state-machine errors are detected on the host before any launch (so they
 * never touch the GPU); argument errors are reported before state-machine errors. Kernels
 * validate each sequence's pointers before any indexed access; a breach (e.g. a pointer array
 * corrupted by the caller) sets a device flag, the affected sequences are skipped, and
 * replayssm_check / replayssm_get_pointers return RSSM_E_STATE; from then on the handle refuses
 * work until replayssm_load_state. A handle is not thread-safe; separate handles are independent.
 */
#ifndef REPLAYSSM_H
#define REPLAYSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct replayssm_layer *replayssm_t;

typedef enum {
    RSSM_OK = 0,
    RSSM_E_INVAL = -1,        /* bad argument, pointer, alignment or shape */
    RSSM_E_WORKSPACE = -2,    /* workspace NULL, misaligned or smaller than required */
    RSSM_E_HIP = -3,          /* a HIP runtime call or kernel launch failed */
    RSSM_E_STATE = -4,        /* state-machine misuse, or the device invariant flag is set */
    RSSM_E_UNSUPPORTED = -5   /* valid but unsupported configuration */
} rssm_status;

/* Precision of the checkpoint copy that serves replay reads; the checkpoint master is always
 * fp32 and every flush re-encodes the copy from it. The pages' 4-bit state reads are NVFP4
 * ([AT Pulse] lede, "Capabilities and access" and "Claims and evidence"), a format gfx950 has no
 * instructions for; the copies here are gfx950-native formats:
 *   BF16      round to nearest even.
 *   FP8_E4M3  OCP E4M3FN codes, one fp32 scale per (sequence, head, block of 64 consecutive rows
 *             p -- the whole head when headdim <= 64) = amax / 448 of the block (1 if amax = 0);
 *             codes = RNE of value / scale clamped to +-448.
 *   MXFP4     OCP MX v1.0 FP4 (E2M1) codes in blocks of 32 consecutive n of a row, one E8M0 scale
 *             byte per block: scale = 2^(e - 127) with e = max(biased fp32 exponent of the block's
 *             amax - 2, 0) (so the largest element lands in [4, 8) before clamping to 6); codes =
 *             RNE of value / scale clamped to +-6, sign kept (a negative rounding to 0 is -0).
 *             Byte i of a block holds element 2i in its low nibble and 2i + 1 in its high nibble. */
typedef enum {
    RSSM_READ_FP32 = 0,
    RSSM_READ_BF16 = 1,
    RSSM_READ_FP8_E4M3 = 2,
    RSSM_READ_MXFP4 = 3
} rssm_read_prec;

/* Precision the checkpoint (master) is kept in ([AT Pulse] "Capabilities and access" and "Claims
 * and evidence": the pages pair 4-bit reads with an FP16 recurrence with stochastic rounding).
 *   FP32     the default.
 *   FP16     IEEE binary16, rounded to nearest even at load and at every flush (values clamped to
 *            +-65504). Reads with read_prec FP32 then come from the fp16 master itself.
 *   FP16_SR  as FP16 at load; at every flush each value rounds stochastically: with q the fp16
 *            magnitude toward zero and ulp the spacing above it, up iff r < (|v| - q) / ulp * 2^16,
 *            r = bits 16*(e mod 2) .. +15 of word (e mod 8) / 2 of Philox4x32-10 (Salmon et al.,
 *            SC'11) with counter (e / 8, sequence, new ckpt_pos, 0) and key (sr_seed, 0),
 *            e = h*P*N + p*N + n. Exactly unbiased over r in fp16's normal range (an fp32 value has
 *            13 bits below the fp16 spacing), within 2^-16 of a spacing below 2^-17; deterministic
 *            for a given seed. Standard steps use the device pointers (the lockstep fast path is
 *            off) so that every flush knows its ckpt_pos.
 *   FP8      ([AT Pulse] "Claims and evidence" names FP8 beside FP16 for the recurrence) the
 *            checkpoint is kept in the FP8_E4M3 read copy's own format: E4M3FN codes with one
 *            fp32 scale per (sequence, head, 64-row block), scale = amax / 448 of the block's
 *            folded values (1 if 0), codes of value * (1 / scale) clamped to +-448, rounded to
 *            nearest even at load and at every flush. Its value is code * scale; reads come from
 *            it directly, so read_prec must be FP32 (RSSM_E_INVAL otherwise: there is no second
 *            copy).
 *   FP8_SR   as FP8 at load; at every flush the scaled value rounds stochastically on the E4M3
 *            grid by FP16_SR's rule and Philox fields (q the E4M3 magnitude toward zero, ulp the
 *            code spacing above it, 2^-9 below 2^-6): an fp32 value keeps 20 bits below E4M3's
 *            spacing, so the mean over r is within 2^-16 of a spacing of the value. Lockstep off
 *            as for FP16_SR.
 * The fp32 and fp16 layouts are [Bt,H,P,N]; an fp8 master's codes take the fp8 copy's chunked
 * layout (see replayssm_layout.read_copy) in the master region, its scales the scale region.
 * RSSM_E_INVAL for a value outside 0..4. */
typedef enum {
    RSSM_MASTER_FP32 = 0,
    RSSM_MASTER_FP16 = 1,
    RSSM_MASTER_FP16_SR = 2,
    RSSM_MASTER_FP8 = 3,
    RSSM_MASTER_FP8_SR = 4
} rssm_master_prec;

typedef struct {
    int32_t batch;       /* Bt >= 0 (0: every call is a no-op) */
    int32_t nheads;      /* H */
    int32_t headdim;     /* P */
    int32_t dstate;      /* N */
    int32_t ngroups;     /* G */
    int32_t buffer_len;  /* L: records kept before a flush ([AT Pulse] "Technical analysis") */
    int32_t max_draft;   /* T_max: 1 = standard decode only; >1 enables spec verify/rollback */
    int32_t read_prec;   /* rssm_read_prec: precision of the checkpoint copy that serves reads */
    int32_t store_C;     /* 1: records also keep C (the record is (x, B, C, dt)); 0: (x, B, dt) */
    int32_t master_prec; /* rssm_master_prec: precision of the checkpoint itself */
    int32_t sr_seed;     /* key of the stochastic-rounding stream (RSSM_MASTER_FP16_SR, FP8_SR) */
    int32_t d_conv;      /* K: 0 = plain step inputs; 2..4 = the mixer edges are fused in (see
                            replayssm_mixer_step; requires buffer_len <= 32) */
} replayssm_config;

/* Byte offsets of the workspace regions (for inspection by tests and tools). */
typedef struct {
    size_t master;     /* checkpoint [Bt,H,P,N], fp32 or fp16 (master_prec), or fp8 codes in the
                          read copy's chunked layout -- updated only by flushes */
    size_t read_copy;  /* bf16 [Bt,H,P,N] row-major; fp8 e4m3fn codes or MXFP4 code bytes in
                          16-byte chunks (16 fp8 / 32 fp4 values of one row), per head ordered
                          [N/VEC][P]: chunk q of row p of head (b,h) at byte offset
                          ((b*H + h)*P*N*s) + (q*P + p)*16, s = 1 (fp8) or 1/2 (fp4);
                          0 bytes for fp32 reads */
    size_t scale;      /* fp8 copy or fp8 master: fp32 [Bt,H,ceil(P/64)] scales, one per 64-row
                          block; MXFP4: E8M0 bytes [Bt,H,P,N/32];
                          0 bytes otherwise */
    size_t ring_x;     /* fp32 [Bt,H,L,P]: record of absolute position q sits in slot q mod L */
    size_t ring_B;     /* fp32 [Bt,G,L,N] */
    size_t ring_C;     /* fp32 [Bt,G,L,N] (0 bytes when store_C = 0) */
    size_t ring_dt;    /* fp32 [Bt,H,L] */
    size_t conv_ring;  /* fp32 [Bt,R,CD], R = d_conv - 1 + max_draft, CD = H*P + 2*G*N: raw
                          in-projection xBC of position q in slot q mod R (0 bytes if d_conv = 0) */
    size_t pos;        /* int32 [Bt]: tokens committed */
    size_t ckpt_pos;   /* int32 [Bt]: tokens folded into the checkpoint */
    size_t counters;   /* uint32 [Bt]: per-launch completion counters (zero between launches) */
    size_t flag;       /* uint32 [1]: device invariant flag */
    size_t total;      /* bytes required */
} replayssm_layout;

/* Workspace bytes for a configuration; 0 if the configuration is invalid. */
size_t replayssm_workspace_bytes(const replayssm_config *cfg);

/* Fill `out` with the workspace layout of a valid configuration. */
rssm_status replayssm_workspace_layout(const replayssm_config *cfg, replayssm_layout *out);

/* Validate `cfg`, carve the caller's device workspace (>= replayssm_workspace_bytes bytes,
 * 256-byte aligned, owned by the caller and outliving the handle) and return a host handle.
 * A and D are device arrays [H] (per-head decay rate, negative, and skip weight), read at every
 * call, so they must outlive the handle too. No device work is done: call replayssm_load_state
 * before the first step. */
rssm_status replayssm_create(const replayssm_config *cfg, void *workspace, size_t bytes,
                             const float *A, const float *D, replayssm_t *out);

/* Free the host handle (the workspace stays the caller's). NULL is accepted. */
rssm_status replayssm_destroy(replayssm_t layer);

/* Start every sequence from `state` (device fp32 [Bt,H,P,N]): the checkpoint master becomes a
 * copy of it, the read copy is encoded from it, pos = ckpt_pos = 0, the buffers are emptied and
 * the device flag and any pending verify are cleared. */
rssm_status replayssm_load_state(replayssm_t layer, const float *state, void *stream);

/* Standard decode step for every sequence ([AT Pulse] lede and "Technical analysis"; [Clarity]
 * claim ledger [18]): store the token's record in ring slot pos mod L, form
 * y (device fp32 [Bt,H,P]) by replay from the checkpoint read copy plus the window's records, and
 * advance pos by 1. When more than L - max_draft records are then pending (for standard decode:
 * when the buffer is full, i.e. every L steps -- [WittyWires] "What happened"), the same launch
 * flushes the sequence: it folds the records into the fp32 master, rewrites the read copy, sets
 * ckpt_pos = pos and reads y from the folded fp32 state. Inputs: x [Bt,H,P], B, C [Bt,G,N],
 * dt [Bt,H]. RSSM_E_STATE if a verify is pending. */
rssm_status replayssm_step(replayssm_t layer, const float *x, const float *B, const float *C,
                           const float *dt, float *y, void *stream);

/* ---- Mixer edges (d_conv = K > 0) ---------------------------------------------------------------
 * The pages give the SSM step itself; in a Mamba-2 mixer it sits between the in-projection and
 * the output gate ([Clarity] "Why it matters": the per-token state read and write of the decode
 * path). A mixer handle fuses the edges of the published Mamba-2 block (Dao and Gu, 2024) into the
 * step, per sequence and token:
 *   in-projection output xBC [CD] (channels: x head-major [H*P], then B [G*N], then C [G*N]),
 *   z [H,P], dt_raw [H];
 *   u[c] = conv_b[c] + sum_{i<K} conv_w[c*K + i] * xBC_{pos-K+1+i}[c]  (causal depthwise conv
 *   over this token and the K-1 before it), (x, B, C) = split(silu(u)), silu(v) = v/(1+e^-v);
 *   dt = softplus(dt_raw + dt_bias[h]), softplus(v) = log(1 + e^v);
 *   the step as replayssm_step on (x, B, C, dt), records as there;
 *   o[h,p] = y[h,p] * silu(z[h,p]).
 * The conv history is the raw xBC of the K-1 committed positions before pos, kept in the
 * workspace ring keyed by position, so a rollback cuts it back with the records (no copy). A
 * mixer handle takes mixer calls: replayssm_step and replayssm_spec_verify return RSSM_E_INVAL.
 * Lockstep graph capture: the step's arguments (window slots and the ring slot pos mod R)
 * repeat every lcm(L, R) steps, so a captured run of such a multiple replays correctly; a replay
 * whose ring slot no longer matches pos mod R raises the device flag (RSSM_E_STATE from
 * replayssm_check), as a mismatched window position does. */

/* Give the edge parameters (device fp32, caller-owned, outliving their use): conv_w [CD,K],
 * conv_b [CD], dt_bias [H]. RSSM_E_INVAL on a handle with d_conv = 0 or a NULL / misaligned
 * pointer. Required before the first replayssm_mixer_step (RSSM_E_STATE otherwise). */
rssm_status replayssm_set_mixer(replayssm_t layer, const float *conv_w, const float *conv_b,
                                const float *dt_bias);

/* Set every sequence's conv history, relative to its current pos: hist (device fp32
 * [Bt,K-1,CD], raw xBC of the K-1 tokens before the next one, oldest first), or zeros if NULL.
 * replayssm_load_state resets the history to zeros. RSSM_E_STATE if a verify is pending. */
rssm_status replayssm_load_conv_state(replayssm_t layer, const float *hist, void *stream);

/* The conv history after the committed tokens into out (device fp32 [Bt,K-1,CD]). */
rssm_status replayssm_materialize_conv_state(replayssm_t layer, float *out, void *stream);

/* Standard decode step with the mixer edges fused: inputs xbc [Bt,CD], z [Bt,H,P],
 * dt_raw [Bt,H]; output o [Bt,H,P] (gated). Stores xbc in the conv ring at slot pos mod R and the
 * token's record (the conv's x, B, C and the softplus dt) as replayssm_step does, with the same
 * flush rule. Float arrays 4-byte aligned. */
rssm_status replayssm_mixer_step(replayssm_t layer, const float *xbc, const float *z,
                                 const float *dt_raw, float *o, void *stream);

/* Speculative verify with the mixer edges (as replayssm_spec_verify): T drafts xbc [Bt,T,CD],
 * z [Bt,T,H,P], dt_raw [Bt,T,H]; draft i's conv runs over the committed history and drafts
 * 0..i; outputs o [Bt,T,H,P] (gated). The drafts' raw xBC enter the conv ring at slots
 * (pos + i) mod R; replayssm_rollback then keeps the accepted prefix's history by the pointer
 * move alone. */
rssm_status replayssm_mixer_spec_verify(replayssm_t layer, int32_t T, const float *xbc, const float *z,
                                        const float *dt_raw, float *o, void *stream);

/* Fold every committed record of the selected sequences into the checkpoint (seq_mask: device
 * int32 [Bt], nonzero = flush; NULL = all), rewrite their read copy, set ckpt_pos = pos.
 * Sequences with no pending record are untouched. RSSM_E_STATE if a verify is pending. */
rssm_status replayssm_flush(replayssm_t layer, const int32_t *seq_mask, void *stream);

/* Speculative verify, output-only ([AT Pulse] "Technical analysis": output-only evaluation that
 * builds no intermediate state): for T draft tokens per sequence (1 <= T <= max_draft), write
 * their records into ring slots (pos + i) mod L and their outputs y [Bt,T,H,P], each formed by
 * replay over the committed window plus the drafts up to and including itself. No state is
 * written and no pointer moves. Requires no pending verify; leaves one pending. */
rssm_status replayssm_spec_verify(replayssm_t layer, int32_t T, const float *x, const float *B,
                                  const float *C, const float *dt, float *y, void *stream);

/* Resolve the pending verify ([AT Pulse] "Technical analysis" and [Clarity] "Why it matters":
 * rejected drafts are discarded by moving the buffer pointer): pos += accepted[b] (device int32
 * [Bt], each in [0, T]); then sequences with more than L - max_draft pending records flush.
 * Accepted counts outside [0, T] set the device flag and leave that sequence unchanged. */
rssm_status replayssm_rollback(replayssm_t layer, const int32_t *accepted, void *stream);

/* Lockstep fast path on (enable = 1, the default) or off (0). While every sequence is known on
 * the host to be at the same window position -- after a load, standard steps and unmasked
 * flushes -- replayssm_step passes (pos mod L, ckpt_pos mod L, window count) to the kernel as
 * arguments instead of reading the device pointers first; the work-group owning head 0 of each
 * sequence checks and advances that sequence's device pointers. These arguments repeat every L
 * steps, so a captured HIP graph of whole windows (starting at a window boundary) replays
 * correctly. A caller that captures other step sequences turns the fast path off: every launch
 * then reads and updates the device pointers in place, which replays correctly for any graph.
 * Switching on takes effect at the next replayssm_load_state. */
rssm_status replayssm_set_lockstep(replayssm_t layer, int enable);

/* Copy pos and ckpt_pos (host int32 [Bt] each; either may be NULL) after synchronizing the
 * stream. RSSM_E_STATE if the device flag is set. */
rssm_status replayssm_get_pointers(replayssm_t layer, int32_t *pos, int32_t *ckpt_pos,
                                   void *stream);

/* Synchronize the stream and report the device flag (RSSM_E_STATE when set). */
rssm_status replayssm_check(replayssm_t layer, void *stream);

/* Write the full current state (checkpoint with all committed records folded in) to `out`
 * (device fp32 [Bt,H,P,N]) without committing anything. For tests and for saving a state. */
rssm_status replayssm_materialize_state(replayssm_t layer, float *out, void *stream);

/* Baseline: conventional Mamba-2 decode step ([Clarity] "Why it matters" and claim ledger [6],
 * [7]): read the state, update it, read the output from it and write it back, in place.
 * state [Bt,H,P,N] in/out; y [Bt,H,P]. Only batch, nheads, headdim, dstate, ngroups of cfg are
 * used. */
rssm_status conventional_step(const replayssm_config *cfg, float *state, const float *x,
                              const float *B, const float *C, const float *dt, const float *A,
                              const float *D, float *y, void *stream);

/* Baseline with the mixer edges: conventional_step with the same fused edges as
 * replayssm_mixer_step. conv_ring [Bt,K,CD] (device fp32, in/out) holds the raw xBC of
 * position q in slot q mod K; t >= 0 is this token's position (the caller
 * keeps it; positions before 0 are the initial history). K = cfg->d_conv (2..4); state, A, D as
 * conventional_step. */
rssm_status conventional_mixer_step(const replayssm_config *cfg, float *state, float *conv_ring, int32_t t,
                                    const float *xbc, const float *z, const float *dt_raw, const float *A,
                                    const float *D, const float *conv_w, const float *conv_b,
                                    const float *dt_bias, float *o, void *stream);

/* Baseline for speculative decoding with per-draft snapshots ([Clarity] "What happened" and claim
 * ledger [13]): slots [Bt,T+1,H,P,N] hold T+1 states per sequence, cur [Bt] (device int32) the
 * committed one. Reads slot cur once, runs the T drafts stepwise, writes the state after draft i
 * to slot (cur + i) mod (T+1) and y [Bt,T,H,P]. cur is not changed. */
rssm_status snapshot_spec_verify(const replayssm_config *cfg, float *slots, const int32_t *cur,
                                 int32_t T, const float *x, const float *B, const float *C,
                                 const float *dt, const float *A, const float *D, float *y,
                                 void *stream);

/* Commit for the snapshot baseline: cur[b] <- (cur[b] + accepted[b]) mod (T+1). Accepted counts
 * outside [0, T] leave cur unchanged. */
rssm_status snapshot_commit(const replayssm_config *cfg, int32_t *cur, const int32_t *accepted,
                            int32_t T, void *stream);

/* Baseline for speculative decoding with per-draft snapshots as one call ([Clarity] "What
 * happened" and claim ledger [13]): snapshot_spec_verify followed by snapshot_commit on the same
 * stream. slots [Bt,T+1,H,P,N] and cur [Bt] as there; drafts x [Bt,T,H,P], B, C [Bt,T,G,N],
 * dt [Bt,T,H]; y [Bt,T,H,P] gets all T outputs; accepted [Bt] (device int32, each in [0, T])
 * then moves cur[b] to (cur[b] + accepted[b]) mod (T+1). Accepted counts outside [0, T] leave
 * that sequence's cur unchanged. Argument errors are reported before either launch. */
rssm_status snapshot_spec_step(const replayssm_config *cfg, float *slots, int32_t *cur, int32_t T,
                               const float *x, const float *B, const float *C, const float *dt,
                               const float *A, const float *D, float *y, const int32_t *accepted,
                               void *stream);

/* Static description of a status code. */
const char *replayssm_status_string(rssm_status status);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_H */
