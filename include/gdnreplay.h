/*
 * gdnreplay.h -- C ABI of the ReplaySSM decode step for Gated DeltaNet (GDN) layers on AMD
 * MI355X (gfx950). Same library, conventions, status codes and state machine as replayssm.h.
 *
 * The pages name Gated DeltaNet as ReplaySSM's second layer type ([AT Pulse] "Capabilities and
 * access": Mamba-2 and Gated DeltaNet kernels for standard and speculative decoding) without a
 * formula. This library computes the published Gated DeltaNet recurrence, per value head h with
 * key head g = h / (H/G) and state S [Dv, Dk] (row p = value index):
 *     S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t * v_t k_t^T,    o_t = S_t q_t
 * (update, then read). The layer keeps a checkpoint S_c plus a ring of per-token records
 * (k, v, alpha, beta); a step forms its output by replay ([AT Pulse] "Technical analysis":
 * output from the checkpoint and the buffered records, only the new record stored): a backward
 * sweep over the window's records j = t..c,
 *     z <- q_t;  c_j = beta_j (k_j . z);  z <- alpha_j (z - c_j k_j),
 * gives o_t = S_c z + sum_j c_j v_j. When the buffer fills, a flush applies the records to the
 * checkpoint in order ([WittyWires] "What happened"). Pointer, flush, verify and rollback rules
 * are those of replayssm.h (T_max = max_draft).
 *
 * Shapes: batch Bt, H value heads of Dv, G key heads of Dk (H a multiple of G), buffer length L.
 * Row-major, last index fastest, all fp32, device memory:
 *     q, k [Bt,G,Dk] (normalized by the caller)   v [Bt,H,Dv]   alpha, beta [Bt,H]
 *     state [Bt,H,Dv,Dk]   o [Bt,H,Dv]
 *     spec-decode inputs: q, k [Bt,T,G,Dk]  v [Bt,T,H,Dv]  alpha, beta [Bt,T,H]  o [Bt,T,H,Dv]
 * Supported: Dk in {16, 32, 64, 128, 256}; Dv a multiple of 4, at most 256; 1 <= L <= 64;
 * 1 <= max_draft <= min(L, 8). Reads: through the fp32 checkpoint (read_prec RSSM_READ_FP32), or
 * through a narrower copy of it ([AT Pulse] "Technical analysis": the recurrence updates a
 * full-precision checkpoint while replayed reads may use a narrower copy; "Capabilities and
 * access": FP8 and 4-bit reads), in the formats of replayssm.h with the value index as the row
 * and the key index as the column: RSSM_READ_BF16 (each value to nearest even), RSSM_READ_FP8_E4M3
 * (one fp32 scale per (sequence, value head, block of 64 value rows)), RSSM_READ_MXFP4 (one E8M0
 * scale per 32 consecutive key columns of a row; Dk >= 32, else RSSM_E_UNSUPPORTED). The copy is
 * written at load and at every flush; replayed outputs and verify read it, flushes fold into and
 * read the fp32 checkpoint.
 *
 * Memory, streams and errors as in replayssm.h: the caller owns every device buffer (16-byte
 * aligned float arrays, 4-byte aligned int32 arrays, 256-byte aligned workspace; NULL allowed
 * at batch 0); calls only enqueue on `stream` except get_pointers / check / materialize's status;
 * argument errors before state errors, all host-side before any launch; a device invariant
 * breach sets the flag and the handle refuses work until the next load.
 */
#ifndef GDNREPLAY_H
#define GDNREPLAY_H

#include <stddef.h>
#include <stdint.h>

#include "replayssm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gdnreplay_layer *gdnreplay_t;

typedef struct {
    int32_t batch;       /* Bt >= 0 */
    int32_t nheads;      /* H value heads */
    int32_t nkheads;     /* G key heads */
    int32_t dv;          /* value size Dv */
    int32_t dk;          /* key size Dk */
    int32_t buffer_len;  /* L */
    int32_t max_draft;   /* T_max: 1 = standard decode only */
    int32_t read_prec;   /* rssm_read_prec (outside 0..3: RSSM_E_INVAL) */
} gdnreplay_config;

/* Byte offsets of the workspace regions. */
typedef struct {
    size_t master;    /* fp32 [Bt,H,Dv,Dk] checkpoint, updated only by flushes */
    size_t read_copy; /* bf16 [Bt,H,Dv,Dk] row-major; fp8 / MXFP4 codes in 16-byte chunks (16 fp8 /
                         32 fp4 values of one row), per head ordered [Dk/VEC][Dv] as in
                         replayssm_layout.read_copy; 0 bytes with fp32 reads */
    size_t scale;     /* fp8: fp32 [Bt,H,ceil(Dv/64)]; MXFP4: E8M0 bytes [Bt,H,Dv,Dk/32]; else 0 bytes */
    size_t ring_k;    /* fp32 [Bt,G,L,Dk]: record of position q in slot q mod L */
    size_t ring_v;    /* fp32 [Bt,H,L,Dv] */
    size_t ring_a;    /* fp32 [Bt,H,L] alpha */
    size_t ring_b;    /* fp32 [Bt,H,L] beta */
    size_t pos;       /* int32 [Bt] tokens committed */
    size_t ckpt_pos;  /* int32 [Bt] tokens folded into the checkpoint */
    size_t counters;  /* uint32 [Bt] per-launch completion counters */
    size_t flag;      /* uint32 [1] device invariant flag */
    size_t total;     /* bytes required */
} gdnreplay_layout;

/* Workspace bytes for a configuration; 0 if invalid. */
size_t gdnreplay_workspace_bytes(const gdnreplay_config *cfg);
rssm_status gdnreplay_workspace_layout(const gdnreplay_config *cfg, gdnreplay_layout *out);

/* Validate, carve the caller's workspace (owned by the caller, outliving the handle), return a
 * host handle. No device work: call gdnreplay_load_state first. */
rssm_status gdnreplay_create(const gdnreplay_config *cfg, void *workspace, size_t bytes, gdnreplay_t *out);
rssm_status gdnreplay_destroy(gdnreplay_t layer);

/* Start every sequence from `state` [Bt,H,Dv,Dk]: checkpoint = state, pos = ckpt_pos = 0,
 * buffers emptied, flag and any pending verify cleared. */
rssm_status gdnreplay_load_state(gdnreplay_t layer, const float *state, void *stream);

/* Standard decode step ([AT Pulse] lede and "Technical analysis"): store the token's record in
 * slot pos mod L, form o [Bt,H,Dv] by replay from the checkpoint and the window's records,
 * pos += 1. When more than L - max_draft records are then pending the same launch applies them
 * to the checkpoint, sets ckpt_pos = pos and reads o from the updated state. */
rssm_status gdnreplay_step(gdnreplay_t layer, const float *q, const float *k, const float *v,
                           const float *alpha, const float *beta, float *o, void *stream);

/* Apply the pending records of the sequences with seq_mask[b] != 0 (all if NULL) to the
 * checkpoint. */
rssm_status gdnreplay_flush(gdnreplay_t layer, const int32_t *seq_mask, void *stream);

/* Output-only evaluation of T <= max_draft drafts ([AT Pulse] "Technical analysis"): draft i's
 * output by replay over the committed window plus drafts 0..i; drafts stored tentatively at
 * slots (pos + i) mod L; nothing folded, no pointer moved. Requires pending + T <= L. */
rssm_status gdnreplay_spec_verify(gdnreplay_t layer, int32_t T, const float *q, const float *k,
                                  const float *v, const float *alpha, const float *beta, float *o,
                                  void *stream);

/* Commit accepted[b] (0..T, device int32 [Bt]) drafts by moving pos; sequences with more than
 * L - max_draft pending records are then flushed. A count out of range sets the flag. */
rssm_status gdnreplay_rollback(gdnreplay_t layer, const int32_t *accepted, void *stream);

/* Lockstep fast path (as replayssm_set_lockstep): while every sequence has done the same standard
 * steps since the last load, the host knows the common window position and the step kernel takes
 * it as arguments, so window loads need no device pointer read first (device pointers are still
 * checked and advanced). enable = 0 forces the device-pointer path; 1 (the default) re-allows the
 * fast path from the next load. RSSM_E_INVAL for other values or a NULL handle. */
rssm_status gdnreplay_set_lockstep(gdnreplay_t layer, int enable);

rssm_status gdnreplay_get_pointers(gdnreplay_t layer, int32_t *pos, int32_t *ckpt_pos, void *stream);
rssm_status gdnreplay_check(gdnreplay_t layer, void *stream);

/* The state after all committed tokens (checkpoint with the pending records applied) into
 * `out` [Bt,H,Dv,Dk]; nothing is committed. */
rssm_status gdnreplay_materialize_state(gdnreplay_t layer, float *out, void *stream);

/* Baseline: one conventional GDN decode step in place ([Clarity] "Why it matters", claim ledger
 * [6]): read state, update with (k, v, alpha, beta), o = S q, write the state back. Uses batch,
 * nheads, nkheads, dv, dk of cfg. */
rssm_status gdn_conventional_step(const gdnreplay_config *cfg, float *state, const float *q, const float *k,
                                  const float *v, const float *alpha, const float *beta, float *o,
                                  void *stream);

/* Baseline: per-draft snapshots ([Clarity] "What happened", claim ledger [13]). slots
 * [Bt,T+1,H,Dv,Dk], cur [Bt] int32 (committed slot): reads slot cur once, writes the state
 * after draft i to slot (cur + i + 1) mod (T + 1), outputs o [Bt,T,H,Dv]. Commit with
 * snapshot_commit (replayssm.h). */
rssm_status gdn_snapshot_spec_verify(const gdnreplay_config *cfg, float *slots, const int32_t *cur, int32_t T,
                                     const float *q, const float *k, const float *v, const float *alpha,
                                     const float *beta, float *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDNREPLAY_H */
