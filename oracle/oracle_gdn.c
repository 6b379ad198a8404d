/*
 * oracle_gdn.c -- float64 CPU oracle for ReplaySSM on Gated DeltaNet (GDN) layers.
 *
 * TEST INFRASTRUCTURE ONLY (as oracle.c): loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library; the two share no source.
 *
 * The pages name GDN as the method's second layer type ([AT Pulse] "Capabilities and access":
 * Mamba-2 and Gated DeltaNet kernels for standard and speculative decoding) but give no formula.
 * Reading G1: the published Gated DeltaNet recurrence, per value head h with key head
 * g = h / (H/G), state S [Dv, Dk] (row p = value index, column n = key index):
 *     S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t * v_t k_t^T
 *     o_t = S_t q_t                          (update, then read, as reading R1 of oracle.c)
 * alpha_t in (0, 1] (gate) and beta_t in (0, 1) (write strength) per (sequence, value head,
 * token); q and k per (sequence, key head, token), already normalized by the caller.
 *
 * Replay form (reading G2, [AT Pulse] "Technical analysis": a checkpoint plus the window's
 * records gives each output): with A_j = alpha_j (I - beta_j k_j k_j^T), unrolling from the
 * checkpoint S_c over records 0..t of the window,
 *     S_t = S_c A_0 ... A_t + sum_j beta_j v_j k_j^T A_{j+1} ... A_t
 * so o_t = S_c z + sum_j c_j v_j, where a backward sweep over the window gives z and c_j:
 *     z <- q_t;  for j = t, ..., 0:  c_j = beta_j (k_j . z);  z <- alpha_j (z - c_j k_j).
 * A flush folds the records into the checkpoint by applying them in order (the recurrence
 * itself); pointer and flush rules are those of oracle.c (readings R2, R5, R6, R10).
 * Reading G4: as for Mamba-2 ([AT Pulse] "Technical analysis": the recurrence is folded into a
 * full-precision checkpoint while replayed reads may use a narrower copy of it), the replay's
 * checkpoint product S_c z may read a copy of the checkpoint, written at load and at every flush
 * from the checkpoint rounded to fp32, in one of oracle.c's read-copy formats with the value
 * index p as the row and the key index n as the column: bf16; fp8 E4M3FN with one scale per
 * (sequence, value head, block of 64 value rows) (reading R6 there); MXFP4 with one E8M0 scale
 * per 32 consecutive key indices of a row (reading R7 there; Dk a multiple of 32). Flushes fold
 * into the checkpoint itself and read their output from it.
 *
 * Layouts (row-major, last index fastest): q, k [Bt,G,Dk]; v [Bt,H,Dv]; alpha, beta [Bt,H];
 * state [Bt,H,Dv,Dk]; o [Bt,H,Dv]. Spec-decode inputs carry the draft index after the batch
 * index: q, k [Bt,T,G,Dk]; v [Bt,T,H,Dv]; alpha, beta [Bt,T,H]; o [Bt,T,H,Dv].
 * All arithmetic is float64 on the exact fp32 input values.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Read-copy codecs of oracle.c (readings R6, R7 there). */
uint16_t oracle_bf16_encode(float v);
float oracle_bf16_decode(uint16_t h);
float oracle_e4m3_scale(const float *tile, size_t n);
uint8_t oracle_e4m3_encode_scaled(float v);
float oracle_e4m3_decode(uint8_t code);
void oracle_encode_mxfp4(const float *in, uint8_t *codes, uint8_t *scales, size_t nblocks);
void oracle_decode_mxfp4(const uint8_t *codes, const uint8_t *scales, double *out, size_t nblocks);

/* One token of one (sequence, value head): the recurrence G1 on the float64 state S [Dv, Dk]. */
static void gdn_update_head(int Dv, int Dk, double *S, const float *k, const float *v, double alpha,
                            double beta)
{
    for (int p = 0; p < Dv; ++p) {
        double *row = S + (size_t)p * Dk;
        double sk = 0.0; /* (S k)[p] before the update */
        for (int n = 0; n < Dk; ++n) sk += row[n] * (double)k[n];
        for (int n = 0; n < Dk; ++n)
            row[n] = alpha * (row[n] - beta * sk * (double)k[n]) + beta * (double)v[p] * (double)k[n];
    }
}

static void gdn_read_head(int Dv, int Dk, const double *S, const float *q, double *o)
{
    for (int p = 0; p < Dv; ++p) {
        double acc = 0.0;
        for (int n = 0; n < Dk; ++n) acc += S[(size_t)p * Dk + n] * (double)q[n];
        o[p] = acc;
    }
}

/* O1g: one token for every (b, h): update with (k, v, alpha, beta), then o = S q. */
void oracle_gdn_step(int Bt, int H, int G, int Dv, int Dk, double *S, const float *q, const float *k,
                     const float *v, const float *alpha, const float *beta, double *o)
{
    const int hpg = H / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < Bt; ++b) {
        for (int h = 0; h < H; ++h) {
            const int g = h / hpg;
            double *Sb = S + ((size_t)b * H + h) * (size_t)Dv * Dk;
            const size_t bh = (size_t)b * H + h, bg = (size_t)b * G + g;
            gdn_update_head(Dv, Dk, Sb, k + bg * Dk, v + bh * Dv, (double)alpha[bh], (double)beta[bh]);
            gdn_read_head(Dv, Dk, Sb, q + bg * Dk, o + bh * Dv);
        }
    }
}

/* O5g: speculative decoding by the plain definition: from the committed state the T drafts run
 * one by one through O1g; all T outputs are produced and the committed state becomes the state
 * after the first accepted[b] drafts ([Clarity] claim ledger [13]'s per-draft snapshots, in
 * float64). Returns 0, or -1 when an accepted count lies outside [0, T]. */
int oracle_gdn_spec_stepwise(int Bt, int H, int G, int Dv, int Dk, int T, double *S, const float *q,
                             const float *k, const float *v, const float *alpha, const float *beta,
                             const int *accepted, double *o)
{
    for (int b = 0; b < Bt; ++b)
        if (accepted[b] < 0 || accepted[b] > T) return -1;
    const size_t tile = (size_t)Dv * Dk;
    const int hpg = H / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < Bt; ++b) {
        for (int h = 0; h < H; ++h) {
            const int g = h / hpg;
            double *committed = S + ((size_t)b * H + h) * tile;
            double *work = (double *)malloc(tile * sizeof(double));
            memcpy(work, committed, tile * sizeof(double));
            for (int i = 0; i < T; ++i) {
                const size_t bth = ((size_t)b * T + i) * H + h, btg = ((size_t)b * T + i) * G + g;
                gdn_update_head(Dv, Dk, work, k + btg * Dk, v + bth * Dv, (double)alpha[bth],
                                (double)beta[bth]);
                gdn_read_head(Dv, Dk, work, q + btg * Dk, o + bth * Dv);
                if (i + 1 == accepted[b]) memcpy(committed, work, tile * sizeof(double));
            }
            free(work);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------- */
/* The replay form with its pointer and flush machine (readings G2, R2, R5 of oracle.c).       */
/* Records are kept by their offset from ckpt_pos (not as a ring); unused entries hold NaN.    */
/* ------------------------------------------------------------------------------------------- */
typedef struct oracle_gdn {
    int Bt, H, G, Dv, Dk, L, Tmax;
    int read_prec;                /* 0: reads from the checkpoint; 1 / 2 / 3: from its bf16 / fp8 /
                                     MXFP4 copy (G4) */
    double *ckpt;                 /* [Bt,H,Dv,Dk] checkpoint */
    double *rcopy;                /* [Bt,H,Dv,Dk] decoded copy (read_prec > 0) */
    float *rk, *rv, *ra, *rb;     /* records: [Bt,L,G,Dk], [Bt,L,H,Dv], [Bt,L,H] x 2 */
    int *pos, *ckpt_pos;
    int pending_T;
} oracle_gdn;

static size_t gk_at(const oracle_gdn *r, int b, int j, int g) { return (((size_t)b * r->L + j) * r->G + g) * r->Dk; }
static size_t gv_at(const oracle_gdn *r, int b, int j, int h) { return (((size_t)b * r->L + j) * r->H + h) * r->Dv; }
static size_t gs_at(const oracle_gdn *r, int b, int j, int h) { return ((size_t)b * r->L + j) * r->H + h; }

static void gdn_poison(oracle_gdn *r, int b, int from)
{
    for (int j = from; j < r->L; ++j) {
        for (int g = 0; g < r->G; ++g)
            for (int n = 0; n < r->Dk; ++n) r->rk[gk_at(r, b, j, g) + n] = NAN;
        for (int h = 0; h < r->H; ++h) {
            for (int p = 0; p < r->Dv; ++p) r->rv[gv_at(r, b, j, h) + p] = NAN;
            r->ra[gs_at(r, b, j, h)] = NAN;
            r->rb[gs_at(r, b, j, h)] = NAN;
        }
    }
}

/* Reading G4: the read copy of sequence b, from its checkpoint rounded to fp32 (the precision the
 * layer keeps it in), encoded and decoded back; written at create and at every flush. */
static void gdn_refresh_copy(oracle_gdn *r, int b)
{
    if (!r->read_prec) return;
    const size_t tile = (size_t)r->Dv * r->Dk;
    float *f = (float *)malloc(tile * sizeof(float));
    for (int h = 0; h < r->H; ++h) {
        const size_t off = ((size_t)b * r->H + h) * tile;
        for (size_t i = 0; i < tile; ++i) f[i] = (float)r->ckpt[off + i];
        double *c = r->rcopy + off;
        if (r->read_prec == 1) {
            for (size_t i = 0; i < tile; ++i) c[i] = (double)oracle_bf16_decode(oracle_bf16_encode(f[i]));
        } else if (r->read_prec == 2) {
            for (int p0 = 0; p0 < r->Dv; p0 += 64) { /* one scale per block of 64 value rows */
                const size_t i0 = (size_t)p0 * r->Dk, i1 = (size_t)(p0 + 64 < r->Dv ? p0 + 64 : r->Dv) * r->Dk;
                const float s = oracle_e4m3_scale(f + i0, i1 - i0);
                const float inv = 1.0f / s;
                for (size_t i = i0; i < i1; ++i)
                    c[i] = (double)oracle_e4m3_decode(oracle_e4m3_encode_scaled(f[i] * inv)) * (double)s;
            }
        } else {
            /* blocks of 32 along the key index never cross a row, since Dk is a multiple of 32 */
            const size_t nb = tile / 32;
            uint8_t *codes = (uint8_t *)malloc(nb * 16), *sc = (uint8_t *)malloc(nb);
            oracle_encode_mxfp4(f, codes, sc, nb);
            oracle_decode_mxfp4(codes, sc, c, nb);
            free(codes);
            free(sc);
        }
    }
    free(f);
}

oracle_gdn *oracle_gdn_create(int Bt, int H, int G, int Dv, int Dk, int L, int Tmax, const float *S0, int read_prec)
{
    if (Bt < 0 || H <= 0 || G <= 0 || H % G || Dv <= 0 || Dk <= 0 || L <= 0 || L > 64 || Tmax <= 0 ||
        Tmax > L || read_prec < 0 || read_prec > 3 || (read_prec == 3 && Dk % 32))
        return NULL;
    oracle_gdn *r = (oracle_gdn *)calloc(1, sizeof(oracle_gdn));
    r->Bt = Bt; r->H = H; r->G = G; r->Dv = Dv; r->Dk = Dk; r->L = L; r->Tmax = Tmax;
    r->read_prec = read_prec;
    const size_t st = (size_t)Bt * H * Dv * Dk;
    r->ckpt = (double *)malloc((st ? st : 1) * sizeof(double));
    for (size_t i = 0; i < st; ++i) r->ckpt[i] = (double)S0[i];
    r->rcopy = read_prec ? (double *)malloc((st ? st : 1) * sizeof(double)) : NULL;
    for (int b = 0; b < Bt; ++b) gdn_refresh_copy(r, b);
    r->rk = (float *)malloc(((size_t)Bt * L * G * Dk + 1) * sizeof(float));
    r->rv = (float *)malloc(((size_t)Bt * L * H * Dv + 1) * sizeof(float));
    r->ra = (float *)malloc(((size_t)Bt * L * H + 1) * sizeof(float));
    r->rb = (float *)malloc(((size_t)Bt * L * H + 1) * sizeof(float));
    r->pos = (int *)calloc(Bt + 1, sizeof(int));
    r->ckpt_pos = (int *)calloc(Bt + 1, sizeof(int));
    for (int b = 0; b < Bt; ++b) gdn_poison(r, b, 0);
    return r;
}

void oracle_gdn_destroy(oracle_gdn *r)
{
    if (!r) return;
    free(r->ckpt); free(r->rcopy); free(r->rk); free(r->rv); free(r->ra); free(r->rb); free(r->pos); free(r->ckpt_pos);
    free(r);
}

static void gdn_store(oracle_gdn *r, int b, int j, const float *k_bg /*[G,Dk]*/, const float *v_bh /*[H,Dv]*/,
                      const float *a_bh /*[H]*/, const float *b_bh /*[H]*/)
{
    memcpy(r->rk + gk_at(r, b, j, 0), k_bg, (size_t)r->G * r->Dk * sizeof(float));
    memcpy(r->rv + gv_at(r, b, j, 0), v_bh, (size_t)r->H * r->Dv * sizeof(float));
    memcpy(r->ra + gs_at(r, b, j, 0), a_bh, (size_t)r->H * sizeof(float));
    memcpy(r->rb + gs_at(r, b, j, 0), b_bh, (size_t)r->H * sizeof(float));
}

/* Output of the query at record index `last` (stored) from the checkpoint and records
 * 0..last, by the backward sweep of reading G2. */
static void gdn_replay_output(const oracle_gdn *r, int b, int last, const float *q_bg /*[G,Dk]*/,
                              double *o_bh /*[H,Dv]*/)
{
    const int hpg = r->H / r->G;
    double *z = (double *)malloc((size_t)r->Dk * sizeof(double));
    double c[64 + 8];
    for (int h = 0; h < r->H; ++h) {
        const int g = h / hpg;
        const float *q = q_bg + (size_t)g * r->Dk;
        for (int n = 0; n < r->Dk; ++n) z[n] = (double)q[n];
        for (int j = last; j >= 0; --j) {
            const float *kj = r->rk + gk_at(r, b, j, g);
            double kz = 0.0;
            for (int n = 0; n < r->Dk; ++n) kz += (double)kj[n] * z[n];
            c[j] = (double)r->rb[gs_at(r, b, j, h)] * kz;
            const double a = (double)r->ra[gs_at(r, b, j, h)];
            for (int n = 0; n < r->Dk; ++n) z[n] = a * (z[n] - c[j] * (double)kj[n]);
        }
        const double *Sc = (r->read_prec ? r->rcopy : r->ckpt) + ((size_t)b * r->H + h) * (size_t)r->Dv * r->Dk;
        for (int p = 0; p < r->Dv; ++p) {
            double acc = 0.0;
            for (int n = 0; n < r->Dk; ++n) acc += Sc[(size_t)p * r->Dk + n] * z[n];
            for (int j = 0; j <= last; ++j) acc += c[j] * (double)r->rv[gv_at(r, b, j, h) + p];
            o_bh[(size_t)h * r->Dv + p] = acc;
        }
    }
    free(z);
}

/* Apply records 0..count-1 of sequence b, in order, to the states at `dst`. */
static void gdn_fold_into(const oracle_gdn *r, int b, int count, double *dst)
{
    const int hpg = r->H / r->G;
    for (int h = 0; h < r->H; ++h) {
        double *S = dst + ((size_t)b * r->H + h) * (size_t)r->Dv * r->Dk;
        for (int j = 0; j < count; ++j)
            gdn_update_head(r->Dv, r->Dk, S, r->rk + gk_at(r, b, j, h / hpg), r->rv + gv_at(r, b, j, h),
                            (double)r->ra[gs_at(r, b, j, h)], (double)r->rb[gs_at(r, b, j, h)]);
    }
}

static void gdn_flush_seq(oracle_gdn *r, int b)
{
    int count = r->pos[b] - r->ckpt_pos[b];
    if (count <= 0) return;
    gdn_fold_into(r, b, count, r->ckpt);
    r->ckpt_pos[b] = r->pos[b];
    gdn_poison(r, b, 0);
    gdn_refresh_copy(r, b);
}

/* Standard decode step: append, pos += 1; flush when more than L - Tmax records are pending and
 * then read the output from the folded checkpoint, else by replay. -1 on a pending verify or
 * broken pointers. */
int oracle_gdn_replay_step(oracle_gdn *r, const float *q, const float *k, const float *v, const float *alpha,
                           const float *beta, double *o)
{
    if (r->pending_T) return -1;
    for (int b = 0; b < r->Bt; ++b) {
        int count = r->pos[b] - r->ckpt_pos[b];
        if (count < 0 || count > r->L - r->Tmax) return -1;
    }
    const int H = r->H, G = r->G, Dv = r->Dv, Dk = r->Dk, hpg = H / G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < r->Bt; ++b) {
        int idx = r->pos[b] - r->ckpt_pos[b];
        gdn_store(r, b, idx, k + (size_t)b * G * Dk, v + (size_t)b * H * Dv, alpha + (size_t)b * H,
                  beta + (size_t)b * H);
        r->pos[b] += 1;
        double *ob = o + (size_t)b * H * Dv;
        if (r->pos[b] - r->ckpt_pos[b] > r->L - r->Tmax) {
            gdn_flush_seq(r, b);
            for (int h = 0; h < H; ++h)
                gdn_read_head(Dv, Dk, r->ckpt + ((size_t)b * H + h) * (size_t)Dv * Dk,
                              q + ((size_t)b * G + h / hpg) * Dk, ob + (size_t)h * Dv);
        } else {
            gdn_replay_output(r, b, idx, q + (size_t)b * G * Dk, ob);
        }
    }
    return 0;
}

/* Speculative verify: T drafts appended after the committed records; draft i's output by replay
 * over the committed window plus drafts 0..i; nothing is folded and no pointer moves. */
int oracle_gdn_replay_verify(oracle_gdn *r, int T, const float *q, const float *k, const float *v,
                             const float *alpha, const float *beta, double *o)
{
    if (r->pending_T || T < 1 || T > r->Tmax) return -1;
    for (int b = 0; b < r->Bt; ++b) {
        int count = r->pos[b] - r->ckpt_pos[b];
        if (count < 0 || count + T > r->L) return -1;
    }
    const int H = r->H, G = r->G, Dv = r->Dv, Dk = r->Dk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < r->Bt; ++b) {
        int count = r->pos[b] - r->ckpt_pos[b];
        for (int i = 0; i < T; ++i) {
            const size_t bt = (size_t)b * T + i;
            gdn_store(r, b, count + i, k + bt * G * Dk, v + bt * H * Dv, alpha + bt * H, beta + bt * H);
        }
        for (int i = 0; i < T; ++i) {
            const size_t bt = (size_t)b * T + i;
            gdn_replay_output(r, b, count + i, q + bt * G * Dk, o + bt * H * Dv);
        }
    }
    r->pending_T = T;
    return 0;
}

/* Rollback and commit: pos += accepted[b] (0..T), drop the rest, flush when more than L - Tmax
 * records are pending. */
int oracle_gdn_replay_rollback(oracle_gdn *r, const int *accepted)
{
    if (!r->pending_T) return -1;
    for (int b = 0; b < r->Bt; ++b)
        if (accepted[b] < 0 || accepted[b] > r->pending_T) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < r->Bt; ++b) {
        r->pos[b] += accepted[b];
        gdn_poison(r, b, r->pos[b] - r->ckpt_pos[b]);
        if (r->pos[b] - r->ckpt_pos[b] > r->L - r->Tmax) gdn_flush_seq(r, b);
    }
    r->pending_T = 0;
    return 0;
}

int oracle_gdn_replay_flush(oracle_gdn *r, const int *seq_mask)
{
    if (r->pending_T) return -1;
    for (int b = 0; b < r->Bt; ++b)
        if (!seq_mask || seq_mask[b]) gdn_flush_seq(r, b);
    return 0;
}

/* Replace every sequence's checkpoint by the fp32 values S [Bt,H,Dv,Dk] as they are, with the */
/* read copy re-encoded from them; records and pointers stay (a test continues the model from   */
/* the GPU's own checkpoint after a flush). Returns 0, or -1 while a verify is pending.         */
int oracle_gdn_replay_set_checkpoint(oracle_gdn *r, const float *S)
{
    if (r->pending_T) return -1;
    const size_t n = (size_t)r->Bt * r->H * r->Dv * r->Dk;
#pragma omp parallel for schedule(static)
    for (size_t i = 0; i < n; ++i) r->ckpt[i] = (double)S[i];
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < r->Bt; ++b) gdn_refresh_copy(r, b);
    return 0;
}

void oracle_gdn_replay_pointers(const oracle_gdn *r, int *pos, int *ckpt_pos)
{
    for (int b = 0; b < r->Bt; ++b) { pos[b] = r->pos[b]; ckpt_pos[b] = r->ckpt_pos[b]; }
}

void oracle_gdn_replay_checkpoint(const oracle_gdn *r, double *out)
{
    memcpy(out, r->ckpt, (size_t)r->Bt * r->H * r->Dv * r->Dk * sizeof(double));
}

/* The state after all committed tokens, without committing anything. */
void oracle_gdn_replay_materialize(const oracle_gdn *r, double *out)
{
    memcpy(out, r->ckpt, (size_t)r->Bt * r->H * r->Dv * r->Dk * sizeof(double));
    for (int b = 0; b < r->Bt; ++b) gdn_fold_into(r, b, r->pos[b] - r->ckpt_pos[b], out);
}

/* The decoded read copy (read_prec > 0) into out [Bt,H,Dv,Dk]. */
void oracle_gdn_replay_read_copy(const oracle_gdn *r, double *out)
{
    if (r->read_prec) memcpy(out, r->rcopy, (size_t)r->Bt * r->H * r->Dv * r->Dk * sizeof(double));
}
