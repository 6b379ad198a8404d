// kernels.hip -- ReplaySSM Mamba-2 decode-step kernels for gfx950, for one state size N.
//
// Compiled once per supported N with -DRSSM_N=<N>; each object exports its launchers
// (launch.h). Page citations refer to the three pages about ReplaySSM named in replayssm.h.
//
// Kernels (one work-group = 256 threads per <= 64 rows of one (sequence, head) state tile):
//   step_kernel         replay + append; the flush-capable variant also folds the sequences
//                       whose buffer fills and reads their output from the folded state
//   flush_kernel        explicit flush, rollback-and-commit, or materialize
//   verify_kernel       output-only evaluation of T draft tokens + tentative append
//   load_state_kernel   master <- state, read copy encoded, pointers reset
//   conventional_kernel read-update-write baseline
//   snapshot_verify_kernel / snapshot_commit_kernel   per-draft snapshot baseline
#include "device.h"
#include "launch.h"

#ifndef RSSM_N
#error "compile with -DRSSM_N=<dstate>"
#endif

namespace rssm {
namespace {

constexpr int NN = RSSM_N;
using GF = Geo<NN, PREC_F32>;  // fp32 geometry (master tile, records)

template <int PREC>
constexpr size_t byte_off(size_t e)
{
    return state_byte_off<PREC>(e);
}

// MXFP4 needs N >= 32 (a scale block is 32 consecutive n of one row).
template <int PREC>
constexpr bool kPrecOk = !(PREC == PREC_FP4 && NN < 32);

template <int PREC>
__device__ inline size_t chunk_off(size_t bh, int p, int q, int P)
{
    return state_chunk_off<NN, PREC>(bh, p, q, P);
}

template <int PREC>
constexpr int kNL = Geo<NN, PREC>::NL;
template <int PREC>
constexpr int kVEC = Geo<NN, PREC>::VEC;

// ------------------------------------------------------------------------------------------
// State rows of this work-group: slot i of a lane covers row i*RPB + wave*RPI + lane/LPR,
// elements [(lane % LPR) * VEC, +VEC). Lanes of rows at or beyond nrows read row 0 instead
// (every load is issued unconditionally, so a wait never covers more loads than it needs):
// rows are independent in every use, and those rows are never stored or reduced across.
// ------------------------------------------------------------------------------------------
template <int PREC>
__device__ inline void load_rows(u32x4 (&v)[kNL<PREC>], const char *rows, int nrows,
                                 int wave, int lane)
{
    using G = Geo<NN, PREC>;
    const int c = lane % G::LPR;
#pragma unroll
    for (int i = 0; i < G::NL; ++i) {
        const int r = i * G::RPB + wave * G::RPI + lane / G::LPR, rr = r < nrows ? r : 0;
        v[i] = load_nt(rows + byte_off<PREC>((size_t)rr * NN + (size_t)c * G::VEC));
    }
}

// MXFP4 block-scale codes of the chunks load_rows reads (a chunk is one block); rows at or
// beyond nrows read row 0's codes, like their chunks (their sums are never used).
template <int PREC>
__device__ inline void load_mxscales(unsigned (&sc)[kNL<PREC>], const unsigned char *rows, int nrows,
                                     int wave, int lane)
{
    using G = Geo<NN, PREC>;
    const int c = lane % G::LPR;
#pragma unroll
    for (int i = 0; i < G::NL; ++i) {
        const int r = i * G::RPB + wave * G::RPI + lane / G::LPR;
        sc[i] = rows[(size_t)(r < nrows ? r : 0) * (NN / 32) + c];
    }
}

template <int PREC>
__device__ inline int row_of(int i, int wave, int lane)
{
    using G = Geo<NN, PREC>;
    return i * G::RPB + wave * G::RPI + lane / G::LPR;
}

// VEC consecutive floats of a C vector at this lane's chunk.
template <int PREC>
__device__ inline void load_cchunk(float (&c)[kVEC<PREC>], const float *C, int lane)
{
    using G = Geo<NN, PREC>;
    const float *p = C + (lane % G::LPR) * G::VEC;
#pragma unroll
    for (int q = 0; q < G::VEC / 4; ++q) {
        const f32x4 f = *(const f32x4 *)(p + 4 * q);
        c[4 * q + 0] = f.x; c[4 * q + 1] = f.y; c[4 * q + 2] = f.z; c[4 * q + 3] = f.w;
    }
}

// Reduce per-slot partial dots to complete row sums and store them (times `scl`) in u[row].
template <int PREC, int M>
__device__ inline void rows_to_lds(float (&part)[M], float *u_base, int u_stride, int nq, int NLv,
                                   float scl, int wave, int lane)
{
    using G = Geo<NN, PREC>;
    transpose_reduce<M, G::LPR>(part, lane);
    bool writer;
    const int first = tr_first<M, G::LPR>(lane, &writer);
    constexpr int cnt = tr_count<M, G::LPR>();
    if (writer) {
#pragma unroll
        for (int e = 0; e < cnt; ++e) {
            const int idx = first + e;
            const int q = idx / NLv, i = idx % NLv;
            const int r = row_of<PREC>(i, wave, lane);
            if (q < nq && r < kRows) u_base[q * u_stride + r] = part[e] * scl;
        }
    }
}

// ------------------------------------------------------------------------------------------
// Record windows. The window of a call is k records: the first `nring` come from the ring
// (absolute position ck + j lives in slot (ck + j) mod L), the rest fresh from the call's inputs.
// ------------------------------------------------------------------------------------------
struct RecSrc {
    const float *rx, *rB, *rdt;   // this (sequence, head / group)'s ring rows, slot 0
    const float *fx, *fB, *fdt;   // first fresh record
    int sx, sB, sdt;              // stride between fresh records (floats)
    int cslot, L, P, nring;  // cslot = ck mod L
    __device__ int slot(int j) const { return ring_slot(cslot, j, L); }
    __device__ const float *x(int j) const
    {
        return j < nring ? rx + (size_t)slot(j) * P : fx + (size_t)(j - nring) * sx;
    }
    __device__ const float *B(int j) const
    {
        return j < nring ? rB + (size_t)slot(j) * NN : fB + (size_t)(j - nring) * sB;
    }
    __device__ float dt(int j) const { return j < nring ? rdt[slot(j)] : fdt[(size_t)(j - nring) * sdt]; }
};

__device__ inline RecSrc ring_src(const Layer &Ld, const Tile &t, int ck, int nring)
{
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    RecSrc s;
    s.rx = Ld.ring_x + bh * Ld.L * Ld.P + t.row0;
    s.rB = Ld.ring_B + ((size_t)t.b * Ld.G + t.g) * Ld.L * NN;
    s.rdt = Ld.ring_dt + bh * Ld.L;
    s.fx = s.fB = s.fdt = nullptr;
    s.sx = s.sB = s.sdt = 0;
    s.cslot = (int)((unsigned)ck % (unsigned)Ld.L); s.L = Ld.L; s.P = Ld.P; s.nring = nring;
    return s;
}

template <int LMAX>
struct Window {
    float xw[LMAX][kRows] __attribute__((aligned(16)));  // x of each record, this work-group's rows
    float Bw[LMAX][NN] __attribute__((aligned(16)));     // B of each record (the head's group)
    float dts[LMAX];
};

// Registers holding a window in flight: issue_window() starts every global load of the k <= LMAX
// records, commit_window() stores them to LDS. Callers issue all their other global loads (state
// rows, C) before committing, so one wait covers every load of the work-group.
template <int LMAX>
struct WindowRegs {
    static constexpr int XU = kRows / 4, BU = NN / 4;
    static constexpr int XS = (LMAX * XU + kThreads - 1) / kThreads;
    static constexpr int BS = (LMAX * BU + kThreads - 1) / kThreads;
    static constexpr int BCH = BS < 8 ? BS : 8;  // B loads held in registers at once
    f32x4 xv[XS];
    f32x4 bv[BCH];
    float dv;
};

template <int LMAX>
__device__ inline void issue_window(WindowRegs<LMAX> &r, const RecSrc &src, int k, int nrows)
{
    using R = WindowRegs<LMAX>;
    const int tid = threadIdx.x;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    r.dv = tid < k ? src.dt(tid) : 0.f;
#pragma unroll
    for (int s = 0; s < R::XS; ++s) {
        const int e = tid + s * kThreads, j = e / R::XU, c = e % R::XU;
        r.xv[s] = (j < k && 4 * c < nrows) ? *(const f32x4 *)(src.x(j) + 4 * c) : zero;
    }
#pragma unroll
    for (int s = 0; s < R::BCH; ++s) {
        const int e = tid + s * kThreads, j = e / R::BU, c = e % R::BU;
        r.bv[s] = (j < k) ? *(const f32x4 *)(src.B(j) + 4 * c) : zero;
    }
}

template <int LMAX>
__device__ inline void commit_window(Window<LMAX> &w, WindowRegs<LMAX> &r, const RecSrc &src, int k)
{
    using R = WindowRegs<LMAX>;
    const int tid = threadIdx.x;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < R::XS; ++s) {
        const int e = tid + s * kThreads, j = e / R::XU, c = e % R::XU;
        if (j < LMAX) *(f32x4 *)&w.xw[j][4 * c] = r.xv[s];
    }
    if (tid < LMAX) w.dts[tid] = r.dv;
    // B rows beyond the first BCH slots (large windows of wide states) go in further chunks.
#pragma unroll
    for (int s0 = 0; s0 < R::BS; s0 += R::BCH) {
        if (s0 > 0) {
#pragma unroll
            for (int s = 0; s < R::BCH; ++s) {
                const int e = tid + (s0 + s) * kThreads, j = e / R::BU, c = e % R::BU;
                r.bv[s] = (s0 + s < R::BS && j < k) ? *(const f32x4 *)(src.B(j) + 4 * c) : zero;
            }
        }
#pragma unroll
        for (int s = 0; s < R::BCH; ++s) {
            const int e = tid + (s0 + s) * kThreads, j = e / R::BU, c = e % R::BU;
            if (s0 + s < R::BS && j < LMAX) *(f32x4 *)&w.Bw[j][4 * c] = r.bv[s];
        }
    }
}

// Unrolled-window weights over records 0..last ([AT Pulse] "Technical analysis": the recurrence
// unrolled over the window): w_j = dt_j * exp(A * sum_{i=j+1..last} dt_i), and the window decay
// exp(A * sum_{i=0..last} dt_i); with SCORES also coef_j = w_j * (B_j . Cq). GS threads share a
// record; requires LMAX >= 4 so a record's threads sit in one wave. last = -1: decay 1.
template <int LMAX, bool SCORES>
__device__ inline void window_weights(const Window<LMAX> &w, const float *Cq, int last, float A,
                                      float *wout, float *coef, float *decay)
{
    constexpr int GS = kThreads / LMAX;
    static_assert(GS <= 64 && (64 % GS) == 0, "record groups must tile a wave");
    const int j = threadIdx.x / GS, sub = threadIdx.x % GS;
    float g = 0.f;
    if (SCORES) {
        if (j <= last)
            for (int n = sub; n < NN; n += GS) g = fmaf(w.Bw[j][n], Cq[n], g);
        g = group_sum<GS>(g);
    }
    if (sub == 0 && j <= last) {
        float tail = 0.f;
        for (int i = j + 1; i <= last; ++i) tail += w.dts[i];
        const float wj = w.dts[j] * expf(A * tail);
        if (wout) wout[j] = wj;
        if (SCORES) coef[j] = wj * g;
        if (j == 0) *decay = expf(A * (tail + w.dts[0]));
    }
    if (last < 0 && threadIdx.x == 0) *decay = 1.0f;
}

// Read-copy writer for fp32 rows held in f32 geometry (device.h: write_copy_rows_n).
template <int PREC>
__device__ inline void write_copy_rows(const Layer &Ld, size_t bh, size_t elem0, const f32x4 (&vf)[GF::NL], int nrows,
                                       int wave, int lane, float *red)
{
    write_copy_rows_n<NN, PREC>(CopyDst{Ld.rcopy, Ld.scale, Ld.mxscale, Ld.P, Ld.psplit}, bh, elem0, vf, nrows, wave,
                                lane, red);
}

// Fold `k` staged records into one head's fp32 rows vf (f32 geometry), in registers:
// S' = decay * S + sum_j (w_j * x_j[p]) * B_j[n]   ([AT Pulse] "Technical analysis": at a flush
// the buffered records are absorbed into the checkpoint). xw rows of this head start at column `col0`. Records
// are the outer loop, so each lane reads its B chunk of a record once for all its rows.
template <int LMAX, int XCOLS>
__device__ inline void fold_head(f32x4 (&vf)[GF::NL], const float (&xw)[LMAX][XCOLS], const float (&Bw)[LMAX][NN],
                                 const float *wts, float decay, int col0, int k, int wave, int lane)
{
    const int c = lane % GF::LPR;
    int col[GF::NL];
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of<PREC_F32>(i, wave, lane);
        col[i] = col0 + (r < kRows ? r : 0);
        vf[i] = vf[i] * decay;
    }
    for (int j = 0; j < k; ++j) {
        const f32x4 bj = *(const f32x4 *)&Bw[j][4 * c];
        const float wj = wts[j];
#pragma unroll
        for (int i = 0; i < GF::NL; ++i) {
            const float wx = wj * xw[j][col[i]];
            vf[i].x = fmaf(wx, bj.x, vf[i].x);
            vf[i].y = fmaf(wx, bj.y, vf[i].y);
            vf[i].z = fmaf(wx, bj.z, vf[i].z);
            vf[i].w = fmaf(wx, bj.w, vf[i].w);
        }
    }
}

__device__ inline void store_rows_f32(float *rows, const f32x4 (&vf)[GF::NL], int nrows, int wave, int lane)
{
    const int c = lane % GF::LPR;
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of<PREC_F32>(i, wave, lane);
        if (r < nrows) store_nt(rows + (size_t)r * NN + 4 * c, as_u32x4(vf[i]));
    }
}

// Master rows in f32 geometry: fp32 16-byte loads, fp16 8-byte loads converted exactly, or fp8
// codes (4 per lane and row, from the head's 16-byte chunks) decoded and times the head's scale.
// F32M: the caller knows the master is fp32 (fp32 read path, all-flush launches), so the other
// formats' code is not compiled in (it would raise the kernel's register count).
template <bool F32M = false>
__device__ inline void load_master_rows(const Layer &Ld, size_t elem0, f32x4 (&vf)[GF::NL], int nrows, int wave,
                                        int lane)
{
    const int c = lane % GF::LPR;
    if (F32M || Ld.mprec == MASTER_F32) {
        u32x4 m[GF::NL];
        load_rows<PREC_F32>(m, (const char *)(Ld.master + elem0), nrows, wave, lane);
#pragma unroll
        for (int i = 0; i < GF::NL; ++i) vf[i] = as_f32x4(m[i]);
        return;
    }
    if (Ld.mprec >= MASTER_F8) {
        const size_t bh = elem0 / ((size_t)Ld.P * NN);
        const int row0 = (int)(elem0 / NN - bh * (size_t)Ld.P);
        const unsigned char *src = (const unsigned char *)Ld.rcopy;
        const float scale = Ld.scale[bh * Ld.psplit + row0 / kRows];
        const int n = 4 * c;
#pragma unroll
        for (int i = 0; i < GF::NL; ++i) {
            const int r = row_of<PREC_F32>(i, wave, lane), rr = r < nrows ? r : 0;
            const unsigned w = __builtin_nontemporal_load(
                (const unsigned *)(src + chunk_off<PREC_FP8>(bh, row0 + rr, n / 16, Ld.P) + n % 16));
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
            vf[i] = f32x4{lo.x * scale, lo.y * scale, hi.x * scale, hi.y * scale};
        }
        return;
    }
    const unsigned short *base = (const unsigned short *)Ld.master + elem0;
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of<PREC_F32>(i, wave, lane), rr = r < nrows ? r : 0;
        const u32x2 w = __builtin_nontemporal_load((const u32x2 *)(base + (size_t)rr * NN + 4 * c));
        const f32x2 lo = f16x2_to_f32(w.x), hi = f16x2_to_f32(w.y);
        vf[i] = f32x4{lo.x, lo.y, hi.x, hi.y};
    }
}

// Store master rows from fp32 values vf. An fp16 master rounds them -- to nearest even, or, when
// `stochastic`, with the Philox stream of sequence b and new checkpoint position `newck` -- and vf
// receives the stored values (the flush's output and the read copy come from the checkpoint as
// stored).
__device__ inline void store_master_rows(const Layer &Ld, int b, size_t elem0, int newck, bool stochastic,
                                         f32x4 (&vf)[GF::NL], int nrows, int wave, int lane)
{
    if (Ld.mprec == MASTER_F32) {
        store_rows_f32(Ld.master + elem0, vf, nrows, wave, lane);
        return;
    }
    const int c = lane % GF::LPR;
    unsigned short *base = (unsigned short *)Ld.master + elem0;
    const size_t seq0 = (size_t)b * Ld.H * Ld.P * NN;
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of<PREC_F32>(i, wave, lane);
        const f32x4 f = vf[i];
        unsigned short h0, h1, h2, h3;
        if (stochastic) {
            // the lane's four elements e .. e+3 are one half of an 8-element Philox group: words
            // 0, 1 for the lower half, 2, 3 for the upper, low 16 bits first
            const size_t e = elem0 - seq0 + (size_t)r * NN + 4 * c;  // element within the sequence
            const U32x4 rnd = philox4x32_10((unsigned)(e / 8), (unsigned)b, (unsigned)newck, 0u, Ld.sr_seed, 0u);
            const unsigned w0 = (e & 4) ? rnd.z : rnd.x, w1 = (e & 4) ? rnd.w : rnd.y;
            h0 = f16_sr(f.x, w0 & 0xFFFFu);
            h1 = f16_sr(f.y, w0 >> 16);
            h2 = f16_sr(f.z, w1 & 0xFFFFu);
            h3 = f16_sr(f.w, w1 >> 16);
        } else {
            h0 = f16_rne(f.x);
            h1 = f16_rne(f.y);
            h2 = f16_rne(f.z);
            h3 = f16_rne(f.w);
        }
        vf[i] = f32x4{f16_value(h0), f16_value(h1), f16_value(h2), f16_value(h3)};
        if (r < nrows) {
            const u32x2 w = {(unsigned)h0 | ((unsigned)h1 << 16), (unsigned)h2 | ((unsigned)h3 << 16)};
            __builtin_nontemporal_store(w, (u32x2 *)(base + (size_t)r * NN + 4 * c));
        }
    }
}

// Store a head's folded fp32 rows vf into an fp8 master (the fp8 read copy's format): the head's
// amax over the work-group (which owns all P rows), scale = amax / 448 (1 if 0), a = v * (1 /
// scale) clamped to +-448, coded to nearest even -- or, when `stochastic`, by e4m3_sr with the
// 16-bit Philox fields of the fp16 master (counter (e / 8, sequence b, newck, 0)). vf receives
// code * scale, the values the checkpoint now holds; there is no separate read copy to refresh.
__device__ inline void store_master_fp8_rows(const Layer &Ld, int b, size_t bh, size_t elem0, int newck,
                                             bool stochastic, f32x4 (&vf)[GF::NL], int nrows, int wave, int lane,
                                             float *red)
{
    const int c = lane % GF::LPR;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const f32x4 f = vf[i];
        const float m = fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w)));
        if (row_of<PREC_F32>(i, wave, lane) < nrows) amax = fmaxf(amax, m);
    }
    amax = block_max(amax, red);
    const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
    const float inv = 1.0f / scale;
    unsigned char *dst = (unsigned char *)Ld.rcopy;
    const int row0 = (int)(elem0 / NN - bh * (size_t)Ld.P);
    const size_t seq0 = (size_t)b * Ld.H * Ld.P * NN;
    const int n = 4 * c;
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of<PREC_F32>(i, wave, lane);
        const f32x4 f = vf[i];
        float a0 = fminf(fmaxf(f.x * inv, -448.0f), 448.0f);
        float a1 = fminf(fmaxf(f.y * inv, -448.0f), 448.0f);
        float a2 = fminf(fmaxf(f.z * inv, -448.0f), 448.0f);
        float a3 = fminf(fmaxf(f.w * inv, -448.0f), 448.0f);
        if (stochastic) {
            // the lane's four elements are one half of an 8-element Philox group (as for fp16)
            const size_t e = elem0 - seq0 + (size_t)r * NN + n;
            const U32x4 rnd = philox4x32_10((unsigned)(e / 8), (unsigned)b, (unsigned)newck, 0u, Ld.sr_seed, 0u);
            const unsigned w0 = (e & 4) ? rnd.z : rnd.x, w1 = (e & 4) ? rnd.w : rnd.y;
            a0 = e4m3_sr(a0, w0 & 0xFFFFu);
            a1 = e4m3_sr(a1, w0 >> 16);
            a2 = e4m3_sr(a2, w1 & 0xFFFFu);
            a3 = e4m3_sr(a3, w1 >> 16);
        }
        int q = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
        q = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, q, true);
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(q, false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(q, true);
        vf[i] = f32x4{lo.x * scale, lo.y * scale, hi.x * scale, hi.y * scale};
        if (r < nrows) *(unsigned *)(dst + chunk_off<PREC_FP8>(bh, row0 + r, n / 16, Ld.P) + n % 16) = (unsigned)q;
    }
    if (threadIdx.x == 0) Ld.scale[bh * Ld.psplit + row0 / kRows] = scale;
}

// Commit a head's folded rows: store them at the master's precision (vf then holds the stored
// values) and refresh the read copy from them -- or, with an fp8 master, which is its own read
// copy, encode them once.
template <int PREC, bool F32M = false>
__device__ inline void commit_rows(const Layer &Ld, int b, size_t bh, size_t elem0, int newck, bool stochastic,
                                   f32x4 (&vf)[GF::NL], int nrows, int wave, int lane, float *red)
{
    if constexpr (F32M) {  // the launch guarantees an fp32 master: no rounding code compiled in
        store_rows_f32(Ld.master + elem0, vf, nrows, wave, lane);
        write_copy_rows<PREC>(Ld, bh, elem0, vf, nrows, wave, lane, red);
        return;
    }
    if constexpr (PREC == PREC_FP8)
        if (Ld.mprec >= MASTER_F8) {
            store_master_fp8_rows(Ld, b, bh, elem0, newck, stochastic, vf, nrows, wave, lane, red);
            return;
        }
    store_master_rows(Ld, b, elem0, newck, stochastic, vf, nrows, wave, lane);
    write_copy_rows<PREC>(Ld, bh, elem0, vf, nrows, wave, lane, red);
}

__device__ inline bool sr_master(const Layer &Ld) { return Ld.mprec == MASTER_F16_SR || Ld.mprec == MASTER_F8_SR; }

// Append one record (LDS row j of the window, C from Cq) into ring slot `slot`. The head's x
// rows and dt are written by each (sequence, head) work-group (dt by split 0 only); B and C by
// the split-0 work-group of the group's first head.
template <int LMAX>
__device__ inline void append_record(const Layer &Ld, const Tile &t, const Window<LMAX> &w, int j,
                                     const float *Cq, int slot)
{
    const int tid = threadIdx.x;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    if (tid < t.nrows) Ld.ring_x[(bh * Ld.L + slot) * Ld.P + t.row0 + tid] = w.xw[j][tid];
    if (t.split == 0) {
        if (tid == 0) Ld.ring_dt[bh * Ld.L + slot] = w.dts[j];
        if (t.h % Ld.hpg == 0 && tid < NN / 4) {
            const size_t off = (((size_t)t.b * Ld.G + t.g) * Ld.L + slot) * NN + 4 * tid;
            *(f32x4 *)(Ld.ring_B + off) = *(const f32x4 *)&w.Bw[j][4 * tid];
            if (Ld.ring_C) *(f32x4 *)(Ld.ring_C + off) = *(const f32x4 *)(Cq + 4 * tid);
        }
    }
}

// ==========================================================================================
// Standard decode step ([AT Pulse] lede and "Technical analysis"; [Clarity] claim ledger [18]):
// y_t = decay * (S_c . C_t) + sum_j w_j (B_j . C_t) x_j + D x_t from the read copy plus the
// window, then store only the new record. FLUSH = the launch may meet sequences whose buffer
// fills ([WittyWires] "What happened": the checkpoint is updated when the buffer fills); those
// fold all records into the fp32 master, rewrite the read copy and read y from the new state.
//
// A work-group covers ROWS/64 heads of one group (ROWS = 64 for fp32; 128 for a bf16 copy and
// 256 for an fp8 copy), so that every work-group streams about 32 KiB of checkpoint whatever the
// read precision, and the group's B window and scores B_j . C_t are staged once for its heads.
// ==========================================================================================
template <int PREC, int ROWS>
struct SGeo {
    using G = Geo<NN, PREC>;
    static constexpr int HPB = ROWS / kRows;                 // heads per work-group
    static constexpr int NL = (ROWS + G::RPB - 1) / G::RPB;  // state load slots per lane
    static_assert(NL <= G::LPR || NL == 1, "transpose-reduce needs NL <= LPR");
};

template <int LMAX, int ROWS>
struct StepLds {
    float xw[LMAX][ROWS] __attribute__((aligned(16)));  // x of each record, rows of every head
    float Bw[LMAX][NN] __attribute__((aligned(16)));    // B of each record (the group's)
    float Cq[NN] __attribute__((aligned(16)));          // C of this token
    float u[ROWS];                                      // S_c . C_t per row
    float w[ROWS / kRows][LMAX];                        // per head: w_j
    float coef[ROWS / kRows][LMAX];                     // per head: w_j * g_j
    float decay[ROWS / kRows];
    float red[kWaves];
};

// Work-group -> (sequence, first head, row split); same XCD-aware order as map_tile.
__device__ inline Tile map_heads(const Layer &Ld, int hpb)
{
    const unsigned nblk = gridDim.x, i = blockIdx.x;
    const unsigned id = (nblk % 8u == 0u) ? (i % 8u) * (nblk / 8u) + i / 8u : i;
    const unsigned hblocks = (unsigned)(Ld.H / hpb);
    Tile t;
    t.split = (int)(id % (unsigned)Ld.psplit);
    const unsigned rest = id / (unsigned)Ld.psplit;
    t.h = (int)(rest % hblocks) * hpb;  // first head
    t.b = (int)(rest / hblocks);
    t.g = t.h / Ld.hpg;
    t.row0 = t.split * kRows;
    t.nrows = min(kRows, Ld.P - t.row0);
    return t;
}

// FLUSH: 0 = no sequence of the launch flushes; 1 = some may (their buffer fills); 2 = every
// sequence flushes (a lockstep flush step with an fp32 master and a narrow read copy: the master
// rows are issued right behind the window, and the replay path is not compiled in); 3 = as 1 with
// a narrow read copy and an fp32 master (the master code carries no fp16 / fp8-master paths).
template <int PREC, int LMAX, int ROWS, int FLUSH, bool MIX>
__global__ void __launch_bounds__(kThreads) step_kernel(Layer Ld, TokenIO io, Lockstep ls)
{
    using G = Geo<NN, PREC>;
    using SG = SGeo<PREC, ROWS>;
    constexpr int HPB = SG::HPB, NL = SG::NL;
    __shared__ StepLds<LMAX, ROWS> s;
    const Tile t = map_heads(Ld, HPB);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh0 = (size_t)t.b * Ld.H + t.h;
    const int c = lane % G::LPR;

    // 1. Checkpoint rows through the read copy, issued first: this is the stream that matters.
    //    Row r of the work-group is row (r % 64) of head r / 64.
    constexpr bool kPreload = !FLUSH || (PREC == PREC_F32 && HPB == 1);
    u32x4 v[NL];
    unsigned sc[NL];  // MXFP4: block-scale code of each chunk
    // All loads are issued unconditionally, so the issue sequence is straight-line and each wait
    // covers exactly the loads it needs. Lanes outside the tile load this tile's first row and
    // keep it: rows are independent in every use below, and those rows are never written.
    auto load_state = [&]() {
        const char *base = (PREC == PREC_F32 || PREC == PREC_F16) ? (const char *)Ld.master : (const char *)Ld.rcopy;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int r = i * G::RPB + wave * G::RPI + lane / G::LPR;
            const bool in = r < ROWS && r % kRows < t.nrows;
            const int hh = in ? r / kRows : 0, pp = t.row0 + (in ? r % kRows : 0);
            v[i] = load_nt(base + chunk_off<PREC>(bh0 + hh, pp, c, Ld.P));
            if constexpr (PREC == PREC_FP4) sc[i] = Ld.mxscale[((bh0 + hh) * Ld.P + pp) * (NN / 32) + c];
        }
    };
    // 2. Pointers. Lockstep: every sequence is at the same, host-known window position, passed
    //    as (pos mod L, ckpt_pos mod L, window count): the window loads need no device read
    //    first, and the arguments are the same on every replay of a captured whole window.
    //    Otherwise: this sequence's device pointers, validated before any address is formed.
    const bool uni = ls.k > 0;
    int pslot = 0, cslot = 0, k = 1, dpos = 0;  // dpos: this sequence's pos (device-pointer mode)
    auto slot_of = [&](int j) { return ring_slot(cslot, j, Ld.L); };  // record j (< L)

    // Two-head flush launches serve fp16 masters only (the host picks them so). Both heads' master
    // rows (8 bytes per lane and slot, in the fold's geometry) are issued as soon as the window
    // position says this step flushes, ahead of the window loads: a work-group then has as many
    // checkpoint bytes in flight as one fp32 head gives.
    constexpr bool kHalfPre = FLUSH && HPB == 2;
    constexpr bool kAll = FLUSH == 2;
    // fp32 master known at compile time: all-flush launches (host-checked) and the fp32 read path
    // (an fp16 or fp8 master is read through the F16 / FP8 kernels)
    constexpr bool kF32M = FLUSH >= 2 || PREC == PREC_F32;
    static_assert(!kAll || (HPB == 1 && !kPreload), "all-flush launches: one head, master rows issued early");
    f32x4 mf[kAll ? GF::NL : 1];
    u32x2 mh[kHalfPre ? HPB : 1][GF::NL];
    auto load_master_half = [&]() {
        const int cf4 = lane % GF::LPR;
#pragma unroll
        for (int hh = 0; hh < (kHalfPre ? HPB : 1); ++hh)
#pragma unroll
            for (int i = 0; i < GF::NL; ++i) {
                const int r = row_of<PREC_F32>(i, wave, lane), rr = r < t.nrows ? r : 0;
                const unsigned short *src =
                    (const unsigned short *)Ld.master + ((bh0 + hh) * Ld.P + t.row0 + rr) * NN + 4 * cf4;
                mh[hh][i] = __builtin_nontemporal_load((const u32x2 *)src);
            }
    };

    // 3. Window loads into registers: x rows of every head, the group's B rows, this token's C,
    //    and (wave w, lane j) <- dt_j of head w.
    constexpr int XS = (LMAX * ROWS / 4 + kThreads - 1) / kThreads;
    constexpr int BS = (LMAX * NN / 4 + kThreads - 1) / kThreads;
    constexpr int BCH = BS < 8 ? BS : 8;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const float *rx = Ld.ring_x + bh0 * Ld.L * Ld.P + t.row0;
    const float *rB = Ld.ring_B + ((size_t)t.b * Ld.G + t.g) * Ld.L * NN;
    // With the mixer edges this token's x, B, C are formed here (the conv prologue below); the
    // unconditional loads that would read them then point at the ring, and their values are unused.
    const float *fx = MIX ? rx : io.x + bh0 * Ld.P + t.row0;
    const float *fB = MIX ? rB : io.B + ((size_t)t.b * Ld.G + t.g) * NN;
    const float *Ct = MIX ? rB : io.C + ((size_t)t.b * Ld.G + t.g) * NN;
    constexpr int KT = MIX ? 1 : 0;  // window records loaded from this token's inputs
    f32x4 xv[XS], bv[BCH], cq;
    float cc[G::VEC];
    float dtj = 0.f, Aw = 0.f, scl_r = 1.0f;
    auto issue_window = [&]() {
#pragma unroll
        for (int sl = 0; sl < XS; ++sl) {
            const int e = tid + sl * kThreads, j = e / (ROWS / 4), rem = e % (ROWS / 4);
            const int hh = rem / (kRows / 4), c4 = rem % (kRows / 4);
            const bool in = j < k - KT && 4 * c4 < t.nrows;
            const float *src = (in && j < k - 1) ? rx + ((size_t)hh * Ld.L + slot_of(j)) * Ld.P + 4 * c4
                                                 : fx + (in ? (size_t)hh * Ld.P + 4 * c4 : 0);
            const f32x4 val = *(const f32x4 *)src;
            xv[sl] = in ? val : zero;
        }
#pragma unroll
        for (int sl = 0; sl < BCH; ++sl) {
            const int e = tid + sl * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
            const float *src = (j < k - 1 ? rB + (size_t)slot_of(j) * NN : fB) + 4 * c4;
            const f32x4 val = *(const f32x4 *)src;
            bv[sl] = j < k - KT ? val : zero;
        }
        if constexpr (!MIX) {
            const f32x4 val = *(const f32x4 *)(Ct + 4 * (tid % (NN / 4)));
            cq = tid < NN / 4 ? val : zero;
            load_cchunk<PREC>(cc, Ct, lane);
        }
        {
            const int hw = wave < HPB ? wave : 0;
            const bool in = wave < HPB && lane < k;
            const float val = (in && lane < k - 1) ? Ld.ring_dt[(bh0 + hw) * Ld.L + slot_of(lane)] : io.dt[bh0 + hw];
            dtj = in ? val : 0.f;
            if constexpr (MIX)  // this token's dt = softplus(dt_raw + dt_bias)
                if (in && lane == k - 1) dtj = softplus_f(val + Ld.dt_bias[t.h + hw]);
            const float a = Ld.A[t.h + hw];
            Aw = wave < HPB ? a : 0.f;
        }
        if (PREC == PREC_FP8) scl_r = Ld.scale[(bh0 + (tid < ROWS ? tid / kRows : 0)) * Ld.psplit + t.split];
    };

    // Mixer edges: this token's x rows (one per thread), the group's B and C (channels e < 2N,
    // B first) from the causal conv over the ring's history and this token's raw xBC, and the
    // gate input z of this thread's output row. Their loads are issued with the window (ahead of
    // the checkpoint stream in lockstep, so consuming them waits for nothing else); the raw
    // values enter the ring at slot pos mod R (x channels by every work-group for its rows, B / C
    // by the group's first work-group) when the results are committed.
    constexpr int BCT = (2 * NN + kThreads - 1) / kThreads;
    ConvIn cx, cbc[BCT];
    float zg = 0.f;
    int mix_rslot = 0;
    auto issue_mix = [&](int rslot) {
        mix_rslot = rslot;
        const float *raw = io.xbc + (size_t)t.b * Ld.CD;
        if (tid < ROWS) {  // whole waves: the threads that own an output row
            const int hh = tid / kRows, p = tid % kRows;
            const int row = t.row0 + (p < t.nrows ? p : 0);
            cx = conv_issue(Ld, t.b, (t.h + hh) * Ld.P + row, rslot, raw);
            zg = io.z[(bh0 + hh) * Ld.P + row];
        }
#pragma unroll
        for (int i = 0; i < BCT; ++i) {
            const int e = tid + i * kThreads, ee = e < 2 * NN ? e : 0;
            const int c = Ld.H * Ld.P + (ee < NN ? t.g * NN + ee : Ld.G * NN + t.g * NN + (ee - NN));
            cbc[i] = conv_issue(Ld, t.b, c, rslot, raw);
        }
    };
    if (uni) {
        // window first: its staging and weights then overlap the checkpoint stream
        pslot = ls.pslot;
        cslot = ls.cslot;
        k = ls.k;
        if constexpr (kHalfPre)
            if (k > Ld.L - Ld.Tmax) load_master_half();
        issue_window();
        if constexpr (MIX) issue_mix(ls.rslot);
        if (kPreload) load_state();
        if constexpr (kAll) load_master_rows<true>(Ld, (bh0 * Ld.P + t.row0) * NN, mf, t.nrows, wave, lane);
    } else {
        // checkpoint stream first; the window addresses wait for this sequence's pointers
        if (kPreload) load_state();
        const int pos = Ld.pos[t.b], ck = Ld.ckpt[t.b];
        const int c0 = pos - ck;
        if (!(ck >= 0 && c0 >= 0 && c0 <= Ld.L - Ld.Tmax) || (!FLUSH && c0 + 1 > Ld.L - Ld.Tmax)) {
            raise_flag(Ld, FLAG_POINTERS);
            seq_done(Ld, t.b, pos, ck, HPB);
            return;
        }
        pslot = (int)((unsigned)pos % (unsigned)Ld.L);
        cslot = (int)((unsigned)ck % (unsigned)Ld.L);
        k = c0 + 1;  // records in the window, this token included
        dpos = pos;
        if constexpr (kHalfPre)
            if (k > Ld.L - Ld.Tmax) load_master_half();
        issue_window();
        if constexpr (MIX) issue_mix((int)((unsigned)pos % (unsigned)Ld.R));
    }
    const bool flush = k > Ld.L - Ld.Tmax;
    if constexpr (kAll) {
        if (!(uni && flush)) {  // launched only for lockstep flush steps
            raise_flag(Ld, FLAG_POINTERS);
            return;
        }
    }

    // Pointer update, once per sequence. Lockstep: the work-group owning head 0 checks the device
    // pointers against the window position -- and, with the mixer edges, the conv ring slot -- (a
    // mismatch means they were corrupted, or a captured graph replays arguments that no longer
    // match: flag, no update) and advances them; device mode: the last work-group of the sequence
    // writes them.
    auto advance_pointers = [&]() {
        if (uni) {
            if (t.h == 0 && t.split == 0 && tid == 0) {
                const int dp = Ld.pos[t.b], dc = Ld.ckpt[t.b];
                const bool ok = dc >= 0 && dp - dc == k - 1 && (int)((unsigned)dp % (unsigned)Ld.L) == pslot &&
                                (int)((unsigned)dc % (unsigned)Ld.L) == cslot &&
                                (!MIX || (int)((unsigned)dp % (unsigned)Ld.R) == ls.rslot);
                if (ok) {
                    Ld.pos[t.b] = dp + 1;
                    Ld.ckpt[t.b] = flush ? dp + 1 : dc;
                } else {
                    __hip_atomic_fetch_or(Ld.flag, FLAG_POINTERS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        } else {
            const int pos = Ld.pos[t.b], ck = Ld.ckpt[t.b];  // unchanged until every work-group counted
            seq_done(Ld, t.b, pos + 1, flush ? pos + 1 : ck, HPB);
        }
    };

    // 4. Commit the window to LDS (B rows beyond the first chunk load here).
#pragma unroll
    for (int sl = 0; sl < XS; ++sl) {
        const int e = tid + sl * kThreads, j = e / (ROWS / 4), rem = e % (ROWS / 4);
        if (j < LMAX && !(MIX && j == k - 1)) *(f32x4 *)&s.xw[j][4 * rem] = xv[sl];
    }
#pragma unroll
    for (int s0 = 0; s0 < BS; s0 += BCH) {
        if (s0 > 0) {
#pragma unroll
            for (int sl = 0; sl < BCH; ++sl) {
                const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
                const float *src = j < k - 1 ? rB + (size_t)slot_of(j) * NN : fB;
                bv[sl] = (s0 + sl < BS && j < k) ? *(const f32x4 *)(src + 4 * c4) : zero;
            }
        }
#pragma unroll
        for (int sl = 0; sl < BCH; ++sl) {
            const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
            if (s0 + sl < BS && j < LMAX && !(MIX && j == k - 1)) *(f32x4 *)&s.Bw[j][4 * c4] = bv[sl];
        }
    }
    if constexpr (MIX) {
        if (tid < ROWS) {
            const int hh = tid / kRows, p = tid % kRows;
            const bool in = p < t.nrows;
            s.xw[k - 1][tid] = in ? conv_finish(cx) : 0.f;
            if (in) Ld.conv_ring[ring_at(Ld, t.b, (t.h + hh) * Ld.P + t.row0 + p, mix_rslot)] = cx.cur;
        }
        const bool leader = t.split == 0 && t.h % Ld.hpg == 0;
#pragma unroll
        for (int i = 0; i < BCT; ++i) {
            const int e = tid + i * kThreads;
            if (e < 2 * NN) {
                const float v = conv_finish(cbc[i]);
                if (e < NN) s.Bw[k - 1][e] = v;
                else s.Cq[e - NN] = v;
                if (leader)
                    Ld.conv_ring[ring_at(Ld, t.b, Ld.H * Ld.P + (e < NN ? t.g * NN + e : Ld.G * NN + t.g * NN + (e - NN)),
                                         mix_rslot)] = cbc[i].cur;
            }
        }
    } else {
        if (tid < NN / 4) *(f32x4 *)&s.Cq[4 * tid] = cq;
    }

    // 5. Window weights of head w in wave w: suffix sums of dt by lane shuffles,
    //    w_j = dt_j * exp(A * sum_{i>j} dt_i), decay = exp(A * sum_i dt_i) ([AT Pulse]
    //    "Technical analysis": the recurrence unrolled over the window).
    float wj = 0.f;
    if (wave < HPB) {
        float tail;
        const float sfx = suffix_sum<LMAX>(dtj, lane, &tail);
        const float total = lane0(sfx);
        wj = lane < k ? dtj * expf(Aw * tail) : 0.f;
        if (lane < LMAX) s.w[wave][lane] = wj;
        if (lane == 0) s.decay[wave] = expf(Aw * total);
    }
    __syncthreads();

    if (FLUSH && flush) {
        // Fused flush, head by head: fold all k records into the master rows (in fp32), store
        // them at the master's precision, rewrite the read copy, and read y from the stored state.
        // (A stochastically rounded master always runs in device-pointer mode: its stream is
        // keyed by the new ckpt_pos, pos + 1.)
        float cf[4];
        load_cchunk<PREC_F32>(cf, MIX ? s.Cq : Ct, lane);
#pragma unroll
        for (int hh = 0; hh < HPB; ++hh) {
            f32x4 vf[GF::NL];
            const size_t elem0 = ((bh0 + hh) * Ld.P + t.row0) * NN;
            if constexpr (kPreload) {
#pragma unroll
                for (int i = 0; i < GF::NL; ++i) vf[i] = as_f32x4(v[i]);
            } else if constexpr (kHalfPre) {
#pragma unroll
                for (int i = 0; i < GF::NL; ++i) {
                    const f32x2 lo = f16x2_to_f32(mh[hh][i].x), hi = f16x2_to_f32(mh[hh][i].y);
                    vf[i] = f32x4{lo.x, lo.y, hi.x, hi.y};
                }
            } else if constexpr (kAll) {
#pragma unroll
                for (int i = 0; i < GF::NL; ++i) vf[i] = mf[i];
            } else {
                load_master_rows<kF32M>(Ld, elem0, vf, t.nrows, wave, lane);
            }
            fold_head<LMAX, ROWS>(vf, s.xw, s.Bw, s.w[hh], s.decay[hh], hh * kRows, k, wave, lane);
            commit_rows<PREC, kF32M>(Ld, t.b, bh0 + hh, elem0, dpos + 1, sr_master(Ld), vf, t.nrows, wave, lane, s.red);
            float part[GF::NL];
#pragma unroll
            for (int i = 0; i < GF::NL; ++i) part[i] = chunk_dot<PREC_F32>(as_u32x4(vf[i]), cf);
            rows_to_lds<PREC_F32, GF::NL>(part, s.u + hh * kRows, 0, 1, GF::NL, 1.0f, wave, lane);
        }
        __syncthreads();
        if (tid < ROWS && tid % kRows < t.nrows) {
            const int hh = tid / kRows;
            const float yv = fmaf(Ld.D[t.h + hh], s.xw[k - 1][tid], s.u[tid]);
            io.y[(bh0 + hh) * Ld.P + t.row0 + tid % kRows] = MIX ? yv * silu_f(zg) : yv;
        }
        // The token's own record is folded already: nothing is appended on a flush step.
        advance_pointers();
        return;
    }

    if constexpr (!kAll) {
        // 6. Replay: the scores B_j . C_t times every head's weights (GS threads per record; LDS
        //    only, while the checkpoint rows may still be in flight), then the row dots with C_t
        //    through the read copy.
        if (!kPreload) load_state();
        if constexpr (MIX) load_cchunk<PREC>(cc, s.Cq, lane);
        {
            constexpr int GS = kThreads / LMAX;
            const int j = tid / GS, sub = tid % GS;
            float gj = 0.f;
            for (int n = sub; n < NN; n += GS) gj = fmaf(s.Bw[j][n], s.Cq[n], gj);
            gj = group_sum<GS>(gj);
            if (sub == 0)
#pragma unroll
                for (int hh = 0; hh < HPB; ++hh) s.coef[hh][j] = s.w[hh][j] * gj;
        }
        float part[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            part[i] = chunk_dot<PREC>(v[i], cc);
            if constexpr (PREC == PREC_FP4) part[i] = mx_scaled(part[i], sc[i]);
        }
        {
            transpose_reduce<NL, G::LPR>(part, lane);
            bool writer;
            const int first = tr_first<NL, G::LPR>(lane, &writer);
            const int r = first * G::RPB + wave * G::RPI + lane / G::LPR;
            if (writer && r < ROWS) s.u[r] = part[0];
        }
        __syncthreads();

        // 7. Combine and append.
        if (tid < ROWS && tid % kRows < t.nrows) {
            const int hh = tid / kRows, p = tid % kRows;
            float acc = s.decay[hh] * (s.u[tid] * scl_r);
#pragma unroll 4
            for (int j = 0; j < k; ++j) acc = fmaf(s.coef[hh][j], s.xw[j][tid], acc);
            const float xt = s.xw[k - 1][tid];
            acc = fmaf(Ld.D[t.h + hh], xt, acc);
            io.y[(bh0 + hh) * Ld.P + t.row0 + p] = MIX ? acc * silu_f(zg) : acc;
            Ld.ring_x[((bh0 + hh) * Ld.L + pslot) * Ld.P + t.row0 + p] = xt;
        }
        if (t.split == 0 && wave < HPB && lane == k - 1) Ld.ring_dt[(bh0 + wave) * Ld.L + pslot] = dtj;
        if (t.split == 0 && t.h % Ld.hpg == 0 && tid < NN / 4) {
            const size_t off = (((size_t)t.b * Ld.G + t.g) * Ld.L + pslot) * NN + 4 * tid;
            *(f32x4 *)(Ld.ring_B + off) = *(const f32x4 *)&s.Bw[k - 1][4 * tid];
            if (Ld.ring_C) *(f32x4 *)(Ld.ring_C + off) = *(const f32x4 *)&s.Cq[4 * tid];
        }
        advance_pointers();
    }
}

// ==========================================================================================
// Replay step through a narrow read copy (fp8 or MXFP4), launches without flushes: one state
// row per lane. Wave w owns head t.h + w and lane p its row p (P <= 64), so every lane of a wave
// walks the same chunk column at the same time: C_t's slice for that column is wave-uniform and
// comes from scalar loads (SGPR operands of the FMAs), the row's dot needs no cross-lane
// reduction, and each lane reads its own row's x window directly. Compared with the lane-along-N
// step this frees the C-chunk registers and the x-window LDS, so more work-groups -- and more
// checkpoint bytes -- are in flight per CU. Same arithmetic as step_kernel ([AT Pulse]
// "Technical analysis": the unrolled window).
// ==========================================================================================
template <int LMAX>
struct NarrowLds {
    float Bw[LMAX][NN] __attribute__((aligned(16)));  // B of each record (the group's)
    float Cq[NN] __attribute__((aligned(16)));        // C of this token
    float g[LMAX];                                    // scores B_j . C_t
};

template <int PREC, int LMAX>
__global__ void __launch_bounds__(kThreads) narrow_step_kernel(Layer Ld, TokenIO io, Lockstep ls)
{
    using G = Geo<NN, PREC>;
    constexpr int NC = NN / G::VEC;  // chunks per row
    constexpr int HPB = kWaves;      // heads per work-group, one per wave
    __shared__ NarrowLds<LMAX> s;
    const Tile t = map_heads(Ld, HPB);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar head index
    const int h = t.h + wave;
    const size_t bh = (size_t)t.b * Ld.H + h;
    const bool prow = lane < Ld.P;
    const int p = prow ? lane : 0;  // lanes beyond P read row 0 and store nothing

    // 1. Checkpoint row through the read copy (and, for MXFP4, the row's block-scale codes).
    u32x4 v[NC];
    unsigned scw[(NC + 3) / 4];
    auto load_state = [&]() {
        const char *base = (const char *)Ld.rcopy;
#pragma unroll
        for (int q = 0; q < NC; ++q) v[q] = load_nt(base + chunk_off<PREC>(bh, p, q, Ld.P));
        if constexpr (PREC == PREC_FP4) {
            const unsigned char *sr = Ld.mxscale + (bh * Ld.P + p) * NC;
            if constexpr (NC >= 4) {
#pragma unroll
                for (int w4 = 0; w4 < NC / 4; ++w4) scw[w4] = *(const unsigned *)(sr + 4 * w4);
            } else if constexpr (NC == 2) {
                scw[0] = *(const unsigned short *)sr;
            } else {
                scw[0] = *sr;
            }
        }
    };

    // 2. Pointers (as in step_kernel: lockstep arguments, or this sequence's device pointers).
    const bool uni = ls.k > 0;
    int pslot = 0, cslot = 0, k = 1;
    auto slot_of = [&](int j) { return ring_slot(cslot, j, Ld.L); };  // record j (< L)

    // 3. Window, in two groups: (a) the group's B rows and C_t, staged through LDS, and (lane j)
    //    dt_j of this head, issued with the checkpoint stream; (b) this lane's x_j (record j of its
    //    row, 0 beyond the window) and the token's x, loaded after the row dots, so that no x
    //    register is held while the stream is in flight (record reads mostly hit the caches).
    constexpr int BS = (LMAX * NN / 4 + kThreads - 1) / kThreads;
    constexpr int BCH = BS < 8 ? BS : 8;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const float *rB = Ld.ring_B + ((size_t)t.b * Ld.G + t.g) * Ld.L * NN;
    const float *fB = io.B + ((size_t)t.b * Ld.G + t.g) * NN;
    const float *Ct = io.C + ((size_t)t.b * Ld.G + t.g) * NN;
    float xj[LMAX], xt = 0.f, dtj = 0.f, Ah = 0.f;
    f32x4 bv[BCH], cq;
    auto issue_bc = [&]() {
#pragma unroll
        for (int sl = 0; sl < BCH; ++sl) {
            const int e = tid + sl * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
            if (j < k) bv[sl] = *(const f32x4 *)((j < k - 1 ? rB + (size_t)slot_of(j) * NN : fB) + 4 * c4);
            else bv[sl] = zero;
        }
        {
            const f32x4 val = *(const f32x4 *)(Ct + 4 * (tid % (NN / 4)));
            cq = tid < NN / 4 ? val : zero;
        }
        {
            const bool in = lane < k;
            const float val = (in && lane < k - 1) ? Ld.ring_dt[bh * Ld.L + slot_of(lane)] : io.dt[bh];
            dtj = in ? val : 0.f;
            Ah = Ld.A[h];
        }
    };
    // k is the same for the work-group's heads (one sequence): the record loops below branch on
    // it uniformly, so a short window costs only its own records.
    auto issue_x = [&]() {
        const float *fx = io.x + bh * Ld.P + p;
        const float *rx = Ld.ring_x + bh * Ld.L * Ld.P + p;
        xt = *fx;
#pragma unroll
        for (int j = 0; j < LMAX; ++j) {
            if (j < k - 1) xj[j] = rx[(size_t)slot_of(j) * Ld.P];
            else xj[j] = j == k - 1 ? xt : 0.f;
        }
    };

    // Invalid device pointers are only noted here and reported after the row dots (with safe
    // window values meanwhile, and no store): no memory write may precede the dots, or the
    // compiler can no longer load C_t through the scalar cache.
    bool bad = false;
    if (uni) {
        pslot = ls.pslot;
        cslot = ls.cslot;
        k = ls.k;
        issue_bc();
        load_state();
    } else {
        load_state();
        const int pos = Ld.pos[t.b], ck = Ld.ckpt[t.b];
        const int c0 = pos - ck;
        bad = !(ck >= 0 && c0 >= 0 && c0 + 1 <= Ld.L - Ld.Tmax);
        pslot = bad ? 0 : (int)((unsigned)pos % (unsigned)Ld.L);
        cslot = bad ? 0 : (int)((unsigned)ck % (unsigned)Ld.L);
        k = bad ? 1 : c0 + 1;
        issue_bc();
    }

    // 4. B window and C_t to LDS; then the x window; this head's weights in its wave meanwhile.
#pragma unroll
    for (int s0 = 0; s0 < BS; s0 += BCH) {
        if (s0 > 0) {
#pragma unroll
            for (int sl = 0; sl < BCH; ++sl) {
                const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
                const float *src = j < k - 1 ? rB + (size_t)slot_of(j) * NN : fB;
                bv[sl] = (s0 + sl < BS && j < k) ? *(const f32x4 *)(src + 4 * c4) : zero;
            }
        }
#pragma unroll
        for (int sl = 0; sl < BCH; ++sl) {
            const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
            if (s0 + sl < BS && j < LMAX) *(f32x4 *)&s.Bw[j][4 * c4] = bv[sl];
        }
    }
    if (tid < NN / 4) *(f32x4 *)&s.Cq[4 * tid] = cq;
    // w_j = dt_j * exp(A * sum_{i>j} dt_i), decay = exp(A * sum_i dt_i): suffix sums by shuffles
    float wj, decay;
    {
        float tail;
        const float sfx = suffix_sum<LMAX>(dtj, lane, &tail);
        wj = lane < k ? dtj * expf(Ah * tail) : 0.f;
        decay = expf(Ah * lane0(sfx));
    }
    __syncthreads();
    // 5. Scores g_j = B_j . C_t (GS threads per record).
    {
        constexpr int GS = kThreads / LMAX;
        const int j = tid / GS, sub = tid % GS;
        float gj = 0.f;
        if (j < k)
            for (int n = sub; n < NN; n += GS) gj = fmaf(s.Bw[j][n], s.Cq[n], gj);
        gj = group_sum<GS>(gj);
        if (sub == 0) s.g[j] = gj;
    }
    __syncthreads();
    const float cj = lane < LMAX ? wj * s.g[lane < LMAX ? lane : 0] : 0.f;  // lane j: w_j * g_j

    // 6. Row dot S_c[p,:] . C_t through the copy. C_t's chunk-column slice is the same for every
    //    lane: it is read from global memory at a wave-uniform address, which the compiler serves
    //    by scalar loads into SGPRs (operands of the FMAs; no LDS traffic, no C registers per
    //    lane -- broadcast LDS reads of the staged C cost 8 LDS cycles per 16 bytes). The empty asm
    //    ties each chunk's decode to the running sums, so chunks are decoded one at a time
    //    instead of all at once (which would hold N decoded values per lane).
    float u0 = 0.f, u1 = 0.f;
#pragma unroll
    for (int q = 0; q < NC; ++q) {
        asm("" : "+v"(v[q]), "+v"(u0), "+v"(u1));
        const float *cs = Ct + q * G::VEC;
        const unsigned w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            if constexpr (PREC == PREC_FP8) {
                const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
                const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
                a0 = fmaf(lo.x, cs[4 * i + 0], a0);
                a1 = fmaf(lo.y, cs[4 * i + 1], a1);
                a0 = fmaf(hi.x, cs[4 * i + 2], a0);
                a1 = fmaf(hi.y, cs[4 * i + 3], a1);
            } else {
                const f32x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 0);
                const f32x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 1);
                const f32x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 2);
                const f32x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 3);
                a0 = fmaf(b0.x, cs[8 * i + 0], a0);
                a1 = fmaf(b0.y, cs[8 * i + 1], a1);
                a0 = fmaf(b1.x, cs[8 * i + 2], a0);
                a1 = fmaf(b1.y, cs[8 * i + 3], a1);
                a0 = fmaf(b2.x, cs[8 * i + 4], a0);
                a1 = fmaf(b2.y, cs[8 * i + 5], a1);
                a0 = fmaf(b3.x, cs[8 * i + 6], a0);
                a1 = fmaf(b3.y, cs[8 * i + 7], a1);
            }
        }
        if constexpr (PREC == PREC_FP4) {
            const unsigned code = (scw[q / 4] >> (8 * (q % 4))) & 0xFFu;
            u0 += mx_scaled(a0 + a1, code);
        } else {
            u0 += a0;
            u1 += a1;
        }
    }
    float u = u0 + u1;
    if constexpr (PREC == PREC_FP8) u *= Ld.scale[bh];  // P <= 64 here: one scale block per head
    issue_x();

    if (bad) {
        raise_flag(Ld, FLAG_POINTERS);
        seq_done(Ld, t.b, Ld.pos[t.b], Ld.ckpt[t.b], HPB);
        return;
    }

    // 7. Combine: y = decay * u + sum_j (w_j g_j) x_j + D x_t; append the record.
    float acc = decay * u;
#pragma unroll
    for (int j = 0; j < LMAX; ++j)
        if (j < k) acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(cj), j)), xj[j], acc);
    acc = fmaf(Ld.D[h], xt, acc);
    if (prow) {
        io.y[bh * Ld.P + p] = acc;
        Ld.ring_x[(bh * Ld.L + pslot) * Ld.P + p] = xt;
    }
    if (lane == k - 1) Ld.ring_dt[bh * Ld.L + pslot] = dtj;
    if (t.h % Ld.hpg == 0 && tid < NN / 4) {
        const size_t off = (((size_t)t.b * Ld.G + t.g) * Ld.L + pslot) * NN + 4 * tid;
        *(f32x4 *)(Ld.ring_B + off) = *(const f32x4 *)&s.Bw[k - 1][4 * tid];
        if (Ld.ring_C) *(f32x4 *)(Ld.ring_C + off) = *(const f32x4 *)&s.Cq[4 * tid];
    }
    // pointer update, once per sequence (see step_kernel)
    if (uni) {
        if (t.h == 0 && tid == 0) {
            const int dp = Ld.pos[t.b], dc = Ld.ckpt[t.b];
            const bool ok = dc >= 0 && dp - dc == k - 1 && (int)((unsigned)dp % (unsigned)Ld.L) == pslot &&
                            (int)((unsigned)dc % (unsigned)Ld.L) == cslot;
            if (ok) Ld.pos[t.b] = dp + 1;
            else __hip_atomic_fetch_or(Ld.flag, FLAG_POINTERS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        const int pos = Ld.pos[t.b], ck = Ld.ckpt[t.b];
        seq_done(Ld, t.b, pos + 1, ck, HPB);
    }
}

// ==========================================================================================
// Flush step of an fp16 or fp8 master when every sequence of the launch flushes (lockstep
// decoding, or a host bound showing every buffer fills): fold all k records of the window into
// the master ([WittyWires] "What happened": the checkpoint is updated when the buffer fills),
// round it to fp16 (nearest even or stochastic) and rewrite the read copy -- or, F8M, encode it
// to E4M3 codes with the head's new scale (nearest even or stochastic), the fp8 master being its
// own read copy -- and read y from the stored master. The fold S' = decay * S + sum_j (w_j x_j)
// (outer) B_j is a rank-k update, a dense contraction: it runs on MFMA
// (v_mfma_f32_16x16x4_f32), leaving the VALU to the conversions, the rounding and its Philox
// stream.
//
// One work-group per (sequence, head), P <= 64: wave w owns rows 16w .. 16w+15. The product is
// formed transposed, D^T[n][p] += sum_j B_j[n] * (w_j x_j[p]), so that an MFMA tile's column is a
// row p of the state (lane l: p = 16w + l % 16) and its four output registers are four
// consecutive n of that row. Tile (q, hf) maps its row r to n = 32q + 8(r / 4) + 4hf + r % 4:
// lane group g = l / 16 then holds n = 32q + 8g .. 32q + 8g + 7 of tiles (q, 0) and (q, 1) --
// eight consecutive fp16 values, one 16-byte load and store per q (fp8 codes: 8 bytes of the
// row's chunk), and one Philox4x32-10 call for the eight 16-bit fields of its stochastic
// rounding. Per fp16 load instruction a wave reads 16 rows x 64 contiguous bytes.
// ==========================================================================================
template <int LMAX>
struct LpFlushLds {
    float w[LMAX];
    float decay;
    float red[kWaves];
    union {
        struct {
            float xw[LMAX][kRows] __attribute__((aligned(16)));  // x of each record, this head's rows
            float Bw[LMAX][NN + 4] __attribute__((aligned(16))); // B of each record; padded: the four
                                                                 // lane groups of a wave read four records
            float Cq[NN] __attribute__((aligned(16)));           // C of this token
        };
        // once the window is consumed: each wave's 16 stored fp16 rows, 16 bytes of padding per
        // row so that the staging writes (16 rows at one column) spread over the banks
        unsigned char tp[kWaves][16 * (2 * NN + 16)] __attribute__((aligned(16)));
    };
};

template <int PREC, int LMAX, bool SR, bool F8M>
__global__ void __launch_bounds__(kThreads) lp_flush_step_kernel(Layer Ld, TokenIO io, Lockstep ls)
{
    static_assert(PREC >= 0 && NN >= 32 && NN % 32 == 0, "lane groups cover 32 consecutive n per load slot");
    static_assert(!F8M || PREC == PREC_FP8, "an fp8 master is read as the fp8 copy");
    constexpr int NQ = NN >= 32 ? NN / 32 : 1;  // 16-byte fp16 loads per lane (eight values each)
    __shared__ LpFlushLds<LMAX> s;
    const Tile t = map_tile(Ld);  // psplit == 1 (host-checked): the work-group owns the head
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int pl = wave * 16 + c16;  // this lane's state row (the MFMA column)
    const bool prow = pl < t.nrows;
    const int pr = prow ? pl : 0;    // rows beyond P read row 0 and store nothing
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    const size_t rowe = (bh * Ld.P + pr) * NN;  // element offset of this lane's row

    // 1. Pointers: the window position (lockstep arguments, or this sequence's device pointers,
    //    validated before any address is formed). Every sequence of the launch must flush.
    const bool uni = ls.k > 0;
    int cslot = 0, k = 1, dpos = 0, dck = 0;
    if (uni) {
        cslot = ls.cslot;
        k = ls.k;
        if (!(k > Ld.L - Ld.Tmax && k <= Ld.L)) {  // the host launches this kernel for flush steps only
            raise_flag(Ld, FLAG_POINTERS);
            return;
        }
    } else {
        dpos = Ld.pos[t.b];
        dck = Ld.ckpt[t.b];
        const int c0 = dpos - dck;
        if (!(dck >= 0 && c0 >= 0 && c0 <= Ld.L - Ld.Tmax && c0 + 1 > Ld.L - Ld.Tmax)) {
            raise_flag(Ld, FLAG_POINTERS);
            seq_done(Ld, t.b, dpos, dck);
            return;
        }
        cslot = (int)((unsigned)dck % (unsigned)Ld.L);
        k = c0 + 1;
    }
    auto slot_of = [&](int j) { return ring_slot(cslot, j, Ld.L); };  // record j (< L)

    // 2. Window loads into registers (x rows, the group's B rows, this token's C, dt in wave 0),
    //    then the master rows: committing the window waits only for the window's loads.
    constexpr int XS = (LMAX * kRows / 4 + kThreads - 1) / kThreads;
    constexpr int BS = (LMAX * NN / 4 + kThreads - 1) / kThreads;
    constexpr int BCH = BS < 8 ? BS : 8;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const float *rx = Ld.ring_x + bh * Ld.L * Ld.P;
    const float *rB = Ld.ring_B + ((size_t)t.b * Ld.G + t.g) * Ld.L * NN;
    const float *fx = io.x + bh * Ld.P;
    const float *fB = io.B + ((size_t)t.b * Ld.G + t.g) * NN;
    const float *Ct = io.C + ((size_t)t.b * Ld.G + t.g) * NN;
    f32x4 xv[XS], bv[BCH], cq;
    float dtj = 0.f;
#pragma unroll
    for (int sl = 0; sl < XS; ++sl) {
        const int e = tid + sl * kThreads, j = e / (kRows / 4), c4 = e % (kRows / 4);
        const bool in = j < k && 4 * c4 < t.nrows;
        const float *src = (in && j < k - 1) ? rx + (size_t)slot_of(j) * Ld.P + 4 * c4 : fx + (in ? 4 * c4 : 0);
        const f32x4 val = *(const f32x4 *)src;
        xv[sl] = in ? val : zero;
    }
#pragma unroll
    for (int sl = 0; sl < BCH; ++sl) {
        const int e = tid + sl * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
        const float *src = (j < k - 1 ? rB + (size_t)slot_of(j) * NN : fB) + 4 * c4;
        const f32x4 val = *(const f32x4 *)src;
        bv[sl] = j < k ? val : zero;
    }
    {
        const f32x4 val = *(const f32x4 *)(Ct + 4 * (tid % (NN / 4)));
        cq = tid < NN / 4 ? val : zero;
    }
    if (wave == 0) {
        const bool in = lane < k;
        const float val = (in && lane < k - 1) ? Ld.ring_dt[bh * Ld.L + slot_of(lane)] : io.dt[bh];
        dtj = in ? val : 0.f;
    }
    const float Ah = Ld.A[t.h];
    // master rows: eight fp16 values (16 bytes) per q, or with an fp8 master eight codes (8 bytes
    // of the row's chunk n0 / 16) and the head's scale
    u32x4 mv[F8M ? 1 : NQ];
    u32x2 m8[F8M ? NQ : 1];
    float mscale = 1.0f;
    if constexpr (F8M) {
        const unsigned char *src = (const unsigned char *)Ld.rcopy;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int n0 = 32 * q + 8 * g;
            m8[q] = __builtin_nontemporal_load((const u32x2 *)(src + chunk_off<PREC_FP8>(bh, pr, n0 / 16, Ld.P) + n0 % 16));
        }
        mscale = Ld.scale[bh];
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            mv[q] = load_nt((const unsigned short *)Ld.master + rowe + 32 * q + 8 * g);
    }

    // SR: the Philox words depend on positions only; they are drawn while the window and master
    // loads are in flight (the empty asm keeps the compiler from sinking them past the barrier).
    const unsigned newck = (unsigned)(dpos + 1);  // stochastic rounding runs in device-pointer mode
    const size_t seq0 = (size_t)t.b * Ld.H * Ld.P * NN;
    unsigned wd[NQ][4];  // SR: the eight 16-bit fields of each group of eight values
    if constexpr (SR) {
        const unsigned e8 = (unsigned)((rowe - seq0) / 8) + (unsigned)g;  // first group's counter
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const U32x4 rnd = philox4x32_10(e8 + 4u * q, (unsigned)t.b, newck, 0u, Ld.sr_seed, 0u);
            wd[q][0] = rnd.x; wd[q][1] = rnd.y; wd[q][2] = rnd.z; wd[q][3] = rnd.w;
            asm volatile("" : "+v"(wd[q][0]), "+v"(wd[q][1]), "+v"(wd[q][2]), "+v"(wd[q][3]));
        }
    }

    // 3. Commit the window to LDS; the window's weights in wave 0 (suffix sums of dt by lane
    //    shuffles: w_j = dt_j exp(A sum_{i>j} dt_i), decay = exp(A sum_i dt_i)).
#pragma unroll
    for (int sl = 0; sl < XS; ++sl) {
        const int e = tid + sl * kThreads, j = e / (kRows / 4), c4 = e % (kRows / 4);
        if (j < LMAX) *(f32x4 *)&s.xw[j][4 * c4] = xv[sl];
    }
#pragma unroll
    for (int s0 = 0; s0 < BS; s0 += BCH) {
        if (s0 > 0) {
#pragma unroll
            for (int sl = 0; sl < BCH; ++sl) {
                const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
                const float *src = j < k - 1 ? rB + (size_t)slot_of(j) * NN : fB;
                bv[sl] = (s0 + sl < BS && j < k) ? *(const f32x4 *)(src + 4 * c4) : zero;
            }
        }
#pragma unroll
        for (int sl = 0; sl < BCH; ++sl) {
            const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
            if (s0 + sl < BS && j < LMAX) *(f32x4 *)&s.Bw[j][4 * c4] = bv[sl];
        }
    }
    if (tid < NN / 4) *(f32x4 *)&s.Cq[4 * tid] = cq;
    if (wave == 0) {
        float tail;
        const float sfx = suffix_sum<LMAX>(dtj, lane, &tail);
        if (lane < LMAX) s.w[lane] = lane < k ? dtj * expf(Ah * tail) : 0.f;
        if (lane == 0) s.decay = expf(Ah * sfx);
    }
    __syncthreads();

    // 4. S' = decay * S + sum_j B_j (outer) (w_j x_j), transposed, on MFMA: the accumulators start
    //    as decay * S (the master rows, converted exactly), then one MFMA per tile and four records.
    const float decay = s.decay;
    f32x4 acc[NQ][2];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if constexpr (F8M) {
            const float sd = mscale * decay;
            const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)m8[q].x, false);
            const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)m8[q].x, true);
            const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)m8[q].y, false);
            const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)m8[q].y, true);
            acc[q][0] = f32x4{a.x, a.y, b.x, b.y} * sd;
            acc[q][1] = f32x4{c.x, c.y, d.x, d.y} * sd;
        } else {
            const f32x2 a = f16x2_to_f32(mv[q].x), b = f16x2_to_f32(mv[q].y);
            const f32x2 c = f16x2_to_f32(mv[q].z), d = f16x2_to_f32(mv[q].w);
            acc[q][0] = f32x4{a.x, a.y, b.x, b.y} * decay;
            acc[q][1] = f32x4{c.x, c.y, d.x, d.y} * decay;
        }
    }
    const int ksteps = (k + 3) / 4;
    for (int kk = 0; kk < ksteps; ++kk) {
        const int j = 4 * kk + g;  // this lane group's record
        const bool jin = j < k;
        const int jr = jin ? j : 0;
        const float bop = jin ? s.w[jr] * s.xw[jr][pl] : 0.f;  // (w_j x_j)[p]
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int n = 32 * q + 8 * (c16 >> 2) + 4 * hf + (c16 & 3);  // tile row c16
                const float aop = jin ? s.Bw[jr][n] : 0.f;                    // B_j[n]
                acc[q][hf] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop, bop, acc[q][hf], 0, 0, 0);
            }
    }

    // 7. y = S_stored[p,:] . C_t + D x_t: partial dots over the lane's n, summed over the four
    //    lane groups of the row (acc holds the checkpoint as stored).
    auto write_output = [&]() {
        float yp = 0.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const f32x4 c0 = *(const f32x4 *)&s.Cq[32 * q + 8 * g];
            const f32x4 c1 = *(const f32x4 *)&s.Cq[32 * q + 8 * g + 4];
            const f32x4 a = acc[q][0], b = acc[q][1];
            yp = fmaf(a.x, c0.x, yp);
            yp = fmaf(a.y, c0.y, yp);
            yp = fmaf(a.z, c0.z, yp);
            yp = fmaf(a.w, c0.w, yp);
            yp = fmaf(b.x, c1.x, yp);
            yp = fmaf(b.y, c1.y, yp);
            yp = fmaf(b.z, c1.z, yp);
            yp = fmaf(b.w, c1.w, yp);
        }
        yp += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(yp), 0x401F));  // xor 16
        yp += __shfl_xor(yp, 32, 64);
        if (g == 0 && prow) io.y[bh * Ld.P + pl] = fmaf(Ld.D[t.h], s.xw[k - 1][pl], yp);
    };
    if constexpr (F8M) {
        // 5'. fp8 master: the head's amax, scale = amax / 448, codes of value / scale to nearest
        //     even (the converter) or by the 16-bit stochastic rule (e4m3_sr), stored in the
        //     row's chunks; acc then holds code * scale, the checkpoint as stored.
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const f32x4 a = acc[q][hf];
                const float m = fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w)));
                amax = prow ? fmaxf(amax, m) : amax;
            }
        amax = block_max(amax, s.red);
        const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
        const float inv = 1.0f / scale;
        unsigned char *dst = (unsigned char *)Ld.rcopy;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const f32x4 a = acc[q][0], b = acc[q][1];
            const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            float c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                c[i] = fminf(fmaxf(f[i] * inv, -448.0f), 448.0f);
                if constexpr (SR) c[i] = e4m3_sr(c[i], (wd[q][i / 2] >> (16 * (i % 2))) & 0xFFFFu);
            }
            int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
            lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
            int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
            hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], hi, true);
            const int n0 = 32 * q + 8 * g;
            if (prow) *(u32x2 *)(dst + chunk_off<PREC_FP8>(bh, pr, n0 / 16, Ld.P) + n0 % 16) = u32x2{(unsigned)lo, (unsigned)hi};
            const f32x2 d0 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false), d1 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
            const f32x2 d2 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false), d3 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
            acc[q][0] = f32x4{d0.x, d0.y, d1.x, d1.y} * scale;
            acc[q][1] = f32x4{d2.x, d2.y, d3.x, d3.y} * scale;
        }
        if (tid == 0) Ld.scale[bh] = scale;
    } else {
        // 5. Round to fp16 and store the master; acc then holds the stored values (the flush's
        //    output and the read copy come from the checkpoint as stored). In fp16's normal range
        //    both roundings are integer operations on the fp32 encoding whose result is the rounded
        //    value itself, exact in fp32 (13 low mantissa bits cleared): nearest even adds
        //    0xFFF + bit 13; the stochastic rule adds 2^13 - 1 - (r16 >> 3) (see f16_sr). The codes
        //    are then packed by the round-toward-zero converter, exact on representable values. A
        //    wave with a value below 2^-14 redoes those values with the general routines.
        bool sub = false;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x4 &a = acc[q][hf];
                float r[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = 4 * hf + i;  // element within the group of eight
                    const float c = __builtin_amdgcn_fmed3f(r[i], -65504.0f, 65504.0f);
                    const unsigned u = __float_as_uint(c);
                    // SR: the 13-bit complement of r16 >> 3 is bits 3 .. 15 of the field, inverted
                    unsigned add;
                    if constexpr (SR) add = (~wd[q][e / 2] >> (3 + 16 * (e % 2))) & 0x1FFFu;
                    else add = 0xFFFu + ((u >> 13) & 1u);
                    sub |= fabsf(c) < 0x1p-14f;
                    r[i] = __uint_as_float((u + add) & ~0x1FFFu);
                }
                // keep the unrounded values for the rare fix-up below
                if (__builtin_expect(__builtin_amdgcn_ballot_w64(sub) != 0, 0)) {
                    const float o[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = 4 * hf + i;
                        if (fabsf(o[i]) < 0x1p-14f) {
                            unsigned short hc;
                            if constexpr (SR) hc = f16_sr(o[i], (wd[q][e / 2] >> (16 * (e % 2))) & 0xFFFFu);
                            else hc = f16_rne(o[i]);
                            r[i] = f16_value(hc);
                        }
                    }
                    sub = false;
                }
                a = f32x4{r[0], r[1], r[2], r[3]};
            }
        write_output();
        // Nearest even: the codes go out in whole rows. A lane's 16 bytes per q cover 64 bytes of
        // each of 16 rows per store instruction (half lines, which the counters show written back
        // at 1.1-1.3x the bytes), so each wave stages its 16 rows through LDS (the window's space,
        // free once every wave has formed its output) and writes them back as 4 rows = 1 KiB per
        // instruction: 253-259 -> 220-227 us at batch 256. The stochastic variants are bound by
        // their VALU work rather than by HBM, and there the extra barrier and LDS round trip cost
        // more than they save (fp16 SR 309-312 -> 314-317 us): they store the fragments directly.
        if constexpr (SR) {
            unsigned short *mdst = (unsigned short *)Ld.master + rowe + 8 * g;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (prow) {
                    const f32x4 a = acc[q][0], b = acc[q][1];
                    u32x4 pk;
                    pk.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a.x, a.y));
                    pk.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a.z, a.w));
                    pk.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(b.x, b.y));
                    pk.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(b.z, b.w));
                    store_nt(mdst + 32 * q, pk);
                }
            }
        } else {
            __syncthreads();
            constexpr int RB = 2 * NN + 16;  // staged row bytes (padded)
            constexpr int GR = 2 * NN / 16;  // 16-byte granules per row
            unsigned char *tw = s.tp[wave];
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 a = acc[q][0], b = acc[q][1];
                u32x4 pk;
                pk.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a.x, a.y));
                pk.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a.z, a.w));
                pk.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(b.x, b.y));
                pk.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(b.z, b.w));
                *(u32x4 *)(tw + c16 * RB + 2 * (32 * q + 8 * g)) = pk;
            }
            // a wave reads back only the rows it staged (its LDS accesses stay in order)
            unsigned char *mrow = (unsigned char *)Ld.master + (bh * Ld.P + wave * 16) * (2 * NN);
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int e = i * 64 + lane, r = e / GR, c = e % GR;
                const u32x4 v = *(const u32x4 *)(tw + r * RB + 16 * c);
                if (wave * 16 + r < t.nrows) store_nt(mrow + r * (2 * NN) + 16 * c, v);
            }
        }

        // 6. Read copy from the stored master.
        if constexpr (PREC == PREC_BF16) {
            unsigned short *dst = (unsigned short *)Ld.rcopy + rowe + 8 * g;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 a = acc[q][0], b = acc[q][1];
                const u32x4 pk = {bf16_rne(a.x) | (bf16_rne(a.y) << 16), bf16_rne(a.z) | (bf16_rne(a.w) << 16),
                                  bf16_rne(b.x) | (bf16_rne(b.y) << 16), bf16_rne(b.z) | (bf16_rne(b.w) << 16)};
                if (prow) *(u32x4 *)(dst + 32 * q) = pk;
            }
        } else if constexpr (PREC == PREC_FP8) {
            float amax = 0.f;
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const f32x4 a = acc[q][hf];
                    const float m = fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w)));
                    amax = prow ? fmaxf(amax, m) : amax;
                }
            amax = block_max(amax, s.red);
            const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
            const float inv = 1.0f / scale;
            unsigned char *dst = (unsigned char *)Ld.rcopy;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 a = acc[q][0], b = acc[q][1];
                const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                float c[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) c[i] = fminf(fmaxf(f[i] * inv, -448.0f), 448.0f);
                int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
                lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
                int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
                hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], hi, true);
                const int n0 = 32 * q + 8 * g;  // 16-value chunk n0 / 16, byte n0 % 16 within it
                if (prow) *(u32x2 *)(dst + chunk_off<PREC_FP8>(bh, pr, n0 / 16, Ld.P) + n0 % 16) = u32x2{(unsigned)lo, (unsigned)hi};
            }
            if (tid == 0) Ld.scale[bh] = scale;
        } else if constexpr (PREC == PREC_FP4) {
            // block q (32 consecutive n of the row) is spread over the four lane groups of this row
            unsigned char *dst = (unsigned char *)Ld.rcopy;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 a = acc[q][0], b = acc[q][1];
                float amax = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                                   fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
                // the row's four lane groups: LDS-pipe exchanges keep these off the VALU
                amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(amax), 0x401F)));
                amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
                const unsigned code = mx_code_of(amax);
                const unsigned lo = mx_encode4(a, code), hi = mx_encode4(b, code);
                if (prow) {
                    *(unsigned *)(dst + chunk_off<PREC_FP4>(bh, pr, q, Ld.P) + 4 * g) = lo | (hi << 16);
                    if (g == 0) Ld.mxscale[(bh * Ld.P + pr) * (NN / 32) + q] = (unsigned char)code;
                }
            }
        }
    }

    if constexpr (F8M) write_output();

    // 8. Pointers (the token's record is folded already: nothing is appended).
    if (uni) {
        if (t.h == 0 && tid == 0) {
            const int dp = Ld.pos[t.b], dc = Ld.ckpt[t.b];
            const bool ok = dc >= 0 && dp - dc == k - 1 && (int)((unsigned)dp % (unsigned)Ld.L) == ls.pslot &&
                            (int)((unsigned)dc % (unsigned)Ld.L) == cslot;
            if (ok) {
                Ld.pos[t.b] = dp + 1;
                Ld.ckpt[t.b] = dp + 1;
            } else {
                __hip_atomic_fetch_or(Ld.flag, FLAG_POINTERS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    } else {
        seq_done(Ld, t.b, dpos + 1, dpos + 1);
    }
}

// ==========================================================================================
// Flush / commit-flush / materialize. MODE_MASK: fold every committed record of the selected
// sequences. MODE_OVERFULL (after a rollback moved pos by the accepted count -- rejected drafts
// are dropped by that pointer move, [AT Pulse] "Technical analysis"): fold the sequences with
// more than L - Tmax pending records. MODE_MATERIALIZE: write checkpoint + committed records to
// `out`, commit nothing. Work-groups of sequences that do not fold exit at once.
// ==========================================================================================
template <int LMAX>
struct FlushLds {
    Window<LMAX> win;
    float w[LMAX];
    float red[kWaves];
    float decay;
};

template <int PREC, int LMAX>
__global__ void __launch_bounds__(kThreads) flush_kernel(Layer Ld, int mode, const int *arg, float *out)
{
    __shared__ FlushLds<LMAX> s;
    const Tile t = map_tile(Ld);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    const size_t elem0 = (bh * Ld.P + t.row0) * NN;

    const int pos = Ld.pos[t.b], ck = Ld.ckpt[t.b];
    const int count = pos - ck;
    const int cap = mode == MODE_OVERFULL ? Ld.L : Ld.L - Ld.Tmax;
    if (!(ck >= 0 && count >= 0 && count <= cap)) {
        raise_flag(Ld, FLAG_POINTERS);
        return;
    }
    bool fold;
    if (mode == MODE_OVERFULL) fold = count > Ld.L - Ld.Tmax;
    else if (mode == MODE_MASK) fold = (arg == nullptr || arg[t.b] != 0) && count > 0;
    else fold = true;
    if (!fold) return;  // pointers unchanged: no completion count needed
    {
        f32x4 vf[GF::NL];
        load_master_rows(Ld, elem0, vf, t.nrows, wave, lane);
        const RecSrc src = ring_src(Ld, t, ck, count);
        WindowRegs<LMAX> wr;
        issue_window<LMAX>(wr, src, count, t.nrows);
        commit_window<LMAX>(s.win, wr, src, count);
        __syncthreads();
        window_weights<LMAX, false>(s.win, nullptr, count - 1, Ld.A[t.h], s.w, nullptr, &s.decay);
        __syncthreads();
        fold_head<LMAX, kRows>(vf, s.win.xw, s.win.Bw, s.w, s.decay, 0, count, wave, lane);
        if (mode == MODE_MATERIALIZE) {
            store_rows_f32(out + elem0, vf, t.nrows, wave, lane);
        } else {
            commit_rows<PREC>(Ld, t.b, bh, elem0, pos, sr_master(Ld), vf, t.nrows, wave, lane, s.red);
        }
    }
    if (mode != MODE_MATERIALIZE) seq_done(Ld, t.b, pos, pos);
}

// Rollback pointer move: pos += accepted[b] (0..T). One thread per sequence; a count out of
// range, or pointers that break the invariant, raise the flag and leave the sequence as it was.
__global__ void advance_kernel(Layer Ld, const int *accepted, int T)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= Ld.Bt) return;
    const int pos = Ld.pos[b], ck = Ld.ckpt[b];
    if (!(ck >= 0 && pos - ck >= 0 && pos - ck <= Ld.L - Ld.Tmax)) {
        __hip_atomic_fetch_or(Ld.flag, FLAG_POINTERS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int a = accepted[b];
    if (a < 0 || a > T) {
        __hip_atomic_fetch_or(Ld.flag, FLAG_ACCEPTED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    Ld.pos[b] = pos + a;
}

// ==========================================================================================
// Speculative verify ([AT Pulse] "Technical analysis": output-only evaluation, no intermediate
// state). One pass over the checkpoint rows serves all T queries: U = S_c . [C_1 .. C_T]. Query
// q's window is the committed records plus drafts 0..q. Drafts are appended tentatively at
// slots (pos + q) mod L; the pointers do not move.
// ==========================================================================================
template <int LMAX, int TQ>
struct VerifyLds {
    Window<LMAX> win;
    float Cq[TQ][NN] __attribute__((aligned(16)));
    float gq[TQ][LMAX];  // B_j . C_q
    float coef[TQ][LMAX];
    float u[TQ][kRows];
    float decay[TQ];
};

template <int PREC, int LMAX, int TQ, bool MIX>
__global__ void __launch_bounds__(kThreads) verify_kernel(Layer Ld, TokenIO io, int T)
{
    using G = Geo<NN, PREC>;
    __shared__ VerifyLds<LMAX, TQ> s;
    const Tile t = map_tile(Ld);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    const size_t elem0 = (bh * Ld.P + t.row0) * NN;
    const char *rbase = (PREC == PREC_F32 || PREC == PREC_F16) ? (const char *)Ld.master : (const char *)Ld.rcopy;
    u32x4 v[G::NL];
#pragma unroll
    for (int i = 0; i < G::NL; ++i) {
        const int r = row_of<PREC>(i, wave, lane), rr = r < t.nrows ? r : 0;
        v[i] = load_nt(rbase + chunk_off<PREC>(bh, t.row0 + rr, lane % G::LPR, Ld.P));
    }
    unsigned sc[G::NL];
    if constexpr (PREC == PREC_FP4) load_mxscales<PREC>(sc, Ld.mxscale + elem0 / 32, t.nrows, wave, lane);

    const int pos = Ld.pos[t.b], ck = Ld.ckpt[t.b];
    const int count0 = pos - ck;
    if (!(ck >= 0 && count0 >= 0 && count0 <= Ld.L - Ld.Tmax && count0 + T <= Ld.L)) {
        raise_flag(Ld, FLAG_POINTERS);
        return;
    }
    const int kw = count0 + T;
    RecSrc src = ring_src(Ld, t, ck, count0);
    constexpr int CQS = (TQ * (NN / 4) + kThreads - 1) / kThreads;
    WindowRegs<LMAX> wr;
    if constexpr (!MIX) {
        src.fx = io.x + ((size_t)t.b * T * Ld.H + t.h) * Ld.P + t.row0;
        src.sx = Ld.H * Ld.P;
        src.fB = io.B + ((size_t)t.b * T * Ld.G + t.g) * NN;
        src.sB = Ld.G * NN;
        src.fdt = io.dt + (size_t)t.b * T * Ld.H + t.h;
        src.sdt = Ld.H;
        f32x4 cqr[CQS];
#pragma unroll
        for (int i = 0; i < CQS; ++i) {
            const int e = tid + i * kThreads, q = e / (NN / 4), c = e % (NN / 4);
            cqr[i] = q < T ? *(const f32x4 *)(io.C + (((size_t)t.b * T + q) * Ld.G + t.g) * NN + 4 * c)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        issue_window<LMAX>(wr, src, kw, t.nrows);
        commit_window<LMAX>(s.win, wr, src, kw);
#pragma unroll
        for (int i = 0; i < CQS; ++i) {
            const int e = tid + i * kThreads, q = e / (NN / 4), c = e % (NN / 4);
            if (q < TQ) *(f32x4 *)&s.Cq[q][4 * c] = cqr[i];
        }
    } else {
        // Mixer edges: the committed records come from the ring; draft q (position pos + q) is
        // formed here by the causal conv over the ring's history (positions < pos) and the
        // drafts' raw xBC (positions >= pos), SiLU, softplus dt. The drafts' raw values enter the
        // ring at slots (pos + q) mod R, which never hold a position the history still needs
        // (R = K - 1 + T_max).
        issue_window<LMAX>(wr, src, count0, t.nrows);
        commit_window<LMAX>(s.win, wr, src, count0);
        __syncthreads();  // the draft rows below overwrite the window's zero fill
        const int R = Ld.R, K = Ld.K;
        const bool leader = t.split == 0 && t.h % Ld.hpg == 0;
        auto draft_channel = [&](int q, int c) {
            const float *w = Ld.conv_w + (size_t)c * K;
            float u = Ld.conv_b[c];
            for (int i = 0; i < K; ++i) {
                const int d = q - (K - 1) + i;  // position pos + d (negative before the first token)
                const int sl = ((pos + d) % R + R) % R;
                const float v = d >= 0 ? io.xbc[((size_t)t.b * T + d) * Ld.CD + c]
                                       : Ld.conv_ring[ring_at(Ld, t.b, c, sl)];
                u = fmaf(w[i], v, u);
            }
            if (leader || c < Ld.H * Ld.P)
                Ld.conv_ring[ring_at(Ld, t.b, c, (int)((unsigned)(pos + q) % (unsigned)R))] =
                    io.xbc[((size_t)t.b * T + q) * Ld.CD + c];
            return silu_f(u);
        };
        for (int e = tid; e < T * kRows; e += kThreads) {
            const int q = e / kRows, p = e % kRows;
            if (p < t.nrows) s.win.xw[count0 + q][p] = draft_channel(q, t.h * Ld.P + t.row0 + p);
        }
        for (int e = tid; e < T * 2 * NN; e += kThreads) {
            const int q = e / (2 * NN), n = e % (2 * NN);
            const int c = Ld.H * Ld.P + (n < NN ? t.g * NN + n : Ld.G * NN + t.g * NN + (n - NN));
            const float v = draft_channel(q, c);
            if (n < NN) s.win.Bw[count0 + q][n] = v;
            else s.Cq[q][n - NN] = v;
        }
        if (tid < T) s.win.dts[count0 + tid] = softplus_f(io.dt[((size_t)t.b * T + tid) * Ld.H + t.h] + Ld.dt_bias[t.h]);
        for (int e = tid; e < (TQ - T) * NN; e += kThreads) s.Cq[T + e / NN][e % NN] = 0.f;
    }
    __syncthreads();  // s.Cq complete

    // Scores B_j . C_q for every query (GS threads per record, the B row read once for all q) and
    // the window weights come first: they need only the window, so they run while the tile's rows
    // are still arriving, and the row products follow.
    {
        constexpr int GS = kThreads / LMAX;
        const int j = tid / GS, sub = tid % GS;
        float g[TQ];
#pragma unroll
        for (int q = 0; q < TQ; ++q) g[q] = 0.f;
        if (j < kw) {
            for (int n = sub; n < NN; n += GS) {
                const float bjn = s.win.Bw[j][n];
#pragma unroll
                for (int q = 0; q < TQ; ++q) g[q] = fmaf(bjn, s.Cq[q][n], g[q]);
            }
        }
#pragma unroll
        for (int q = 0; q < TQ; ++q)
            g[q] = group_sum<GS>(g[q]);
        if (sub == 0)
#pragma unroll
            for (int q = 0; q < TQ; ++q) s.gq[q][j] = g[q];
    }
    __syncthreads();

    // Weights of query q (its window: records 0 .. count0 + q) in wave q mod 4: suffix sums of
    // dt by lane shuffles ([AT Pulse] "Technical analysis": the unrolled window).
    const float A = Ld.A[t.h];
    for (int q = wave; q < T; q += kWaves) {
        const int last = count0 + q;
        const float d = lane <= last && lane < LMAX ? s.win.dts[lane] : 0.f;
        float tail;
        const float sfx = suffix_sum<LMAX>(d, lane, &tail);
        const float total = lane0(sfx);
        if (lane < LMAX) s.coef[q][lane] = lane <= last ? d * expf(A * tail) * s.gq[q][lane] : 0.f;
        if (lane == 0) s.decay[q] = expf(A * total);
    }
    __syncthreads();

    // S_c C_q one query at a time (its C chunk from LDS): the tile's rows stay in registers while a
    // pass holds one chunk set and NL partial sums -- 62 registers at fp32 against 78 with every
    // query's chunks and partial sums live at once, so 8 waves per SIMD instead of 6.
    constexpr int QB = 1;
    const float scl = PREC == PREC_FP8 ? Ld.scale[bh * Ld.psplit + t.split] : 1.0f;
#pragma unroll
    for (int q0 = 0; q0 < TQ; q0 += QB) {
        if (q0 >= T) break;
        float cc[QB][G::VEC];
#pragma unroll
        for (int q = 0; q < QB; ++q) load_cchunk<PREC>(cc[q], s.Cq[q0 + q], lane);
        float part[G::NL * QB];
#pragma unroll
        for (int q = 0; q < QB; ++q)
#pragma unroll
            for (int i = 0; i < G::NL; ++i) {
                part[q * G::NL + i] = chunk_dot<PREC>(v[i], cc[q]);
                if constexpr (PREC == PREC_FP4) part[q * G::NL + i] = mx_scaled(part[q * G::NL + i], sc[i]);
            }
        rows_to_lds<PREC, G::NL * QB>(part, &s.u[q0][0], kRows, T - q0, G::NL, scl, wave, lane);
    }
    __syncthreads();

    // Combine: wave q mod 4 forms query q's output rows; then the tentative appends.
    const float Dh = Ld.D[t.h];
    const int pslot0 = (int)((unsigned)pos % (unsigned)Ld.L);  // draft q goes to slot (pos + q) mod L
    for (int q = wave; q < T; q += kWaves) {
        if (lane < t.nrows) {
            const int last = count0 + q;
            float acc = s.decay[q] * s.u[q][lane];
            for (int j = 0; j <= last; ++j) acc = fmaf(s.coef[q][j], s.win.xw[j][lane], acc);
            acc = fmaf(Dh, s.win.xw[last][lane], acc);
            if constexpr (MIX) acc *= silu_f(io.z[(((size_t)t.b * T + q) * Ld.H + t.h) * Ld.P + t.row0 + lane]);
            io.y[(((size_t)t.b * T + q) * Ld.H + t.h) * Ld.P + t.row0 + lane] = acc;
            Ld.ring_x[(bh * Ld.L + ring_slot(pslot0, q, Ld.L)) * Ld.P + t.row0 + lane] = s.win.xw[last][lane];
        }
        if (t.split == 0 && lane == 0) Ld.ring_dt[bh * Ld.L + ring_slot(pslot0, q, Ld.L)] = s.win.dts[count0 + q];
    }
    if (t.split == 0 && t.h % Ld.hpg == 0) {
        for (int e = tid; e < T * (NN / 4); e += kThreads) {
            const int q = e / (NN / 4), c4 = e % (NN / 4);
            const size_t off = (((size_t)t.b * Ld.G + t.g) * Ld.L + ring_slot(pslot0, q, Ld.L)) * NN + 4 * c4;
            *(f32x4 *)(Ld.ring_B + off) = *(const f32x4 *)&s.win.Bw[count0 + q][4 * c4];
            if (Ld.ring_C) *(f32x4 *)(Ld.ring_C + off) = *(const f32x4 *)&s.Cq[q][4 * c4];
        }
    }
}

// ==========================================================================================
// Load: master <- state, read copy encoded from it, pointers and counters reset, flag cleared.
// ==========================================================================================
template <int PREC>
__global__ void __launch_bounds__(kThreads) load_state_kernel(Layer Ld, const float *state)
{
    __shared__ float red[kWaves];
    const Tile t = map_tile(Ld);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    const size_t elem0 = (bh * Ld.P + t.row0) * NN;
    u32x4 m[GF::NL];
    load_rows<PREC_F32>(m, (const char *)(state + elem0), t.nrows, wave, lane);
    f32x4 vf[GF::NL];
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) vf[i] = as_f32x4(m[i]);
    commit_rows<PREC, PREC == PREC_F32>(Ld, t.b, bh, elem0, 0, false, vf, t.nrows, wave, lane, red);  // nearest even at load
    if (t.h == 0 && t.split == 0 && threadIdx.x == 0) {
        Ld.pos[t.b] = 0;
        Ld.ckpt[t.b] = 0;
        Ld.counter[t.b] = 0u;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *Ld.flag = 0u;
}

// ==========================================================================================
// Baseline: conventional decode step, in place ([Clarity] "Why it matters", claim ledger [6],
// [7]): S <- exp(dt A) S + dt x (outer) B; y = S . C + D x.
// ==========================================================================================
__global__ void __launch_bounds__(kThreads) conventional_kernel(Layer Ld, float *state, TokenIO io)
{
    __shared__ float u[kRows];
    const Tile t = map_tile(Ld);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    float *rows = state + (bh * Ld.P + t.row0) * NN;
    u32x4 m[GF::NL];
    load_rows<PREC_F32>(m, (const char *)rows, t.nrows, wave, lane);
    const float dtv = io.dt[bh];
    const float a = expf(dtv * Ld.A[t.h]);
    const float *Bt = io.B + ((size_t)t.b * Ld.G + t.g) * NN;
    const float *Ct = io.C + ((size_t)t.b * Ld.G + t.g) * NN;
    const float *xr = io.x + bh * Ld.P + t.row0;
    float bc[4], cc[4];
    load_cchunk<PREC_F32>(bc, Bt, lane);
    load_cchunk<PREC_F32>(cc, Ct, lane);
    float part[GF::NL];
    f32x4 vf[GF::NL];
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of<PREC_F32>(i, wave, lane);
        const float dx = r < t.nrows ? dtv * xr[r] : 0.f;
        f32x4 sv = as_f32x4(m[i]);
        sv.x = fmaf(dx, bc[0], a * sv.x);
        sv.y = fmaf(dx, bc[1], a * sv.y);
        sv.z = fmaf(dx, bc[2], a * sv.z);
        sv.w = fmaf(dx, bc[3], a * sv.w);
        vf[i] = sv;
        part[i] = chunk_dot<PREC_F32>(as_u32x4(sv), cc);
    }
    store_rows_f32(rows, vf, t.nrows, wave, lane);
    rows_to_lds<PREC_F32, GF::NL>(part, u, 0, 1, GF::NL, 1.0f, wave, lane);
    __syncthreads();
    if (tid < t.nrows) io.y[bh * Ld.P + t.row0 + tid] = fmaf(Ld.D[t.h], xr[tid], u[tid]);
}

// ==========================================================================================
// Baseline with the mixer edges: the conventional step of the same layer with the same fused
// edges as the replay's mixer step (conv over a ring of K raw inputs at slot rslot = t mod K,
// softplus dt, gated output), so that the comparison measures the state traffic only.
// ==========================================================================================
__global__ void __launch_bounds__(kThreads) conventional_mixer_kernel(Layer Ld, float *state, TokenIO io, int rslot)
{
    __shared__ float u[kRows], xs[kRows], bs[NN], cs[NN];
    const Tile t = map_tile(Ld);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    float *rows = state + (bh * Ld.P + t.row0) * NN;
    u32x4 m[GF::NL];
    load_rows<PREC_F32>(m, (const char *)rows, t.nrows, wave, lane);
    const float dtv = softplus_f(io.dt[bh] + Ld.dt_bias[t.h]);
    const float a = expf(dtv * Ld.A[t.h]);
    const float *raw = io.xbc + (size_t)t.b * Ld.CD;
    float zg = 0.f;
    if (tid < kRows) {
        const bool in = tid < t.nrows;
        const int c = t.h * Ld.P + t.row0 + (in ? tid : 0);
        const ConvIn ci = conv_issue(Ld, t.b, c, rslot, raw);
        zg = io.z[bh * Ld.P + t.row0 + (in ? tid : 0)];
        xs[tid] = in ? conv_finish(ci) : 0.f;
        if (in) Ld.conv_ring[ring_at(Ld, t.b, c, rslot)] = ci.cur;
    }
    const bool leader = t.split == 0 && t.h % Ld.hpg == 0;
    for (int e = tid; e < 2 * NN; e += kThreads) {
        const int c = Ld.H * Ld.P + (e < NN ? t.g * NN + e : Ld.G * NN + t.g * NN + (e - NN));
        const ConvIn ci = conv_issue(Ld, t.b, c, rslot, raw);
        const float v = conv_finish(ci);
        if (e < NN) bs[e] = v;
        else cs[e - NN] = v;
        if (leader) Ld.conv_ring[ring_at(Ld, t.b, c, rslot)] = ci.cur;
    }
    __syncthreads();
    float bc[4], cc[4];
    load_cchunk<PREC_F32>(bc, bs, lane);
    load_cchunk<PREC_F32>(cc, cs, lane);
    float part[GF::NL];
    f32x4 vf[GF::NL];
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of<PREC_F32>(i, wave, lane);
        const float dx = r < t.nrows ? dtv * xs[r] : 0.f;
        f32x4 sv = as_f32x4(m[i]);
        sv.x = fmaf(dx, bc[0], a * sv.x);
        sv.y = fmaf(dx, bc[1], a * sv.y);
        sv.z = fmaf(dx, bc[2], a * sv.z);
        sv.w = fmaf(dx, bc[3], a * sv.w);
        vf[i] = sv;
        part[i] = chunk_dot<PREC_F32>(as_u32x4(sv), cc);
    }
    store_rows_f32(rows, vf, t.nrows, wave, lane);
    rows_to_lds<PREC_F32, GF::NL>(part, u, 0, 1, GF::NL, 1.0f, wave, lane);
    __syncthreads();
    if (tid < t.nrows) io.y[bh * Ld.P + t.row0 + tid] = fmaf(Ld.D[t.h], xs[tid], u[tid]) * silu_f(zg);
}

// ==========================================================================================
// Baseline: per-draft snapshots ([Clarity] "What happened", claim ledger [13]). Reads the
// committed slot once, runs the T drafts stepwise and writes the state after draft q to slot
// (cur + q + 1) mod (T + 1): one read and T writes of the state per verify.
// ==========================================================================================
template <int TQ>
__global__ void __launch_bounds__(kThreads) snapshot_verify_kernel(Layer Ld, float *slots, const int *cur,
                                                                   int T, TokenIO io)
{
    __shared__ float u[TQ][kRows];
    const Tile t = map_tile(Ld);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c0 = cur[t.b];
    if (c0 < 0 || c0 > T) return;  // invalid slot index: nothing is read or written
    const size_t tile = (size_t)Ld.P * NN;
    auto slot_rows = [&](int sl) {
        return slots + (((size_t)t.b * (T + 1) + sl) * Ld.H + t.h) * tile + (size_t)t.row0 * NN;
    };
    u32x4 m[GF::NL];
    load_rows<PREC_F32>(m, (const char *)slot_rows(c0), t.nrows, wave, lane);
    f32x4 vf[GF::NL];
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) vf[i] = as_f32x4(m[i]);
    const float A = Ld.A[t.h];
    float part[GF::NL * TQ];
#pragma unroll
    for (int q = 0; q < TQ; ++q) {
        if (q < T) {
            const size_t bq = (size_t)t.b * T + q;
            const float dtv = io.dt[bq * Ld.H + t.h];
            const float a = expf(dtv * A);
            float bc[4], cc[4];
            load_cchunk<PREC_F32>(bc, io.B + (bq * Ld.G + t.g) * NN, lane);
            load_cchunk<PREC_F32>(cc, io.C + (bq * Ld.G + t.g) * NN, lane);
            const float *xr = io.x + (bq * Ld.H + t.h) * Ld.P + t.row0;
#pragma unroll
            for (int i = 0; i < GF::NL; ++i) {
                const int r = row_of<PREC_F32>(i, wave, lane);
                const float dx = r < t.nrows ? dtv * xr[r] : 0.f;
                f32x4 sv = vf[i];
                sv.x = fmaf(dx, bc[0], a * sv.x);
                sv.y = fmaf(dx, bc[1], a * sv.y);
                sv.z = fmaf(dx, bc[2], a * sv.z);
                sv.w = fmaf(dx, bc[3], a * sv.w);
                vf[i] = sv;
                part[q * GF::NL + i] = chunk_dot<PREC_F32>(as_u32x4(sv), cc);
            }
            store_rows_f32(slot_rows((c0 + q + 1) % (T + 1)), vf, t.nrows, wave, lane);
        } else {
#pragma unroll
            for (int i = 0; i < GF::NL; ++i) part[q * GF::NL + i] = 0.f;
        }
    }
    rows_to_lds<PREC_F32, GF::NL * TQ>(part, &u[0][0], kRows, T, GF::NL, 1.0f, wave, lane);
    __syncthreads();
    if (tid < t.nrows) {
        const float Dh = Ld.D[t.h];
        for (int q = 0; q < T; ++q) {
            const size_t bq = (size_t)t.b * T + q;
            const float xv = io.x[(bq * Ld.H + t.h) * Ld.P + t.row0 + tid];
            io.y[(bq * Ld.H + t.h) * Ld.P + t.row0 + tid] = fmaf(Dh, xv, u[q][tid]);
        }
    }
}

// ------------------------------------------------------------------------------------------
// Launch helpers.
// ------------------------------------------------------------------------------------------
inline unsigned nblocks(const Layer &Ld) { return (unsigned)Ld.Bt * (unsigned)Ld.H * (unsigned)Ld.psplit; }

template <int PREC, int LMAX, int ROWS, int FLUSH, bool MIX>
hipError_t step_rows(const Layer &Ld, const TokenIO &io, Lockstep ls, hipStream_t st)
{
    const unsigned grid = nblocks(Ld) / (ROWS / kRows);
    hipLaunchKernelGGL((step_kernel<PREC, LMAX, ROWS, FLUSH, MIX>), dim3(grid), dim3(kThreads), 0, st, Ld, io, ls);
    return hipGetLastError();
}

// Heads per work-group: 1 for fp32 (two fp32 heads per work-group measured no faster: the
// occupancy drops from 8 to 4 work-groups per CU); for the narrow copies as many as make
// ~32 KiB of checkpoint per work-group (bf16 2, fp8 4; fp4 4 as well, 16 KiB, since the
// transpose-reduce needs at most LPR load slots per lane), when the head tile fits one work-group
// (P <= 64), the group divides evenly, the launch keeps at least 2048 work-groups (8 per CU) and
// the window bucket is at most 32 (at 64 the x window of four heads fills 100 KiB of LDS).
// Flush-capable launches use one head per work-group (their fold loop is per head), except with an
// fp16 master: a head's fp16 rows are half the bytes, so two heads per work-group with their rows
// issued together keep the flush's bytes in flight (one head each: 2.6 TB/s on the flush step).
// MIX: the mixer edges fused in (no one-row-per-lane variant).
template <int PREC, int LMAX, bool MIX>
hipError_t step_t(const Layer &Ld, const TokenIO &io, bool flush_capable, bool all_flush, Lockstep ls,
                  hipStream_t st)
{
    constexpr int wide = PREC == PREC_F32 ? 1 : (PREC == PREC_BF16 || PREC == PREC_F16) ? 2 : 4;  // fp8, fp4: 4
    if (flush_capable) {
        // fp16 master, every sequence flushes: the fold on MFMA, one work-group per head
        if constexpr (!MIX && NN >= 32)
            if (all_flush && (Ld.mprec == MASTER_F16 || Ld.mprec == MASTER_F16_SR) && Ld.psplit == 1 &&
                (Ld.mprec != MASTER_F16_SR || ls.k == 0)) {
                if (Ld.mprec == MASTER_F16_SR)
                    hipLaunchKernelGGL((lp_flush_step_kernel<PREC, LMAX, true, false>), dim3(nblocks(Ld)), dim3(kThreads),
                                       0, st, Ld, io, ls);
                else
                    hipLaunchKernelGGL((lp_flush_step_kernel<PREC, LMAX, false, false>), dim3(nblocks(Ld)),
                                       dim3(kThreads), 0, st, Ld, io, ls);
                return hipGetLastError();
            }
        // fp8 master, every sequence flushes: the same MFMA fold, read from and encoded to E4M3
        if constexpr (!MIX && NN >= 32 && PREC == PREC_FP8)
            if (all_flush && (Ld.mprec == MASTER_F8 || Ld.mprec == MASTER_F8_SR) && Ld.psplit == 1 &&
                (Ld.mprec != MASTER_F8_SR || ls.k == 0)) {
                if (Ld.mprec == MASTER_F8_SR)
                    hipLaunchKernelGGL((lp_flush_step_kernel<PREC, LMAX, true, true>), dim3(nblocks(Ld)), dim3(kThreads),
                                       0, st, Ld, io, ls);
                else
                    hipLaunchKernelGGL((lp_flush_step_kernel<PREC, LMAX, false, true>), dim3(nblocks(Ld)),
                                       dim3(kThreads), 0, st, Ld, io, ls);
                return hipGetLastError();
            }
        // fp16 master: two heads per work-group with the master rows issued early (see step_kernel)
        if constexpr (LMAX <= 32)
            if ((Ld.mprec == MASTER_F16 || Ld.mprec == MASTER_F16_SR) && Ld.psplit == 1 && Ld.hpg % 2 == 0)
                return step_rows<PREC, LMAX, 2 * kRows, true, MIX>(Ld, io, ls, st);
        // lockstep flush step, fp32 master, narrow copy: every sequence flushes
        if constexpr (PREC == PREC_BF16 || PREC == PREC_FP8 || PREC == PREC_FP4)
            if (Ld.mprec == MASTER_F32) {
                if (ls.k > 0) return step_rows<PREC, LMAX, kRows, 2, MIX>(Ld, io, ls, st);
                return step_rows<PREC, LMAX, kRows, 3, MIX>(Ld, io, ls, st);
            }
        return step_rows<PREC, LMAX, kRows, true, MIX>(Ld, io, ls, st);
    }
    if constexpr (!MIX && (PREC == PREC_FP8 || PREC == PREC_FP4) && LMAX == 16 && NN <= 128) {
        // one row per lane: P <= 64, four heads of one group per work-group; at N = 256 a row's
        // chunks would hold 64 (fp8) registers per lane
        if (Ld.P <= kRows && Ld.hpg % kWaves == 0) {
            const unsigned grid = nblocks(Ld) / kWaves;
            hipLaunchKernelGGL((narrow_step_kernel<PREC, LMAX>), dim3(grid), dim3(kThreads), 0, st, Ld, io, ls);
            return hipGetLastError();
        }
    }
    if (wide > 1 && LMAX <= 32 && Ld.psplit == 1 && Ld.hpg % wide == 0 && nblocks(Ld) / wide >= 2048)
        return step_rows<PREC, LMAX, kRows * wide, false, MIX>(Ld, io, ls, st);
    return step_rows<PREC, LMAX, kRows, false, MIX>(Ld, io, ls, st);
}

template <int PREC, int LMAX>
hipError_t flush_t(const Layer &Ld, int mode, const int *arg, int T, float *out, hipStream_t st)
{
    if (mode == MODE_OVERFULL) {
        hipLaunchKernelGGL(advance_kernel, dim3((Ld.Bt + 255) / 256), dim3(256), 0, st, Ld, arg, T);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((flush_kernel<PREC, LMAX>), dim3(nblocks(Ld)), dim3(kThreads), 0, st, Ld, mode,
                       mode == MODE_OVERFULL ? nullptr : arg, out);
    return hipGetLastError();
}

template <int PREC, int LMAX, int TQ, bool MIX>
hipError_t verify_t(const Layer &Ld, const TokenIO &io, int T, hipStream_t st)
{
    hipLaunchKernelGGL((verify_kernel<PREC, LMAX, TQ, MIX>), dim3(nblocks(Ld)), dim3(kThreads), 0, st, Ld, io, T);
    return hipGetLastError();
}

template <int PREC, int LMAX, bool MIX>
hipError_t verify_tq(const Layer &Ld, const TokenIO &io, int T, hipStream_t st)
{
    if (T <= 2) return verify_t<PREC, LMAX, 2, MIX>(Ld, io, T, st);
    if (T <= 4) return verify_t<PREC, LMAX, 4, MIX>(Ld, io, T, st);
    return verify_t<PREC, LMAX, 8, MIX>(Ld, io, T, st);
}

template <template <int, int> class F, typename... Args>
hipError_t by_prec_lmax(int prec, int lmax, Args... args)
{
    switch (prec * 100 + lmax) {
    case PREC_F32 * 100 + 16: return F<PREC_F32, 16>::run(args...);
    case PREC_F32 * 100 + 32: return F<PREC_F32, 32>::run(args...);
    case PREC_F32 * 100 + 64: return F<PREC_F32, 64>::run(args...);
    case PREC_BF16 * 100 + 16: return F<PREC_BF16, 16>::run(args...);
    case PREC_BF16 * 100 + 32: return F<PREC_BF16, 32>::run(args...);
    case PREC_BF16 * 100 + 64: return F<PREC_BF16, 64>::run(args...);
    case PREC_FP8 * 100 + 16: return F<PREC_FP8, 16>::run(args...);
    case PREC_FP8 * 100 + 32: return F<PREC_FP8, 32>::run(args...);
    case PREC_FP8 * 100 + 64: return F<PREC_FP8, 64>::run(args...);
    case PREC_FP4 * 100 + 16: return F<PREC_FP4, 16>::run(args...);
    case PREC_FP4 * 100 + 32: return F<PREC_FP4, 32>::run(args...);
    case PREC_FP4 * 100 + 64: return F<PREC_FP4, 64>::run(args...);
    case PREC_F16 * 100 + 16: return F<PREC_F16, 16>::run(args...);
    case PREC_F16 * 100 + 32: return F<PREC_F16, 32>::run(args...);
    case PREC_F16 * 100 + 64: return F<PREC_F16, 64>::run(args...);
    default: return hipErrorInvalidValue;
    }
}

template <int PREC, int LMAX>
struct StepF {
    static hipError_t run(const Layer &Ld, const TokenIO &io, bool fc, bool af, bool mix, Lockstep ls, hipStream_t st)
    {
        if constexpr (!kPrecOk<PREC>) {
            return hipErrorInvalidValue;
        } else {
            if (!mix) return step_t<PREC, LMAX, false>(Ld, io, fc, af, ls, st);
            if constexpr (LMAX <= 32) return step_t<PREC, LMAX, true>(Ld, io, fc, af, ls, st);
            else return hipErrorInvalidValue;  // the mixer edges need L <= 32 (host-checked)
        }
    }
};
template <int PREC, int LMAX>
struct FlushF {
    static hipError_t run(const Layer &Ld, int mode, const int *arg, int T, float *out, hipStream_t st)
    {
        if constexpr (!kPrecOk<PREC>) return hipErrorInvalidValue;
        else return flush_t<PREC, LMAX>(Ld, mode, arg, T, out, st);
    }
};
template <int PREC, int LMAX>
struct VerifyF {
    static hipError_t run(const Layer &Ld, const TokenIO &io, int T, bool mix, hipStream_t st)
    {
        if constexpr (!kPrecOk<PREC>) {
            return hipErrorInvalidValue;
        } else {
            if (!mix) return verify_tq<PREC, LMAX, false>(Ld, io, T, st);
            if constexpr (LMAX <= 32) return verify_tq<PREC, LMAX, true>(Ld, io, T, st);
            else return hipErrorInvalidValue;  // the mixer edges need L <= 32 (host-checked)
        }
    }
};

template <int PREC>
hipError_t load_p(const Layer &Ld, const float *state, hipStream_t st)
{
    if constexpr (!kPrecOk<PREC>) {
        return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((load_state_kernel<PREC>), dim3(nblocks(Ld)), dim3(kThreads), 0, st, Ld, state);
        return hipGetLastError();
    }
}

}  // namespace

// Exported launchers for this N.
#define RSSM_CAT2(a, b) a##b
#define RSSM_CAT(a, b) RSSM_CAT2(a, b)

hipError_t RSSM_CAT(launch_step_n, RSSM_N)(int prec, int lmax, const Layer &Ld, const TokenIO &io, bool flush_capable,
                                           bool all_flush, bool mix, Lockstep ls, hipStream_t st)
{
    return by_prec_lmax<StepF>(prec, lmax, Ld, io, flush_capable, all_flush, mix, ls, st);
}

hipError_t RSSM_CAT(launch_flush_n, RSSM_N)(int prec, int lmax, const Layer &Ld, int mode, const int *arg, int T, float *out, hipStream_t st)
{
    return by_prec_lmax<FlushF>(prec, lmax, Ld, mode, arg, T, out, st);
}

hipError_t RSSM_CAT(launch_verify_n, RSSM_N)(int prec, int lmax, const Layer &Ld, const TokenIO &io, int T, bool mix,
                                             hipStream_t st)
{
    return by_prec_lmax<VerifyF>(prec, lmax, Ld, io, T, mix, st);
}

hipError_t RSSM_CAT(launch_load_n, RSSM_N)(int prec, const Layer &Ld, const float *state, hipStream_t st)
{
    switch (prec) {
    case PREC_F32: return load_p<PREC_F32>(Ld, state, st);
    case PREC_BF16: return load_p<PREC_BF16>(Ld, state, st);
    case PREC_FP8: return load_p<PREC_FP8>(Ld, state, st);
    case PREC_FP4: return load_p<PREC_FP4>(Ld, state, st);
    case PREC_F16: return load_p<PREC_F16>(Ld, state, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t RSSM_CAT(launch_conventional_n, RSSM_N)(const Layer &Ld, float *state, const TokenIO &io, hipStream_t st)
{
    hipLaunchKernelGGL(conventional_kernel, dim3(nblocks(Ld)), dim3(kThreads), 0, st, Ld, state, io);
    return hipGetLastError();
}

hipError_t RSSM_CAT(launch_conventional_mixer_n, RSSM_N)(const Layer &Ld, float *state, const TokenIO &io, int rslot,
                                                       hipStream_t st)
{
    hipLaunchKernelGGL(conventional_mixer_kernel, dim3(nblocks(Ld)), dim3(kThreads), 0, st, Ld, state, io, rslot);
    return hipGetLastError();
}

hipError_t RSSM_CAT(launch_snapshot_n, RSSM_N)(const Layer &Ld, float *slots, const int *cur, int T, const TokenIO &io, hipStream_t st)
{
    const dim3 grid(nblocks(Ld)), block(kThreads);
    if (T <= 2) hipLaunchKernelGGL((snapshot_verify_kernel<2>), grid, block, 0, st, Ld, slots, cur, T, io);
    else if (T <= 4) hipLaunchKernelGGL((snapshot_verify_kernel<4>), grid, block, 0, st, Ld, slots, cur, T, io);
    else hipLaunchKernelGGL((snapshot_verify_kernel<8>), grid, block, 0, st, Ld, slots, cur, T, io);
    return hipGetLastError();
}

}  // namespace rssm
