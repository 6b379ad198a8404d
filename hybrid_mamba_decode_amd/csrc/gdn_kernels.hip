// gdn_kernels.hip -- ReplaySSM decode-step kernels for Gated DeltaNet layers on gfx950, for one
// key size Dk (compiled once per supported Dk with -DRSSM_N=<Dk>).
//
// Layer (per value head h, key head g = h / (H/G); the published Gated DeltaNet recurrence, the
// plain reading of the pages' second layer type, [AT Pulse] "Capabilities and access"):
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
// with S [Dv, Dk] per (sequence, value head), row p = value index. Replay form ([AT Pulse]
// "Technical analysis": output from a checkpoint plus the window's records): a backward sweep
// over the window's records j = t..c gives z and c_j,
//     z <- q_t;  c_j = beta_j (k_j . z);  z <- alpha_j (z - c_j k_j);   o_t = S_c z + sum_j c_j v_j
// and a flush applies the records to the checkpoint in order.
//
// Tiling as for the Mamba-2 kernels (device.h): one 256-thread work-group per <= 64 rows of one
// (sequence, value head) tile, lanes along Dk, 16-byte non-temporal loads, transpose-reduce for
// row dots, XCD-aware tile order.
//
// Kernels:
//   gdn_step_kernel       replay + append; the flush-capable variant folds the sequences whose
//                         buffer fills and reads their output from the folded state
//   gdn_flush_kernel      explicit flush, rollback commit, or materialize
//   gdn_verify_kernel     output-only evaluation of T draft tokens + tentative append
//   gdn_step_copy_kernel, gdn_verify_copy_kernel   the same through a bf16 / fp8 / MXFP4 copy,
//                         128-row tiles
//   gdn_load_kernel       master <- state, pointers reset
//   gdn_conventional_kernel   read-update-write baseline
//   gdn_snapshot_kernel   per-draft snapshot baseline (one read, T writes)
#include "device.h"
#include "gdn_launch.h"

#ifndef RSSM_N
#error "compile with -DRSSM_N=<Dk>"
#endif

namespace rssm {
namespace {

constexpr int NN = RSSM_N;
using GF = Geo<NN, PREC_F32>;
constexpr int ZPL = NN >= 64 ? NN / 64 : 1;  // sweep vector elements per lane (n = lane + 64 e)

// State row held by load slot i of a lane (f32 geometry).
__device__ inline int row_of_f32(int i, int wave, int lane) { return i * GF::RPB + wave * GF::RPI + lane / GF::LPR; }

// Tiles of RT value rows, `splits` = ceil(Dv / RT) per (sequence, value head).
template <int RT>
__device__ inline Tile gmap_tile_rows(const GLayer &Ld, int splits)
{
    const unsigned nblk = gridDim.x, i = blockIdx.x;
    const unsigned id = (nblk % 8u == 0u) ? (i % 8u) * (nblk / 8u) + i / 8u : i;
    Tile t;
    t.split = (int)(id % (unsigned)splits);
    const unsigned bh = id / (unsigned)splits;
    t.h = (int)(bh % (unsigned)Ld.H);
    t.b = (int)(bh / (unsigned)Ld.H);
    t.g = t.h / Ld.hpg;
    t.row0 = t.split * RT;
    t.nrows = min(RT, Ld.Dv - t.row0);
    return t;
}

__device__ inline Tile gmap_tile(const GLayer &Ld) { return gmap_tile_rows<kRows>(Ld, Ld.psplit); }

__device__ inline void graise(const GLayer &Ld, unsigned bits)
{
    if (threadIdx.x == 0) __hip_atomic_fetch_or(Ld.flag, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-sequence completion (as seq_done in device.h): the last work-group of sequence b to finish
// writes the new pointers and re-arms the counter.
__device__ inline void gseq_done(const GLayer &Ld, int b, int new_pos, int new_ckpt, int splits)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned expected = (unsigned)(Ld.H * splits);
        const unsigned prev = __hip_atomic_fetch_add(&Ld.counter[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev + 1u == expected) {
            Ld.pos[b] = new_pos;
            Ld.ckpt[b] = new_ckpt;
            __hip_atomic_store(&Ld.counter[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__device__ inline void gseq_done(const GLayer &Ld, int b, int new_pos, int new_ckpt)
{
    gseq_done(Ld, b, new_pos, new_ckpt, Ld.psplit);
}

template <int LMAX, int RT = kRows>
struct GWin {
    float K[LMAX][NN] __attribute__((aligned(16)));  // k_j of the key head
    float V[LMAX][RT] __attribute__((aligned(16)));  // v_j, this work-group's RT rows
    float a[LMAX], b[LMAX];                          // alpha_j, beta_j of the value head
};

// Stage records 0..k-1 of the window in LDS: record j < nring from ring slot (ck + j) mod L, the
// rest from the call's fresh inputs (fresh record f at fk + f*sk, fv + f*sv, fa/fb + f*ss).
template <int LMAX>
__device__ inline void stage_window(GWin<LMAX> &w, const GLayer &Ld, const Tile &t, int ck, int nring, int k,
                                    const float *fk, int sk, const float *fv, int sv, const float *fa,
                                    const float *fb, int ss)
{
    const int tid = threadIdx.x;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    const float *rk = Ld.ring_k + ((size_t)t.b * Ld.G + t.g) * Ld.L * NN;
    const float *rv = Ld.ring_v + bh * Ld.L * Ld.Dv + t.row0;
    const int cs0 = (int)((unsigned)ck % (unsigned)Ld.L);
    auto slot = [&](int j) { return ring_slot(cs0, j, Ld.L); };  // record j (< L)
    for (int e = tid; e < k * (NN / 4); e += kThreads) {
        const int j = e / (NN / 4), c4 = e % (NN / 4);
        const float *src = j < nring ? rk + (size_t)slot(j) * NN : fk + (size_t)(j - nring) * sk;
        *(f32x4 *)&w.K[j][4 * c4] = *(const f32x4 *)(src + 4 * c4);
    }
    for (int e = tid; e < k * kRows; e += kThreads) {
        const int j = e / kRows, p = e % kRows;
        float val = 0.f;
        if (p < t.nrows) val = j < nring ? rv[(size_t)slot(j) * Ld.Dv + p] : fv[(size_t)(j - nring) * sv + p];
        w.V[j][p] = val;
    }
    if (tid < k) {
        const int j = tid;
        w.a[j] = j < nring ? Ld.ring_a[bh * Ld.L + slot(j)] : fa[(size_t)(j - nring) * ss];
        w.b[j] = j < nring ? Ld.ring_b[bh * Ld.L + slot(j)] : fb[(size_t)(j - nring) * ss];
    }
}

// Sum over aligned groups of W lanes for the record loops below (every lane of a group receives
// it): DPP within the row of 16, then ds_swizzle (xor 16) and ds_bpermute (xor 32) -- in these
// dependent per-record chains the LDS-pipe exchanges measured faster than gfx950's permlane swaps
// that device.h's group_sum uses (spec verify + commit at batch 512, T 4: 352 -> 338 us fp32,
// 292 -> 284 us bf16).
template <int W>
__device__ inline float record_sum(float v)
{
    if constexpr (W >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
    if constexpr (W >= 16) v += dpp_f<0x140>(v); // row_mirror
    if constexpr (W >= 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // xor 16
    if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Sum of a value over the LPR consecutive lanes of a row (all of them receive it).
__device__ inline float row_allreduce(float v) { return record_sum<GF::LPR>(v); }

// Backward sweep of one query over records last..0 in the calling wave: z <- q; c_j = beta_j
// (k_j . z); z <- alpha_j (z - c_j k_j). Writes c_j to c[j] and the final z to z_out (lane 0 and
// lanes holding z elements; wave-wide shuffles, so the whole wave must call it).
template <int LMAX, int RT>
__device__ inline void gdn_sweep(const GWin<LMAX, RT> &w, const float *q, int last, float *c, float *z_out, int lane)
{
    float z[ZPL];
#pragma unroll
    for (int e = 0; e < ZPL; ++e) {
        const int n = lane + 64 * e;
        z[e] = n < NN ? q[n] : 0.f;
    }
    for (int j = last; j >= 0; --j) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < ZPL; ++e) {
            const int n = lane + 64 * e;
            if (n < NN) part = fmaf(z[e], w.K[j][n], part);
        }
        part = record_sum<64>(part);
        const float cj = w.b[j] * part;
        const float aj = w.a[j];
#pragma unroll
        for (int e = 0; e < ZPL; ++e) {
            const int n = lane + 64 * e;
            if (n < NN) z[e] = aj * (z[e] - cj * w.K[j][n]);
        }
        if (lane == 0) c[j] = cj;
    }
#pragma unroll
    for (int e = 0; e < ZPL; ++e) {
        const int n = lane + 64 * e;
        if (n < NN) z_out[n] = z[e];
    }
}



// Apply records 0..k-1 to fp32 rows held in f32 geometry (vf), in order:
// S_row <- alpha_j (S_row - beta_j (S_row . k_j) k_j) + beta_j v_j[row] k_j.
template <int LMAX>
__device__ inline void gdn_fold_rows(f32x4 (&vf)[GF::NL], const GWin<LMAX> &w, int k, int wave, int lane)
{
    const int c = lane % GF::LPR;
    int row[GF::NL];
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of_f32(i, wave, lane);
        row[i] = r < kRows ? r : 0;
    }
    for (int j = 0; j < k; ++j) {
        const f32x4 kj = *(const f32x4 *)&w.K[j][4 * c];
        const float aj = w.a[j], bj = w.b[j];
#pragma unroll
        for (int i = 0; i < GF::NL; ++i) {
            float part = vf[i].x * kj.x;
            part = fmaf(vf[i].y, kj.y, part);
            part = fmaf(vf[i].z, kj.z, part);
            part = fmaf(vf[i].w, kj.w, part);
            const float sk = row_allreduce(part);
            // alpha (S - beta sk k) + beta v k = alpha S + (beta v - alpha beta sk) k
            const float coef = bj * (w.V[j][row[i]] - aj * sk);
            vf[i].x = fmaf(coef, kj.x, aj * vf[i].x);
            vf[i].y = fmaf(coef, kj.y, aj * vf[i].y);
            vf[i].z = fmaf(coef, kj.z, aj * vf[i].z);
            vf[i].w = fmaf(coef, kj.w, aj * vf[i].w);
        }
    }
}

__device__ inline void store_rows(float *rows, const f32x4 (&vf)[GF::NL], int nrows, int wave, int lane)
{
    const int c = lane % GF::LPR;
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of_f32(i, wave, lane);
        if (r < nrows) store_nt(rows + (size_t)r * NN + 4 * c, as_u32x4(vf[i]));
    }
}

// fp32 rows of a tile, one 16-byte load per lane and slot, all issued unconditionally: lanes of rows
// at or beyond nrows read row 0 again (rows are independent in every use, and those are never
// stored), so the issue sequence is straight-line and no wait covers more loads than it needs.
__device__ inline void load_rows_f32(f32x4 (&vf)[GF::NL], const float *rows, int nrows, int wave, int lane)
{
    const int c = lane % GF::LPR;
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of_f32(i, wave, lane), rr = r < nrows ? r : 0;
        vf[i] = as_f32x4(load_nt(rows + (size_t)rr * NN + 4 * c));
    }
}

// bf16 copy rows in the same geometry: 8 bytes (4 values) per lane and slot, widened exactly (rows
// beyond the tile as in load_rows_f32).
__device__ inline void load_rows_bf16(f32x4 (&vf)[GF::NL], const unsigned short *rows, int nrows, int wave, int lane)
{
    const int c = lane % GF::LPR;
#pragma unroll
    for (int i = 0; i < GF::NL; ++i) {
        const int r = row_of_f32(i, wave, lane), rr = r < nrows ? r : 0;
        const u32x2 w = __builtin_nontemporal_load((const u32x2 *)(rows + (size_t)rr * NN + 4 * c));
        vf[i] = f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    }
}

// Store folded master rows of head bh and, with a read copy, their encoding (write_copy_rows_n:
// bf16, fp8 with this 64-row block's scale, MXFP4). red: kWaves floats of LDS for the fp8 amax.
__device__ inline void store_checkpoint(const GLayer &Ld, size_t bh, size_t elem0, const f32x4 (&vf)[GF::NL],
                                        int nrows, int wave, int lane, float *red)
{
    store_rows(Ld.master + elem0, vf, nrows, wave, lane);
    const CopyDst d{Ld.rcopy, Ld.scale, Ld.mxscale, Ld.Dv, Ld.psplit};
    switch (Ld.rprec) {
    case PREC_BF16: write_copy_rows_n<NN, PREC_BF16>(d, bh, elem0, vf, nrows, wave, lane, red); break;
    case PREC_FP8: write_copy_rows_n<NN, PREC_FP8>(d, bh, elem0, vf, nrows, wave, lane, red); break;
    case PREC_FP4:
        if constexpr (NN >= 32) write_copy_rows_n<NN, PREC_FP4>(d, bh, elem0, vf, nrows, wave, lane, red);
        break;
    default: break;
    }
}

// Rows of a tile of head bh through the read copy, decoded exactly into f32 geometry (4 values
// per lane and slot; rows beyond the tile as in load_rows_f32): bf16 widened; fp8 codes (4 bytes
// of the row's chunk) times the block's scale; MXFP4 codes (2 bytes) times 2^(code - 127) of
// their block.
template <int RP>
__device__ inline void load_rows_copy(f32x4 (&vf)[GF::NL], const GLayer &Ld, size_t bh, int row0, int nrows, int wave,
                                      int lane)
{
    const int n = 4 * (lane % GF::LPR);
    if constexpr (RP == PREC_BF16) {
        load_rows_bf16(vf, (const unsigned short *)Ld.rcopy + (bh * Ld.Dv + row0) * NN, nrows, wave, lane);
    } else if constexpr (RP == PREC_FP8) {
        const unsigned char *src = (const unsigned char *)Ld.rcopy;
        const float scale = Ld.scale[bh * Ld.psplit + row0 / kRows];
#pragma unroll
        for (int i = 0; i < GF::NL; ++i) {
            const int r = row_of_f32(i, wave, lane), rr = r < nrows ? r : 0;
            const unsigned w = __builtin_nontemporal_load(
                (const unsigned *)(src + state_chunk_off<NN, PREC_FP8>(bh, row0 + rr, n / 16, Ld.Dv) + n % 16));
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
            vf[i] = f32x4{lo.x * scale, lo.y * scale, hi.x * scale, hi.y * scale};
        }
    } else if constexpr (RP == PREC_FP4) {
        const unsigned char *src = (const unsigned char *)Ld.rcopy;
#pragma unroll
        for (int i = 0; i < GF::NL; ++i) {
            const int r = row_of_f32(i, wave, lane), rr = r < nrows ? r : 0;
            const unsigned w = __builtin_nontemporal_load((const unsigned short *)(
                src + state_chunk_off<NN, PREC_FP4>(bh, row0 + rr, n / 32, Ld.Dv) + (n % 32) / 2));
            const unsigned code = Ld.mxscale[(bh * Ld.Dv + row0 + rr) * (NN / 32) + n / 32];
            const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
            const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
            vf[i] = f32x4{mx_scaled(a.x, code), mx_scaled(a.y, code), mx_scaled(b.x, code), mx_scaled(b.y, code)};
        }
    }
}

// Row dots of the tile with M vectors (vectors[m] in LDS, NN floats each), reduced into
// u[m * kRows + row].
template <int M>
__device__ inline void rows_dot(const f32x4 (&vf)[GF::NL], const float *vectors, int nvec, float *u, int wave,
                                int lane)
{
    const int c = lane % GF::LPR;
    float part[GF::NL * M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const f32x4 z = m < nvec ? *(const f32x4 *)(vectors + (size_t)m * NN + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < GF::NL; ++i) {
            float s = vf[i].x * z.x;
            s = fmaf(vf[i].y, z.y, s);
            s = fmaf(vf[i].z, z.z, s);
            part[m * GF::NL + i] = fmaf(vf[i].w, z.w, s);
        }
    }
    transpose_reduce<GF::NL * M, GF::LPR>(part, lane);
    bool writer;
    const int first = tr_first<GF::NL * M, GF::LPR>(lane, &writer);
    constexpr int cnt = tr_count<GF::NL * M, GF::LPR>();
    if (writer) {
#pragma unroll
        for (int e = 0; e < cnt; ++e) {
            const int idx = first + e, m = idx / GF::NL, i = idx % GF::NL;
            const int r = row_of_f32(i, wave, lane);
            if (m < nvec && r < kRows) u[m * kRows + r] = part[e];
        }
    }
}

// ==========================================================================================
// Standard decode step. FLUSH = the launch may meet sequences whose buffer fills ([WittyWires]
// "What happened": the checkpoint is updated when the buffer fills); those apply all records to
// the fp32 master and read o from the folded state (no record is stored for that token).
// ==========================================================================================
template <int LMAX, int RT = kRows>
struct GStepLds {
    GWin<LMAX, RT> w;
    float q[NN] __attribute__((aligned(16)));
    float z[NN] __attribute__((aligned(16)));
    float c[LMAX];
    float u[RT];
    float red[kWaves];
};

// The step's window staged through registers: issued before the checkpoint stream (global loads
// complete in issue order, so the window can be written to LDS while the stream is still in
// flight) and committed to LDS afterwards. Record j < k-1 comes from ring slot (cslot + j) mod L,
// record k-1 (this token) and q from the call's inputs; v covers the tile's RT rows.
template <int LMAX, int RT>
struct StepWindow {
    static constexpr int KS = (LMAX * NN / 4 + kThreads - 1) / kThreads;
    static constexpr int KCH = KS < 8 ? KS : 8;  // k slots held at once; the rest load at commit
    static constexpr int VS = (LMAX * RT / 4 + kThreads - 1) / kThreads;
    f32x4 kr[KCH], vr[VS], qr;
    float ar, br;
    size_t bh, bg;
    const float *rk, *rv;  // ring k of the key head; ring v at the tile's first row
    int cslot, k, tid;

    __device__ StepWindow(const GLayer &Ld, const Tile &t, int tid_) : tid(tid_)
    {
        bh = (size_t)t.b * Ld.H + t.h;
        bg = (size_t)t.b * Ld.G + t.g;
        rk = Ld.ring_k + bg * Ld.L * NN;
        rv = Ld.ring_v + bh * Ld.L * Ld.Dv + t.row0;
    }
    __device__ int slot_of(const GLayer &Ld, int j) const { return ring_slot(cslot, j, Ld.L); }  // j < L
    __device__ const float *kaddr(const GLayer &Ld, const GTokenIO &io, int j, int c4) const
    {
        return (j < k - 1 ? rk + (size_t)slot_of(Ld, j) * NN : io.k + bg * NN) + 4 * c4;
    }

    __device__ void issue(const GLayer &Ld, const GTokenIO &io, const Tile &t, int cslot_, int k_)
    {
        cslot = cslot_;
        k = k_;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sl = 0; sl < KCH; ++sl) {
            const int e = tid + sl * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
            const f32x4 val = *(const f32x4 *)kaddr(Ld, io, j < k ? j : k - 1, c4);
            kr[sl] = j < k ? val : zero;
        }
#pragma unroll
        for (int sl = 0; sl < VS; ++sl) {
            const int e = tid + sl * kThreads, j = e / (RT / 4), c4 = e % (RT / 4);
            const bool in = j < k && 4 * c4 < t.nrows;
            const float *src = (in && j < k - 1) ? rv + (size_t)slot_of(Ld, j) * Ld.Dv + 4 * c4
                                                 : io.v + bh * Ld.Dv + t.row0 + (in ? 4 * c4 : 0);
            const f32x4 val = *(const f32x4 *)src;
            vr[sl] = in ? val : zero;
        }
        const bool in = tid < k;
        const bool ring = in && tid < k - 1;
        const size_t ri = bh * Ld.L + (ring ? slot_of(Ld, tid) : 0);
        const float a = ring ? Ld.ring_a[ri] : io.alpha[bh];
        const float b = ring ? Ld.ring_b[ri] : io.beta[bh];
        ar = in ? a : 0.f;
        br = in ? b : 0.f;
        const f32x4 q = *(const f32x4 *)(io.q + bg * NN + 4 * (tid % (NN / 4)));
        qr = tid < NN / 4 ? q : zero;
    }

    __device__ void commit(GWin<LMAX, RT> &w, float *q, const GLayer &Ld, const GTokenIO &io)
    {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s0 = 0; s0 < KS; s0 += KCH) {
            if (s0 > 0) {
#pragma unroll
                for (int sl = 0; sl < KCH; ++sl) {
                    const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
                    kr[sl] = (s0 + sl < KS && j < k) ? *(const f32x4 *)kaddr(Ld, io, j, c4) : zero;
                }
            }
#pragma unroll
            for (int sl = 0; sl < KCH; ++sl) {
                const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
                if (s0 + sl < KS && j < LMAX) *(f32x4 *)&w.K[j][4 * c4] = kr[sl];
            }
        }
#pragma unroll
        for (int sl = 0; sl < VS; ++sl) {
            const int e = tid + sl * kThreads, j = e / (RT / 4), c4 = e % (RT / 4);
            if (j < LMAX) *(f32x4 *)&w.V[j][4 * c4] = vr[sl];
        }
        if (tid < LMAX) {
            w.a[tid] = ar;
            w.b[tid] = br;
        }
        if (tid < NN / 4) *(f32x4 *)&q[4 * tid] = qr;
    }
};

// Pointer update once per sequence after a step. Lockstep: the first tile of head 0 checks the
// device pointers against the window position (a mismatch raises the flag) and advances them;
// otherwise the last work-group of the sequence writes them.
__device__ inline void step_advance(const GLayer &Ld, const Tile &t, bool uni, int pslot, int cslot, int k,
                                    bool flush, int pos, int ck, int splits)
{
    if (uni) {
        if (t.h == 0 && t.split == 0 && threadIdx.x == 0) {
            const int dp = Ld.pos[t.b], dc = Ld.ckpt[t.b];
            const bool ok = dc >= 0 && dp - dc == k - 1 && (int)((unsigned)dp % (unsigned)Ld.L) == pslot &&
                            (int)((unsigned)dc % (unsigned)Ld.L) == cslot;
            if (ok) {
                Ld.pos[t.b] = dp + 1;
                Ld.ckpt[t.b] = flush ? dp + 1 : dc;
            } else {
                __hip_atomic_fetch_or(Ld.flag, FLAG_POINTERS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    } else {
        gseq_done(Ld, t.b, pos + 1, flush ? pos + 1 : ck, splits);
    }
}

// Replayed output o = S_c z + sum_j c_j v_j from the row dots in s.u, and the token's record
// appended at ring slot pslot (v by every tile, alpha / beta by the first tile, k by the first
// tile of the key head's first value head).
template <int LMAX, int RT>
__device__ inline void step_output_append(const GStepLds<LMAX, RT> &s, const GLayer &Ld, const GTokenIO &io,
                                          const Tile &t, int pslot, int k)
{
    const int tid = threadIdx.x;
    const size_t bh = (size_t)t.b * Ld.H + t.h, bg = (size_t)t.b * Ld.G + t.g;
    if (tid < t.nrows) {
        float acc = s.u[tid];
        for (int j = 0; j < k; ++j) acc = fmaf(s.c[j], s.w.V[j][tid], acc);
        io.o[bh * Ld.Dv + t.row0 + tid] = acc;
        Ld.ring_v[(bh * Ld.L + pslot) * Ld.Dv + t.row0 + tid] = s.w.V[k - 1][tid];
    }
    if (t.split == 0 && tid == 0) {
        Ld.ring_a[bh * Ld.L + pslot] = s.w.a[k - 1];
        Ld.ring_b[bh * Ld.L + pslot] = s.w.b[k - 1];
    }
    if (t.split == 0 && t.h % Ld.hpg == 0 && tid < NN / 4)
        *(f32x4 *)(Ld.ring_k + (bg * Ld.L + pslot) * NN + 4 * tid) = *(const f32x4 *)&s.w.K[k - 1][4 * tid];
}

// RP: the read copy's precision (PREC_F32: none). With a copy the checkpoint product reads it
// (replayed outputs); a flushing sequence reads and folds the fp32 master.
template <int LMAX, bool FLUSH, int RP>
__global__ void __launch_bounds__(kThreads) gdn_step_kernel(GLayer Ld, GTokenIO io, Lockstep ls)
{
    constexpr bool CP = RP != PREC_F32;
    __shared__ GStepLds<LMAX> s;
    const Tile t = gmap_tile(Ld);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    const size_t elem0 = (bh * Ld.Dv + t.row0) * NN;
    float *rows = Ld.master + elem0;
    auto load_state = [&](f32x4 (&dst)[GF::NL], bool master) {
        if (CP && !master) load_rows_copy<RP>(dst, Ld, bh, t.row0, t.nrows, wave, lane);
        else load_rows_f32(dst, rows, t.nrows, wave, lane);
    };

    StepWindow<LMAX, kRows> win(Ld, t, tid);
    const bool uni = ls.k > 0;
    int pslot = 0, cslot = 0, k = 1;
    f32x4 vf[GF::NL];
    int pos = 0, ck = 0;
    // With a read copy a flush-capable launch reads the master only for sequences that flush: in
    // device-pointer mode their pointers come first.
    constexpr bool kLate = CP && FLUSH;
    if (uni) {
        pslot = ls.pslot;
        cslot = ls.cslot;
        k = ls.k;
        win.issue(Ld, io, t, cslot, k);
        load_state(vf, FLUSH && k > Ld.L - Ld.Tmax);
    } else {
        if (!kLate) load_state(vf, false);  // the checkpoint stream first
        pos = Ld.pos[t.b];
        ck = Ld.ckpt[t.b];
        const int c0 = pos - ck;
        if (!(ck >= 0 && c0 >= 0 && c0 <= Ld.L - Ld.Tmax) || (!FLUSH && c0 + 1 > Ld.L - Ld.Tmax)) {
            graise(Ld, FLAG_POINTERS);
            gseq_done(Ld, t.b, pos, ck);
            return;
        }
        pslot = (int)((unsigned)pos % (unsigned)Ld.L);
        cslot = (int)((unsigned)ck % (unsigned)Ld.L);
        k = c0 + 1;  // records in the window, this token included
        if (kLate) load_state(vf, k > Ld.L - Ld.Tmax);
        win.issue(Ld, io, t, cslot, k);
    }
    win.commit(s.w, s.q, Ld, io);
    __syncthreads();
    const bool flush = k > Ld.L - Ld.Tmax;

    if (FLUSH && flush) {
        gdn_fold_rows<LMAX>(vf, s.w, k, wave, lane);
        store_checkpoint(Ld, bh, elem0, vf, t.nrows, wave, lane, s.red);
        rows_dot<1>(vf, s.q, 1, s.u, wave, lane);
        __syncthreads();
        if (tid < t.nrows) io.o[bh * Ld.Dv + t.row0 + tid] = s.u[tid];
        step_advance(Ld, t, uni, pslot, cslot, k, true, pos, ck, Ld.psplit);
        return;
    }

    // The sweep needs only the window: wave 0 runs it while the checkpoint rows may still be in
    // flight.
    if (wave == 0) gdn_sweep<LMAX>(s.w, s.q, k - 1, s.c, s.z, lane);
    __syncthreads();
    rows_dot<1>(vf, s.z, 1, s.u, wave, lane);
    __syncthreads();
    step_output_append(s, Ld, io, t, pslot, k);
    step_advance(Ld, t, uni, pslot, cslot, k, flush, pos, ck, Ld.psplit);
}

// ==========================================================================================
// Flush step when every sequence of the launch flushes (lockstep decoding, or a host bound showing
// every buffer fills), Dk >= 128: the fold with 16 values per lane, LW = Dk / 16 lanes per row
// (8 at Dk = 128), lane c of a row holding chunks c + LW i (i = 0..3, four consecutive key
// columns each), so every load instruction still reads 128 contiguous bytes of each row. The
// delta rule's per-record row dot S_row . k_j then needs a reduction over LW lanes -- three
// exchange steps at Dk = 128 instead of five over the 32 lanes of the f32 geometry -- which is
// most of the fold's VALU work. Same arithmetic as gdn_fold_rows (records applied in order).
// ==========================================================================================
constexpr int kW = 16;                          // values per lane and row
constexpr int kLW = NN / kW;                    // lanes per row
constexpr int kRW = kThreads / (kLW > 0 ? kLW : 1);  // rows per work-group instruction
constexpr int kNW = (kRows + kRW - 1) / kRW;    // row slots per lane
constexpr bool kWideFold = NN >= 128;

template <int LMAX>
__global__ void __launch_bounds__(kThreads) gdn_flush_step_kernel(GLayer Ld, GTokenIO io, Lockstep ls)
{
    static_assert(kWideFold, "16 values per lane: Dk >= 128 (an MXFP4 block is 8 consecutive lanes)");
    __shared__ GStepLds<LMAX> s;
    const Tile t = gmap_tile(Ld);
    const int tid = threadIdx.x, lane = tid & 63;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    const size_t elem0 = (bh * Ld.Dv + t.row0) * NN;
    const int c = tid % kLW;
    auto row_of = [&](int sl) { return sl * kRW + tid / kLW; };  // tile row of slot sl
    auto ncol = [&](int i) { return 4 * (c + kLW * i); };         // first key column of chunk i

    // 1. Pointers and window (as gdn_step_kernel), then the master rows.
    StepWindow<LMAX, kRows> win(Ld, t, tid);
    const bool uni = ls.k > 0;
    int pslot = 0, cslot = 0, k = 1, pos = 0, ck = 0;
    if (uni) {
        pslot = ls.pslot;
        cslot = ls.cslot;
        k = ls.k;
        if (!(k > Ld.L - Ld.Tmax && k <= Ld.L)) {  // the host launches this kernel for flush steps only
            graise(Ld, FLAG_POINTERS);
            return;
        }
    } else {
        pos = Ld.pos[t.b];
        ck = Ld.ckpt[t.b];
        const int c0 = pos - ck;
        if (!(ck >= 0 && c0 >= 0 && c0 <= Ld.L - Ld.Tmax && c0 + 1 > Ld.L - Ld.Tmax)) {
            graise(Ld, FLAG_POINTERS);
            gseq_done(Ld, t.b, pos, ck);
            return;
        }
        pslot = (int)((unsigned)pos % (unsigned)Ld.L);
        cslot = (int)((unsigned)ck % (unsigned)Ld.L);
        k = c0 + 1;
    }
    win.issue(Ld, io, t, cslot, k);
    f32x4 vf[kNW][4];
#pragma unroll
    for (int sl = 0; sl < kNW; ++sl) {
        const int r = row_of(sl), rr = r < t.nrows ? r : 0;
        const float *rowp = Ld.master + elem0 + (size_t)rr * NN;
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[sl][i] = as_f32x4(load_nt(rowp + ncol(i)));
    }
    win.commit(s.w, s.q, Ld, io);
    __syncthreads();

    // 2. Fold: S_row <- alpha_j (S_row - beta_j (S_row . k_j) k_j) + beta_j v_j[row] k_j, j in order.
    int rowc[kNW];
#pragma unroll
    for (int sl = 0; sl < kNW; ++sl) rowc[sl] = row_of(sl) < kRows ? row_of(sl) : 0;
    for (int j = 0; j < k; ++j) {
        f32x4 kv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kv[i] = *(const f32x4 *)&s.w.K[j][ncol(i)];
        const float aj = s.w.a[j], bj = s.w.b[j];
#pragma unroll
        for (int sl = 0; sl < kNW; ++sl) {
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                part = fmaf(vf[sl][i].x, kv[i].x, part);
                part = fmaf(vf[sl][i].y, kv[i].y, part);
                part = fmaf(vf[sl][i].z, kv[i].z, part);
                part = fmaf(vf[sl][i].w, kv[i].w, part);
            }
            const float sk = group_sum<kLW>(part);
            // alpha (S - beta sk k) + beta v k = alpha S + (beta v - alpha beta sk) k
            const float coef = bj * (s.w.V[j][rowc[sl]] - aj * sk);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vf[sl][i].x = fmaf(coef, kv[i].x, aj * vf[sl][i].x);
                vf[sl][i].y = fmaf(coef, kv[i].y, aj * vf[sl][i].y);
                vf[sl][i].z = fmaf(coef, kv[i].z, aj * vf[sl][i].z);
                vf[sl][i].w = fmaf(coef, kv[i].w, aj * vf[sl][i].w);
            }
        }
    }

    // 3. Store the master, encode the read copy, o = S_new q.
#pragma unroll
    for (int sl = 0; sl < kNW; ++sl) {
        const int r = row_of(sl);
        if (r < t.nrows) {
#pragma unroll
            for (int i = 0; i < 4; ++i) store_nt(Ld.master + elem0 + (size_t)r * NN + ncol(i), as_u32x4(vf[sl][i]));
        }
    }
    {
        f32x4 units[kNW * 4];
#pragma unroll
        for (int u = 0; u < kNW * 4; ++u) units[u] = vf[u / 4][u % 4];
        auto at = [&](int u) { return int2{row_of(u / 4), ncol(u % 4)}; };
        const CopyDst d{Ld.rcopy, Ld.scale, Ld.mxscale, Ld.Dv, Ld.psplit};
        switch (Ld.rprec) {
        case PREC_BF16: write_copy_units<NN, PREC_BF16, kNW * 4>(d, bh, elem0, units, t.nrows, at, s.red); break;
        case PREC_FP8: write_copy_units<NN, PREC_FP8, kNW * 4>(d, bh, elem0, units, t.nrows, at, s.red); break;
        case PREC_FP4: write_copy_units<NN, PREC_FP4, kNW * 4>(d, bh, elem0, units, t.nrows, at, s.red); break;
        default: break;
        }
    }
    {
        f32x4 qv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[i] = *(const f32x4 *)&s.q[ncol(i)];
#pragma unroll
        for (int sl = 0; sl < kNW; ++sl) {
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                part = fmaf(vf[sl][i].x, qv[i].x, part);
                part = fmaf(vf[sl][i].y, qv[i].y, part);
                part = fmaf(vf[sl][i].z, qv[i].z, part);
                part = fmaf(vf[sl][i].w, qv[i].w, part);
            }
            const float o = group_sum<kLW>(part);
            const int r = row_of(sl);
            if (c == 0 && r < t.nrows) io.o[bh * Ld.Dv + t.row0 + r] = o;
        }
    }
    // 4. Pointers (the token's record is folded already: nothing is appended).
    step_advance(Ld, t, uni, pslot, cslot, k, true, pos, ck, Ld.psplit);
    (void)lane;
}

// Non-flush step reading the copy (bf16, fp8 or MXFP4) with one work-group per kRowsC = 128 value
// rows (a whole head at Dv = 128): 16-byte loads of one chunk per lane (8 bf16, 16 fp8 or 32 fp4
// values), so each work-group streams twice the rows of a 64-row tile for the same fixed window
// cost, and the backward sweep runs once per head instead of once per 64 rows. Used for Dk <= 128
// and windows of up to 32 records (the LDS window of 128 rows stays under 64 KiB).
constexpr int kRowsC = 128;
template <int RP>
struct CopyTile {
    using G = Geo<NN, RP>;
    static constexpr int NL = (kRowsC + G::RPB - 1) / G::RPB;  // copy load slots per lane
    static_assert(NL <= G::LPR || NL == 1 || G::LPR == 1, "transpose-reduce needs NL <= LPR");
};
template <int RP>
constexpr bool kCopyTiles = NN <= 128 && RP != PREC_F32 && (RP != PREC_FP4 || NN >= 32);

// The copy rows of a 128-row tile: raw chunks (and MXFP4 block-scale codes) per lane and slot;
// rows beyond the tile read its first row.
template <int RP>
struct CopyRows {
    using G = Geo<NN, RP>;
    static constexpr int NL = CopyTile<RP>::NL;
    u32x4 raw[NL];
    unsigned sc[RP == PREC_FP4 ? NL : 1];
    __device__ static int row_of(int i, int wave, int lane) { return i * G::RPB + wave * G::RPI + lane / G::LPR; }
    __device__ void load(const GLayer &Ld, const Tile &t, size_t bh, int wave, int lane)
    {
        const int c = lane % G::LPR;
        const char *base = (const char *)Ld.rcopy;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int r = row_of(i, wave, lane), rr = r < t.nrows ? r : 0;
            raw[i] = load_nt(base + state_chunk_off<NN, RP>(bh, t.row0 + rr, c, Ld.Dv));
            if constexpr (RP == PREC_FP4) sc[i] = Ld.mxscale[(bh * Ld.Dv + t.row0 + rr) * (NN / 32) + c];
        }
    }
    // Row dot of slot i with the vector z (NN floats in LDS), before the fp8 block scale.
    __device__ float dot(int i, const float *z, int lane) const
    {
        const int c = lane % G::LPR;
        const float p = chunk_dot<RP>(raw[i], z + G::VEC * c);
        if constexpr (RP == PREC_FP4) return mx_scaled(p, sc[i]);
        else return p;
    }
    // The finished row sum of tile row r: times its 64-row block's scale for fp8 (rows beyond the
    // tile, whose sums are never used, read the tile's first block).
    __device__ static float finish(const GLayer &Ld, const Tile &t, size_t bh, int r, float sum)
    {
        if constexpr (RP == PREC_FP8) return sum * Ld.scale[bh * Ld.psplit + (t.row0 + (r < t.nrows ? r : 0)) / kRows];
        else return sum;
    }
};

template <int LMAX, int RP>
__global__ void __launch_bounds__(kThreads) gdn_step_copy_kernel(GLayer Ld, GTokenIO io, Lockstep ls, int splits)
{
    using CR = CopyRows<RP>;
    using G = typename CR::G;
    constexpr int NLC = CR::NL;
    __shared__ GStepLds<LMAX, kRowsC> s;
    const Tile t = gmap_tile_rows<kRowsC>(Ld, splits);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    CR cr;

    StepWindow<LMAX, kRowsC> win(Ld, t, tid);
    const bool uni = ls.k > 0;
    int pslot, cslot, k, pos = 0, ck = 0;
    if (uni) {
        pslot = ls.pslot;
        cslot = ls.cslot;
        k = ls.k;
        win.issue(Ld, io, t, cslot, k);
        cr.load(Ld, t, bh, wave, lane);
    } else {
        cr.load(Ld, t, bh, wave, lane);  // the copy stream first
        pos = Ld.pos[t.b];
        ck = Ld.ckpt[t.b];
        const int c0 = pos - ck;
        if (!(ck >= 0 && c0 >= 0 && c0 + 1 <= Ld.L - Ld.Tmax)) {  // no sequence of this launch flushes
            graise(Ld, FLAG_POINTERS);
            gseq_done(Ld, t.b, pos, ck, splits);
            return;
        }
        pslot = (int)((unsigned)pos % (unsigned)Ld.L);
        cslot = (int)((unsigned)ck % (unsigned)Ld.L);
        k = c0 + 1;
        win.issue(Ld, io, t, cslot, k);
    }
    win.commit(s.w, s.q, Ld, io);
    __syncthreads();
    if (wave == 0) gdn_sweep<LMAX>(s.w, s.q, k - 1, s.c, s.z, lane);
    __syncthreads();

    // S_c z: each lane's chunk against the matching slice of z, summed over the row's lanes.
    float part[NLC];
#pragma unroll
    for (int i = 0; i < NLC; ++i) part[i] = cr.dot(i, s.z, lane);
    transpose_reduce<NLC, G::LPR>(part, lane);
    bool writer;
    const int first = tr_first<NLC, G::LPR>(lane, &writer);
    if (writer) {
#pragma unroll
        for (int e = 0; e < tr_count<NLC, G::LPR>(); ++e) {
            const int r = CR::row_of(first + e, wave, lane);
            if (r < kRowsC) s.u[r] = CR::finish(Ld, t, bh, r, part[e]);
        }
    }
    __syncthreads();
    step_output_append(s, Ld, io, t, pslot, k);
    step_advance(Ld, t, uni, pslot, cslot, k, false, pos, ck, splits);
}

// ==========================================================================================
// Flush / rollback commit / materialize (modes as for the Mamba-2 flush, launch.h).
// ==========================================================================================
template <int LMAX>
__global__ void __launch_bounds__(kThreads) gdn_flush_kernel(GLayer Ld, int mode, const int *arg, float *out)
{
    __shared__ GWin<LMAX> w;
    __shared__ float red[kWaves];
    const Tile t = gmap_tile(Ld);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    const size_t elem0 = (bh * Ld.Dv + t.row0) * NN;
    const int pos = Ld.pos[t.b], ck = Ld.ckpt[t.b];
    const int count = pos - ck;
    const int cap = mode == MODE_OVERFULL ? Ld.L : Ld.L - Ld.Tmax;
    if (!(ck >= 0 && count >= 0 && count <= cap)) {
        graise(Ld, FLAG_POINTERS);
        return;
    }
    bool fold;
    if (mode == MODE_OVERFULL) fold = count > Ld.L - Ld.Tmax;
    else if (mode == MODE_MASK) fold = (arg == nullptr || arg[t.b] != 0) && count > 0;
    else fold = true;
    if (!fold) return;
    // The window (every record from the ring: record j at slot (ck + j) mod L) into registers
    // first, then the checkpoint rows; the window reaches LDS while the rows are in flight.
    constexpr int KS = (LMAX * NN / 4 + kThreads - 1) / kThreads;
    constexpr int KCH = KS < 8 ? KS : 8;  // k slots held at once; the rest load at the commit
    constexpr int VS = (LMAX * kRows / 4 + kThreads - 1) / kThreads;
    const int tid = threadIdx.x;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const float *rk = Ld.ring_k + ((size_t)t.b * Ld.G + t.g) * Ld.L * NN;
    const float *rv = Ld.ring_v + bh * Ld.L * Ld.Dv + t.row0;
    const int cs0 = (int)((unsigned)ck % (unsigned)Ld.L);
    auto slot_of = [&](int j) { return ring_slot(cs0, j < count ? j : 0, Ld.L); };
    f32x4 kr[KCH], vr[VS];
#pragma unroll
    for (int sl = 0; sl < KCH; ++sl) {
        const int e = tid + sl * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
        const f32x4 val = *(const f32x4 *)(rk + (size_t)slot_of(j) * NN + 4 * c4);
        kr[sl] = j < count ? val : zero;
    }
#pragma unroll
    for (int sl = 0; sl < VS; ++sl) {
        const int e = tid + sl * kThreads, j = e / (kRows / 4), c4 = e % (kRows / 4);
        const bool in = j < count && 4 * c4 < t.nrows;
        const f32x4 val = *(const f32x4 *)(rv + (size_t)slot_of(j) * Ld.Dv + (in ? 4 * c4 : 0));
        vr[sl] = in ? val : zero;
    }
    const float ar = Ld.ring_a[bh * Ld.L + slot_of(tid)], br = Ld.ring_b[bh * Ld.L + slot_of(tid)];
    f32x4 vf[GF::NL];
    load_rows_f32(vf, Ld.master + elem0, t.nrows, wave, lane);
#pragma unroll
    for (int s0 = 0; s0 < KS; s0 += KCH) {
        if (s0 > 0) {
#pragma unroll
            for (int sl = 0; sl < KCH; ++sl) {
                const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
                kr[sl] = (s0 + sl < KS && j < count) ? *(const f32x4 *)(rk + (size_t)slot_of(j) * NN + 4 * c4) : zero;
            }
        }
#pragma unroll
        for (int sl = 0; sl < KCH; ++sl) {
            const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
            if (s0 + sl < KS && j < LMAX) *(f32x4 *)&w.K[j][4 * c4] = kr[sl];
        }
    }
#pragma unroll
    for (int sl = 0; sl < VS; ++sl) {
        const int e = tid + sl * kThreads, j = e / (kRows / 4), c4 = e % (kRows / 4);
        if (j < LMAX) *(f32x4 *)&w.V[j][4 * c4] = vr[sl];
    }
    if (tid < LMAX) {
        w.a[tid] = tid < count ? ar : 0.f;
        w.b[tid] = tid < count ? br : 0.f;
    }
    __syncthreads();
    gdn_fold_rows<LMAX>(vf, w, count, wave, lane);
    if (mode == MODE_MATERIALIZE) {
        store_rows(out + elem0, vf, t.nrows, wave, lane);
    } else {
        store_checkpoint(Ld, bh, elem0, vf, t.nrows, wave, lane, red);
        gseq_done(Ld, t.b, pos, pos);
    }
}

__global__ void gdn_advance_kernel(GLayer Ld, const int *accepted, int T)
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
// Speculative verify ([AT Pulse] "Technical analysis": output-only evaluation). Query q's window
// is the committed records plus drafts 0..q; its sweep runs in wave q mod 4. One pass over the
// checkpoint rows serves all T queries: U = S_c [z_1 .. z_T]. Drafts are appended tentatively at
// slots (pos + q) mod L; no pointer moves.
// ==========================================================================================
template <int LMAX, int TQ, int RT = kRows>
struct GVerifyLds {
    GWin<LMAX, RT> w;
    float q[TQ][NN] __attribute__((aligned(16)));
    float z[TQ][NN] __attribute__((aligned(16)));
    float c[TQ][LMAX];
    float u[TQ][RT];
};

// The verify's window through registers: the count0 committed records from the ring (record j at
// slot (ck + j) mod L), then the T drafts from the call's inputs, and the T queries. Issued before
// the checkpoint stream (global loads complete in issue order), committed to LDS after it.
template <int LMAX, int TQ, int RT>
struct VerifyWindow {
    static constexpr int KS = (LMAX * NN / 4 + kThreads - 1) / kThreads;
    static constexpr int KCH = KS < 8 ? KS : 8;  // k slots held at once; the rest load at commit
    static constexpr int VS = (LMAX * RT / 4 + kThreads - 1) / kThreads;
    static constexpr int QS = (TQ * NN / 4 + kThreads - 1) / kThreads;
    f32x4 kr[KCH], vr[VS], qr[QS];
    float ar, br;
    const float *rk, *rv;
    size_t bh, bT;
    int cslot, count0, kw, T, tid;  // cslot = ckpt_pos mod L

    __device__ int slot_of(const GLayer &Ld, int j) const { return ring_slot(cslot, j, Ld.L); }  // j < L
    __device__ const float *kaddr(const GLayer &Ld, const GTokenIO &io, const Tile &t, int j) const
    {
        return j < count0 ? rk + (size_t)slot_of(Ld, j) * NN : io.k + ((bT + (j - count0)) * Ld.G + t.g) * NN;
    }

    __device__ void issue(const GLayer &Ld, const GTokenIO &io, const Tile &t, int ck_, int count0_, int T_)
    {
        tid = threadIdx.x;
        cslot = (int)((unsigned)ck_ % (unsigned)Ld.L);
        count0 = count0_;
        T = T_;
        kw = count0 + T;
        bh = (size_t)t.b * Ld.H + t.h;
        bT = (size_t)t.b * T;
        rk = Ld.ring_k + ((size_t)t.b * Ld.G + t.g) * Ld.L * NN;
        rv = Ld.ring_v + bh * Ld.L * Ld.Dv + t.row0;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sl = 0; sl < KCH; ++sl) {
            const int e = tid + sl * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
            const f32x4 val = *(const f32x4 *)(kaddr(Ld, io, t, j < kw ? j : kw - 1) + 4 * c4);
            kr[sl] = j < kw ? val : zero;
        }
#pragma unroll
        for (int sl = 0; sl < VS; ++sl) {
            const int e = tid + sl * kThreads, j = e / (RT / 4), c4 = e % (RT / 4);
            const bool in = j < kw && 4 * c4 < t.nrows;
            const int jj = in ? j : 0, cc = in ? 4 * c4 : 0;
            const float *src = jj < count0 ? rv + (size_t)slot_of(Ld, jj) * Ld.Dv + cc
                                           : io.v + ((bT + (jj - count0)) * Ld.H + t.h) * Ld.Dv + t.row0 + cc;
            const f32x4 val = *(const f32x4 *)src;
            vr[sl] = in ? val : zero;
        }
        {
            const bool in = tid < kw;
            const int jj = in ? tid : 0;
            const size_t ri = jj < count0 ? bh * Ld.L + slot_of(Ld, jj) : 0;
            const size_t fi = jj < count0 ? 0 : (bT + (jj - count0)) * Ld.H + t.h;
            const float a = jj < count0 ? Ld.ring_a[ri] : io.alpha[fi];
            const float b = jj < count0 ? Ld.ring_b[ri] : io.beta[fi];
            ar = in ? a : 0.f;
            br = in ? b : 0.f;
        }
#pragma unroll
        for (int sl = 0; sl < QS; ++sl) {
            const int e = tid + sl * kThreads, q = e / (NN / 4), c4 = e % (NN / 4);
            const int qq = q < T ? q : 0;
            const f32x4 val = *(const f32x4 *)(io.q + ((bT + qq) * Ld.G + t.g) * NN + 4 * c4);
            qr[sl] = q < T ? val : zero;
        }
    }

    __device__ void commit(GVerifyLds<LMAX, TQ, RT> &s, const GLayer &Ld, const GTokenIO &io, const Tile &t)
    {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s0 = 0; s0 < KS; s0 += KCH) {
            if (s0 > 0) {
#pragma unroll
                for (int sl = 0; sl < KCH; ++sl) {
                    const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
                    kr[sl] = (s0 + sl < KS && j < kw) ? *(const f32x4 *)(kaddr(Ld, io, t, j) + 4 * c4) : zero;
                }
            }
#pragma unroll
            for (int sl = 0; sl < KCH; ++sl) {
                const int e = tid + (s0 + sl) * kThreads, j = e / (NN / 4), c4 = e % (NN / 4);
                if (s0 + sl < KS && j < LMAX) *(f32x4 *)&s.w.K[j][4 * c4] = kr[sl];
            }
        }
#pragma unroll
        for (int sl = 0; sl < VS; ++sl) {
            const int e = tid + sl * kThreads, j = e / (RT / 4), c4 = e % (RT / 4);
            if (j < LMAX) *(f32x4 *)&s.w.V[j][4 * c4] = vr[sl];
        }
        if (tid < LMAX) {
            s.w.a[tid] = ar;
            s.w.b[tid] = br;
        }
#pragma unroll
        for (int sl = 0; sl < QS; ++sl) {
            const int e = tid + sl * kThreads, q = e / (NN / 4), c4 = e % (NN / 4);
            if (q < TQ) *(f32x4 *)&s.q[q][4 * c4] = qr[sl];
        }
    }
};

// Outputs of a verify from the row dots in s.u and the window (o_q = S_c z_q + sum_j c_qj v_j for
// the tile's rows), and the T drafts appended at ring slots (pos + q) mod L (v by every tile,
// alpha / beta by the first tile, k by the first tile of the key head's first value head).
template <int LMAX, int TQ, int RT>
__device__ inline void verify_output_append(const GVerifyLds<LMAX, TQ, RT> &s, const GLayer &Ld, const GTokenIO &io,
                                            const Tile &t, int pos, int count0, int T)
{
    const int tid = threadIdx.x;
    const size_t bh = (size_t)t.b * Ld.H + t.h, bT = (size_t)t.b * T;
    const int pslot0 = (int)((unsigned)pos % (unsigned)Ld.L);  // draft q goes to slot (pos + q) mod L
    for (int e = tid; e < T * RT; e += kThreads) {
        const int q = e / RT, r = e % RT;
        if (r < t.nrows) {
            const int last = count0 + q;
            float acc = s.u[q][r];
            for (int j = 0; j <= last; ++j) acc = fmaf(s.c[q][j], s.w.V[j][r], acc);
            io.o[((bT + q) * Ld.H + t.h) * Ld.Dv + t.row0 + r] = acc;
            const int slot = ring_slot(pslot0, q, Ld.L);
            Ld.ring_v[(bh * Ld.L + slot) * Ld.Dv + t.row0 + r] = s.w.V[last][r];
        }
    }
    if (t.split == 0 && tid < T) {
        const int slot = ring_slot(pslot0, tid, Ld.L);
        Ld.ring_a[bh * Ld.L + slot] = s.w.a[count0 + tid];
        Ld.ring_b[bh * Ld.L + slot] = s.w.b[count0 + tid];
    }
    if (t.split == 0 && t.h % Ld.hpg == 0) {
        for (int e = tid; e < T * (NN / 4); e += kThreads) {
            const int q = e / (NN / 4), c4 = e % (NN / 4);
            const int slot = ring_slot(pslot0, q, Ld.L);
            *(f32x4 *)(Ld.ring_k + (((size_t)t.b * Ld.G + t.g) * Ld.L + slot) * NN + 4 * c4) =
                *(const f32x4 *)&s.w.K[count0 + q][4 * c4];
        }
    }
}

template <int LMAX, int TQ, int RP>
__global__ void __launch_bounds__(kThreads) gdn_verify_kernel(GLayer Ld, GTokenIO io, int T)
{
    __shared__ GVerifyLds<LMAX, TQ> s;
    const Tile t = gmap_tile(Ld);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    // Pointers first, then the window and the queries into registers, then the checkpoint stream:
    // global loads complete in issue order, so the window reaches LDS and the T backward sweeps
    // run while the stream is still in flight.
    const int pos = Ld.pos[t.b], ck = Ld.ckpt[t.b];
    const int count0 = pos - ck;
    if (!(ck >= 0 && count0 >= 0 && count0 <= Ld.L - Ld.Tmax && count0 + T <= Ld.L)) {
        graise(Ld, FLAG_POINTERS);
        return;
    }
    VerifyWindow<LMAX, TQ, kRows> win;
    win.issue(Ld, io, t, ck, count0, T);
    f32x4 vf[GF::NL];
    if constexpr (RP != PREC_F32) load_rows_copy<RP>(vf, Ld, bh, t.row0, t.nrows, wave, lane);
    else load_rows_f32(vf, Ld.master + (bh * Ld.Dv + t.row0) * NN, t.nrows, wave, lane);
    win.commit(s, Ld, io, t);
    __syncthreads();
    for (int q = wave; q < T; q += kWaves) gdn_sweep<LMAX>(s.w, s.q[q], count0 + q, s.c[q], s.z[q], lane);
    __syncthreads();
    rows_dot<TQ>(vf, &s.z[0][0], T, &s.u[0][0], wave, lane);
    __syncthreads();
    verify_output_append(s, Ld, io, t, pos, count0, T);
}

// Verify through the copy with one work-group per 128 value rows (as gdn_step_copy_kernel): one
// 16-byte chunk per lane and slot, the T sweeps once per head.
template <int LMAX, int TQ, int RP>
__global__ void __launch_bounds__(kThreads) gdn_verify_copy_kernel(GLayer Ld, GTokenIO io, int T, int splits)
{
    using CR = CopyRows<RP>;
    using G = typename CR::G;
    constexpr int NLC = CR::NL;
    __shared__ GVerifyLds<LMAX, TQ, kRowsC> s;
    const Tile t = gmap_tile_rows<kRowsC>(Ld, splits);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    const int pos = Ld.pos[t.b], ck = Ld.ckpt[t.b];
    const int count0 = pos - ck;
    if (!(ck >= 0 && count0 >= 0 && count0 <= Ld.L - Ld.Tmax && count0 + T <= Ld.L)) {
        graise(Ld, FLAG_POINTERS);
        return;
    }
    VerifyWindow<LMAX, TQ, kRowsC> win;
    win.issue(Ld, io, t, ck, count0, T);
    CR cr;
    cr.load(Ld, t, bh, wave, lane);
    win.commit(s, Ld, io, t);
    __syncthreads();
    for (int q = wave; q < T; q += kWaves) gdn_sweep<LMAX>(s.w, s.q[q], count0 + q, s.c[q], s.z[q], lane);
    __syncthreads();
    // S_c z_q for every query: each lane's chunk against the matching slice of z_q.
    float part[NLC * TQ];
#pragma unroll
    for (int q = 0; q < TQ; ++q)
#pragma unroll
        for (int i = 0; i < NLC; ++i) part[q * NLC + i] = q < T ? cr.dot(i, s.z[q], lane) : 0.f;
    transpose_reduce<NLC * TQ, G::LPR>(part, lane);
    bool writer;
    const int first = tr_first<NLC * TQ, G::LPR>(lane, &writer);
    if (writer) {
#pragma unroll
        for (int e = 0; e < tr_count<NLC * TQ, G::LPR>(); ++e) {
            const int idx = first + e, q = idx / NLC, r = CR::row_of(idx % NLC, wave, lane);
            if (q < T && r < kRowsC) s.u[q][r] = CR::finish(Ld, t, bh, r, part[e]);
        }
    }
    __syncthreads();
    verify_output_append(s, Ld, io, t, pos, count0, T);
}

// ==========================================================================================
// Load: master <- state; pointers, counters and the flag reset.
// ==========================================================================================
__global__ void __launch_bounds__(kThreads) gdn_load_kernel(GLayer Ld, const float *state)
{
    __shared__ float red[kWaves];
    const Tile t = gmap_tile(Ld);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h;
    const size_t elem0 = (bh * Ld.Dv + t.row0) * NN;
    f32x4 vf[GF::NL];
    load_rows_f32(vf, state + elem0, t.nrows, wave, lane);
    store_checkpoint(Ld, bh, elem0, vf, t.nrows, wave, lane, red);
    if (t.h == 0 && t.split == 0 && threadIdx.x == 0) {
        Ld.pos[t.b] = 0;
        Ld.ckpt[t.b] = 0;
        Ld.counter[t.b] = 0u;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *Ld.flag = 0u;
}

// ==========================================================================================
// Baseline: conventional GDN decode step in place ([Clarity] "Why it matters", claim ledger [6]:
// read the state, update it, read the output, write it back).
// ==========================================================================================
__global__ void __launch_bounds__(kThreads) gdn_conventional_kernel(GLayer Ld, float *state, GTokenIO io)
{
    __shared__ GWin<1> w;
    __shared__ float q[NN] __attribute__((aligned(16)));
    __shared__ float u[kRows];
    const Tile t = gmap_tile(Ld);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = (size_t)t.b * Ld.H + t.h, bg = (size_t)t.b * Ld.G + t.g;
    float *rows = state + (bh * Ld.Dv + t.row0) * NN;
    f32x4 vf[GF::NL];
    load_rows_f32(vf, rows, t.nrows, wave, lane);
    stage_window<1>(w, Ld, t, 0, 0, 1, io.k + bg * NN, 0, io.v + bh * Ld.Dv + t.row0, 0, io.alpha + bh, io.beta + bh, 0);
    if (tid < NN / 4) *(f32x4 *)&q[4 * tid] = *(const f32x4 *)(io.q + bg * NN + 4 * tid);
    __syncthreads();
    gdn_fold_rows<1>(vf, w, 1, wave, lane);
    store_rows(rows, vf, t.nrows, wave, lane);
    rows_dot<1>(vf, q, 1, u, wave, lane);
    __syncthreads();
    if (tid < t.nrows) io.o[bh * Ld.Dv + t.row0 + tid] = u[tid];
}

// ==========================================================================================
// Baseline: per-draft snapshots ([Clarity] "What happened", claim ledger [13]): read the
// committed slot once, run the T drafts stepwise, write the state after draft q to slot
// (cur + q + 1) mod (T + 1). One read and T writes of the state per verify.
// ==========================================================================================
template <int TQ>
__global__ void __launch_bounds__(kThreads) gdn_snapshot_kernel(GLayer Ld, float *slots, const int *cur, int T,
                                                                 GTokenIO io)
{
    __shared__ GWin<TQ> w;
    __shared__ float q[TQ][NN] __attribute__((aligned(16)));
    __shared__ float u[TQ][kRows];
    const Tile t = gmap_tile(Ld);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c0 = cur[t.b];
    if (c0 < 0 || c0 > T) return;
    const size_t tile = (size_t)Ld.Dv * NN;
    auto slot_rows = [&](int sl) {
        return slots + (((size_t)t.b * (T + 1) + sl) * Ld.H + t.h) * tile + (size_t)t.row0 * NN;
    };
    f32x4 vf[GF::NL];
    load_rows_f32(vf, slot_rows(c0), t.nrows, wave, lane);
    const size_t bT = (size_t)t.b * T;
    stage_window<TQ>(w, Ld, t, 0, 0, T, io.k + (bT * Ld.G + t.g) * NN, Ld.G * NN,
                     io.v + (bT * Ld.H + t.h) * Ld.Dv + t.row0, Ld.H * Ld.Dv, io.alpha + bT * Ld.H + t.h,
                     io.beta + bT * Ld.H + t.h, Ld.H);
    for (int e = tid; e < T * (NN / 4); e += kThreads) {
        const int qi = e / (NN / 4), c4 = e % (NN / 4);
        *(f32x4 *)&q[qi][4 * c4] = *(const f32x4 *)(io.q + ((bT + qi) * Ld.G + t.g) * NN + 4 * c4);
    }
    __syncthreads();
    const int c = lane % GF::LPR;
    float part[GF::NL * TQ];
#pragma unroll
    for (int qi = 0; qi < TQ; ++qi) {
        if (qi < T) {
            // one record: the fold of record qi alone
            const f32x4 kj = *(const f32x4 *)&w.K[qi][4 * c];
            const float aj = w.a[qi], bj = w.b[qi];
            const f32x4 qq = *(const f32x4 *)&q[qi][4 * c];
#pragma unroll
            for (int i = 0; i < GF::NL; ++i) {
                const int r = row_of_f32(i, wave, lane);
                float pk = vf[i].x * kj.x;
                pk = fmaf(vf[i].y, kj.y, pk);
                pk = fmaf(vf[i].z, kj.z, pk);
                pk = fmaf(vf[i].w, kj.w, pk);
                const float sk = row_allreduce(pk);
                const float coef = bj * (w.V[qi][r < kRows ? r : 0] - aj * sk);
                vf[i].x = fmaf(coef, kj.x, aj * vf[i].x);
                vf[i].y = fmaf(coef, kj.y, aj * vf[i].y);
                vf[i].z = fmaf(coef, kj.z, aj * vf[i].z);
                vf[i].w = fmaf(coef, kj.w, aj * vf[i].w);
                float s = vf[i].x * qq.x;
                s = fmaf(vf[i].y, qq.y, s);
                s = fmaf(vf[i].z, qq.z, s);
                part[qi * GF::NL + i] = fmaf(vf[i].w, qq.w, s);
            }
            store_rows(slot_rows((c0 + qi + 1) % (T + 1)), vf, t.nrows, wave, lane);
        } else {
#pragma unroll
            for (int i = 0; i < GF::NL; ++i) part[qi * GF::NL + i] = 0.f;
        }
    }
    transpose_reduce<GF::NL * TQ, GF::LPR>(part, lane);
    bool writer;
    const int first = tr_first<GF::NL * TQ, GF::LPR>(lane, &writer);
    constexpr int cnt = tr_count<GF::NL * TQ, GF::LPR>();
    if (writer) {
#pragma unroll
        for (int e = 0; e < cnt; ++e) {
            const int idx = first + e, qi = idx / GF::NL, i = idx % GF::NL;
            const int r = row_of_f32(i, wave, lane);
            if (qi < T && r < kRows) u[qi][r] = part[e];
        }
    }
    __syncthreads();
    if (tid < t.nrows)
        for (int qi = 0; qi < T; ++qi) io.o[((bT + qi) * Ld.H + t.h) * Ld.Dv + t.row0 + tid] = u[qi][tid];
}

inline unsigned gblocks(const GLayer &Ld) { return (unsigned)Ld.Bt * (unsigned)Ld.H * (unsigned)Ld.psplit; }

template <int LMAX, int RP>
hipError_t step_lc(const GLayer &Ld, const GTokenIO &io, bool fc, bool all_flush, Lockstep ls, hipStream_t st)
{
    if constexpr (kWideFold) {
        if (fc && all_flush) {
            hipLaunchKernelGGL((gdn_flush_step_kernel<LMAX>), dim3(gblocks(Ld)), dim3(kThreads), 0, st, Ld, io, ls);
            return hipGetLastError();
        }
    }
    if constexpr (kCopyTiles<RP> && LMAX <= 32) {
        if (!fc) {
            const int splits = (Ld.Dv + kRowsC - 1) / kRowsC;
            const unsigned grid = (unsigned)Ld.Bt * (unsigned)Ld.H * (unsigned)splits;
            hipLaunchKernelGGL((gdn_step_copy_kernel<LMAX, RP>), dim3(grid), dim3(kThreads), 0, st, Ld, io, ls, splits);
            return hipGetLastError();
        }
    }
    if (fc) hipLaunchKernelGGL((gdn_step_kernel<LMAX, true, RP>), dim3(gblocks(Ld)), dim3(kThreads), 0, st, Ld, io, ls);
    else hipLaunchKernelGGL((gdn_step_kernel<LMAX, false, RP>), dim3(gblocks(Ld)), dim3(kThreads), 0, st, Ld, io, ls);
    return hipGetLastError();
}

// The copy precisions a key size supports (MXFP4: blocks of 32 key columns, Dk >= 32).
template <template <int> class F, typename... Args>
hipError_t by_rprec(int rprec, Args &&...args)
{
    switch (rprec) {
    case PREC_F32: return F<PREC_F32>::run(args...);
    case PREC_BF16: return F<PREC_BF16>::run(args...);
    case PREC_FP8: return F<PREC_FP8>::run(args...);
    case PREC_FP4:
        if constexpr (NN >= 32) return F<PREC_FP4>::run(args...);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int LMAX>
struct StepL {
    template <int RP>
    struct F {
        static hipError_t run(const GLayer &Ld, const GTokenIO &io, bool fc, bool af, Lockstep ls, hipStream_t st)
        {
            return step_lc<LMAX, RP>(Ld, io, fc, af, ls, st);
        }
    };
};

template <int LMAX>
hipError_t step_l(const GLayer &Ld, const GTokenIO &io, bool fc, bool af, Lockstep ls, hipStream_t st)
{
    return by_rprec<StepL<LMAX>::template F>(Ld.rprec, Ld, io, fc, af, ls, st);
}

template <int LMAX>
hipError_t flush_l(const GLayer &Ld, int mode, const int *arg, int T, float *out, hipStream_t st)
{
    if (mode == MODE_OVERFULL) {
        hipLaunchKernelGGL(gdn_advance_kernel, dim3((Ld.Bt + 255) / 256), dim3(256), 0, st, Ld, arg, T);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gdn_flush_kernel<LMAX>), dim3(gblocks(Ld)), dim3(kThreads), 0, st, Ld, mode,
                       mode == MODE_OVERFULL ? nullptr : arg, out);
    return hipGetLastError();
}

template <int LMAX, int RP>
hipError_t verify_lc(const GLayer &Ld, const GTokenIO &io, int T, hipStream_t st)
{
    if constexpr (kCopyTiles<RP> && LMAX <= 32) {
        const int splits = (Ld.Dv + kRowsC - 1) / kRowsC;
        const dim3 grid((unsigned)Ld.Bt * (unsigned)Ld.H * (unsigned)splits), block(kThreads);
        if (T <= 2) hipLaunchKernelGGL((gdn_verify_copy_kernel<LMAX, 2, RP>), grid, block, 0, st, Ld, io, T, splits);
        else if (T <= 4) hipLaunchKernelGGL((gdn_verify_copy_kernel<LMAX, 4, RP>), grid, block, 0, st, Ld, io, T, splits);
        else hipLaunchKernelGGL((gdn_verify_copy_kernel<LMAX, 8, RP>), grid, block, 0, st, Ld, io, T, splits);
        return hipGetLastError();
    }
    const dim3 grid(gblocks(Ld)), block(kThreads);
    if (T <= 2) hipLaunchKernelGGL((gdn_verify_kernel<LMAX, 2, RP>), grid, block, 0, st, Ld, io, T);
    else if (T <= 4) hipLaunchKernelGGL((gdn_verify_kernel<LMAX, 4, RP>), grid, block, 0, st, Ld, io, T);
    else hipLaunchKernelGGL((gdn_verify_kernel<LMAX, 8, RP>), grid, block, 0, st, Ld, io, T);
    return hipGetLastError();
}

template <int LMAX>
struct VerifyL {
    template <int RP>
    struct F {
        static hipError_t run(const GLayer &Ld, const GTokenIO &io, int T, hipStream_t st)
        {
            return verify_lc<LMAX, RP>(Ld, io, T, st);
        }
    };
};

template <int LMAX>
hipError_t verify_l(const GLayer &Ld, const GTokenIO &io, int T, hipStream_t st)
{
    return by_rprec<VerifyL<LMAX>::template F>(Ld.rprec, Ld, io, T, st);
}

}  // namespace

#define RSSM_CAT2(a, b) a##b
#define RSSM_CAT(a, b) RSSM_CAT2(a, b)

hipError_t RSSM_CAT(gdn_launch_step_n, RSSM_N)(int lmax, const GLayer &Ld, const GTokenIO &io, bool flush_capable,
                                               bool all_flush, Lockstep ls, hipStream_t st)
{
    switch (lmax) {
    case 16: return step_l<16>(Ld, io, flush_capable, all_flush, ls, st);
    case 32: return step_l<32>(Ld, io, flush_capable, all_flush, ls, st);
    case 64: return step_l<64>(Ld, io, flush_capable, all_flush, ls, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t RSSM_CAT(gdn_launch_flush_n, RSSM_N)(int lmax, const GLayer &Ld, int mode, const int *arg, int T,
                                                float *out, hipStream_t st)
{
    switch (lmax) {
    case 16: return flush_l<16>(Ld, mode, arg, T, out, st);
    case 32: return flush_l<32>(Ld, mode, arg, T, out, st);
    case 64: return flush_l<64>(Ld, mode, arg, T, out, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t RSSM_CAT(gdn_launch_verify_n, RSSM_N)(int lmax, const GLayer &Ld, const GTokenIO &io, int T, hipStream_t st)
{
    switch (lmax) {
    case 16: return verify_l<16>(Ld, io, T, st);
    case 32: return verify_l<32>(Ld, io, T, st);
    case 64: return verify_l<64>(Ld, io, T, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t RSSM_CAT(gdn_launch_load_n, RSSM_N)(const GLayer &Ld, const float *state, hipStream_t st)
{
    hipLaunchKernelGGL(gdn_load_kernel, dim3(gblocks(Ld)), dim3(kThreads), 0, st, Ld, state);
    return hipGetLastError();
}

hipError_t RSSM_CAT(gdn_launch_conventional_n, RSSM_N)(const GLayer &Ld, float *state, const GTokenIO &io, hipStream_t st)
{
    hipLaunchKernelGGL(gdn_conventional_kernel, dim3(gblocks(Ld)), dim3(kThreads), 0, st, Ld, state, io);
    return hipGetLastError();
}

hipError_t RSSM_CAT(gdn_launch_snapshot_n, RSSM_N)(const GLayer &Ld, float *slots, const int *cur, int T,
                                                   const GTokenIO &io, hipStream_t st)
{
    const dim3 grid(gblocks(Ld)), block(kThreads);
    if (T <= 2) hipLaunchKernelGGL((gdn_snapshot_kernel<2>), grid, block, 0, st, Ld, slots, cur, T, io);
    else if (T <= 4) hipLaunchKernelGGL((gdn_snapshot_kernel<4>), grid, block, 0, st, Ld, slots, cur, T, io);
    else hipLaunchKernelGGL((gdn_snapshot_kernel<8>), grid, block, 0, st, Ld, slots, cur, T, io);
    return hipGetLastError();
}

}  // namespace rssm
