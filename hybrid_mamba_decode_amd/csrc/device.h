// device.h -- device-side building blocks shared by the ReplaySSM kernels (gfx950, wave64).
//
// Tiling. One work-group (256 threads = 4 wave64s) owns up to kRows = 64 rows (headdim entries
// p) of one (sequence, head) state tile [P, N]; a head with P > 64 is split over ceil(P/64)
// work-groups. Within a wave the lanes run along N: each lane loads one 16-byte chunk of a row
// per load slot (4 fp32, 8 bf16, 16 fp8 or 32 fp4 values -- one fp4 chunk is exactly one MXFP4
// scale block), LPR = N / VEC lanes cover a row and one wave
// instruction covers RPI = 64 / LPR consecutive rows, so every wave instruction reads a
// contiguous, fully coalesced 1 KiB. Per-row dot products are finished by a transpose-reduce
// across the LPR lanes of a row (NL - 1 + log2(LPR/NL) lane exchanges instead of
// NL * log2(LPR)).
//
// Work-group -> tile order is XCD-aware: MI355X dispatches consecutive work-groups round-robin
// over its 8 XCDs (each with its own L2), so block i is given tile (i % 8) * (nblk / 8) + i / 8.
// Each XCD then walks a contiguous range of tiles, and the heads of one group -- which share that
// group's B window -- hit the same L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 64;

// Read precisions of the replay kernels. PREC_F16 reads an fp16 master directly (no copy).
enum { PREC_F32 = 0, PREC_BF16 = 1, PREC_FP8 = 2, PREC_FP4 = 3, PREC_F16 = 4 };

// Master (checkpoint) precisions: fp32, fp16 or fp8 (E4M3FN codes with a per-head scale, kept in
// the fp8 read copy's place), the narrow ones rounded to nearest even / stochastically.
enum { MASTER_F32 = 0, MASTER_F16 = 1, MASTER_F16_SR = 2, MASTER_F8 = 3, MASTER_F8_SR = 4 };

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Everything a kernel needs to know about one layer's workspace (passed by value).
struct Layer {
    float *master;      // [Bt,H,P,N] checkpoint: fp32, or fp16 (reinterpret) when mprec != 0
    void *rcopy;        // [Bt,H,P,N] bf16 / e4m3 read copy, or [Bt,H,P,N/2] MXFP4 bytes
    float *scale;       // [Bt,H] fp8 per-head scale
    unsigned char *mxscale;  // [Bt,H,P,N/32] MXFP4 E8M0 block-scale codes
    float *ring_x;      // [Bt,H,L,P]
    float *ring_B;      // [Bt,G,L,N]
    float *ring_C;      // [Bt,G,L,N] or nullptr
    float *ring_dt;     // [Bt,H,L]
    int *pos;           // [Bt]
    int *ckpt;          // [Bt]
    unsigned *counter;  // [Bt]
    unsigned *flag;     // [1]
    const float *A;     // [H]
    const float *D;     // [H]
    int Bt, H, P, G, L, Tmax, hpg, psplit;
    int mprec;          // MASTER_*
    unsigned sr_seed;   // key of the stochastic-rounding stream
    // Mixer edges (K > 0): raw in-projection xBC of recent positions, position q at slot q mod R
    float *conv_ring;       // [Bt,R,CD]
    const float *conv_w;    // [CD,K]
    const float *conv_b;    // [CD]
    const float *dt_bias;   // [H]
    int K, R, CD;
    int wvec;               // K == 4 and conv_w 16-byte aligned: a channel's weights in one load
};

// Per-token inputs of one call (layouts in replayssm.h).
struct TokenIO {
    const float *x, *B, *C, *dt;  // with the mixer edges: dt holds dt_raw, x/B/C are unused
    float *y;
    const float *xbc, *z;         // mixer edges: raw in-projection xBC [..,CD] and gate input z
};

// Lockstep window position: when every sequence is known (on the host) to be at the same window
// position, kernels take it as (pos mod L, ckpt_pos mod L, records in the window including this
// token); k = 0 means "read each sequence's device pointers".
struct Lockstep {
    int pslot, cslot, k;
    int rslot;  // pos mod R (mixer edges' conv ring)
};

// Mixer-edge activations in fp32: silu(v) = v / (1 + e^-v); softplus(v) = log(1 + e^v), in the
// overflow-free form v + log(1 + e^-v) for v > 0.
__device__ inline float silu_f(float v) { return v / (1.0f + expf(-v)); }
__device__ inline float softplus_f(float v) { return v > 0.f ? v + log1pf(expf(-v)) : log1pf(expf(v)); }

// One conv channel's operands in registers (K <= 4): issued early by conv_issue, consumed by
// conv_finish, so that the loads go out with a kernel's other early loads.
struct ConvIn {
    float cur, wc, b, tap[3], wt[3];
};

// Ring element of sequence b, channel c, slot sl ([Bt,R,CD]: a wave's channels are contiguous).
__device__ inline size_t ring_at(const Layer &Ld, int b, int c, int sl)
{
    return ((size_t)b * Ld.R + sl) * Ld.CD + c;
}

// Operands of channel c for sequence b at position pos (ring slot rslot): this token's raw value
// from raw, its weight and the bias, and the K-1 history taps (oldest first) with their weights.
// K = 4 with aligned weights: the channel's weights in one 16-byte load. Unused taps
// (i >= K-1) read slot 0 and weight 0 of the channel, so every address stays inside its rows.
__device__ inline ConvIn conv_issue(const Layer &Ld, int b, int c, int rslot, const float *raw)
{
    ConvIn r;
    r.cur = raw[c];
    r.b = Ld.conv_b[c];
    bool in[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        in[i] = i < Ld.K - 1;
        const int d = Ld.K - 1 - i;  // position pos - d
        const int sl = !in[i] ? 0 : rslot >= d ? rslot - d : rslot - d + Ld.R;
        const float v = Ld.conv_ring[ring_at(Ld, b, c, sl)];
        r.tap[i] = in[i] ? v : 0.f;
    }
    const float *w = Ld.conv_w + (size_t)c * Ld.K;
    if (Ld.wvec) {
        const f32x4 w4 = *(const f32x4 *)w;
        r.wt[0] = w4.x;
        r.wt[1] = w4.y;
        r.wt[2] = w4.z;
        r.wc = w4.w;
    } else {
        r.wc = w[Ld.K - 1];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const float wv = w[in[i] ? i : 0];
            r.wt[i] = in[i] ? wv : 0.f;
        }
    }
    return r;
}

__device__ inline float conv_finish(const ConvIn &r)
{
    float u = fmaf(r.wc, r.cur, r.b);
#pragma unroll
    for (int i = 0; i < 3; ++i) u = fmaf(r.wt[i], r.tap[i], u);
    return silu_f(u);
}

// Ring slot of the record j places after the one in slot `base` (base < L, 0 <= j < L): one
// compare and subtract instead of an integer division by the runtime L.
__device__ inline int ring_slot(int base, int j, int L)
{
    const int sl = base + j;
    return sl >= L ? sl - L : sl;
}

// Device flag bits.
enum : unsigned { FLAG_POINTERS = 1u, FLAG_ACCEPTED = 2u };

template <int N, int PREC>
struct Geo {
    static constexpr int VEC = PREC == PREC_F32 ? 4 : (PREC == PREC_BF16 || PREC == PREC_F16) ? 8 : PREC == PREC_FP8 ? 16 : 32;
    static constexpr int LPR = N / VEC;          // lanes per row
    static constexpr int RPI = 64 / LPR;         // rows per wave instruction
    static constexpr int RPB = kWaves * RPI;     // rows per work-group instruction
    static constexpr int NL = (kRows + RPB - 1) / RPB;  // load slots per lane for kRows rows
    static_assert(N % VEC == 0 && LPR >= 1 && LPR <= 64, "unsupported N for this precision");
    static_assert(NL <= LPR || LPR == 1 || NL == 1, "transpose-reduce needs NL <= LPR");
};

struct Tile {
    int b, h, g, split, row0, nrows;
};

__device__ inline Tile map_tile(const Layer &Ld)
{
    const unsigned nblk = gridDim.x, i = blockIdx.x;
    const unsigned id = (nblk % 8u == 0u) ? (i % 8u) * (nblk / 8u) + i / 8u : i;
    Tile t;
    t.split = (int)(id % (unsigned)Ld.psplit);
    const unsigned bh = id / (unsigned)Ld.psplit;
    t.h = (int)(bh % (unsigned)Ld.H);
    t.b = (int)(bh / (unsigned)Ld.H);
    t.g = t.h / Ld.hpg;
    t.row0 = t.split * kRows;
    t.nrows = min(kRows, Ld.P - t.row0);
    return t;
}

// ------------------------------------------------------------------------------------------
// Loads and stores. State tiles stream through once per call: non-temporal, so they do not
// evict the record windows that several work-groups share from L2.
// ------------------------------------------------------------------------------------------
__device__ inline u32x4 load_nt(const void *p) { return __builtin_nontemporal_load((const u32x4 *)p); }
__device__ inline void store_nt(void *p, u32x4 v) { __builtin_nontemporal_store(v, (u32x4 *)p); }
__device__ inline f32x4 as_f32x4(u32x4 v) { return __builtin_bit_cast(f32x4, v); }
__device__ inline u32x4 as_u32x4(f32x4 v) { return __builtin_bit_cast(u32x4, v); }

// ------------------------------------------------------------------------------------------
// Read-copy codecs.
// bf16: the top half of an fp32 word, rounded to nearest, ties to the even 16-bit code.
// e4m3: OCP FP8 E4M3FN (bias 7, 3 mantissa bits, max 448, no infinities), saturating; both
// directions use gfx950's fp8 converters.
// ------------------------------------------------------------------------------------------
__device__ inline unsigned bf16_rne(float f)
{
    const unsigned u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// e4m3 encode: the fp32 value (already multiplied by 1/scale) is clamped to +-448 and converted
// by gfx950's v_cvt_pk_fp8_f32, which rounds to nearest even into OCP E4M3FN (checked on the GPU
// against the format definition for every fp32 pattern below 464 in magnitude, subnormals
// included); see write_copy_rows.

// Dot product of one 16-byte chunk of a state row with the matching slice of C.
template <int PREC>
__device__ inline float chunk_dot(u32x4 v, const float *c);

template <>
__device__ inline float chunk_dot<PREC_F32>(u32x4 v, const float *c)
{
    const f32x4 f = as_f32x4(v);
    float s = f.x * c[0];
    s = fmaf(f.y, c[1], s);
    s = fmaf(f.z, c[2], s);
    return fmaf(f.w, c[3], s);
}

template <>
__device__ inline float chunk_dot<PREC_BF16>(u32x4 v, const float *c)
{
    float s = bf16_lo(v.x) * c[0];
    s = fmaf(bf16_hi(v.x), c[1], s);
    s = fmaf(bf16_lo(v.y), c[2], s);
    s = fmaf(bf16_hi(v.y), c[3], s);
    s = fmaf(bf16_lo(v.z), c[4], s);
    s = fmaf(bf16_hi(v.z), c[5], s);
    s = fmaf(bf16_lo(v.w), c[6], s);
    return fmaf(bf16_hi(v.w), c[7], s);
}

// fp16 (the master read directly): eight values per chunk, converted exactly.
__device__ inline f32x2 f16x2_to_f32(unsigned w)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = __builtin_bit_cast(h2, w);
    return f32x2{(float)h.x, (float)h.y};
}

template <>
__device__ inline float chunk_dot<PREC_F16>(u32x4 v, const float *c)
{
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 f = f16x2_to_f32(w[i]);
        s = fmaf(f.x, c[2 * i], s);
        s = fmaf(f.y, c[2 * i + 1], s);
    }
    return s;
}

// ------------------------------------------------------------------------------------------
// fp16 master rounding. Nearest even by gfx950's converter (values clamped to +-65504 first).
// Stochastic: with q the fp16 magnitude toward zero from |v| and ulp the spacing above it, round
// up iff r16 < (|v| - q) / ulp * 2^16. Both factors are exact in fp32 (Sterbenz; scaling by a
// power of two), so the decision is exact. In fp16's normal range the threshold is a multiple of
// 8 (fp32 keeps 13 bits below the fp16 spacing), so the rounding is exactly unbiased over r16;
// below 2^-17 the bias is under 2^-16 of a spacing.
// r16 = 16-bit field of Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2,
// 3", SC'11) of counter (element / 8, sequence, new ckpt_pos, 0) and key (seed, 0): element e
// takes bits 16 * (e % 2) .. +15 of word (e % 8) / 2 (elements numbered h*P*N + p*N + n within
// the sequence).
// ------------------------------------------------------------------------------------------
__device__ inline unsigned short f16_bits(float v) { return __builtin_bit_cast(unsigned short, (_Float16)v); }
__device__ inline float f16_value(unsigned short h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ inline unsigned short f16_rne(float v)
{
    return f16_bits(fminf(fmaxf(v, -65504.0f), 65504.0f));
}

__device__ inline unsigned short f16_sr(float v, unsigned r16)
{
    const float a = fminf(fabsf(v), 65504.0f);
    if (a >= 0x1p-14f) {
        // fp16 normal range: the spacing is 2^13 fp32 spacings of a and |v| - q is the low 13 bits
        // of a's encoding (low13 of them), so the rule reads r16 < low13 * 2^3, i.e.
        // (r16 >> 3) < low13: adding 2^13 - 1 - (r16 >> 3) to the encoding carries into bit 13
        // exactly then; the truncated sum is the chosen fp16 value, converted exactly.
        const unsigned u = (__float_as_uint(a) + (0x1FFFu - (r16 >> 3))) & ~0x1FFFu;
        return (unsigned short)(f16_bits(__uint_as_float(u)) | (__float_as_uint(v) >> 31 << 15));
    }
    unsigned short h = f16_bits(a);  // nearest even
    float q = f16_value(h);
    if (q > a) {
        h = (unsigned short)(h - 1);
        q = f16_value(h);
    }
    if (a > q) {
        const float ulp = f16_value((unsigned short)(h + 1)) - q;
        if ((float)r16 < (a - q) * (65536.0f / ulp)) h = (unsigned short)(h + 1);
    }
    return (unsigned short)(h | (__float_as_uint(v) >> 31 << 15));
}

// Stochastic rounding of a (already divided by the scale and clamped to +-448) onto the E4M3FN
// grid, with the same 16-bit rule: up iff r16 < (|a| - q) / ulp * 2^16. Returns the chosen E4M3
// value as fp32 (the converter then encodes it exactly). For |a| >= 2^-6 the spacing is 2^20
// fp32 spacings of a, so the rule reads (r16 << 4) < low20 and one carry into bit 20 decides it;
// below, the spacing is 2^-9 and a * 2^9 splits exactly into its floor and fraction.
__device__ inline float e4m3_sr(float a, unsigned r16)
{
    const unsigned u = __float_as_uint(a), sgn = u & 0x80000000u, m = u & 0x7FFFFFFFu;
    if (m >= 0x3C800000u)  // 2^-6
        return __uint_as_float(((m + (0xFFFFFu - (r16 << 4))) & ~0xFFFFFu) | sgn);
    const float t = __uint_as_float(m) * 512.0f;
    const float fl = floorf(t);
    const float q = (float)r16 < (t - fl) * 65536.0f ? fl + 1.0f : fl;
    return __uint_as_float(__float_as_uint(q * (1.0f / 512.0f)) | sgn);
}

struct U32x4 {
    unsigned x, y, z, w;
};

__device__ inline U32x4 philox4x32_10(unsigned c0, unsigned c1, unsigned c2, unsigned c3, unsigned k0, unsigned k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // one 32x32 -> 64-bit multiply per product (v_mad_u64_u32), high and low halves
        const unsigned long long p0 = (unsigned long long)0xD2511F53u * c0;
        const unsigned long long p1 = (unsigned long long)0xCD9E8D57u * c2;
        // three-input xor in one v_bitop3_b32 (truth table 0x96 = a ^ b ^ c)
        const unsigned n0 = __builtin_amdgcn_bitop3_b32((unsigned)(p1 >> 32), c1, k0, 0x96);
        const unsigned n2 = __builtin_amdgcn_bitop3_b32((unsigned)(p0 >> 32), c3, k1, 0x96);
        c0 = n0;
        c1 = (unsigned)p1;
        c2 = n2;
        c3 = (unsigned)p0;
    }
    return U32x4{c0, c1, c2, c3};
}

// e4m3 codes are decoded by gfx950's converter, two per instruction (OCP E4M3FN on this
// target: checked against the format's table for all 256 codes); the per-head scale is applied
// once to the finished row sum.
template <>
__device__ inline float chunk_dot<PREC_FP8>(u32x4 v, const float *c)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    float s = 0.0f;
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        s = fmaf(lo.x, c[4 * i + 0], s);
        s = fmaf(lo.y, c[4 * i + 1], s);
        s = fmaf(hi.x, c[4 * i + 2], s);
        s = fmaf(hi.y, c[4 * i + 3], s);
    }
    return s;
}

// MXFP4 codes: 32 E2M1 values per chunk (one scale block), decoded by gfx950's converter two per
// instruction, low nibble first (checked on the GPU against the E2M1 table for every byte value
// and byte position, signed zeros included). The block scale 2^(code - 127) is applied to the
// lane's partial sum (mx_scaled).
template <>
__device__ inline float chunk_dot<PREC_FP4>(u32x4 v, const float *c)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    float s = 0.0f;
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 0);
        const f32x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 1);
        const f32x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 2);
        const f32x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 3);
        s = fmaf(b0.x, c[8 * i + 0], s);
        s = fmaf(b0.y, c[8 * i + 1], s);
        s = fmaf(b1.x, c[8 * i + 2], s);
        s = fmaf(b1.y, c[8 * i + 3], s);
        s = fmaf(b2.x, c[8 * i + 4], s);
        s = fmaf(b2.y, c[8 * i + 5], s);
        s = fmaf(b3.x, c[8 * i + 6], s);
        s = fmaf(b3.y, c[8 * i + 7], s);
    }
    return s;
}

// A partial sum over one MXFP4 block times the block scale 2^(code - 127) (exact: v_ldexp_f32).
__device__ inline float mx_scaled(float part, unsigned code) { return __builtin_amdgcn_ldexpf(part, (int)code - 127); }

// MXFP4 encode of four consecutive fp32 values of one block, given the block's amax: returns the
// E8M0 code; `codes` gets the two code bytes (element order low nibble first). Scale exponent =
// max(biased exponent of amax - 2, 0), so every value / scale is below 8; the division is exact
// (multiplication by 2^(127 - code), a normal fp32 for codes 0..253; a product that underflows
// is below 0.25 either way). gfx950's v_cvt_scalef32_pk_fp4_f32 rounds to nearest even and
// clamps to +-6 (checked on the GPU against that rule over dense sweeps of [2^-4, 8], ties
// included); every fp32 value of magnitude below 0.25 -- signed zeros and denormals too -- gives
// the signed zero code (0 or 8: checked on the GPU over all 2 x 1,048,576,000 of them).
__device__ inline unsigned mx_code_of(float amax)
{
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
    return (unsigned)(e > 2 ? e - 2 : 0);
}

__device__ inline unsigned short mx_encode4(f32x4 f, unsigned code)
{
    const float inv = __uint_as_float((254u - code) << 23);  // 2^(127 - code)
    const float a[4] = {f.x * inv, f.y * inv, f.z * inv, f.w * inv};
    const unsigned lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a[0], a[1], 1.0f, 0) & 0xFFu;
    const unsigned hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a[2], a[3], 1.0f, 0) & 0xFFu;
    return (unsigned short)(lo | (hi << 8));
}

// ------------------------------------------------------------------------------------------
// Cross-lane exchanges that stay in the VALU. On gfx950 a __shfl_* lowers to ds_bpermute: an
// LDS round trip plus address arithmetic per call, which serializes reductions inside record
// loops. Within a row of 16 lanes DPP moves the data; across rows and halves of the wave the
// permlane swaps do (v_permlane16_swap / v_permlane32_swap, new in gfx950).
// ------------------------------------------------------------------------------------------
// DPP move of v (dpp_ctrl CTRL); a lane whose source lies outside its row reads 0.
template <int CTRL>
__device__ inline float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Both values of the lane pair (l, l ^ O), O = 16 or 32, from one swap of two copies of v: the
// lane with bit O clear holds its own value in .x and its partner's in .y, the other lane the
// reverse (the swap exchanges the odd rows of the first copy with the even rows of the second,
// or the upper half of the first with the lower half of the second).
template <int O>
__device__ inline f32x2 pair_far(float v)
{
    static_assert(O == 16 || O == 32, "permlane swaps exchange rows of 16 or halves of 32");
    const unsigned u = __float_as_uint(v);
    if constexpr (O == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
    }
}

// Value of lane l ^ O for O = 1, 2, 16, 32. For O = 4 and 8 the partner is l ^ 7 and l ^ 15 (the
// half-row and row mirrors): still a lane whose bit O differs and whose bits above O agree, so a
// butterfly or transpose that runs its offsets from high to low down to 1 pairs the same sets.
template <int O>
__device__ inline float partner(float v, int lane)
{
    if constexpr (O == 1) return dpp_f<0xB1>(v);        // quad_perm [1,0,3,2]
    else if constexpr (O == 2) return dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    else if constexpr (O == 4) return dpp_f<0x141>(v);  // row_half_mirror
    else if constexpr (O == 8) return dpp_f<0x140>(v);  // row_mirror
    else {
        const f32x2 p = pair_far<O>(v);
        return (lane & O) ? p.x : p.y;
    }
}

// Sum over aligned groups of W lanes (W a power of two, <= 64); every lane of a group receives
// the same value (each exchange adds a symmetric pair).
template <int W>
__device__ inline float group_sum(float v)
{
    if constexpr (W >= 64) { const f32x2 p = pair_far<32>(v); v = p.x + p.y; }
    if constexpr (W >= 32) { const f32x2 p = pair_far<16>(v); v = p.x + p.y; }
    if constexpr (W >= 16) v += dpp_f<0x140>(v);
    if constexpr (W >= 8) v += dpp_f<0x141>(v);
    if constexpr (W >= 4) v += dpp_f<0x4E>(v);
    if constexpr (W >= 2) v += dpp_f<0xB1>(v);
    return v;
}

template <int W>
__device__ inline float group_max(float v)
{
    if constexpr (W >= 64) { const f32x2 p = pair_far<32>(v); v = fmaxf(p.x, p.y); }
    if constexpr (W >= 32) { const f32x2 p = pair_far<16>(v); v = fmaxf(p.x, p.y); }
    if constexpr (W >= 16) v = fmaxf(v, dpp_f<0x140>(v));
    if constexpr (W >= 8) v = fmaxf(v, dpp_f<0x141>(v));
    if constexpr (W >= 4) v = fmaxf(v, dpp_f<0x4E>(v));
    if constexpr (W >= 2) v = fmaxf(v, dpp_f<0xB1>(v));
    return v;
}

// Inclusive suffix sums over the window's lanes: lane l receives sum_{i >= l} v_i. Records sit
// in lanes 0 .. W-1 (W the window bound) and every other lane of the wave holds 0. For W <= 16
// the four row shifts of the first row suffice (row_shl: lane l reads l + o, 0 past the row's
// end); `next` receives the suffix sum from lane l + 1.
template <int W>
__device__ inline float suffix_sum(float v, int lane, float *next)
{
    if constexpr (W <= 16) {
        v += dpp_f<0x101>(v);
        v += dpp_f<0x102>(v);
        v += dpp_f<0x104>(v);
        v += dpp_f<0x108>(v);
        *next = dpp_f<0x101>(v);
    } else {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float nb = __shfl_down(v, o, 64);
            v += lane + o < 64 ? nb : 0.f;
        }
        const float nxt = __shfl_down(v, 1, 64);
        *next = lane + 1 < 64 ? nxt : 0.f;
    }
    return v;
}

// Lane 0's value, in every lane (a scalar read of the register).
__device__ inline float lane0(float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)); }

// ------------------------------------------------------------------------------------------
// Transpose-reduce. Each lane holds M partial sums (M a power of two); the LPR consecutive lanes
// of a row group must each sum over the group. At every exchange step with lane offset o the
// pair (l, partner<o>(l)) splits its list: the lane with bit o clear keeps the first half and
// receives the partner's first half, the other keeps the second half. Once one value is left, the remaining
// offsets are plain butterflies. Afterwards a lane holds max(1, M/LPR) complete sums: those of
// list entries [first, first + count) with first = its selected bits, see tr_first().
// ------------------------------------------------------------------------------------------
template <int M, int O, int NCUR>
struct TransposeStep {
    __device__ static inline void run(float (&v)[M], int lane)
    {
        if constexpr (O >= 1) {
            if constexpr (NCUR > 1) {
                constexpr int half = NCUR / 2;
                const bool upper = (lane & O) != 0;
#pragma unroll
                for (int m = 0; m < half; ++m) {
                    const float send = upper ? v[m] : v[half + m];
                    const float keep = upper ? v[half + m] : v[m];
                    v[m] = keep + partner<O>(send, lane);
                }
                TransposeStep<M, O / 2, half>::run(v, lane);
            } else {
                v[0] += partner<O>(v[0], lane);
                TransposeStep<M, O / 2, 1>::run(v, lane);
            }
        }
    }
};

template <int M, int LPR>
__device__ inline void transpose_reduce(float (&v)[M], int lane)
{
    TransposeStep<M, LPR / 2, M>::run(v, lane);
}

// Index (into the original list) of the first complete sum a lane holds after transpose_reduce,
// and whether the lane is the designated writer among its replicas.
template <int M, int LPR>
__device__ inline int tr_first(int lane, bool *writer)
{
    int n = M, first = 0;
    bool w = true;
    for (int o = LPR / 2; o >= 1; o >>= 1) {
        if (n > 1) {
            if (lane & o) first += n / 2;
            n /= 2;
        } else if (lane & o) {
            w = false;
        }
    }
    *writer = w;
    return first;
}

template <int M, int LPR>
constexpr int tr_count() { return M / LPR > 1 ? M / LPR : 1; }

// Block-wide max of a non-negative value (all threads return it). `red` holds kWaves floats.
__device__ inline float block_max(float v, float *red)
{
    v = group_max<64>(v);
    const int wave = threadIdx.x / 64;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w]);
    __syncthreads();
    return m;
}

// ------------------------------------------------------------------------------------------
// Per-sequence completion: every work-group of sequence b increments counter[b] once per
// launch, after all its reads of the pointers; the last one to arrive writes the new pointers
// and re-arms the counter. Pointers can therefore be updated in place within the launch that
// reads them, which keeps every call a single launch and safe to replay in a captured graph.
//
// The increment is a relaxed device-scope atomic. Ordering needs no fence: the pointer loads of
// every thread have returned before the work-group barrier below (it waits for all outstanding
// memory operations), so they precede the increment, and the new values are read only by later
// launches, which see them through the kernel-boundary cache maintenance. An acquire/release
// atomic here would add an L2 write-back and invalidate per work-group (MI355X keeps one L2
// per XCD), which costs more than the whole tile stream.
// ------------------------------------------------------------------------------------------
__device__ inline void seq_done(const Layer &Ld, int b, int new_pos, int new_ckpt, int heads_per_group = 1)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned expected = (unsigned)(Ld.H / heads_per_group * Ld.psplit);
        const unsigned prev = __hip_atomic_fetch_add(&Ld.counter[b], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (prev + 1u == expected) {
            Ld.pos[b] = new_pos;
            Ld.ckpt[b] = new_ckpt;
            __hip_atomic_store(&Ld.counter[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__device__ inline void raise_flag(const Layer &Ld, unsigned bits)
{
    if (threadIdx.x == 0) __hip_atomic_fetch_or(Ld.flag, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float fast_exp(float v) { return __expf(v); }

// ------------------------------------------------------------------------------------------
// State arrays and read copies, shared by the Mamba-2 (P rows of N) and Gated DeltaNet (Dv value
// rows of Dk key columns) kernels.
//
// Byte offset of element e of a state array in precision PREC (fp4: two elements per byte; e is
// always a chunk start, hence even).
// ------------------------------------------------------------------------------------------
template <int PREC>
constexpr size_t state_byte_off(size_t e)
{
    return PREC == PREC_F32 ? e * 4 : (PREC == PREC_BF16 || PREC == PREC_F16) ? e * 2 : PREC == PREC_FP8 ? e : e / 2;
}

// Byte offset of 16-byte chunk q (elements [q*VEC, (q+1)*VEC)) of row p of head bh in a state
// array of precision PREC with N columns and P rows per head. The fp32 master and the bf16 copy
// are row-major ([P][N] per head). The fp8 and MXFP4 copies are chunk-column-major per head
// ([N/VEC][P] chunks): one wave instruction over 64 consecutive rows of one chunk column then
// reads 1 KiB contiguously, which is what a one-row-per-lane kernel issues; lane-along-N kernels
// read them in runs of RPI rows (128-256 bytes).
template <int N, int PREC>
__device__ inline size_t state_chunk_off(size_t bh, int p, int q, int P)
{
    using G = Geo<N, PREC>;
    const size_t head = state_byte_off<PREC>(bh * (size_t)P * N);
    if constexpr (PREC == PREC_FP8 || PREC == PREC_FP4) return head + ((size_t)q * P + p) * 16;
    else return head + ((size_t)p * (N / G::VEC) + q) * 16;
}

// A layer's read copy as a write destination: codes, fp8 scales [Bt,H,psplit] (one per block of
// kRows rows), MXFP4 scale bytes [Bt,H,P,N/32], rows per head and row blocks per head.
struct CopyDst {
    void *rcopy;
    float *scale;
    unsigned char *mxscale;
    int P, psplit;
};

// Read-copy writer for fp32 values of one work-group's tile held in 4-value units: unit u of a
// lane holds the four consecutive values n .. n + 3 of tile row r, with (r, n) = at(u). The tile's
// first element is `elem0` of head bh, and it is one block of kRows rows (tiles start at row 0);
// the work-group holds every value of its tile's valid rows (r < nrows) exactly once. For MXFP4
// the eight units of a 32-value block sit, in order of n, in eight consecutive lanes with the
// same u. bf16: each value to nearest even. fp8: the block's scale = amax / 448 over the
// work-group, codes RNE-saturated by gfx950's converter. MXFP4: one E8M0 scale per 32 values.
template <int N, int PREC, int NU, class At>
__device__ inline void write_copy_units(const CopyDst &d, size_t bh, size_t elem0, const f32x4 (&vf)[NU], int nrows,
                                        At at, float *red)
{
    if constexpr (PREC == PREC_BF16) {
        unsigned short *dst = (unsigned short *)d.rcopy + elem0;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int2 rn = at(u);
            if (rn.x < nrows) {
                const f32x4 f = vf[u];
                u32x2 pk;
                pk.x = bf16_rne(f.x) | (bf16_rne(f.y) << 16);
                pk.y = bf16_rne(f.z) | (bf16_rne(f.w) << 16);
                *(u32x2 *)(dst + (size_t)rn.x * N + rn.y) = pk;
            }
        }
    } else if constexpr (PREC == PREC_FP8) {
        float amax = 0.f;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const f32x4 f = vf[u];
            const float m = fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w)));
            if (at(u).x < nrows) amax = fmaxf(amax, m);
        }
        amax = block_max(amax, red);
        const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
        const float inv = 1.0f / scale;
        unsigned char *dst = (unsigned char *)d.rcopy;
        const int row0 = (int)(elem0 / N - bh * (size_t)d.P);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int2 rn = at(u);
            if (rn.x < nrows) {
                const f32x4 f = vf[u];
                // clamp to the largest finite code, then the converter rounds to nearest even
                // (four codes per dword, two per instruction)
                const float a0 = fminf(fmaxf(f.x * inv, -448.0f), 448.0f);
                const float a1 = fminf(fmaxf(f.y * inv, -448.0f), 448.0f);
                const float a2 = fminf(fmaxf(f.z * inv, -448.0f), 448.0f);
                const float a3 = fminf(fmaxf(f.w * inv, -448.0f), 448.0f);
                int q = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
                q = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, q, true);
                *(unsigned *)(dst + state_chunk_off<N, PREC_FP8>(bh, row0 + rn.x, rn.y / 16, d.P) + rn.y % 16) =
                    (unsigned)q;
            }
        }
        if (threadIdx.x == 0) d.scale[bh * d.psplit + row0 / kRows] = scale;
    } else if constexpr (PREC == PREC_FP4) {
        // A 32-value block is 8 consecutive lanes (4 values each): its amax by three lane
        // exchanges, then each lane encodes its 4 values into 2 bytes and the block's first lane
        // writes the scale byte.
        unsigned char *dst = (unsigned char *)d.rcopy;
        unsigned char *sdst = d.mxscale + elem0 / 32;
        const int row0 = (int)(elem0 / N - bh * (size_t)d.P);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int2 rn = at(u);
            const f32x4 f = vf[u];
            float amax = fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w)));
            amax = group_max<8>(amax);
            const unsigned code = mx_code_of(amax);
            if (rn.x < nrows) {
                *(unsigned short *)(dst + state_chunk_off<N, PREC_FP4>(bh, row0 + rn.x, rn.y / 32, d.P) +
                                    (rn.y % 32) / 2) = mx_encode4(f, code);
                if (rn.y % 32 == 0) sdst[((size_t)rn.x * N + rn.y) / 32] = (unsigned char)code;
            }
        }
        (void)red;
    }
}

// The same for f32 geometry (Geo<N, PREC_F32>: unit i of a lane is row i*RPB + wave*RPI +
// lane/LPR, values from n = 4 (lane % LPR)).
template <int N, int PREC>
__device__ inline void write_copy_rows_n(const CopyDst &d, size_t bh, size_t elem0,
                                         const f32x4 (&vf)[Geo<N, PREC_F32>::NL], int nrows, int wave, int lane,
                                         float *red)
{
    using GF = Geo<N, PREC_F32>;
    const int c = lane % GF::LPR;
    auto at = [&](int i) { return int2{i * GF::RPB + wave * GF::RPI + lane / GF::LPR, 4 * c}; };
    write_copy_units<N, PREC, GF::NL>(d, bh, elem0, vf, nrows, at, red);
}

}  // namespace rssm
