/*
 * oracle.c -- float64 CPU oracle for the ReplaySSM Mamba-2 decode step.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the CPU-baseline leg of the
 * benchmark are the only code that loads this library. The GPU library never links it, includes
 * nothing from it and shares no source with it; the two meet only in the tests, which feed both
 * the same seeded fp32 inputs.
 *
 * Sources. The method is described in prose by three web pages; nothing below copies code from
 * anywhere (the pages print none):
 *   [AT Pulse]   "NVIDIA and Princeton's ReplaySSM stores a checkpoint and recent inputs instead of
 *                full SSM state to speed up hybrid-model decoding" (at-pulse.com, story 2558)
 *   [Clarity]    "NVIDIA and Princeton cache SSM inputs in place of state to speed hybrid-model
 *                decoding" (theclarity.today)
 *   [WittyWires] "ReplaySSM cuts memory traffic to speed up hybrid-model decoding"
 *                (wittywires.com forums)
 *
 * The pages print no formulas. What is computed here is the plain Mamba-2 reading of their prose;
 * each reading is stated where it is used:
 *   R1  update, then read: the output of token t already includes token t ([Clarity] "Why it
 *       matters" and claim ledger [6]: a conventional step updates the state, reads the output
 *       from it and stores it).
 *   R2  the flush happens on the step whose append fills the buffer, and that step's output is
 *       read from the folded state ([WittyWires] "What happened": the checkpoint is updated when
 *       the buffer fills; [AT Pulse] "Technical analysis": a flush every L steps).
 *   R3  a record is (x, B, C, dt); replay and flush read x, B and dt of stored records. The pages
 *       call the record "(decay, value, key)": decay <-> dt*A, value <-> x, key <-> B, query <-> C.
 *   R4  dt arrives positive (softplus applied by the caller); A and D are scalars per head;
 *       head h uses group g(h) = h / (H/G).
 *   R5  spec-decode buffer capacity is L; after a commit the layer flushes when more than L - T
 *       records are pending, so T drafts always fit; with T = 1 this is rule R2.
 *   R6  read copy: bf16 by round-to-nearest-even, or OCP fp8 E4M3FN with one fp32 scale per
 *       (sequence, head, block of 64 consecutive rows p -- rows 64i .. 64i + 63, the whole head
 *       when P <= 64) = amax/448 of the block (1 when amax is 0), values multiplied by 1/scale in
 *       fp32, clamped to +-448 and rounded to nearest even, or OCP MXFP4 (reading R7). It is
 *       written from the master when a state is loaded and at every flush, never otherwise.
 *   R7  MXFP4 read copy (the pages' 4-bit state reads are NVFP4, which has no gfx950 form; MXFP4
 *       is the OCP microscaling format gfx950 converts natively): per state row, blocks of 32
 *       consecutive n share one E8M0 scale; elements are FP4 E2M1. Scale and rounding follow the
 *       OCP "Microscaling Formats (MX)" specification v1.0: shared exponent = floor(log2(block
 *       amax)) - 2 (2 = the exponent of E2M1's largest value, 6 = 1.5 * 2^2), elements = the value
 *       divided by the scale, rounded to nearest with ties to even, clamped to +-6. The spec
 *       leaves the scale of an all-zero block open: it takes the smallest code. Two elements per
 *       byte, element 2i in the low nibble.
 *   R8  low-precision master recurrence (the pages' FP16-with-stochastic-rounding recurrence,
 *       [AT Pulse] "Capabilities and access" and "Claims and evidence"): the checkpoint itself is
 *       kept in IEEE fp16. At load the fp32 state is rounded to nearest even; at every flush the
 *       fold is computed at full precision from the fp16 checkpoint and the records, rounded to
 *       fp32, clamped to +-65504 and rounded to fp16 either to nearest even or stochastically:
 *       with q the fp16 value toward zero and ulp the fp16 spacing above it, the magnitude rounds
 *       up iff r < (|v| - |q|) / ulp * 2^16, r a 16-bit random integer: Philox4x32-10 (Salmon et
 *       al., SC'11) with counter (element / 8, sequence, new ckpt_pos, 0) and key (seed, 0) gives
 *       eight 16-bit fields, element e taking bits 16*(e % 2) .. +15 of word (e % 8) / 2 (elements
 *       numbered h*P*N + p*N + n within the sequence). The threshold is exact in fp32. In fp16's
 *       normal range an fp32 magnitude has 13 bits below the fp16 spacing, so the threshold is a
 *       multiple of 8 and the rounding is exactly unbiased over r -- the same distribution as any
 *       wider random integer gives; below 2^-17 (deep in fp16's subnormal range) fp32 keeps finer
 *       bits and the bias is below 2^-16 of a spacing. Reads and the read copy then come from the
 *       fp16 checkpoint; a flush step's output is read from the rounded checkpoint.
 *   R9  FP8 master recurrence (the pages' FP8 alternative to the FP16 recurrence, [AT Pulse]
 *       "Claims and evidence"): the checkpoint itself is kept as OCP E4M3FN codes with one fp32
 *       scale per (sequence, head, 64-row block), in the format of the fp8 read copy (R6): scale
 *       = amax / 448 of the block's fold rounded to fp32 (1 if amax is 0), a = v * (1 / scale) in fp32, clamped to
 *       +-448. A load rounds a to nearest even; a flush to nearest even (FP8) or stochastically
 *       (FP8_SR): with q the E4M3 magnitude toward zero and ulp the code spacing above it, the
 *       magnitude rounds up iff r16 < (|a| - q) / ulp * 2^16, with the 16-bit fields of R8's
 *       Philox stream. The checkpoint's value is code * scale; reads come from it directly.
 *
 * Layouts (row-major, last index fastest): x [Bt,H,P]; B, C [Bt,G,N]; dt [Bt,H]; A, D [H];
 * state [Bt,H,P,N]; y [Bt,H,P]. Spec-decode inputs carry the draft index after the batch index:
 * x [Bt,T,H,P]; B, C [Bt,T,G,N]; dt [Bt,T,H]; y [Bt,T,H,P].
 *
 * All arithmetic is float64 on the exact fp32 input values, with libm exp.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------------- */
/* O1: the stepwise Mamba-2 recurrence (the truth).                                             */
/* For one token and every (b, h, p, n), with a = exp(dt*A_h):                                 */
/*     S[p,n] <- a*S[p,n] + dt * x[p] * B[n]       (state update)                              */
/*     y[p]    = sum_n S[p,n]*C[n] + D_h*x[p]      (read from the updated state, reading R1)   */
/* [Clarity] claim ledger [6] and "Why it matters": the conventional step updates, reads and   */
/* stores the state in one pass.                                                               */
/* ------------------------------------------------------------------------------------------- */
void oracle_step(int Bt, int H, int P, int N, int G, double *S, const float *x, const float *B,
                 const float *C, const float *dt, const float *A, const float *D, double *y)
{
    const int hpg = H / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < Bt; ++b) {
        for (int h = 0; h < H; ++h) {
            const int g = h / hpg;
            const double dtv = (double)dt[(size_t)b * H + h];
            const double a = exp(dtv * (double)A[h]);
            const float *xb = x + ((size_t)b * H + h) * P;
            const float *Bb = B + ((size_t)b * G + g) * N;
            const float *Cb = C + ((size_t)b * G + g) * N;
            double *Sb = S + ((size_t)b * H + h) * (size_t)P * N;
            double *yb = y + ((size_t)b * H + h) * P;
            for (int p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    double s = a * Sb[(size_t)p * N + n] + dtv * (double)xb[p] * (double)Bb[n];
                    Sb[(size_t)p * N + n] = s;
                    acc += s * (double)Cb[n];
                }
                yb[p] = acc + (double)D[h] * (double)xb[p];
            }
        }
    }
}

/* O5: speculative decoding by the plain definition. From the committed state, the T drafts are */
/* run one by one with O1; all T outputs are produced (rejected drafts included), and the       */
/* committed state becomes the state after the first accepted[b] drafts. This is the per-draft  */
/* snapshot method of [Clarity] claim ledger [13], carried out in float64.                      */
/* Returns 0, or -1 when an accepted count lies outside [0, T].                                 */
int oracle_spec_stepwise(int Bt, int H, int P, int N, int G, int T, double *S, const float *x,
                         const float *B, const float *C, const float *dt, const float *A,
                         const float *D, const int *accepted, double *y)
{
    for (int b = 0; b < Bt; ++b)
        if (accepted[b] < 0 || accepted[b] > T) return -1;
    const size_t tile = (size_t)P * N;
    const size_t seq_state = (size_t)H * tile;
    double *work = (double *)malloc(seq_state * sizeof(double));
    float *xs = (float *)malloc((size_t)H * P * sizeof(float));
    float *Bs = (float *)malloc((size_t)G * N * sizeof(float));
    float *Cs = (float *)malloc((size_t)G * N * sizeof(float));
    float *ds = (float *)malloc((size_t)H * sizeof(float));
    double *ys = (double *)malloc((size_t)H * P * sizeof(double));
    for (int b = 0; b < Bt; ++b) {
        memcpy(work, S + b * seq_state, seq_state * sizeof(double));
        for (int i = 0; i < T; ++i) {
            memcpy(xs, x + ((size_t)b * T + i) * H * P, (size_t)H * P * sizeof(float));
            memcpy(Bs, B + ((size_t)b * T + i) * G * N, (size_t)G * N * sizeof(float));
            memcpy(Cs, C + ((size_t)b * T + i) * G * N, (size_t)G * N * sizeof(float));
            memcpy(ds, dt + ((size_t)b * T + i) * H, (size_t)H * sizeof(float));
            oracle_step(1, H, P, N, G, work, xs, Bs, Cs, ds, A, D, ys);
            memcpy(y + ((size_t)b * T + i) * H * P, ys, (size_t)H * P * sizeof(double));
            if (i + 1 == accepted[b]) memcpy(S + b * seq_state, work, seq_state * sizeof(double));
        }
    }
    free(work); free(xs); free(Bs); free(Cs); free(ds); free(ys);
    return 0;
}

/* ------------------------------------------------------------------------------------------- */
/* O7: read-copy quantizers, written from the format definitions.                               */
/* ------------------------------------------------------------------------------------------- */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 keeps the top 16 bits of an fp32 value. Round to nearest, ties to the even 16-bit code:  */
/* the dropped low half is compared with one half of the kept unit. NaN is out of contract.     */
uint16_t oracle_bf16_encode(float f)
{
    uint32_t u = f32_bits(f);
    uint32_t kept = u >> 16, dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u; /* may carry into */
    return (uint16_t)kept;                                             /* the exponent: correct */
}

float oracle_bf16_decode(uint16_t v) { return bits_f32((uint32_t)v << 16); }

/* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is   */
/* subnormal (value m * 2^-9); no infinities; S.1111.111 is NaN, so the largest finite value is */
/* 1.75 * 2^8 = 448.                                                                             */
float oracle_e4m3_decode(uint8_t code)
{
    int sign = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (float)(sign ? -mag : mag);
}

/* Encode an fp32 value already divided by the scale: clamp to +-448, then round to the nearest  */
/* representable magnitude with ties to the even code. Within one binade [2^e, 2^(e+1)) the      */
/* codes are spaced 2^(e-3) apart; below 2^-6 the spacing is the subnormal step 2^-9. The        */
/* quotient |v| / spacing is exact in float64, and rint() rounds it to nearest even.             */
uint8_t oracle_e4m3_encode_scaled(float v)
{
    double t = (double)v;
    int sign = t < 0.0 || (t == 0.0 && signbit(t));
    double mag = fabs(t);
    if (mag > 448.0) mag = 448.0;
    int e;
    if (mag < ldexp(1.0, -6)) {
        e = -6; /* subnormal range shares the spacing of the lowest binade */
    } else {
        e = (int)floor(log2(mag));
        if (ldexp(1.0, e) > mag) e -= 1;      /* guard log2 rounding at binade edges */
        if (ldexp(1.0, e + 1) <= mag) e += 1;
    }
    double spacing = ldexp(1.0, e - 3);
    double k = rint(mag / spacing);           /* round half to even on the multiple */
    double q = k * spacing;                   /* may reach 2^(e+1): the next binade's first code */
    /* convert the quantized magnitude to a code */
    uint8_t code;
    if (q < ldexp(1.0, -6)) {
        code = (uint8_t)(int)(q / ldexp(1.0, -9));               /* subnormal: m = q / 2^-9 */
    } else {
        int qe = (int)floor(log2(q));
        if (ldexp(1.0, qe) > q) qe -= 1;
        if (ldexp(1.0, qe + 1) <= q) qe += 1;
        int m = (int)(q / ldexp(1.0, qe - 3)) - 8;
        code = (uint8_t)(((qe + 7) << 3) | m);
    }
    return (uint8_t)(code | (sign ? 0x80 : 0));
}

/* Stochastic rounding to E4M3FN of an fp32 value already divided by the scale (reading R9):   */
/* clamp to +-448; with q the code magnitude toward zero and ulp the spacing of its binade (the   */
/* subnormal step 2^-9 below 2^-6), round up iff r16 < (|v| - q) / ulp * 2^16 (exact in float64). */
/* q + ulp may be the next binade's first code; the sign is kept (a negative that stays at zero  */
/* is -0).                                                                                        */
uint8_t oracle_e4m3_encode_sr(float v, uint32_t r16)
{
    double t = (double)v;
    int neg = t < 0.0 || (t == 0.0 && signbit(t));
    double mag = fabs(t);
    if (mag > 448.0) mag = 448.0;
    int e;
    if (mag < ldexp(1.0, -6)) {
        e = -6;
    } else {
        e = (int)floor(log2(mag));
        if (ldexp(1.0, e) > mag) e -= 1;
        if (ldexp(1.0, e + 1) <= mag) e += 1;
    }
    double spacing = ldexp(1.0, e - 3);
    double q = floor(mag / spacing) * spacing;
    double out = q;
    if (mag > q && (double)r16 < (mag - q) / spacing * 65536.0) out = q + spacing;
    /* out is an E4M3 magnitude: its nearest-even encoding is its own code */
    return oracle_e4m3_encode_scaled((float)(neg ? -out : out));
}

/* Per-(sequence, head) scale for the fp8 read copy (reading R6): scale = amax / 448 in fp32,    */
/* or 1 when amax is 0; codes are RNE(clamp(S * (1/scale))) with the product taken in fp32.    */
float oracle_e4m3_scale(const float *tile, size_t n)
{
    float amax = 0.0f;
    for (size_t i = 0; i < n; ++i) {
        float a = fabsf(tile[i]);
        if (a > amax) amax = a;
    }
    return amax == 0.0f ? 1.0f : amax / 448.0f;
}

void oracle_encode_bf16(const float *in, uint16_t *out, size_t n)
{
#pragma omp parallel for schedule(static)
    for (size_t i = 0; i < n; ++i) out[i] = oracle_bf16_encode(in[i]);
}

/* Encode ntiles tiles of tile_elems values each with the per-tile scale. */
void oracle_encode_e4m3_tiles(const float *in, uint8_t *out, float *scale, size_t ntiles,
                              size_t tile_elems)
{
#pragma omp parallel for schedule(static)
    for (size_t t = 0; t < ntiles; ++t) {
        const float *tl = in + t * tile_elems;
        float s = oracle_e4m3_scale(tl, tile_elems);
        float inv = 1.0f / s;
        scale[t] = s;
        for (size_t i = 0; i < tile_elems; ++i)
            out[t * tile_elems + i] = oracle_e4m3_encode_scaled(tl[i] * inv);
    }
}

/* Element-wise e4m3 encode at a given inverse scale (used by the quantizer pins). */
void oracle_encode_e4m3_at(const float *in, uint8_t *out, size_t n, float inv)
{
#pragma omp parallel for schedule(static)
    for (size_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode_scaled(in[i] * inv);
}

/* OCP FP4 E2M1 (MX specification v1.0, element data types): 1 sign bit, 2 exponent bits with */
/* bias 1, 1 mantissa bit; exponent field 0 is subnormal (value m * 0.5); no infinities or NaN. */
float oracle_e2m1_decode(uint8_t code)
{
    int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (float)(sign ? -mag : mag);
}

/* Code of a value already divided by its block scale (reading R7): the nearest of the eight    */
/* magnitudes, on a tie the one with an even code (mantissa bit 0); beyond 6 the nearest is 6,  */
/* which is the clamp. The sign bit follows the value's sign, so a negative that rounds to zero */
/* is -0.                                                                                        */
uint8_t oracle_e2m1_encode_scaled(double v)
{
    double mag = fabs(v), best_d = INFINITY;
    int best = 0;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(mag - (double)oracle_e2m1_decode((uint8_t)c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 8 : 0));
}

void oracle_encode_e2m1_scaled(const double *in, uint8_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i) out[i] = oracle_e2m1_encode_scaled(in[i]);
}

/* E8M0 scale code of one block of 32 (reading R7): X = 2^(floor(log2 amax) - 2), code = the    */
/* exponent + 127, limited to the finite codes 0..254; 0 for an all-zero block.                 */
uint8_t oracle_mx_scale_code(const float *blk, size_t n)
{
    double amax = 0.0;
    for (size_t i = 0; i < n; ++i) amax = fmax(amax, fabs((double)blk[i]));
    if (amax == 0.0) return 0;
    int e;
    frexp(amax, &e); /* amax = f * 2^e with 0.5 <= f < 1, so floor(log2 amax) = e - 1 */
    int code = (e - 1) - 2 + 127;
    if (code < 0) code = 0;
    if (code > 254) code = 254;
    return (uint8_t)code;
}

/* Encode nblocks blocks of 32 values: codes (16 bytes per block, element 2i in the low nibble  */
/* of byte i) and one scale code per block. The division by the scale is exact in float64.      */
void oracle_encode_mxfp4(const float *in, uint8_t *codes, uint8_t *scales, size_t nblocks)
{
#pragma omp parallel for schedule(static)
    for (size_t b = 0; b < nblocks; ++b) {
        const float *blk = in + b * 32;
        uint8_t sc = oracle_mx_scale_code(blk, 32);
        scales[b] = sc;
        double inv = ldexp(1.0, 127 - (int)sc);
        for (int i = 0; i < 32; i += 2) {
            uint8_t lo = oracle_e2m1_encode_scaled((double)blk[i] * inv);
            uint8_t hi = oracle_e2m1_encode_scaled((double)blk[i + 1] * inv);
            codes[b * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

/* Decoded values of nblocks encoded blocks, in float64: E2M1 value times 2^(scale code - 127). */
void oracle_decode_mxfp4(const uint8_t *codes, const uint8_t *scales, double *out, size_t nblocks)
{
    for (size_t b = 0; b < nblocks; ++b) {
        for (int i = 0; i < 32; ++i) {
            uint8_t byte = codes[b * 16 + i / 2];
            uint8_t c = (i & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
            out[b * 32 + i] = ldexp((double)oracle_e2m1_decode(c), (int)scales[b] - 127);
        }
    }
}

/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",  */
/* SC'11): ten rounds of two 32x32->64 multiplications; the key is bumped by the Weyl constants */
/* between rounds.                                                                               */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits; exponent field 0 is  */
/* subnormal (m * 2^-24); the largest finite value is 65504.                                    */
float oracle_f16_decode(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double mag = e == 31 ? (m ? NAN : INFINITY) : e == 0 ? ldexp((double)m, -24) : ldexp(1.0 + m / 1024.0, e - 15);
    return (float)(sign ? -mag : mag);
}

/* fp16 spacing at magnitude q (an fp16 value): 2^(e - 10) in the binade [2^e, 2^(e+1)), 2^-24  */
/* below 2^-14.                                                                                  */
static double f16_spacing(double q)
{
    if (q < ldexp(1.0, -14)) return ldexp(1.0, -24);
    int e;
    frexp(q, &e); /* q = f * 2^e, 0.5 <= f < 1 */
    return ldexp(1.0, e - 1 - 10);
}

static uint16_t f16_code_of(double mag) /* an exactly representable magnitude <= 65504 */
{
    if (mag < ldexp(1.0, -14)) return (uint16_t)(int)(mag / ldexp(1.0, -24));
    int e;
    frexp(mag, &e);
    e -= 1; /* mag in [2^e, 2^(e+1)) */
    int m = (int)(mag / ldexp(1.0, e - 10)) - 1024;
    return (uint16_t)(((e + 15) << 10) | m);
}

/* Largest fp16 magnitude <= mag (mag <= 65504). */
static double f16_toward_zero(double mag)
{
    double sp = f16_spacing(mag);
    double q = floor(mag / sp) * sp;
    if (f16_spacing(q) != sp) q = floor(mag / f16_spacing(q)) * f16_spacing(q); /* binade edge */
    return q;
}

/* Round an fp32 value to fp16, to nearest even (reading R8; clamped to +-65504 first). */
uint16_t oracle_f16_encode_rne(float v)
{
    double t = (double)v, mag = fabs(t);
    int sign = signbit(t) ? 1 : 0;
    if (mag > 65504.0) mag = 65504.0;
    double q = f16_toward_zero(mag), sp = f16_spacing(q), up = q + sp;
    double r = mag - q;
    double out = q;
    if (r > sp / 2 || (r == sp / 2 && (f16_code_of(q) & 1))) out = up;
    if (out > 65504.0) out = 65504.0;
    return (uint16_t)(f16_code_of(out) | (sign << 15));
}

/* Round an fp32 value to fp16 stochastically with the 16-bit random integer r16 (reading R8). */
uint16_t oracle_f16_encode_sr(float v, uint32_t r16)
{
    double t = (double)v, mag = fabs(t);
    int sign = signbit(t) ? 1 : 0;
    if (mag > 65504.0) mag = 65504.0;
    double q = f16_toward_zero(mag);
    double out = q;
    if (mag > q) {
        double threshold = (mag - q) / f16_spacing(q) * 65536.0; /* exact */
        if ((double)r16 < threshold) out = q + f16_spacing(q);
    }
    return (uint16_t)(f16_code_of(out) | (sign << 15));
}

void oracle_encode_f16(const float *in, uint16_t *out, size_t n, int stochastic, const uint32_t *r16)
{
    for (size_t i = 0; i < n; ++i) out[i] = stochastic ? oracle_f16_encode_sr(in[i], r16[i]) : oracle_f16_encode_rne(in[i]);
}

/* ------------------------------------------------------------------------------------------- */
/* O3 + O4: the replay form with its pointer and flush state machine.                           */
/*                                                                                             */
/* [AT Pulse] "Technical analysis" and [Clarity] claim ledger [17], [18]: the state of a       */
/* sequence is kept as a checkpoint together with the input records of the tokens since it;    */
/* an ordinary step derives its output from both by expanding the recurrence across those      */
/* records and writes nothing but its own record; once L records have gathered they are        */
/* merged into the checkpoint; discarding rejected drafts only moves the buffer pointer.       */
/*                                                                                             */
/* Unrolling O1 from the checkpoint S_c (all tokens before c folded) over records c..t gives,   */
/* per (b, h), with g = g(h):                                                                   */
/*     decay_t = exp(A_h * sum_{i=c..t} dt_i)                                                   */
/*     w_j     = dt_j * exp(A_h * sum_{i=j+1..t} dt_i)              (so w_t = dt_t)            */
/*     y_t[p]  = decay_t * (S_c[p,:] . C_t) + sum_{j=c..t} w_j * (B_j . C_t) * x_j[p]            */
/*               + D_h * x_t[p]                                                                 */
/*     fold:     S_c <- decay_t * S_c + sum_{j=c..t} w_j * x_j (outer) B_j ;  c <- t + 1        */
/*                                                                                             */
/* Pointers per sequence: pos = tokens committed, ckpt_pos = tokens folded into S_c;           */
/* count = pos - ckpt_pos, always in [0, L - Tmax] between calls (readings R2, R5).            */
/* Records are kept by their offset from ckpt_pos (not as a ring): the record of absolute      */
/* position q sits at index q - ckpt_pos. Unused entries hold NaN so a stray read shows up.    */
/* ------------------------------------------------------------------------------------------- */

typedef struct oracle_replay {
    int Bt, H, P, N, G, L, Tmax, read_prec; /* 0 fp32 master, 1 bf16, 2 fp8 e4m3, 3 mxfp4 */
    float *mscale;                          /* fp8 master: scale per (sequence, head, 64-row block)
                                               [Bt,H,ceil(P/64)] */
    int master_prec;                        /* 0 fp32, 1 fp16 nearest even, 2 fp16 stochastic (R8),
                                               3 fp8 nearest even, 4 fp8 stochastic (R9) */
    uint32_t seed;
    int *seq_id;                            /* [Bt] sequence index in the Philox counter */
    double *A, *D;                          /* [H] */
    double *ckpt;                           /* [Bt,H,P,N] master */
    double *rcopy;                          /* [Bt,H,P,N] decoded read copy (read_prec != 0) */
    float *rx, *rB, *rC, *rdt;              /* records: [Bt,L,H,P], [Bt,L,G,N] x2, [Bt,L,H] */
    int *pos, *ckpt_pos;                    /* [Bt] */
    int pending_T;                          /* drafts of an unresolved verify, else 0 */
} oracle_replay;

static size_t rx_at(const oracle_replay *r, int b, int idx, int h)
{ return (((size_t)b * r->L + idx) * r->H + h) * r->P; }
static size_t rg_at(const oracle_replay *r, int b, int idx, int g)
{ return (((size_t)b * r->L + idx) * r->G + g) * r->N; }
static size_t rdt_at(const oracle_replay *r, int b, int idx, int h)
{ return ((size_t)b * r->L + idx) * r->H + h; }

static void poison_records(oracle_replay *r, int b, int from_idx)
{
    for (int idx = from_idx; idx < r->L; ++idx) {
        for (int h = 0; h < r->H; ++h) {
            for (int p = 0; p < r->P; ++p) r->rx[rx_at(r, b, idx, h) + p] = NAN;
            r->rdt[rdt_at(r, b, idx, h)] = NAN;
        }
        for (int g = 0; g < r->G; ++g)
            for (int n = 0; n < r->N; ++n) {
                r->rB[rg_at(r, b, idx, g) + n] = NAN;
                r->rC[rg_at(r, b, idx, g) + n] = NAN;
            }
    }
}

/* Keep sequence b's checkpoint in the master precision (reading R8): fp32 (rounded from the     */
/* float64 fold), or fp16 to nearest even / stochastically with the Philox stream of flush      */
/* position `ck` (stochastic rounding only after a flush; a load rounds to nearest even).       */
static void round_master(oracle_replay *r, int b, int ck, int stochastic)
{
    const size_t n = (size_t)r->H * r->P * r->N;
    double *m = r->ckpt + (size_t)b * n;
    if (r->master_prec >= 3) { /* fp8 (R9): per-block scale of the fold rounded to fp32 */
        const size_t tile = (size_t)r->P * r->N;
        const int nblk = (r->P + 63) / 64;
        float *v = (float *)malloc(tile * sizeof(float));
        for (int h = 0; h < r->H; ++h) {
            double *mh = m + (size_t)h * tile;
            for (size_t i = 0; i < tile; ++i) v[i] = (float)mh[i];
            for (int kb = 0; kb < nblk; ++kb) {
                const size_t i0 = (size_t)kb * 64 * r->N;
                const size_t i1 = (size_t)(kb * 64 + 64 < r->P ? kb * 64 + 64 : r->P) * r->N;
                const float scale = oracle_e4m3_scale(v + i0, i1 - i0);
                const float inv = 1.0f / scale;
                r->mscale[((size_t)b * r->H + h) * nblk + kb] = scale;
                for (size_t i = i0; i < i1; i += 8) {
                    const size_t e = (size_t)h * tile + i; /* element within the sequence */
                    uint32_t words[4] = {0, 0, 0, 0};
                    if (r->master_prec == 4 && stochastic) {
                        const uint32_t ctr[4] = {(uint32_t)(e / 8), (uint32_t)r->seq_id[b], (uint32_t)ck, 0u};
                        const uint32_t key[2] = {r->seed, 0u};
                        oracle_philox4x32_10(ctr, key, words);
                    }
                    for (int w = 0; w < 8 && i + w < i1; ++w) {
                        const float a = v[i + w] * inv;
                        const uint32_t r16 = (words[w / 2] >> (16 * (w % 2))) & 0xFFFFu;
                        const uint8_t code = (r->master_prec == 4 && stochastic) ? oracle_e4m3_encode_sr(a, r16)
                                                                               : oracle_e4m3_encode_scaled(a);
                        mh[i + w] = (double)oracle_e4m3_decode(code) * (double)scale;
                    }
                }
            }
        }
        free(v);
        return;
    }
    for (size_t e = 0; e < n; e += 8) {
        uint32_t words[4] = {0, 0, 0, 0};
        if (r->master_prec == 2 && stochastic) {
            const uint32_t ctr[4] = {(uint32_t)(e / 8), (uint32_t)r->seq_id[b], (uint32_t)ck, 0u};
            const uint32_t key[2] = {r->seed, 0u};
            oracle_philox4x32_10(ctr, key, words);
        }
        for (int w = 0; w < 8 && e + w < n; ++w) {
            const float v = (float)m[e + w];
            const uint32_t r16 = (words[w / 2] >> (16 * (w % 2))) & 0xFFFFu;
            if (r->master_prec == 0) m[e + w] = (double)v;
            else if (r->master_prec == 2 && stochastic) m[e + w] = (double)oracle_f16_decode(oracle_f16_encode_sr(v, r16));
            else m[e + w] = (double)oracle_f16_decode(oracle_f16_encode_rne(v));
        }
    }
}

/* Refresh sequence b's read copy from its master (reading R6): the master value is rounded to */
/* fp32 (the precision the layer keeps it in), encoded, and decoded back to float64.           */
static void refresh_copy(oracle_replay *r, int b)
{
    if (r->read_prec == 0) return;
    const size_t tile = (size_t)r->P * r->N;
    float *f = (float *)malloc(tile * sizeof(float));
    for (int h = 0; h < r->H; ++h) {
        const double *m = r->ckpt + ((size_t)b * r->H + h) * tile;
        double *c = r->rcopy + ((size_t)b * r->H + h) * tile;
        for (size_t i = 0; i < tile; ++i) f[i] = (float)m[i];
        if (r->read_prec == 1) {
            for (size_t i = 0; i < tile; ++i)
                c[i] = (double)oracle_bf16_decode(oracle_bf16_encode(f[i]));
        } else if (r->read_prec == 3) {
            /* blocks of 32 along n never cross a row, since N is a multiple of 32 */
            const size_t nb = tile / 32;
            uint8_t *codes = (uint8_t *)malloc(nb * 16), *sc = (uint8_t *)malloc(nb);
            oracle_encode_mxfp4(f, codes, sc, nb);
            oracle_decode_mxfp4(codes, sc, c, nb);
            free(codes);
            free(sc);
        } else {
            for (int p0 = 0; p0 < r->P; p0 += 64) { /* one scale per block of 64 rows */
                const size_t i0 = (size_t)p0 * r->N, i1 = (size_t)(p0 + 64 < r->P ? p0 + 64 : r->P) * r->N;
                const float s = oracle_e4m3_scale(f + i0, i1 - i0);
                const float inv = 1.0f / s;
                for (size_t i = i0; i < i1; ++i)
                    c[i] = (double)oracle_e4m3_decode(oracle_e4m3_encode_scaled(f[i] * inv)) * (double)s;
            }
        }
    }
    free(f);
}

oracle_replay *oracle_replay_create(int Bt, int H, int P, int N, int G, int L, int Tmax,
                                    int read_prec, const float *S0, const float *A, const float *D,
                                    int master_prec, uint32_t seed)
{
    if (Bt < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G || L <= 0 || L > 64 ||
        Tmax <= 0 || Tmax > L || read_prec < 0 || read_prec > 3 || (read_prec == 3 && N % 32) ||
        master_prec < 0 || master_prec > 4 || (master_prec != 0 && N % 4) || (master_prec >= 3 && N % 8) ||
        (master_prec >= 3 && read_prec != 0))
        return NULL;
    oracle_replay *r = (oracle_replay *)calloc(1, sizeof(oracle_replay));
    r->Bt = Bt; r->H = H; r->P = P; r->N = N; r->G = G; r->L = L; r->Tmax = Tmax;
    r->read_prec = read_prec;
    r->master_prec = master_prec;
    r->seed = seed;
    const size_t st = (size_t)Bt * H * P * N;
    r->A = (double *)malloc(H * sizeof(double));
    r->D = (double *)malloc(H * sizeof(double));
    for (int h = 0; h < H; ++h) { r->A[h] = A[h]; r->D[h] = D[h]; }
    r->ckpt = (double *)malloc((st ? st : 1) * sizeof(double));
    r->mscale = (float *)calloc((size_t)Bt * H * ((P + 63) / 64) + 1, sizeof(float));
    for (size_t i = 0; i < st; ++i) r->ckpt[i] = (double)S0[i];
    r->rcopy = read_prec ? (double *)malloc((st ? st : 1) * sizeof(double)) : NULL;
    r->rx = (float *)malloc(((size_t)Bt * L * H * P + 1) * sizeof(float));
    r->rB = (float *)malloc(((size_t)Bt * L * G * N + 1) * sizeof(float));
    r->rC = (float *)malloc(((size_t)Bt * L * G * N + 1) * sizeof(float));
    r->rdt = (float *)malloc(((size_t)Bt * L * H + 1) * sizeof(float));
    r->pos = (int *)calloc(Bt + 1, sizeof(int));
    r->ckpt_pos = (int *)calloc(Bt + 1, sizeof(int));
    r->seq_id = (int *)calloc(Bt + 1, sizeof(int));
    for (int b = 0; b < Bt; ++b) r->seq_id[b] = b;
    for (int b = 0; b < Bt; ++b) { round_master(r, b, 0, 0); poison_records(r, b, 0); refresh_copy(r, b); }
    return r;
}

/* Stand the oracle's rows for sequences ids[0..Bt) of a larger batch: only the stochastic   */
/* rounding stream depends on a sequence's index, so a sample of a batch is modelled exactly. */
void oracle_replay_set_seq_ids(oracle_replay *r, const int *ids)
{
    for (int b = 0; b < r->Bt; ++b) r->seq_id[b] = ids[b];
}

void oracle_replay_destroy(oracle_replay *r)
{
    if (!r) return;
    free(r->seq_id);
    free(r->mscale);
    free(r->A); free(r->D); free(r->ckpt); free(r->rcopy);
    free(r->rx); free(r->rB); free(r->rC); free(r->rdt); free(r->pos); free(r->ckpt_pos);
    free(r);
}

static void store_record(oracle_replay *r, int b, int idx, const float *x_bh /*[H,P]*/,
                         const float *B_bg /*[G,N]*/, const float *C_bg, const float *dt_bh /*[H]*/)
{
    memcpy(r->rx + rx_at(r, b, idx, 0), x_bh, (size_t)r->H * r->P * sizeof(float));
    memcpy(r->rB + rg_at(r, b, idx, 0), B_bg, (size_t)r->G * r->N * sizeof(float));
    memcpy(r->rC + rg_at(r, b, idx, 0), C_bg, (size_t)r->G * r->N * sizeof(float));
    memcpy(r->rdt + rdt_at(r, b, idx, 0), dt_bh, (size_t)r->H * sizeof(float));
}

/* Unrolled-window weights for records idx 0..last (relative to ckpt_pos) of (b, h):          */
/* w[j] = dt_j * exp(A * sum_{i=j+1..last} dt_i) and the window decay exp(A * sum_{0..last}). */
static double window_weights(const oracle_replay *r, int b, int h, int last, double *w)
{
    double tail = 0.0; /* sum of dt strictly after record j */
    for (int j = last; j >= 0; --j) {
        double dtj = (double)r->rdt[rdt_at(r, b, j, h)];
        w[j] = dtj * exp(r->A[h] * tail);
        tail += dtj;
    }
    return exp(r->A[h] * tail);
}

/* Output of the query token at record index `last` (its record is stored): reads the           */
/* checkpoint through `S` (the master or the decoded read copy), and the records 0..last.      */
static void replay_output(const oracle_replay *r, const double *S, int b, int last,
                          const float *Cq_bg /*[G,N]: the query token's C*/, double *y_bh /*[H,P]*/)
{
    const int hpg = r->H / r->G;
    double w[64 + 8];
    for (int h = 0; h < r->H; ++h) {
        const int g = h / hpg;
        const double *Sc = S + ((size_t)b * r->H + h) * (size_t)r->P * r->N;
        const float *Cq = Cq_bg + (size_t)g * r->N;
        double decay = window_weights(r, b, h, last, w);
        double score[64 + 8]; /* (B_j . C_t) */
        for (int j = 0; j <= last; ++j) {
            const float *Bj = r->rB + rg_at(r, b, j, g);
            double s = 0.0;
            for (int n = 0; n < r->N; ++n) s += (double)Bj[n] * (double)Cq[n];
            score[j] = s;
        }
        for (int p = 0; p < r->P; ++p) {
            double u = 0.0;
            for (int n = 0; n < r->N; ++n) u += Sc[(size_t)p * r->N + n] * (double)Cq[n];
            double acc = decay * u;
            for (int j = 0; j <= last; ++j)
                acc += w[j] * score[j] * (double)r->rx[rx_at(r, b, j, h) + p];
            const double x_last = (double)r->rx[rx_at(r, b, last, h) + p];
            y_bh[(size_t)h * r->P + p] = acc + r->D[h] * x_last;
        }
    }
}

/* Fold records 0..count-1 of sequence b into `dst` (the master when committing). */
static void fold_into(const oracle_replay *r, int b, int count, double *dst)
{
    if (count <= 0) return;
    const int hpg = r->H / r->G;
    double w[64 + 8];
    for (int h = 0; h < r->H; ++h) {
        const int g = h / hpg;
        double *S = dst + ((size_t)b * r->H + h) * (size_t)r->P * r->N;
        double decay = window_weights(r, b, h, count - 1, w);
        for (int p = 0; p < r->P; ++p)
            for (int n = 0; n < r->N; ++n) {
                double s = decay * S[(size_t)p * r->N + n];
                for (int j = 0; j < count; ++j)
                    s += w[j] * (double)r->rx[rx_at(r, b, j, h) + p] *
                         (double)r->rB[rg_at(r, b, j, g) + n];
                S[(size_t)p * r->N + n] = s;
            }
    }
}

/* Commit a flush of sequence b: fold its pos - ckpt_pos records, advance ckpt_pos to pos,     */
/* forget the records and refresh the read copy.                                               */
static void flush_seq(oracle_replay *r, int b)
{
    int count = r->pos[b] - r->ckpt_pos[b];
    if (count <= 0) return;
    fold_into(r, b, count, r->ckpt);
    r->ckpt_pos[b] = r->pos[b];
    if (r->master_prec) round_master(r, b, r->ckpt_pos[b], 1);
    poison_records(r, b, 0);
    refresh_copy(r, b);
}

/* Standard decode step for all sequences: append the token's record, pos += 1; if more than   */
/* L - Tmax records are now pending, flush and read the output from the folded master (R2,    */
/* R5); else form the output by replay through the read copy. Returns 0, or -1 when a verify  */
/* is pending or a sequence's pointers break the invariant.                                    */
int oracle_replay_step(oracle_replay *r, const float *x, const float *B, const float *C,
                       const float *dt, double *y)
{
    if (r->pending_T) return -1;
    for (int b = 0; b < r->Bt; ++b) {
        int count = r->pos[b] - r->ckpt_pos[b];
        if (count < 0 || count > r->L - r->Tmax) return -1;
    }
    const int H = r->H, P = r->P, N = r->N, G = r->G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < r->Bt; ++b) {
        int idx = r->pos[b] - r->ckpt_pos[b];
        store_record(r, b, idx, x + (size_t)b * H * P, B + (size_t)b * G * N,
                     C + (size_t)b * G * N, dt + (size_t)b * H);
        r->pos[b] += 1;
        double *yb = y + (size_t)b * H * P;
        if (r->pos[b] - r->ckpt_pos[b] > r->L - r->Tmax) {
            flush_seq(r, b);
            /* y_t = S_new . C_t + D x_t, from the fresh master */
            const int hpg = H / G;
            for (int h = 0; h < H; ++h) {
                const double *S = r->ckpt + ((size_t)b * H + h) * (size_t)P * N;
                const float *Ct = C + ((size_t)b * G + h / hpg) * N;
                for (int p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int n = 0; n < N; ++n) acc += S[(size_t)p * N + n] * (double)Ct[n];
                    yb[(size_t)h * P + p] =
                        acc + r->D[h] * (double)x[((size_t)b * H + h) * P + p];
                }
            }
        } else {
            const double *Sread = r->read_prec ? r->rcopy : r->ckpt;
            replay_output(r, Sread, b, idx, C + (size_t)b * G * N, yb);
        }
    }
    return 0;
}

/* Speculative verify (output-only evaluation): T draft records go after the committed ones,   */
/* and each draft's output is formed by replay over the committed window plus the drafts up to */
/* and including itself. No state is stored and no pointer moves ([AT Pulse] "Technical        */
/* analysis": verification uses output-only evaluation and builds no intermediate state).      */
/* Returns 0, or -1 (verify already pending, T out of range, or drafts would not fit).         */
int oracle_replay_verify(oracle_replay *r, int T, const float *x, const float *B, const float *C,
                         const float *dt, double *y)
{
    if (r->pending_T || T < 1 || T > r->Tmax) return -1;
    for (int b = 0; b < r->Bt; ++b) {
        int count = r->pos[b] - r->ckpt_pos[b];
        if (count < 0 || count + T > r->L) return -1;
    }
    const int H = r->H, P = r->P, N = r->N, G = r->G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < r->Bt; ++b) {
        int count = r->pos[b] - r->ckpt_pos[b];
        for (int i = 0; i < T; ++i)
            store_record(r, b, count + i, x + ((size_t)b * T + i) * H * P,
                         B + ((size_t)b * T + i) * G * N, C + ((size_t)b * T + i) * G * N,
                         dt + ((size_t)b * T + i) * H);
        const double *Sread = r->read_prec ? r->rcopy : r->ckpt;
        for (int i = 0; i < T; ++i)
            replay_output(r, Sread, b, count + i, C + ((size_t)b * T + i) * G * N,
                          y + ((size_t)b * T + i) * H * P);
    }
    r->pending_T = T;
    return 0;
}

/* Rollback and commit: the first accepted[b] drafts become committed (pos moves forward by    */
/* accepted[b]; the rest are forgotten), then the sequence flushes when more than L - Tmax     */
/* records are pending (R5). [AT Pulse] "Technical analysis": rollback is a pointer move.      */
int oracle_replay_rollback(oracle_replay *r, const int *accepted)
{
    if (!r->pending_T) return -1;
    for (int b = 0; b < r->Bt; ++b)
        if (accepted[b] < 0 || accepted[b] > r->pending_T) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < r->Bt; ++b) {
        r->pos[b] += accepted[b];
        poison_records(r, b, r->pos[b] - r->ckpt_pos[b]);
        if (r->pos[b] - r->ckpt_pos[b] > r->L - r->Tmax) flush_seq(r, b);
    }
    r->pending_T = 0;
    return 0;
}

/* Replace checkpoints by given fp32 values, held as they are (no rounding to the master       */
/* precision), and re-encode the read copy from them; records and pointers stay. rows == NULL:  */
/* S is [Bt,H,P,N] and every sequence is set; else S is [nrows,H,P,N] and its row i sets       */
/* sequence rows[i]. A test uses it to continue the replay-form model from the GPU's own        */
/* checkpoint after a flush: the model then reads exactly the copy the layer must hold (the     */
/* master encoded by R6/R7), so later replayed outputs can be compared at fp32 rounding.        */
/* Returns 0, or -1 while a verify is pending or for a row index out of range.                  */
int oracle_replay_set_checkpoint(oracle_replay *r, const float *S, const int *rows, int nrows)
{
    if (r->pending_T) return -1;
    if (!rows) nrows = r->Bt;
    for (int i = 0; i < nrows; ++i)
        if (rows && (rows[i] < 0 || rows[i] >= r->Bt)) return -1;
    const size_t seq = (size_t)r->H * r->P * r->N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nrows; ++i) {
        const int b = rows ? rows[i] : i;
        for (size_t e = 0; e < seq; ++e) r->ckpt[(size_t)b * seq + e] = (double)S[(size_t)i * seq + e];
        refresh_copy(r, b);
    }
    return 0;
}

/* fp8 master (reading R9): export E4M3FN codes [Bt,H,P,N] and scales [Bt,H,ceil(P/64)] -- each */
/* value is code * scale exactly, so its code is the nearest-even code of value / scale.        */
/* -1 for another master precision.                                                             */
int oracle_replay_master_fp8(const oracle_replay *r, uint8_t *codes, float *scales)
{
    if (r->master_prec < 3) return -1;
    const int nblk = (r->P + 63) / 64;
    for (size_t bh = 0; bh < (size_t)r->Bt * r->H; ++bh)
        for (int p = 0; p < r->P; ++p) {
            const float s = r->mscale[bh * nblk + p / 64];
            const size_t row = (bh * r->P + p) * r->N;
            for (int n = 0; n < r->N; ++n) codes[row + n] = oracle_e4m3_encode_scaled((float)(r->ckpt[row + n] / (double)s));
        }
    memcpy(scales, r->mscale, (size_t)r->Bt * r->H * nblk * sizeof(float));
    return 0;
}

/* fp8 master: set the checkpoints of sequences rows[0..nrows) (all when rows is NULL) to     */
/* codes [nrows,H,P,N] times scales [nrows,H,ceil(P/64)], exactly in float64; records and      */
/* pointers stay. A test continues the model from the GPU's own fp8 master this way. -1 while  */
/* a verify is pending, for a row out of range, or for another master precision.             */
int oracle_replay_set_master_fp8(oracle_replay *r, const uint8_t *codes, const float *scales, const int *rows,
                                 int nrows)
{
    if (r->pending_T || r->master_prec < 3) return -1;
    if (!rows) nrows = r->Bt;
    for (int i = 0; i < nrows; ++i)
        if (rows && (rows[i] < 0 || rows[i] >= r->Bt)) return -1;
    const int nblk = (r->P + 63) / 64;
    for (int i = 0; i < nrows; ++i) {
        const int b = rows ? rows[i] : i;
        for (int h = 0; h < r->H; ++h)
            for (int p = 0; p < r->P; ++p) {
                const float s = scales[((size_t)i * r->H + h) * nblk + p / 64];
                r->mscale[((size_t)b * r->H + h) * nblk + p / 64] = s;
                const size_t src = (((size_t)i * r->H + h) * r->P + p) * r->N;
                const size_t dst = (((size_t)b * r->H + h) * r->P + p) * r->N;
                for (int n = 0; n < r->N; ++n) r->ckpt[dst + n] = (double)oracle_e4m3_decode(codes[src + n]) * (double)s;
            }
    }
    return 0;
}

/* Explicit flush of the selected sequences (all when mask is NULL). */
int oracle_replay_flush(oracle_replay *r, const int *seq_mask)
{
    if (r->pending_T) return -1;
    for (int b = 0; b < r->Bt; ++b)
        if (!seq_mask || seq_mask[b]) flush_seq(r, b);
    return 0;
}

void oracle_replay_pointers(const oracle_replay *r, int *pos, int *ckpt_pos)
{
    for (int b = 0; b < r->Bt; ++b) { pos[b] = r->pos[b]; ckpt_pos[b] = r->ckpt_pos[b]; }
}

void oracle_replay_checkpoint(const oracle_replay *r, double *out)
{
    memcpy(out, r->ckpt, (size_t)r->Bt * r->H * r->P * r->N * sizeof(double));
}

/* The decoded read copy (equals the master when reads are fp32). */
void oracle_replay_read_copy(const oracle_replay *r, double *out)
{
    memcpy(out, r->read_prec ? r->rcopy : r->ckpt,
           (size_t)r->Bt * r->H * r->P * r->N * sizeof(double));
}

/* The full state after all committed tokens: the master with the pending committed records   */
/* folded in, without committing anything.                                                    */
void oracle_replay_materialize(const oracle_replay *r, double *out)
{
    memcpy(out, r->ckpt, (size_t)r->Bt * r->H * r->P * r->N * sizeof(double));
    for (int b = 0; b < r->Bt; ++b) fold_into(r, b, r->pos[b] - r->ckpt_pos[b], out);
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for later parallel regions (n >= 1); for timing the oracle on a given core count. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
