/*
 * oracle_mixer.c -- float64 CPU oracle for the Mamba-2 mixer edges around the decode step.
 *
 * TEST INFRASTRUCTURE ONLY (as oracle.c): loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library; the two share no source.
 *
 * The pages give the SSM step only ([Clarity] "Why it matters": a conventional step updates the
 * state, reads the output and stores the state). In a Mamba-2 mixer that step sits between the
 * in-projection and the output gate; reading M1 takes the published Mamba-2 block (Dao and Gu,
 * "Transformers are SSMs", 2024) for the two edges, per token and sequence:
 *
 *   in-projection output: z [H*P], xBC [CD] with CD = H*P + 2*G*N (channels: x head-major, then
 *   B group-major, then C), dt_raw [H].
 *   causal depthwise conv1d of width K over xBC, weights w [CD][K], bias b [CD]:
 *       u_t[c] = b[c] + sum_{i=0}^{K-1} w[c][i] * xBC_{t-K+1+i}[c]
 *   with the K-1 previous tokens' raw inputs as history (zeros before the first token);
 *       (x_t, B_t, C_t) = split(silu(u_t)),   silu(v) = v / (1 + exp(-v))
 *       dt_t = softplus(dt_raw + dt_bias[h]),  softplus(v) = log(1 + exp(v))
 *   the SSM step (oracle.c) on (x_t, B_t, C_t, dt_t), and the gated output
 *       o_t[h,p] = y_t[h,p] * silu(z_t[h,p]).
 *
 * The edge works in float64 and hands the SSM fp32 values (reading M2: the layer's inputs and
 * records are fp32, as when the in-projection writes them). The history is the raw fp32 inputs
 * of the last K-1 tokens, oldest first.
 */
#include <math.h>
#include <stddef.h>
#include <string.h>

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* log(1 + exp(v)) without overflow: for v > 0 it equals v + log(1 + exp(-v)). */
static double softplus(double v) { return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }

double oracle_silu(double v) { return silu(v); }
double oracle_softplus(double v) { return softplus(v); }

/* One token of the input edge for every sequence. hist [Bt][K-1][CD] is updated in place (the  */
/* oldest row drops out, this token's xbc enters last). Outputs: x [Bt][H*P], B and C           */
/* [Bt][G*N], dt [Bt][H], fp32 (reading M2).                                                     */
void oracle_mixer_edge(int Bt, int H, int P, int N, int G, int K, float *hist, const float *xbc,
                       const float *dt_raw, const float *conv_w, const float *conv_b,
                       const float *dt_bias, float *x, float *B, float *C, float *dt)
{
    const size_t HP = (size_t)H * P, GN = (size_t)G * N, CD = HP + 2 * GN;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < Bt; ++b) {
        float *hb = hist + (size_t)b * (K - 1) * CD;
        const float *in = xbc + (size_t)b * CD;
        for (size_t c = 0; c < CD; ++c) {
            /* taps i = 0..K-2 read the history (oldest first), tap K-1 this token */
            double u = (double)conv_b[c];
            for (int i = 0; i < K - 1; ++i) u += (double)conv_w[c * K + i] * (double)hb[(size_t)i * CD + c];
            u += (double)conv_w[c * K + K - 1] * (double)in[c];
            const float v = (float)silu(u);
            if (c < HP) x[(size_t)b * HP + c] = v;
            else if (c < HP + GN) B[(size_t)b * GN + (c - HP)] = v;
            else C[(size_t)b * GN + (c - HP - GN)] = v;
        }
        for (int h = 0; h < H; ++h)
            dt[(size_t)b * H + h] = (float)softplus((double)dt_raw[(size_t)b * H + h] + (double)dt_bias[h]);
        if (K > 1) {
            memmove(hb, hb + CD, (size_t)(K - 2) * CD * sizeof(float));
            memcpy(hb + (size_t)(K - 2) * CD, in, CD * sizeof(float));
        }
    }
}

/* Output gate: o = y * silu(z), elementwise over n values. */
void oracle_mixer_gate(size_t n, const double *y, const float *z, double *o)
{
    for (size_t i = 0; i < n; ++i) o[i] = y[i] * silu((double)z[i]);
}
