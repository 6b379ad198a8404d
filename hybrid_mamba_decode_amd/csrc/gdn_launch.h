// gdn_launch.h -- Gated DeltaNet layer descriptor and internal launchers, one set per supported
// key size Dk (gdn_kernels.hip, compiled once per Dk). The C ABI (gdn_api.hip) validates first.
#pragma once

#include "device.h"
#include "launch.h"  // MODE_MASK / MODE_OVERFULL / MODE_MATERIALIZE

namespace rssm {

// One GDN layer's workspace (passed by value). H value heads of Dv, G key heads of Dk.
struct GLayer {
    float *master;      // [Bt,H,Dv,Dk] fp32 checkpoint
    void *rcopy;        // read copy, else nullptr: bf16 [Bt,H,Dv,Dk] row-major, or fp8 / MXFP4 codes
                        // in 16-byte chunks, chunk-column-major per head (state_chunk_off)
    int rprec;          // PREC_F32 (reads from the checkpoint), PREC_BF16, PREC_FP8 or PREC_FP4
    float *scale;       // fp8: [Bt,H,psplit], one per 64 value rows
    unsigned char *mxscale;  // MXFP4: [Bt,H,Dv,Dk/32] E8M0 block-scale codes
    float *ring_k;      // [Bt,G,L,Dk]
    float *ring_v;      // [Bt,H,L,Dv]
    float *ring_a;      // [Bt,H,L] gate alpha
    float *ring_b;      // [Bt,H,L] write strength beta
    int *pos;           // [Bt]
    int *ckpt;          // [Bt]
    unsigned *counter;  // [Bt]
    unsigned *flag;     // [1]
    int Bt, H, Dv, G, L, Tmax, hpg, psplit;
};

// Per-token inputs of one call (layouts in gdnreplay.h).
struct GTokenIO {
    const float *q, *k, *v, *alpha, *beta;
    float *o;
};

#define RSSM_DECLARE_GDN_LAUNCHERS(NV)                                                                       \
    hipError_t gdn_launch_step_n##NV(int lmax, const GLayer &Ld, const GTokenIO &io, bool flush_capable,     \
                                     bool all_flush, Lockstep ls, hipStream_t st);                           \
    hipError_t gdn_launch_flush_n##NV(int lmax, const GLayer &Ld, int mode, const int *arg, int T, float *out, \
                                      hipStream_t st);                                                       \
    hipError_t gdn_launch_verify_n##NV(int lmax, const GLayer &Ld, const GTokenIO &io, int T, hipStream_t st);  \
    hipError_t gdn_launch_load_n##NV(const GLayer &Ld, const float *state, hipStream_t st);                  \
    hipError_t gdn_launch_conventional_n##NV(const GLayer &Ld, float *state, const GTokenIO &io, hipStream_t st); \
    hipError_t gdn_launch_snapshot_n##NV(const GLayer &Ld, float *slots, const int *cur, int T,               \
                                         const GTokenIO &io, hipStream_t st);

RSSM_DECLARE_GDN_LAUNCHERS(16)
RSSM_DECLARE_GDN_LAUNCHERS(32)
RSSM_DECLARE_GDN_LAUNCHERS(64)
RSSM_DECLARE_GDN_LAUNCHERS(128)
RSSM_DECLARE_GDN_LAUNCHERS(256)

#undef RSSM_DECLARE_GDN_LAUNCHERS

}  // namespace rssm
