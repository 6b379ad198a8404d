// launch.h -- internal launchers, one set per supported state size N (kernels.hip, compiled
// once per N). The C ABI (api.hip) validates everything first, then calls these.
#pragma once

#include "device.h"

namespace rssm {

// MODE_OVERFULL: advance pos by the accepted counts, then fold sequences with more than L - Tmax
// pending records (the rollback commit).
enum { MODE_MASK = 0, MODE_OVERFULL = 1, MODE_MATERIALIZE = 2 };

#define RSSM_DECLARE_LAUNCHERS(NV)                                                                     \
    hipError_t launch_step_n##NV(int prec, int lmax, const Layer &Ld, const TokenIO &io,               \
                                 bool flush_capable, bool all_flush, bool mix, Lockstep ls,            \
                                 hipStream_t st);                                                      \
    hipError_t launch_flush_n##NV(int prec, int lmax, const Layer &Ld, int mode, const int *arg, int T,  \
                                  float *out, hipStream_t st);                                         \
    hipError_t launch_verify_n##NV(int prec, int lmax, const Layer &Ld, const TokenIO &io, int T,       \
                                   bool mix, hipStream_t st);                                          \
    hipError_t launch_load_n##NV(int prec, const Layer &Ld, const float *state, hipStream_t st);        \
    hipError_t launch_conventional_n##NV(const Layer &Ld, float *state, const TokenIO &io,             \
                                         hipStream_t st);                                              \
    hipError_t launch_conventional_mixer_n##NV(const Layer &Ld, float *state, const TokenIO &io,       \
                                               int rslot, hipStream_t st);                             \
    hipError_t launch_snapshot_n##NV(const Layer &Ld, float *slots, const int *cur, int T,              \
                                     const TokenIO &io, hipStream_t st);

RSSM_DECLARE_LAUNCHERS(16)
RSSM_DECLARE_LAUNCHERS(32)
RSSM_DECLARE_LAUNCHERS(64)
RSSM_DECLARE_LAUNCHERS(128)
RSSM_DECLARE_LAUNCHERS(256)

#undef RSSM_DECLARE_LAUNCHERS

}  // namespace rssm
