// api.hip -- the C ABI of replayssm.h: argument and state-machine validation, workspace layout,
// the host-side flush hint, and kernel dispatch by state size N.
//
// Everything that can be checked on the host is checked before any HIP call, so the error paths
// run without a GPU.
#include "../../include/replayssm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>

#include "host_state.h"
#include "launch.h"

using namespace rssm;

struct replayssm_layer {
    replayssm_config cfg;
    replayssm_layout lay;
    Layer dev;
    int lmax;       // window bucket for kernel instances (16, 32 or 64)
    // Host state machine (host_state.h). Lockstep arguments: with T_max = 1 and no mixer edges they
    // repeat every L steps, so a captured run of whole windows replays correctly; with the mixer
    // edges the conv ring slot pos mod R repeats every R steps, so a captured run must span a
    // multiple of lcm(L, R) steps. A replay whose arguments no longer match the device pointers
    // (or ring slot) raises the device flag.
    HostState hs;
    int mixer_set;  // replayssm_set_mixer has given the edge parameters
};

namespace {

bool supported_n(int n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }

int psplit_of(const replayssm_config &c) { return (c.headdim + kRows - 1) / kRows; }

// Shape checks shared by every entry point (the baselines use only these fields).
rssm_status check_shape(const replayssm_config *c)
{
    if (!c) return RSSM_E_INVAL;
    if (c->batch < 0 || c->nheads <= 0 || c->headdim <= 0 || c->dstate <= 0 || c->ngroups <= 0)
        return RSSM_E_INVAL;
    if (c->nheads % c->ngroups) return RSSM_E_INVAL;
    if (c->headdim % 4) return RSSM_E_INVAL;
    if (!supported_n(c->dstate) || c->headdim > 256) return RSSM_E_UNSUPPORTED;
    const uint64_t blocks = (uint64_t)c->batch * c->nheads * psplit_of(*c);
    if (blocks * kThreads >= (1ull << 32)) return RSSM_E_UNSUPPORTED;
    return RSSM_OK;
}

rssm_status check_config(const replayssm_config *c)
{
    rssm_status s = check_shape(c);
    if (s != RSSM_OK) return s;
    if (c->buffer_len < 1 || c->max_draft < 1 || c->max_draft > c->buffer_len) return RSSM_E_INVAL;
    if (c->read_prec < RSSM_READ_FP32 || c->read_prec > RSSM_READ_MXFP4) return RSSM_E_INVAL;
    if (c->store_C != 0 && c->store_C != 1) return RSSM_E_INVAL;
    if (c->buffer_len > 64 || c->max_draft > 8) return RSSM_E_UNSUPPORTED;
    if (c->read_prec == RSSM_READ_MXFP4 && c->dstate < 32) return RSSM_E_UNSUPPORTED;
    if (c->master_prec < RSSM_MASTER_FP32 || c->master_prec > RSSM_MASTER_FP8_SR) return RSSM_E_INVAL;
    // an fp8 master is its own read copy: no second copy
    if (c->master_prec >= RSSM_MASTER_FP8 && c->read_prec != RSSM_READ_FP32) return RSSM_E_INVAL;
    if (c->d_conv < 0 || c->d_conv == 1) return RSSM_E_INVAL;
    if (c->d_conv > 4 || (c->d_conv > 0 && c->buffer_len > 32)) return RSSM_E_UNSUPPORTED;
    return RSSM_OK;
}

// Mixer edges: conv channels CD = H*P + 2*G*N and ring slots R = K - 1 + T_max.
size_t conv_dim(const replayssm_config &c) { return (size_t)c.nheads * c.headdim + 2 * (size_t)c.ngroups * c.dstate; }
int conv_slots(const replayssm_config &c) { return c.d_conv > 0 ? c.d_conv - 1 + c.max_draft : 0; }

bool fp8_master(const replayssm_config &c) { return c.master_prec >= RSSM_MASTER_FP8; }
bool sr_master(const replayssm_config &c)
{
    return c.master_prec == RSSM_MASTER_FP16_SR || c.master_prec == RSSM_MASTER_FP8_SR;
}

// Read precision of the kernels: the copy's, or the fp16 / fp8 master read directly.
int kernel_prec(const replayssm_config &c)
{
    if (fp8_master(c)) return PREC_FP8;
    return c.read_prec == RSSM_READ_FP32 && c.master_prec != RSSM_MASTER_FP32 ? PREC_F16 : c.read_prec;
}

void make_layout(const replayssm_config &c, replayssm_layout *L)
{
    const size_t Bt = (size_t)c.batch, H = c.nheads, P = c.headdim, N = c.dstate, G = c.ngroups,
                 Lb = c.buffer_len;
    const size_t elems = Bt * H * P * N;
    RegionCarver rc;
    auto take = [&](size_t bytes) { return rc.take(bytes); };
    // an fp8 master takes the fp8 copy's layout (chunked codes) in the master region and its
    // per-head scales in the scale region
    L->master = take(elems * (c.master_prec == RSSM_MASTER_FP32 ? 4 : fp8_master(c) ? 1 : 2));
    const int rp = fp8_master(c) ? RSSM_READ_FP8_E4M3 : c.read_prec;
    L->read_copy = take(fp8_master(c) ? 0 : rp == RSSM_READ_BF16 ? elems * 2 : rp == RSSM_READ_FP8_E4M3 ? elems
                        : rp == RSSM_READ_MXFP4 ? elems / 2 : 0);
    L->scale = take(rp == RSSM_READ_FP8_E4M3 ? Bt * H * psplit_of(c) * 4 : rp == RSSM_READ_MXFP4 ? elems / 32 : 0);
    L->ring_x = take(Bt * H * Lb * P * 4);
    L->ring_B = take(Bt * G * Lb * N * 4);
    L->ring_C = take(c.store_C ? Bt * G * Lb * N * 4 : 0);
    L->ring_dt = take(Bt * H * Lb * 4);
    L->conv_ring = take(Bt * conv_slots(c) * conv_dim(c) * 4);
    L->pos = take(Bt * 4);
    L->ckpt_pos = take(Bt * 4);
    L->counters = take(Bt * 4);
    L->flag = take(4);
    L->total = rc.off;
}

// A Layer carrying only shapes and A/D, for the baselines.
Layer shape_layer(const replayssm_config &c, const float *A, const float *D)
{
    Layer L;
    std::memset(&L, 0, sizeof(L));
    L.A = A;
    L.D = D;
    L.Bt = c.batch;
    L.H = c.nheads;
    L.P = c.headdim;
    L.G = c.ngroups;
    L.L = 1;
    L.Tmax = 1;
    L.hpg = c.nheads / c.ngroups;
    L.psplit = psplit_of(c);
    return L;
}

// Snapshot baseline commit: the committed slot moves forward by the accepted count, modulo the
// T + 1 slots. One thread per sequence; out-of-range counts leave the slot unchanged.
__global__ void snapshot_commit_kernel(int *cur, const int *accepted, int T, int Bt)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= Bt) return;
    const int a = accepted[b], c = cur[b];
    if (a >= 0 && a <= T && c >= 0 && c <= T) cur[b] = (c + a) % (T + 1);
}

hipError_t launch_snapshot_commit(int *cur, const int *accepted, int T, int Bt, hipStream_t st)
{
    hipLaunchKernelGGL(snapshot_commit_kernel, dim3((Bt + 255) / 256), dim3(256), 0, st, cur, accepted, T, Bt);
    return hipGetLastError();
}

#define RSSM_BY_N(NV, CALL)                 \
    switch (NV) {                           \
    case 16: return hip_status(CALL(16));   \
    case 32: return hip_status(CALL(32));   \
    case 64: return hip_status(CALL(64));   \
    case 128: return hip_status(CALL(128)); \
    case 256: return hip_status(CALL(256)); \
    default: return RSSM_E_UNSUPPORTED;     \
    }

rssm_status ready(replayssm_t h)
{
    if (!h) return RSSM_E_INVAL;
    return h->hs.ready();
}

// Conv history of every sequence, relative to its device pos: row i (oldest first) is the raw
// xBC of position pos - (K-1) + i, at ring slot (that position) mod R. load: from hist (zeros
// when NULL); materialize (out != NULL): into out. One thread per (sequence, row, channel).
__global__ void conv_hist_kernel(Layer Ld, const float *hist, float *out)
{
    const size_t rows = (size_t)Ld.K - 1, e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (size_t)Ld.Bt * rows * Ld.CD) return;
    const int c = (int)(e % Ld.CD);
    const int i = (int)(e / Ld.CD % rows);
    const int b = (int)(e / Ld.CD / rows);
    const int q = Ld.pos[b] - (Ld.K - 1) + i;
    const int slot = ((q % Ld.R) + Ld.R) % Ld.R;
    float *ring = Ld.conv_ring + ((size_t)b * Ld.R + slot) * Ld.CD + c;
    if (out) out[e] = *ring;
    else *ring = hist ? hist[e] : 0.f;
}

hipError_t launch_conv_hist(const Layer &Ld, const float *hist, float *out, hipStream_t st)
{
    const size_t n = (size_t)Ld.Bt * (Ld.K - 1) * Ld.CD;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(conv_hist_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Ld, hist, out);
    return hipGetLastError();
}

rssm_status read_flag(replayssm_t h, hipStream_t st) { return h->hs.read_flag(h->dev.flag, h->cfg.batch, st); }

}  // namespace

extern "C" {

size_t replayssm_workspace_bytes(const replayssm_config *cfg)
{
    if (check_config(cfg) != RSSM_OK) return 0;
    replayssm_layout L;
    make_layout(*cfg, &L);
    return L.total;
}

rssm_status replayssm_workspace_layout(const replayssm_config *cfg, replayssm_layout *out)
{
    const rssm_status s = check_config(cfg);
    if (s != RSSM_OK) return s;
    if (!out) return RSSM_E_INVAL;
    make_layout(*cfg, out);
    return RSSM_OK;
}

rssm_status replayssm_create(const replayssm_config *cfg, void *workspace, size_t bytes,
                             const float *A, const float *D, replayssm_t *out)
{
    if (!out) return RSSM_E_INVAL;
    *out = nullptr;
    const rssm_status s = check_config(cfg);
    if (s != RSSM_OK) return s;
    if (!A || !D || !aligned(A, 4) || !aligned(D, 4)) return RSSM_E_INVAL;
    replayssm_layout lay;
    make_layout(*cfg, &lay);
    if (!workspace || !aligned(workspace, kWsAlign) || bytes < lay.total) return RSSM_E_WORKSPACE;
    replayssm_layer *h = new (std::nothrow) replayssm_layer();
    if (!h) return RSSM_E_INVAL;
    h->cfg = *cfg;
    h->hs.init(cfg->buffer_len, cfg->max_draft);
    h->lay = lay;
    char *ws = (char *)workspace;
    Layer &d = h->dev;
    d.master = (float *)(ws + lay.master);
    d.rcopy = fp8_master(*cfg) ? (void *)(ws + lay.master)
              : cfg->read_prec == RSSM_READ_FP32 ? nullptr : (void *)(ws + lay.read_copy);
    d.scale = cfg->read_prec == RSSM_READ_FP8_E4M3 || fp8_master(*cfg) ? (float *)(ws + lay.scale) : nullptr;
    d.mxscale = cfg->read_prec == RSSM_READ_MXFP4 ? (unsigned char *)(ws + lay.scale) : nullptr;
    d.ring_x = (float *)(ws + lay.ring_x);
    d.ring_B = (float *)(ws + lay.ring_B);
    d.ring_C = cfg->store_C ? (float *)(ws + lay.ring_C) : nullptr;
    d.ring_dt = (float *)(ws + lay.ring_dt);
    d.pos = (int *)(ws + lay.pos);
    d.ckpt = (int *)(ws + lay.ckpt_pos);
    d.counter = (unsigned *)(ws + lay.counters);
    d.flag = (unsigned *)(ws + lay.flag);
    d.A = A;
    d.D = D;
    d.Bt = cfg->batch;
    d.H = cfg->nheads;
    d.P = cfg->headdim;
    d.G = cfg->ngroups;
    d.L = cfg->buffer_len;
    d.Tmax = cfg->max_draft;
    d.hpg = cfg->nheads / cfg->ngroups;
    d.psplit = psplit_of(*cfg);
    d.mprec = cfg->master_prec;
    d.sr_seed = (unsigned)cfg->sr_seed;
    d.conv_ring = cfg->d_conv > 0 ? (float *)(ws + lay.conv_ring) : nullptr;
    d.K = cfg->d_conv;
    d.R = conv_slots(*cfg);
    d.CD = (int)conv_dim(*cfg);
    h->lmax = cfg->buffer_len <= 16 ? 16 : cfg->buffer_len <= 32 ? 32 : 64;
    *out = h;
    return RSSM_OK;
}

rssm_status replayssm_destroy(replayssm_t h)
{
    delete h;
    return RSSM_OK;
}

rssm_status replayssm_load_state(replayssm_t h, const float *state, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!ok_ptr(state, h->cfg.batch)) return RSSM_E_INVAL;
    // a stochastically rounded master keys its stream by each sequence's device ckpt_pos
    h->hs.on_load(!sr_master(h->cfg));
    if (h->cfg.batch == 0) return RSSM_OK;
    const hipStream_t st = (hipStream_t)stream;
    rssm_status s = RSSM_OK;
    {
#define CALL(NV) launch_load_n##NV(kernel_prec(h->cfg), h->dev, state, st)
        s = [&]() -> rssm_status { RSSM_BY_N(h->cfg.dstate, CALL) }();
#undef CALL
    }
    if (s != RSSM_OK || h->cfg.d_conv == 0) return s;
    return hip_status(launch_conv_hist(h->dev, nullptr, nullptr, st));  // a fresh conv history: zeros
}

namespace {

// One standard step (plain or with the mixer edges), after the entry point's argument checks.
rssm_status do_step(replayssm_t h, const TokenIO &io, bool mix, void *stream)
{
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->hs.pending_T) return RSSM_E_STATE;
    const StepPlan p = h->hs.begin_step();
    const Lockstep ls{p.pslot, p.cslot, p.k, p.k > 0 && h->dev.R > 0 ? p.upos % h->dev.R : 0};
    if (h->cfg.batch == 0) return RSSM_OK;
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) launch_step_n##NV(kernel_prec(h->cfg), h->lmax, h->dev, io, p.flush_capable, p.all_flush, mix, ls, st)
    RSSM_BY_N(h->cfg.dstate, CALL)
#undef CALL
}

}  // namespace

rssm_status replayssm_step(replayssm_t h, const float *x, const float *B, const float *C,
                           const float *dt, float *y, void *stream)
{
    if (!h || h->cfg.d_conv > 0) return RSSM_E_INVAL;  // a mixer handle steps through replayssm_mixer_step
    const int bt = h->cfg.batch;
    if (!ok_ptr(x, bt) || !ok_ptr(B, bt) || !ok_ptr(C, bt) || !ok_ptr(dt, bt) || !ok_ptr(y, bt))
        return RSSM_E_INVAL;
    return do_step(h, TokenIO{x, B, C, dt, y, nullptr, nullptr}, false, stream);
}

rssm_status replayssm_set_mixer(replayssm_t h, const float *conv_w, const float *conv_b, const float *dt_bias)
{
    if (!h || h->cfg.d_conv == 0) return RSSM_E_INVAL;
    if (!conv_w || !conv_b || !dt_bias || !aligned(conv_w, 4) || !aligned(conv_b, 4) || !aligned(dt_bias, 4))
        return RSSM_E_INVAL;
    h->dev.conv_w = conv_w;
    h->dev.conv_b = conv_b;
    h->dev.dt_bias = dt_bias;
    h->dev.wvec = h->cfg.d_conv == 4 && aligned(conv_w, 16);
    h->mixer_set = 1;
    return RSSM_OK;
}

rssm_status replayssm_load_conv_state(replayssm_t h, const float *hist, void *stream)
{
    if (!h || h->cfg.d_conv == 0) return RSSM_E_INVAL;
    if (hist && !aligned(hist, 4)) return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->hs.pending_T) return RSSM_E_STATE;
    if (h->cfg.batch == 0) return RSSM_OK;
    return hip_status(launch_conv_hist(h->dev, hist, nullptr, (hipStream_t)stream));
}

rssm_status replayssm_materialize_conv_state(replayssm_t h, float *out, void *stream)
{
    if (!h || h->cfg.d_conv == 0) return RSSM_E_INVAL;
    if (!ok_ptr4(out, h->cfg.batch)) return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->hs.pending_T) return RSSM_E_STATE;
    if (h->cfg.batch == 0) return RSSM_OK;
    return hip_status(launch_conv_hist(h->dev, nullptr, out, (hipStream_t)stream));
}

rssm_status replayssm_mixer_step(replayssm_t h, const float *xbc, const float *z, const float *dt_raw, float *o,
                                 void *stream)
{
    if (!h || h->cfg.d_conv == 0) return RSSM_E_INVAL;
    const int bt = h->cfg.batch;
    if (!ok_ptr4(xbc, bt) || !ok_ptr4(z, bt) || !ok_ptr4(dt_raw, bt) || !ok_ptr4(o, bt)) return RSSM_E_INVAL;
    if (!h->mixer_set) return RSSM_E_STATE;
    return do_step(h, TokenIO{nullptr, nullptr, nullptr, dt_raw, o, xbc, z}, true, stream);
}

rssm_status replayssm_flush(replayssm_t h, const int32_t *seq_mask, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (seq_mask && !aligned(seq_mask, 4)) return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->hs.pending_T) return RSSM_E_STATE;
    h->hs.on_flush(seq_mask != nullptr);
    if (h->cfg.batch == 0) return RSSM_OK;
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) launch_flush_n##NV(kernel_prec(h->cfg), h->lmax, h->dev, MODE_MASK, seq_mask, 0, nullptr, st)
    RSSM_BY_N(h->cfg.dstate, CALL)
#undef CALL
}

rssm_status replayssm_spec_verify(replayssm_t h, int32_t T, const float *x, const float *B,
                                  const float *C, const float *dt, float *y, void *stream)
{
    if (!h || h->cfg.d_conv > 0) return RSSM_E_INVAL;
    const int bt = h->cfg.batch;
    if (T < 1 || T > h->cfg.max_draft) return RSSM_E_INVAL;
    if (!ok_ptr(x, bt) || !ok_ptr(B, bt) || !ok_ptr(C, bt) || !ok_ptr(dt, bt) || !ok_ptr(y, bt))
        return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->hs.pending_T) return RSSM_E_STATE;
    h->hs.pending_T = T;
    if (h->cfg.batch == 0) return RSSM_OK;
    const TokenIO io{x, B, C, dt, y};
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) launch_verify_n##NV(kernel_prec(h->cfg), h->lmax, h->dev, io, T, false, st)
    RSSM_BY_N(h->cfg.dstate, CALL)
#undef CALL
}

rssm_status replayssm_mixer_spec_verify(replayssm_t h, int32_t T, const float *xbc, const float *z,
                                        const float *dt_raw, float *o, void *stream)
{
    if (!h || h->cfg.d_conv == 0) return RSSM_E_INVAL;
    const int bt = h->cfg.batch;
    if (T < 1 || T > h->cfg.max_draft) return RSSM_E_INVAL;
    if (!ok_ptr4(xbc, bt) || !ok_ptr4(z, bt) || !ok_ptr4(dt_raw, bt) || !ok_ptr4(o, bt)) return RSSM_E_INVAL;
    if (!h->mixer_set) return RSSM_E_STATE;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->hs.pending_T) return RSSM_E_STATE;
    h->hs.pending_T = T;
    if (h->cfg.batch == 0) return RSSM_OK;
    const TokenIO io{nullptr, nullptr, nullptr, dt_raw, o, xbc, z};
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) launch_verify_n##NV(kernel_prec(h->cfg), h->lmax, h->dev, io, T, true, st)
    RSSM_BY_N(h->cfg.dstate, CALL)
#undef CALL
}

rssm_status replayssm_rollback(replayssm_t h, const int32_t *accepted, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!ok_ptr4(accepted, h->cfg.batch)) return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (!h->hs.pending_T) return RSSM_E_STATE;
    const int T = h->hs.pending_T;
    h->hs.on_rollback(T);
    if (h->cfg.batch == 0) return RSSM_OK;
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) launch_flush_n##NV(kernel_prec(h->cfg), h->lmax, h->dev, MODE_OVERFULL, accepted, T, nullptr, st)
    RSSM_BY_N(h->cfg.dstate, CALL)
#undef CALL
}

rssm_status replayssm_set_lockstep(replayssm_t h, int enable)
{
    if (!h || (enable != 0 && enable != 1)) return RSSM_E_INVAL;
    h->hs.set_lockstep(enable);
    return RSSM_OK;
}

rssm_status replayssm_get_pointers(replayssm_t h, int32_t *pos, int32_t *ckpt_pos, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!h->hs.loaded) return RSSM_E_STATE;
    const hipStream_t st = (hipStream_t)stream;
    const rssm_status s = read_flag(h, st);
    if (s != RSSM_OK) return s;
    const size_t bytes = (size_t)h->cfg.batch * sizeof(int32_t);
    if (bytes == 0) return RSSM_OK;
    if (pos && hipMemcpy(pos, h->dev.pos, bytes, hipMemcpyDeviceToHost) != hipSuccess) return RSSM_E_HIP;
    if (ckpt_pos && hipMemcpy(ckpt_pos, h->dev.ckpt, bytes, hipMemcpyDeviceToHost) != hipSuccess) return RSSM_E_HIP;
    return RSSM_OK;
}

rssm_status replayssm_check(replayssm_t h, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!h->hs.loaded || h->hs.poisoned) return RSSM_E_STATE;
    return read_flag(h, (hipStream_t)stream);
}

rssm_status replayssm_materialize_state(replayssm_t h, float *out, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!ok_ptr(out, h->cfg.batch)) return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->cfg.batch == 0) return RSSM_OK;
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) launch_flush_n##NV(kernel_prec(h->cfg), h->lmax, h->dev, MODE_MATERIALIZE, nullptr, 0, out, st)
    RSSM_BY_N(h->cfg.dstate, CALL)
#undef CALL
}

rssm_status conventional_step(const replayssm_config *cfg, float *state, const float *x,
                              const float *B, const float *C, const float *dt, const float *A,
                              const float *D, float *y, void *stream)
{
    const rssm_status s = check_shape(cfg);
    if (s != RSSM_OK) return s;
    const int bt = cfg->batch;
    if (!ok_ptr(state, bt) || !ok_ptr(x, bt) || !ok_ptr(B, bt) || !ok_ptr(C, bt) || !ok_ptr(dt, bt) ||
        !ok_ptr(y, bt))
        return RSSM_E_INVAL;
    if (!A || !D || !aligned(A, 4) || !aligned(D, 4)) return RSSM_E_INVAL;
    if (cfg->batch == 0) return RSSM_OK;
    const Layer Ld = shape_layer(*cfg, A, D);
    const TokenIO io{x, B, C, dt, y};
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) launch_conventional_n##NV(Ld, state, io, st)
    RSSM_BY_N(cfg->dstate, CALL)
#undef CALL
}

rssm_status conventional_mixer_step(const replayssm_config *cfg, float *state, float *conv_ring, int32_t t,
                                    const float *xbc, const float *z, const float *dt_raw, const float *A,
                                    const float *D, const float *conv_w, const float *conv_b,
                                    const float *dt_bias, float *o, void *stream)
{
    const rssm_status s = check_shape(cfg);
    if (s != RSSM_OK) return s;
    if (cfg->d_conv < 2) return RSSM_E_INVAL;
    if (cfg->d_conv > 4) return RSSM_E_UNSUPPORTED;
    if (t < 0) return RSSM_E_INVAL;
    const int bt = cfg->batch;
    if (!ok_ptr(state, bt) || !ok_ptr4(conv_ring, bt) || !ok_ptr4(xbc, bt) || !ok_ptr4(z, bt) ||
        !ok_ptr4(dt_raw, bt) || !ok_ptr4(o, bt))
        return RSSM_E_INVAL;
    if (!A || !D || !conv_w || !conv_b || !dt_bias || !aligned(A, 4) || !aligned(D, 4) || !aligned(conv_w, 4) ||
        !aligned(conv_b, 4) || !aligned(dt_bias, 4))
        return RSSM_E_INVAL;
    if (cfg->batch == 0) return RSSM_OK;
    Layer Ld = shape_layer(*cfg, A, D);
    Ld.conv_ring = conv_ring;
    Ld.conv_w = conv_w;
    Ld.conv_b = conv_b;
    Ld.dt_bias = dt_bias;
    Ld.K = Ld.R = cfg->d_conv;
    Ld.CD = (int)conv_dim(*cfg);
    Ld.wvec = cfg->d_conv == 4 && aligned(conv_w, 16);
    const TokenIO io{nullptr, nullptr, nullptr, dt_raw, o, xbc, z};
    const int rslot = t % cfg->d_conv;
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) launch_conventional_mixer_n##NV(Ld, state, io, rslot, st)
    RSSM_BY_N(cfg->dstate, CALL)
#undef CALL
}

rssm_status snapshot_spec_verify(const replayssm_config *cfg, float *slots, const int32_t *cur,
                                 int32_t T, const float *x, const float *B, const float *C,
                                 const float *dt, const float *A, const float *D, float *y,
                                 void *stream)
{
    const rssm_status s = check_shape(cfg);
    if (s != RSSM_OK) return s;
    if (T < 1 || T > 8) return RSSM_E_INVAL;
    const int bt = cfg->batch;
    if (!ok_ptr(slots, bt) || !ok_ptr4(cur, bt) || !ok_ptr(x, bt) || !ok_ptr(B, bt) || !ok_ptr(C, bt) ||
        !ok_ptr(dt, bt) || !ok_ptr(y, bt))
        return RSSM_E_INVAL;
    if (!A || !D || !aligned(A, 4) || !aligned(D, 4)) return RSSM_E_INVAL;
    if (cfg->batch == 0) return RSSM_OK;
    const Layer Ld = shape_layer(*cfg, A, D);
    const TokenIO io{x, B, C, dt, y};
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) launch_snapshot_n##NV(Ld, slots, cur, T, io, st)
    RSSM_BY_N(cfg->dstate, CALL)
#undef CALL
}

rssm_status snapshot_commit(const replayssm_config *cfg, int32_t *cur, const int32_t *accepted,
                            int32_t T, void *stream)
{
    const rssm_status s = check_shape(cfg);
    if (s != RSSM_OK) return s;
    if (T < 1 || T > 8) return RSSM_E_INVAL;
    if (!ok_ptr4(cur, cfg->batch) || !ok_ptr4(accepted, cfg->batch)) return RSSM_E_INVAL;
    if (cfg->batch == 0) return RSSM_OK;
    return hip_status(launch_snapshot_commit(cur, accepted, T, cfg->batch, (hipStream_t)stream));
}

rssm_status snapshot_spec_step(const replayssm_config *cfg, float *slots, int32_t *cur, int32_t T,
                               const float *x, const float *B, const float *C, const float *dt,
                               const float *A, const float *D, float *y, const int32_t *accepted,
                               void *stream)
{
    // every argument check of both halves before the first launch
    const rssm_status s = check_shape(cfg);
    if (s != RSSM_OK) return s;
    if (T < 1 || T > 8) return RSSM_E_INVAL;
    if (!ok_ptr4(accepted, cfg->batch)) return RSSM_E_INVAL;
    const rssm_status v = snapshot_spec_verify(cfg, slots, cur, T, x, B, C, dt, A, D, y, stream);
    if (v != RSSM_OK) return v;
    return snapshot_commit(cfg, cur, accepted, T, stream);
}

const char *replayssm_status_string(rssm_status s)
{
    switch (s) {
    case RSSM_OK: return "ok";
    case RSSM_E_INVAL: return "invalid argument, pointer, alignment or shape";
    case RSSM_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case RSSM_E_HIP: return "HIP runtime error";
    case RSSM_E_STATE: return "state-machine misuse or device invariant flag set";
    case RSSM_E_UNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
    }
}

}  // extern "C"
