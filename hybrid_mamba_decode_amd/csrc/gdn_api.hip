// gdn_api.hip -- the C ABI of gdnreplay.h: argument and state-machine validation, workspace
// layout, the host-side flush hint, and kernel dispatch by key size Dk. Every host-checkable
// error is reported before any HIP call (argument errors before state errors).
#include "../../include/gdnreplay.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>

#include "gdn_launch.h"
#include "host_state.h"

using namespace rssm;

struct gdnreplay_layer {
    gdnreplay_config cfg;
    gdnreplay_layout lay;
    GLayer dev;
    int lmax;      // window bucket of the kernel instances (16, 32 or 64)
    HostState hs;  // host state machine (host_state.h), as for the Mamba-2 handle
};

namespace {

bool supported_dk(int n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }
int psplit_of(const gdnreplay_config &c) { return (c.dv + kRows - 1) / kRows; }

rssm_status check_shape(const gdnreplay_config *c)
{
    if (!c) return RSSM_E_INVAL;
    if (c->batch < 0 || c->nheads <= 0 || c->nkheads <= 0 || c->dv <= 0 || c->dk <= 0) return RSSM_E_INVAL;
    if (c->nheads % c->nkheads || c->dv % 4) return RSSM_E_INVAL;
    if (!supported_dk(c->dk) || c->dv > 256) return RSSM_E_UNSUPPORTED;
    const uint64_t blocks = (uint64_t)c->batch * c->nheads * psplit_of(*c);
    if (blocks * kThreads >= (1ull << 32)) return RSSM_E_UNSUPPORTED;
    return RSSM_OK;
}

rssm_status check_config(const gdnreplay_config *c)
{
    const rssm_status s = check_shape(c);
    if (s != RSSM_OK) return s;
    if (c->buffer_len < 1 || c->max_draft < 1 || c->max_draft > c->buffer_len) return RSSM_E_INVAL;
    if (c->buffer_len > 64 || c->max_draft > 8) return RSSM_E_UNSUPPORTED;
    if (c->read_prec < RSSM_READ_FP32 || c->read_prec > RSSM_READ_MXFP4) return RSSM_E_INVAL;
    if (c->read_prec == RSSM_READ_MXFP4 && c->dk < 32) return RSSM_E_UNSUPPORTED;  // blocks of 32 key columns
    return RSSM_OK;
}

void make_layout(const gdnreplay_config &c, gdnreplay_layout *L)
{
    const size_t Bt = (size_t)c.batch, H = c.nheads, G = c.nkheads, Dv = c.dv, Dk = c.dk, Lb = c.buffer_len;
    RegionCarver rc;
    auto take = [&](size_t bytes) { return rc.take(bytes); };
    const size_t elems = Bt * H * Dv * Dk;
    const int rp = c.read_prec;
    L->master = take(elems * 4);
    L->read_copy = take(rp == RSSM_READ_BF16 ? elems * 2 : rp == RSSM_READ_FP8_E4M3 ? elems
                        : rp == RSSM_READ_MXFP4 ? elems / 2 : 0);
    L->scale = take(rp == RSSM_READ_FP8_E4M3 ? Bt * H * psplit_of(c) * 4 : rp == RSSM_READ_MXFP4 ? elems / 32 : 0);
    L->ring_k = take(Bt * G * Lb * Dk * 4);
    L->ring_v = take(Bt * H * Lb * Dv * 4);
    L->ring_a = take(Bt * H * Lb * 4);
    L->ring_b = take(Bt * H * Lb * 4);
    L->pos = take(Bt * 4);
    L->ckpt_pos = take(Bt * 4);
    L->counters = take(Bt * 4);
    L->flag = take(4);
    L->total = rc.off;
}

// A GLayer carrying shapes only, for the baselines.
GLayer shape_layer(const gdnreplay_config &c)
{
    GLayer L;
    std::memset(&L, 0, sizeof(L));
    L.Bt = c.batch;
    L.H = c.nheads;
    L.Dv = c.dv;
    L.G = c.nkheads;
    L.L = 1;
    L.Tmax = 1;
    L.hpg = c.nheads / c.nkheads;
    L.psplit = psplit_of(c);
    return L;
}

#define GDN_BY_N(NV, CALL)                  \
    switch (NV) {                           \
    case 16: return hip_status(CALL(16));   \
    case 32: return hip_status(CALL(32));   \
    case 64: return hip_status(CALL(64));   \
    case 128: return hip_status(CALL(128)); \
    case 256: return hip_status(CALL(256)); \
    default: return RSSM_E_UNSUPPORTED;     \
    }

rssm_status ready(gdnreplay_t h)
{
    if (!h) return RSSM_E_INVAL;
    return h->hs.ready();
}

rssm_status read_flag(gdnreplay_t h, hipStream_t st) { return h->hs.read_flag(h->dev.flag, h->cfg.batch, st); }

bool ok_io(int bt, const float *q, const float *k, const float *v, const float *a, const float *b, const float *o)
{
    return ok_ptr(q, bt) && ok_ptr(k, bt) && ok_ptr(v, bt) && ok_ptr(a, bt) && ok_ptr(b, bt) && ok_ptr(o, bt);
}

}  // namespace

extern "C" {

size_t gdnreplay_workspace_bytes(const gdnreplay_config *cfg)
{
    if (check_config(cfg) != RSSM_OK) return 0;
    gdnreplay_layout L;
    make_layout(*cfg, &L);
    return L.total;
}

rssm_status gdnreplay_workspace_layout(const gdnreplay_config *cfg, gdnreplay_layout *out)
{
    const rssm_status s = check_config(cfg);
    if (s != RSSM_OK) return s;
    if (!out) return RSSM_E_INVAL;
    make_layout(*cfg, out);
    return RSSM_OK;
}

rssm_status gdnreplay_create(const gdnreplay_config *cfg, void *workspace, size_t bytes, gdnreplay_t *out)
{
    if (!out) return RSSM_E_INVAL;
    *out = nullptr;
    const rssm_status s = check_config(cfg);
    if (s != RSSM_OK) return s;
    gdnreplay_layout lay;
    make_layout(*cfg, &lay);
    if (!workspace || !aligned(workspace, kWsAlign) || bytes < lay.total) return RSSM_E_WORKSPACE;
    gdnreplay_layer *h = new (std::nothrow) gdnreplay_layer();
    if (!h) return RSSM_E_INVAL;
    h->cfg = *cfg;
    h->hs.init(cfg->buffer_len, cfg->max_draft);
    h->lay = lay;
    char *ws = (char *)workspace;
    GLayer &d = h->dev;
    d.master = (float *)(ws + lay.master);
    static_assert(PREC_BF16 == RSSM_READ_BF16 && PREC_FP8 == RSSM_READ_FP8_E4M3 && PREC_FP4 == RSSM_READ_MXFP4,
                  "read precisions map onto the kernels' codes");
    d.rprec = cfg->read_prec;
    d.rcopy = d.rprec ? (void *)(ws + lay.read_copy) : nullptr;
    d.scale = d.rprec == PREC_FP8 ? (float *)(ws + lay.scale) : nullptr;
    d.mxscale = d.rprec == PREC_FP4 ? (unsigned char *)(ws + lay.scale) : nullptr;
    d.ring_k = (float *)(ws + lay.ring_k);
    d.ring_v = (float *)(ws + lay.ring_v);
    d.ring_a = (float *)(ws + lay.ring_a);
    d.ring_b = (float *)(ws + lay.ring_b);
    d.pos = (int *)(ws + lay.pos);
    d.ckpt = (int *)(ws + lay.ckpt_pos);
    d.counter = (unsigned *)(ws + lay.counters);
    d.flag = (unsigned *)(ws + lay.flag);
    d.Bt = cfg->batch;
    d.H = cfg->nheads;
    d.Dv = cfg->dv;
    d.G = cfg->nkheads;
    d.L = cfg->buffer_len;
    d.Tmax = cfg->max_draft;
    d.hpg = cfg->nheads / cfg->nkheads;
    d.psplit = psplit_of(*cfg);
    h->lmax = cfg->buffer_len <= 16 ? 16 : cfg->buffer_len <= 32 ? 32 : 64;
    *out = h;
    return RSSM_OK;
}

rssm_status gdnreplay_destroy(gdnreplay_t h)
{
    delete h;
    return RSSM_OK;
}

rssm_status gdnreplay_load_state(gdnreplay_t h, const float *state, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!ok_ptr(state, h->cfg.batch)) return RSSM_E_INVAL;
    h->hs.on_load(true);
    if (h->cfg.batch == 0) return RSSM_OK;
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) gdn_launch_load_n##NV(h->dev, state, st)
    GDN_BY_N(h->cfg.dk, CALL)
#undef CALL
}

rssm_status gdnreplay_step(gdnreplay_t h, const float *q, const float *k, const float *v, const float *alpha,
                           const float *beta, float *o, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!ok_io(h->cfg.batch, q, k, v, alpha, beta, o)) return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->hs.pending_T) return RSSM_E_STATE;
    const StepPlan p = h->hs.begin_step();
    const Lockstep ls{p.pslot, p.cslot, p.k};
    if (h->cfg.batch == 0) return RSSM_OK;
    const GTokenIO io{q, k, v, alpha, beta, o};
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) gdn_launch_step_n##NV(h->lmax, h->dev, io, p.flush_capable, p.all_flush, ls, st)
    GDN_BY_N(h->cfg.dk, CALL)
#undef CALL
}

rssm_status gdnreplay_flush(gdnreplay_t h, const int32_t *seq_mask, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (seq_mask && !aligned(seq_mask, 4)) return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->hs.pending_T) return RSSM_E_STATE;
    h->hs.on_flush(seq_mask != nullptr);
    if (h->cfg.batch == 0) return RSSM_OK;
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) gdn_launch_flush_n##NV(h->lmax, h->dev, MODE_MASK, seq_mask, 0, nullptr, st)
    GDN_BY_N(h->cfg.dk, CALL)
#undef CALL
}

rssm_status gdnreplay_spec_verify(gdnreplay_t h, int32_t T, const float *q, const float *k, const float *v,
                                  const float *alpha, const float *beta, float *o, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (T < 1 || T > h->cfg.max_draft) return RSSM_E_INVAL;
    if (!ok_io(h->cfg.batch, q, k, v, alpha, beta, o)) return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->hs.pending_T) return RSSM_E_STATE;
    h->hs.pending_T = T;
    if (h->cfg.batch == 0) return RSSM_OK;
    const GTokenIO io{q, k, v, alpha, beta, o};
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) gdn_launch_verify_n##NV(h->lmax, h->dev, io, T, st)
    GDN_BY_N(h->cfg.dk, CALL)
#undef CALL
}

rssm_status gdnreplay_rollback(gdnreplay_t h, const int32_t *accepted, void *stream)
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
#define CALL(NV) gdn_launch_flush_n##NV(h->lmax, h->dev, MODE_OVERFULL, accepted, T, nullptr, st)
    GDN_BY_N(h->cfg.dk, CALL)
#undef CALL
}

rssm_status gdnreplay_set_lockstep(gdnreplay_t h, int enable)
{
    if (!h || (enable != 0 && enable != 1)) return RSSM_E_INVAL;
    h->hs.set_lockstep(enable);
    return RSSM_OK;
}

rssm_status gdnreplay_get_pointers(gdnreplay_t h, int32_t *pos, int32_t *ckpt_pos, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!h->hs.loaded) return RSSM_E_STATE;
    const rssm_status s = read_flag(h, (hipStream_t)stream);
    if (s != RSSM_OK) return s;
    const size_t bytes = (size_t)h->cfg.batch * sizeof(int32_t);
    if (bytes == 0) return RSSM_OK;
    if (pos && hipMemcpy(pos, h->dev.pos, bytes, hipMemcpyDeviceToHost) != hipSuccess) return RSSM_E_HIP;
    if (ckpt_pos && hipMemcpy(ckpt_pos, h->dev.ckpt, bytes, hipMemcpyDeviceToHost) != hipSuccess) return RSSM_E_HIP;
    return RSSM_OK;
}

rssm_status gdnreplay_check(gdnreplay_t h, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!h->hs.loaded || h->hs.poisoned) return RSSM_E_STATE;
    return read_flag(h, (hipStream_t)stream);
}

rssm_status gdnreplay_materialize_state(gdnreplay_t h, float *out, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!ok_ptr(out, h->cfg.batch)) return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->cfg.batch == 0) return RSSM_OK;
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) gdn_launch_flush_n##NV(h->lmax, h->dev, MODE_MATERIALIZE, nullptr, 0, out, st)
    GDN_BY_N(h->cfg.dk, CALL)
#undef CALL
}

rssm_status gdn_conventional_step(const gdnreplay_config *cfg, float *state, const float *q, const float *k,
                                  const float *v, const float *alpha, const float *beta, float *o, void *stream)
{
    const rssm_status s = check_shape(cfg);
    if (s != RSSM_OK) return s;
    if (!ok_ptr(state, cfg->batch) || !ok_io(cfg->batch, q, k, v, alpha, beta, o)) return RSSM_E_INVAL;
    if (cfg->batch == 0) return RSSM_OK;
    const GLayer Ld = shape_layer(*cfg);
    const GTokenIO io{q, k, v, alpha, beta, o};
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) gdn_launch_conventional_n##NV(Ld, state, io, st)
    GDN_BY_N(cfg->dk, CALL)
#undef CALL
}

rssm_status gdn_snapshot_spec_verify(const gdnreplay_config *cfg, float *slots, const int32_t *cur, int32_t T,
                                     const float *q, const float *k, const float *v, const float *alpha,
                                     const float *beta, float *o, void *stream)
{
    const rssm_status s = check_shape(cfg);
    if (s != RSSM_OK) return s;
    if (T < 1 || T > 8) return RSSM_E_INVAL;
    if (!ok_ptr(slots, cfg->batch) || !ok_ptr4(cur, cfg->batch) || !ok_io(cfg->batch, q, k, v, alpha, beta, o))
        return RSSM_E_INVAL;
    if (cfg->batch == 0) return RSSM_OK;
    const GLayer Ld = shape_layer(*cfg);
    const GTokenIO io{q, k, v, alpha, beta, o};
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) gdn_launch_snapshot_n##NV(Ld, slots, cur, T, io, st)
    GDN_BY_N(cfg->dk, CALL)
#undef CALL
}

}  // extern "C"
