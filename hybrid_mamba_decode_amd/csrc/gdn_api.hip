// gdn_api.hip -- the C ABI of gdnreplay.h: argument and state-machine validation, workspace
// layout, the host-side flush hint, and kernel dispatch by key size Dk. Every host-checkable
// error is reported before any HIP call (argument errors before state errors).
#include "../../include/gdnreplay.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>

#include "gdn_launch.h"

using namespace rssm;

struct gdnreplay_layer {
    gdnreplay_config cfg;
    gdnreplay_layout lay;
    GLayer dev;
    int lmax;       // window bucket of the kernel instances (16, 32 or 64)
    int loaded;     // gdnreplay_load_state has run
    int poisoned;   // device flag observed: refuse work until the next load
    int pending_T;  // drafts of an unresolved verify, else 0
    // Bounds on the pending-record count over all sequences: they only choose whether a step
    // launch may meet a flush (the device decides each flush per sequence).
    int cmin, cmax;
    // Lockstep: after a load, standard steps and unmasked flushes keep every sequence at the same
    // window position (pos mod L, ckpt_pos mod L, pending count), tracked here and passed to the
    // step kernel; a rollback or masked flush ends it until the next load.
    int uni, pslot, cslot, lcount;
    int lockstep_ok;
};

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool ok_ptr(const void *p, int batch) { return p ? aligned(p, 16) : batch == 0; }
bool ok_ptr4(const void *p, int batch) { return p ? aligned(p, 4) : batch == 0; }
bool supported_dk(int n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }
int psplit_of(const gdnreplay_config &c) { return (c.dv + kRows - 1) / kRows; }
rssm_status hip_status(hipError_t e) { return e == hipSuccess ? RSSM_OK : RSSM_E_HIP; }

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
    if (c->read_prec != RSSM_READ_FP32 && c->read_prec != RSSM_READ_BF16) return RSSM_E_INVAL;
    return RSSM_OK;
}

void make_layout(const gdnreplay_config &c, gdnreplay_layout *L)
{
    const size_t Bt = (size_t)c.batch, H = c.nheads, G = c.nkheads, Dv = c.dv, Dk = c.dk, Lb = c.buffer_len;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    L->master = take(Bt * H * Dv * Dk * 4);
    L->read_copy = take(c.read_prec == RSSM_READ_BF16 ? Bt * H * Dv * Dk * 2 : 0);
    L->ring_k = take(Bt * G * Lb * Dk * 4);
    L->ring_v = take(Bt * H * Lb * Dv * 4);
    L->ring_a = take(Bt * H * Lb * 4);
    L->ring_b = take(Bt * H * Lb * 4);
    L->pos = take(Bt * 4);
    L->ckpt_pos = take(Bt * 4);
    L->counters = take(Bt * 4);
    L->flag = take(4);
    L->total = off;
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
    if (!h->loaded || h->poisoned) return RSSM_E_STATE;
    return RSSM_OK;
}

void commit_bounds(gdnreplay_t h, int lo, int hi)
{
    const int lim = h->cfg.buffer_len - h->cfg.max_draft;
    const int nmin = h->cmin + lo, nmax = h->cmax + hi;
    if (nmax <= lim) {
        h->cmin = nmin;
        h->cmax = nmax;
    } else if (nmin > lim) {
        h->cmin = h->cmax = 0;
    } else {
        h->cmin = 0;
        h->cmax = lim;
    }
}

rssm_status read_flag(gdnreplay_t h, hipStream_t st)
{
    if (hipStreamSynchronize(st) != hipSuccess) return RSSM_E_HIP;
    unsigned flag = 0;
    if (h->cfg.batch > 0 && hipMemcpy(&flag, h->dev.flag, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess)
        return RSSM_E_HIP;
    if (flag) {
        h->poisoned = 1;
        return RSSM_E_STATE;
    }
    return RSSM_OK;
}

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
    if (!workspace || !aligned(workspace, kAlign) || bytes < lay.total) return RSSM_E_WORKSPACE;
    gdnreplay_layer *h = new (std::nothrow) gdnreplay_layer;
    if (!h) return RSSM_E_INVAL;
    std::memset(h, 0, sizeof(*h));
    h->cfg = *cfg;
    h->lay = lay;
    char *ws = (char *)workspace;
    GLayer &d = h->dev;
    d.master = (float *)(ws + lay.master);
    d.rprec = cfg->read_prec == RSSM_READ_BF16 ? 1 : 0;
    d.rcopy = d.rprec ? (unsigned short *)(ws + lay.read_copy) : nullptr;
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
    h->lockstep_ok = 1;
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
    h->loaded = 1;
    h->poisoned = 0;
    h->pending_T = 0;
    h->cmin = h->cmax = 0;
    h->uni = h->lockstep_ok;
    h->pslot = h->cslot = h->lcount = 0;
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
    if (h->pending_T) return RSSM_E_STATE;
    const int lim = h->cfg.buffer_len - h->cfg.max_draft;
    bool flush_capable = h->cmax + 1 > lim;
    Lockstep ls{0, 0, 0};
    if (h->uni) {
        ls = Lockstep{h->pslot, h->cslot, h->lcount + 1};
        flush_capable = h->lcount + 1 > lim;  // every sequence flushes, or none does
        h->pslot = (h->pslot + 1) % h->cfg.buffer_len;
        if (flush_capable) {
            h->lcount = 0;
            h->cslot = h->pslot;
        } else {
            h->lcount += 1;
        }
    }
    commit_bounds(h, 1, 1);
    if (h->cfg.batch == 0) return RSSM_OK;
    const GTokenIO io{q, k, v, alpha, beta, o};
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) gdn_launch_step_n##NV(h->lmax, h->dev, io, flush_capable, ls, st)
    GDN_BY_N(h->cfg.dk, CALL)
#undef CALL
}

rssm_status gdnreplay_flush(gdnreplay_t h, const int32_t *seq_mask, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (seq_mask && !aligned(seq_mask, 4)) return RSSM_E_INVAL;
    rssm_status s = ready(h);
    if (s != RSSM_OK) return s;
    if (h->pending_T) return RSSM_E_STATE;
    if (!seq_mask) {
        h->cmin = h->cmax = 0;
        h->lcount = 0;
        h->cslot = h->pslot;
    } else {
        h->cmin = 0;
        h->uni = 0;
    }
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
    if (h->pending_T) return RSSM_E_STATE;
    h->pending_T = T;
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
    if (!h->pending_T) return RSSM_E_STATE;
    const int T = h->pending_T;
    h->pending_T = 0;
    h->uni = 0;
    commit_bounds(h, 0, T);
    if (h->cfg.batch == 0) return RSSM_OK;
    const hipStream_t st = (hipStream_t)stream;
#define CALL(NV) gdn_launch_flush_n##NV(h->lmax, h->dev, MODE_OVERFULL, accepted, T, nullptr, st)
    GDN_BY_N(h->cfg.dk, CALL)
#undef CALL
}

rssm_status gdnreplay_set_lockstep(gdnreplay_t h, int enable)
{
    if (!h || (enable != 0 && enable != 1)) return RSSM_E_INVAL;
    h->lockstep_ok = enable;
    if (!enable) h->uni = 0;
    return RSSM_OK;
}

rssm_status gdnreplay_get_pointers(gdnreplay_t h, int32_t *pos, int32_t *ckpt_pos, void *stream)
{
    if (!h) return RSSM_E_INVAL;
    if (!h->loaded) return RSSM_E_STATE;
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
    if (!h->loaded || h->poisoned) return RSSM_E_STATE;
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
