// host_state.h -- the host side of a layer handle's state machine, shared by the Mamba-2
// (replayssm.h) and Gated DeltaNet (gdnreplay.h) C ABIs: argument helpers, workspace carving, the
// loaded / poisoned / pending-verify flags, the flush hint and lockstep tracking, and the device
// flag read. Host code only; nothing here launches a kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/replayssm.h"

namespace rssm {

constexpr size_t kWsAlign = 256;  // workspace and region alignment

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
// Device array arguments: non-NULL and aligned; with batch 0 (empty arrays) NULL is accepted too.
inline bool ok_ptr(const void *p, int batch) { return p ? aligned(p, 16) : batch == 0; }
inline bool ok_ptr4(const void *p, int batch) { return p ? aligned(p, 4) : batch == 0; }
inline rssm_status hip_status(hipError_t e) { return e == hipSuccess ? RSSM_OK : RSSM_E_HIP; }

// Consecutive workspace regions, each starting on a kWsAlign boundary.
struct RegionCarver {
    size_t off = 0;
    size_t take(size_t bytes)
    {
        const size_t at = off;
        off = (off + bytes + kWsAlign - 1) / kWsAlign * kWsAlign;
        return at;
    }
};

// What the next standard step launch must be able to do, from the host's knowledge alone.
struct StepPlan {
    bool flush_capable;  // some sequence may flush in this launch
    bool all_flush;      // every sequence flushes in this launch
    int pslot, cslot, k; // lockstep window position (k = records incl. this token); k = 0: the
                         // kernels read each sequence's device pointers
    int upos;            // lockstep: the common pos before this step
};

struct HostState {
    int L = 1, Tmax = 1;   // buffer length, maximum drafts
    int loaded = 0;        // load_state has run
    int poisoned = 0;      // device flag observed: refuse work until the next load
    int pending_T = 0;     // drafts of an unresolved verify, else 0
    // Bounds on the pending-record count over all sequences: exact for lockstep decoding,
    // conservative otherwise. They only select kernel variants; the device decides each flush
    // per sequence.
    int cmin = 0, cmax = 0;
    // Lockstep: after a load, standard steps and unmasked flushes keep every sequence at the same
    // window position (pos mod L, ckpt_pos mod L, pending count), tracked here and passed to the
    // kernels as arguments; a rollback or a masked flush makes sequences diverge.
    int uni = 0, pslot = 0, cslot = 0, lcount = 0, upos = 0;
    int lockstep_ok = 1;   // set_lockstep: the fast path may be used at all

    void init(int buffer_len, int max_draft)
    {
        *this = HostState();
        L = buffer_len;
        Tmax = max_draft;
    }

    int limit() const { return L - Tmax; }  // a sequence flushes when more records are pending

    rssm_status ready() const { return (!loaded || poisoned) ? RSSM_E_STATE : RSSM_OK; }

    // A load: every sequence at pos = ckpt_pos = 0, no verify pending, the flag cleared.
    void on_load(bool lockstep_allowed)
    {
        loaded = 1;
        poisoned = 0;
        pending_T = 0;
        cmin = cmax = 0;
        uni = lockstep_ok && lockstep_allowed;
        pslot = cslot = lcount = upos = 0;
    }

    // Bounds after every sequence commits lo..hi more records and those with more than
    // L - Tmax pending flush.
    void commit_bounds(int lo, int hi)
    {
        const int lim = limit();
        const int nmin = cmin + lo, nmax = cmax + hi;
        if (nmax <= lim) {
            cmin = nmin;
            cmax = nmax;
        } else if (nmin > lim) {
            cmin = cmax = 0;
        } else {
            cmin = 0;
            cmax = lim;
        }
    }

    // One standard step: its launch plan, and the state after it.
    StepPlan begin_step()
    {
        const int lim = limit();
        StepPlan p{cmax + 1 > lim, cmin + 1 > lim, 0, 0, 0, 0};
        if (uni) {
            p.pslot = pslot;
            p.cslot = cslot;
            p.k = lcount + 1;
            p.upos = upos;
            p.flush_capable = p.all_flush = lcount + 1 > lim;  // every sequence flushes, or none does
            upos += 1;
            pslot = (pslot + 1) % L;
            if (p.flush_capable) {
                lcount = 0;
                cslot = pslot;
            } else {
                lcount += 1;
            }
        }
        commit_bounds(1, 1);
        return p;
    }

    // An explicit flush of all sequences (masked = false) or of a subset.
    void on_flush(bool masked)
    {
        if (!masked) {
            cmin = cmax = 0;
            lcount = 0;
            cslot = pslot;
        } else {
            cmin = 0;
            uni = 0;
        }
    }

    // Resolving a verify of T drafts: pointers move by per-sequence counts, lockstep ends.
    void on_rollback(int T)
    {
        pending_T = 0;
        uni = 0;
        commit_bounds(0, T);
    }

    void set_lockstep(int enable)
    {
        lockstep_ok = enable;
        if (!enable) uni = 0;
    }

    // Synchronize the stream and read the device flag (batch > 0); a set flag poisons the handle.
    rssm_status read_flag(const unsigned *dflag, int batch, hipStream_t st)
    {
        if (hipStreamSynchronize(st) != hipSuccess) return RSSM_E_HIP;
        unsigned flag = 0;
        if (batch > 0 && hipMemcpy(&flag, dflag, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess)
            return RSSM_E_HIP;
        if (flag) {
            poisoned = 1;
            return RSSM_E_STATE;
        }
        return RSSM_OK;
    }
};

}  // namespace rssm
