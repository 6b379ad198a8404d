"""Secondary benchmark workloads (each prints JSON lines; the headline line is bench.py's default).

spec:  speculative decode on the serving layer -- batch 512, T = 4 drafts, accepted prefix uniform
       in {0..4} per sequence (seeded), 128 verify steps. Buffer-pointer rollback (verify launch +
       rollback/commit-flush launch) against per-draft state snapshots (verify-with-snapshots launch
       + commit launch), same inputs, same stream.
gdn:   a Gated DeltaNet layer (32 value heads, 16 key heads, Dv = Dk = 128) at batch 256, L = 16:
       the replay step (non-flush and flush launches, 256 steps = 16 windows) against the
       conventional step, and speculative decode at batch 512, T = 4 against per-draft snapshots.
mixer: the serving layer with the Mamba-2 mixer edges fused (conv1d width 4 over xBC, softplus
       dt, output gate), batch 256, L = 16: the fused mixer step (256 steps = 16 windows) against
       the plain replay step on precomputed x, B, C, dt and the conventional step with the same
       fused edges.
sweep: the serving head shape stacked as 10 independent layers, batch in {1, 8, 64, 256, 512} x
       buffer length in {4, 8, 16, 32}, 64 decode steps: per-layer tokens/s of the replay step
       (amortized over whole windows) and of the conventional step, eager and as HIP graphs
       (a captured window of L steps x 10 layers), the flush-step time per layer, and the
       crossover batch.

States and per-step inputs are drawn on the GPU from a seeded torch generator with the layer
definition's distributions (x ~ N(0,1); B, C ~ N(0, 1/N); dt = softplus(N(0,1) - 4); S0 ~ N(0,1)),
so that large stacks are set up in seconds.
"""
import json
import time

import numpy as np
import torch

import hybrid_mamba_decode_amd as rs
from hybrid_mamba_decode_amd import traffic
import workload

H, P, N, G = 128, 64, 128, 8
PEAK = 8000.0


def _gen(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _tokens(g, lead, n):
    x = torch.randn(*lead, H, P, device="cuda", generator=g)
    B = torch.randn(*lead, G, N, device="cuda", generator=g) / n ** 0.5
    C = torch.randn(*lead, G, N, device="cuda", generator=g) / n ** 0.5
    dt = torch.nn.functional.softplus(torch.randn(*lead, H, device="cuda", generator=g) - 4.0)
    return x, B, C, dt


def _layer_params():
    A, D = workload.layer_params(workload.config_seed(1), H)
    return torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()


def _calib_copy():
    """Counter calibration: a plain kernel that reads exactly 1 GiB and writes exactly 1 GiB."""
    a = torch.ones(1 << 28, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def _timed(fn, reps):
    st = torch.cuda.current_stream()
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(reps):
        e0[r].record(st)
        fn(r)
        e1[r].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, np.array([e0[r].elapsed_time(e1[r]) * 1e-3 for r in range(reps)])


def spec(args):
    Bt, T, L, iters = 512, 4, 16, 128
    A, D = _layer_params()
    g = _gen(3007)
    S0 = torch.randn(Bt, H, P, N, device="cuda", generator=g)
    pool = [_tokens(g, (Bt, T), N) for _ in range(8)]
    acc = torch.from_numpy(np.stack([workload.accepted_counts(workload.config_seed(3), it, Bt, T)
                                     for it in range(iters)])).cuda()
    y = torch.empty(Bt, T, H, P, device="cuda")
    lay = rs.ReplaySSM(Bt, H, P, N, G, A, D, buffer_len=L, max_draft=T)
    ev = {"verify": [], "rollback": []}
    st = torch.cuda.current_stream()

    def run_replay(warm):
        lay.load_state(S0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        marks = []
        for it in range(iters):
            x, B, C, dt = pool[it % len(pool)]
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(st)
            rs.replayssm_spec_verify(lay.handle, T, x, B, C, dt, y)
            e[1].record(st)
            rs.replayssm_rollback(lay.handle, acc[it])
            e[2].record(st)
            marks.append(e)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, marks

    run_replay(True)
    wall_r, marks = run_replay(False)
    assert lay.check() == rs.RSSM_OK
    tv = np.array([m[0].elapsed_time(m[1]) for m in marks]) * 1e-3
    tr = np.array([m[1].elapsed_time(m[2]) for m in marks]) * 1e-3
    accepted = int(acc.sum().item())
    # per-draft snapshot baseline
    cfg = rs.make_config(Bt, H, P, N, G)
    slots = torch.empty(Bt, T + 1, H, P, N, device="cuda")
    slots[:, 0].copy_(S0)
    cur = torch.zeros(Bt, dtype=torch.int32, device="cuda")

    def run_snap():
        cur.zero_()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        marks = []
        for it in range(iters):
            x, B, C, dt = pool[it % len(pool)]
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(st)
            rs.snapshot_spec_verify(cfg, slots, cur, T, x, B, C, dt, A, D, y)
            e[1].record(st)
            rs.snapshot_commit(cfg, cur, acc[it], T)
            e[2].record(st)
            marks.append(e)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, marks

    run_snap()
    wall_s, smarks = run_snap()
    sv = np.array([m[0].elapsed_time(m[1]) for m in smarks]) * 1e-3
    # verify bytes at the mean committed window (k_old ~ count before verify)
    snap_bytes = traffic.snapshot_verify(H, P, N, G, T) * Bt
    out = {
        "workload": "spec decode, serving layer, batch 512, T=4, accepted ~ U{0..4}, 128 verify steps, fp32",
        "replay": {"verify_steps_per_s": round(iters / wall_r, 1),
                   "accepted_tokens_per_s_layer": round(accepted / wall_r, 1),
                   "verify_mean_us": round(tv.mean() * 1e6, 2),
                   "verify_gbps_at_state_read": round(traffic.verify(H, P, N, G, T, 0) * Bt / tv.mean() / 1e9, 1),
                   "rollback_mean_us": round(tr.mean() * 1e6, 2),
                   "rollback_max_us": round(tr.max() * 1e6, 2)},
        "snapshot": {"verify_steps_per_s": round(iters / wall_s, 1),
                     "accepted_tokens_per_s_layer": round(accepted / wall_s, 1),
                     "verify_mean_us": round(sv.mean() * 1e6, 2),
                     "gbps": round(snap_bytes / sv.mean() / 1e9, 1),
                     "state_memory_gib": round(slots.numel() * 4 / 2 ** 30, 2)},
        "replay_state_memory_gib": round(lay.workspace.numel() / 2 ** 30, 2),
        "speedup_vs_snapshot": round(wall_s / wall_r, 3),
        "accepted_tokens": accepted,
    }
    print(json.dumps(out), flush=True)


def sweep(args):
    A, D = _layer_params()
    layers = 10
    steps = 64
    results = []
    for Bt in (1, 8, 64, 256, 512):
        g = _gen(4007 + Bt)
        states = [torch.randn(Bt, H, P, N, device="cuda", generator=g) for _ in range(layers)]
        pool = [_tokens(g, (Bt,), N) for _ in range(4)]
        y = torch.empty(Bt, H, P, device="cuda")
        # conventional: 10 independent layers per step, in place
        cfg = rs.make_config(Bt, H, P, N, G)
        cst = [s.clone() for s in states]

        def conv_step(r):
            x, B, C, dt = pool[r % len(pool)]
            for l in range(layers):
                rs.conventional_step(cfg, cst[l], x, B, C, dt, A, D, y)
        _timed(conv_step, 4)
        wall_c, _ = _timed(conv_step, steps)
        conv_tps = Bt * steps * layers / wall_c   # tokens/s per layer: each step runs every layer
        gc = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gc):
            for r in range(16):
                conv_step(r)
        gc.replay()
        wall_cg, _ = _timed(lambda r: gc.replay(), max(1, steps // 16))
        conv_graph_tps = Bt * max(1, steps // 16) * 16 * layers / wall_cg
        del gc
        del cst
        for L in (4, 8, 16, 32):
            lays = [rs.ReplaySSM(Bt, H, P, N, G, A, D, buffer_len=L) for _ in range(layers)]
            for l in range(layers):
                lays[l].load_state(states[l])

            def rep_step(r):
                x, B, C, dt = pool[r % len(pool)]
                for l in range(layers):
                    rs.replayssm_step(lays[l].handle, x, B, C, dt, y)
            _timed(rep_step, L)                      # warm one whole window
            wall_r, d = _timed(rep_step, steps)      # 64 steps = whole windows for every L
            flush_idx = [r for r in range(steps) if (r + 1) % L == 0]
            nonflush_idx = [r for r in range(steps) if (r + 1) % L != 0]
            # the same window captured once as a HIP graph (from a window boundary: the lockstep
            # arguments repeat every window, so the graph replays correctly)
            for l in range(layers):
                lays[l].load_state(states[l])
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for r in range(L):
                    rep_step(r)
            gr.replay()
            reps = max(1, steps // L)
            wall_g, _ = _timed(lambda r: gr.replay(), reps)
            graph_tps = Bt * reps * L * layers / wall_g
            rec = {"batch": Bt, "L": L, "layers": layers,
                   "replay_graph_tokens_per_s_layer": round(graph_tps, 1),
                   "conventional_graph_tokens_per_s_layer": round(conv_graph_tps, 1),
                   "speedup_graph": round(graph_tps / conv_graph_tps, 3),
                   "replay_tokens_per_s_layer": round(Bt * steps * layers / wall_r, 1),
                   "conventional_tokens_per_s_layer": round(conv_tps, 1),
                   "speedup": round((Bt * steps * layers / wall_r) / conv_tps, 3),
                   "flush_step_us_per_layer": round(float(d[flush_idx].mean()) * 1e6 / layers, 2),
                   "nonflush_step_us_per_layer": round(float(d[nonflush_idx].mean()) * 1e6 / layers, 2),
                   "replay_gbps_amortized": round(traffic.replay_window_amortized(H, P, N, G, L) * Bt * layers * steps / wall_r / 1e9, 1),
                   "working_set_mib": round(layers * lays[0].workspace.numel() / 2 ** 20, 1)}
            for l in range(layers):
                assert lays[l].check() == rs.RSSM_OK
            print(json.dumps(rec), flush=True)
            results.append(rec)
            del gr, lays
        del states
        torch.cuda.empty_cache()
    for L in (4, 8, 16, 32):
        wins = [r["batch"] for r in results if r["L"] == L and r["speedup"] > 1.0]
        print(json.dumps({"L": L, "smallest_batch_where_replay_wins": min(wins) if wins else None}), flush=True)


def _gdn_tokens(g, lead, Hv, Gk, Dv, Dk, rates):
    q = torch.nn.functional.normalize(torch.randn(*lead, Gk, Dk, device="cuda", generator=g), dim=-1)
    k = torch.nn.functional.normalize(torch.randn(*lead, Gk, Dk, device="cuda", generator=g), dim=-1)
    v = torch.randn(*lead, Hv, Dv, device="cuda", generator=g)
    alpha = torch.exp(rates * torch.nn.functional.softplus(torch.randn(*lead, Hv, device="cuda", generator=g) - 4.0))
    beta = torch.sigmoid(torch.randn(*lead, Hv, device="cuda", generator=g))
    return q, k, v, alpha, beta


def gdn(args):
    c = workload.GDN_SERVING
    Bt, Hv, Gk, Dv, Dk, L = c["Bt"], c["H"], c["G"], c["Dv"], c["Dk"], c["L"]
    rates = torch.from_numpy(workload.gdn_gate_rates(workload.config_seed(6), Hv)).float().cuda()
    g = _gen(6007)
    S0 = torch.randn(Bt, Hv, Dv, Dk, device="cuda", generator=g)
    pool = [_gdn_tokens(g, (Bt,), Hv, Gk, Dv, Dk, rates) for _ in range(8)]
    o = torch.empty(Bt, Hv, Dv, device="cuda")
    prec = args.read_prec
    lay = rs.GDNReplay(Bt, Hv, Gk, Dv, Dk, buffer_len=L, read_prec=prec)
    lay.load_state(S0)

    def rep_step(r):
        rs.gdnreplay_step(lay.handle, *pool[r % len(pool)], o)
    _timed(rep_step, 2 * L)
    steps = 16 * L
    wall, d = _timed(rep_step, steps)      # starts at a window boundary: step r has k = r % L + 1
    assert lay.check() == rs.RSSM_OK
    ks = np.array([r % L + 1 for r in range(steps)])
    fl = ks == L
    nf_bytes = np.array([traffic.gdn_replay_nonflush(Hv, Gk, Dv, Dk, int(k), prec) * Bt for k in ks[~fl]])
    fl_bytes = traffic.gdn_replay_flush_step(Hv, Gk, Dv, Dk, L, prec) * Bt
    cfg = rs.make_gdn_config(Bt, Hv, Gk, Dv, Dk)
    cst = S0.clone()

    def conv_step(r):
        rs.gdn_conventional_step(cfg, cst, *pool[r % len(pool)], o)
    _timed(conv_step, 4)
    wall_c, dc = _timed(conv_step, 64)
    conv_bytes = traffic.gdn_conventional(Hv, Gk, Dv, Dk) * Bt
    nf_gbps = float((nf_bytes / d[~fl]).mean()) / 1e9
    out = {
        "workload": f"Gated DeltaNet layer decode step, batch {Bt}, {Hv} value heads x {Gk} key heads, "
                    f"Dv {Dv}, Dk {Dk}, L {L}, fp32 checkpoint (2 MiB per sequence), {prec} reads",
        "replay": {"tokens_per_s_layer": round(Bt * steps / wall, 1),
                   "nonflush_mean_us": round(float(d[~fl].mean()) * 1e6, 2),
                   "nonflush_gbps": round(nf_gbps, 1), "nonflush_frac_of_8tbs": round(nf_gbps / PEAK, 4),
                   "nonflush_alg_bytes_per_launch": int(nf_bytes.mean()),
                   "flush_mean_us": round(float(d[fl].mean()) * 1e6, 2),
                   "flush_gbps": round(fl_bytes / float(d[fl].mean()) / 1e9, 1),
                   "nonflush_us_by_k": {int(k): round(float(d[ks == k].mean()) * 1e6, 1) for k in (1, 4, 8, 12, 15)}},
        "conventional": {"tokens_per_s_layer": round(Bt * 64 / wall_c, 1),
                         "mean_us": round(float(dc.mean()) * 1e6, 2),
                         "gbps": round(conv_bytes / float(dc.mean()) / 1e9, 1)},
        "speedup_vs_conventional": round((Bt * steps / wall) / (Bt * 64 / wall_c), 3),
    }
    print(json.dumps(out), flush=True)
    del lay, cst
    torch.cuda.empty_cache()
    if getattr(args, "calib_copy", False):
        _calib_copy()

    # speculative decode: batch 512, T = 4, accepted ~ U{0..4}
    s = workload.GDN_SPEC
    Bt, T, iters = s["Bt"], s["T"], s["steps"]
    S0 = torch.randn(Bt, Hv, Dv, Dk, device="cuda", generator=g)
    dpool = [_gdn_tokens(g, (Bt, T), Hv, Gk, Dv, Dk, rates) for _ in range(4)]
    acc = torch.from_numpy(np.stack([workload.accepted_counts(workload.config_seed(7), it, Bt, T)
                                     for it in range(iters)])).cuda()
    od = torch.empty(Bt, T, Hv, Dv, device="cuda")
    lay = rs.GDNReplay(Bt, Hv, Gk, Dv, Dk, buffer_len=L, max_draft=T, read_prec=prec)

    def spec_iter(it):
        rs.gdnreplay_spec_verify(lay.handle, T, *dpool[it % len(dpool)], od)
        rs.gdnreplay_rollback(lay.handle, acc[it])
    lay.load_state(S0)
    _timed(spec_iter, 8)
    lay.load_state(S0)
    wall_r, dr = _timed(spec_iter, iters)
    assert lay.check() == rs.RSSM_OK
    accepted = int(acc.sum().item())
    del lay
    torch.cuda.empty_cache()
    cfg = rs.make_gdn_config(Bt, Hv, Gk, Dv, Dk)
    slots = torch.empty(Bt, T + 1, Hv, Dv, Dk, device="cuda")
    slots[:, 0].copy_(S0)
    cur = torch.zeros(Bt, dtype=torch.int32, device="cuda")
    ccfg = rs.make_config(Bt, 4, 4, 16, 1)   # snapshot_commit reads only the batch size

    def snap_iter(it):
        rs.gdn_snapshot_spec_verify(cfg, slots, cur, T, *dpool[it % len(dpool)], od)
        rs.snapshot_commit(ccfg, cur, acc[it], T)
    _timed(snap_iter, 4)
    cur.zero_()
    wall_s, ds = _timed(snap_iter, iters)
    out = {
        "workload": f"Gated DeltaNet spec decode, batch {Bt}, T={T}, accepted ~ U{{0..{T}}}, {iters} verify steps, "
                    f"fp32 checkpoint, {prec} reads",
        "replay": {"accepted_tokens_per_s_layer": round(accepted / wall_r, 1),
                   "verify_plus_rollback_mean_us": round(float(dr.mean()) * 1e6, 2)},
        "snapshot": {"accepted_tokens_per_s_layer": round(accepted / wall_s, 1),
                     "verify_plus_commit_mean_us": round(float(ds.mean()) * 1e6, 2),
                     "gbps": round(traffic.gdn_snapshot_verify(Hv, Gk, Dv, Dk, T) * Bt / float(ds.mean()) / 1e9, 1),
                     "state_memory_gib": round(slots.numel() * 4 / 2 ** 30, 2)},
        "speedup_vs_snapshot": round(wall_s / wall_r, 3),
    }
    print(json.dumps(out), flush=True)


def mixer(args):
    c = workload.MIXER
    Bt, L, K = c["Bt"], c["L"], c["K"]
    CD = rs.conv_dim(rs.make_config(Bt, H, P, N, G))
    A, D = _layer_params()
    w, b, bias = (torch.from_numpy(a).cuda() for a in workload.mixer_params(workload.config_seed(8), H, P, G, N, K))
    g = _gen(8008)
    S0 = torch.randn(Bt, H, P, N, device="cuda", generator=g)
    hist = torch.randn(Bt, K - 1, CD, device="cuda", generator=g)
    pool = [(torch.randn(Bt, CD, device="cuda", generator=g), torch.randn(Bt, H, P, device="cuda", generator=g),
             torch.randn(Bt, H, device="cuda", generator=g)) for _ in range(16)]
    plain_pool = [_tokens(g, (Bt,), N) for _ in range(16)]
    o = torch.empty(Bt, H, P, device="cuda")
    lay = rs.ReplaySSM(Bt, H, P, N, G, A, D, buffer_len=L, d_conv=K)
    lay.set_mixer(w, b, bias)

    def mix_step(r):
        rs.replayssm_mixer_step(lay.handle, *pool[r % len(pool)], o)
    lay.load_state(S0)
    lay.load_conv_state(hist)
    _timed(mix_step, 2 * L)
    lay.load_state(S0)
    lay.load_conv_state(hist)
    steps = 16 * L
    wall, d = _timed(mix_step, steps)
    assert lay.check() == rs.RSSM_OK
    assert torch.isfinite(o).all().item()
    del lay
    ks = np.array([r % L + 1 for r in range(steps)])
    fl = ks == L
    pb = traffic.mixer_param_bytes(H, P, N, G, K)
    nf_bytes = np.array([traffic.replay_mixer_nonflush(H, P, N, G, int(k), K) * Bt + pb for k in ks[~fl]])
    fl_bytes = traffic.replay_mixer_flush_step(H, P, N, G, L, K) * Bt + pb
    nf_gbps = float((nf_bytes / d[~fl]).mean()) / 1e9

    plain = rs.ReplaySSM(Bt, H, P, N, G, A, D, buffer_len=L)

    def plain_step(r):
        rs.replayssm_step(plain.handle, *plain_pool[r % len(plain_pool)], o)
    plain.load_state(S0)
    _timed(plain_step, 2 * L)
    plain.load_state(S0)
    wall_p, dp = _timed(plain_step, steps)
    del plain

    cfg = rs.make_config(Bt, H, P, N, G, d_conv=K)
    ring = torch.zeros(Bt, K, CD, device="cuda")
    cst = S0.clone()

    def conv_step(r):
        rs.conventional_mixer_step(cfg, cst, ring, r, *pool[r % len(pool)], A, D, w, b, bias, o)
    _timed(conv_step, 4)
    wall_c, dc = _timed(conv_step, 64)
    conv_bytes = traffic.conventional_mixer(H, P, N, G, K) * Bt + pb
    unfused = np.array([traffic.unfused_mixer_nonflush(H, P, N, G, int(k), K) for k in ks[~fl]]).mean() * Bt
    out = {
        "workload": f"Mamba-2 layer decode step with the mixer edges fused (conv1d width {K} over {CD} xBC "
                    f"channels, softplus dt, output gate), batch {Bt}, 128 heads, P 64, N 128, 8 groups, L {L}, fp32",
        "replay_mixer": {"tokens_per_s_layer": round(Bt * steps / wall, 1),
                         "nonflush_mean_us": round(float(d[~fl].mean()) * 1e6, 2),
                         "nonflush_gbps": round(nf_gbps, 1), "nonflush_frac_of_8tbs": round(nf_gbps / PEAK, 4),
                         "nonflush_alg_bytes_per_launch": int(nf_bytes.mean()),
                         "flush_mean_us": round(float(d[fl].mean()) * 1e6, 2),
                         "flush_gbps": round(fl_bytes / float(d[fl].mean()) / 1e9, 1)},
        "replay_plain_step": {"tokens_per_s_layer": round(Bt * steps / wall_p, 1),
                              "nonflush_mean_us": round(float(dp[~fl].mean()) * 1e6, 2),
                              "flush_mean_us": round(float(dp[fl].mean()) * 1e6, 2)},
        "conventional_mixer": {"tokens_per_s_layer": round(Bt * 64 / wall_c, 1),
                               "mean_us": round(float(dc.mean()) * 1e6, 2),
                               "gbps": round(conv_bytes / float(dc.mean()) / 1e9, 1)},
        "speedup_vs_conventional_mixer": round((Bt * steps / wall) / (Bt * 64 / wall_c), 3),
        "edge_cost_vs_plain_step": round(float(d[~fl].mean()) / float(dp[~fl].mean()), 4),
        "alg_bytes_per_launch_unfused_pipeline_model": int(unfused),
    }
    print(json.dumps(out), flush=True)
    if getattr(args, "calib_copy", False):
        _calib_copy()


def ceilings(args):
    """Bandwidth ceilings on this GPU, the context for the replay kernels' fractions of 8 TB/s:
    the streaming probes of libbwprobe.so (32 KiB contiguous per work-group, 16-byte
    non-temporal accesses: the checkpoint stream's pattern without its arithmetic) -- a read of
    2 GiB, a copy of 1 GiB and an in-place read-modify-write of 1 GiB -- and, beside them, the
    same three through plain PyTorch kernels (torch.amax, copy_, mul_). Each figure is the median
    of 20 launches after 5 warm-up launches, in TB/s of bytes moved."""
    from hybrid_mamba_decode_amd import bwprobe
    n = 1 << 28                                    # 1 GiB of fp32
    x = torch.randn(2 * n, device="cuda")
    a, b = x[:n], torch.empty(n, device="cuda")
    sink = torch.empty(2 * n // 2048, device="cuda")

    def rate(fn, nbytes):
        _timed(fn, 5)
        _, d = _timed(fn, 20)
        return round(nbytes / float(np.median(d)) / 1e12, 3)

    out = {"probe": {"read_tbs": rate(lambda r: bwprobe.read(x, sink), 8 * n),
                     "copy_tbs": rate(lambda r: bwprobe.copy(a, b), 8 * n),
                     "rmw_tbs": rate(lambda r: bwprobe.rmw(a, 1.0), 8 * n)},
           "torch": {"read_tbs": rate(lambda r: torch.amax(x), 8 * n),
                     "copy_tbs": rate(lambda r: b.copy_(a), 8 * n),
                     "rmw_tbs": rate(lambda r: a.mul_(1.0), 8 * n)},
           "peak_tbs": PEAK / 1e3}
    print(json.dumps({"workload": "bandwidth ceilings: streaming probes (32 KiB per work-group, "
                                  "non-temporal 16-byte accesses) and plain PyTorch kernels", **out}), flush=True)


def run(args):
    if args.workload == "ceilings":
        ceilings(args)
    elif args.workload == "mixer":
        mixer(args)
    elif args.workload == "spec":
        spec(args)
    elif args.workload == "gdn":
        gdn(args)
    elif args.workload == "sweep":
        sweep(args)
