"""Benchmark: ReplaySSM Mamba-2 decode step on one MI355X.

Workload (default): one serving-size Mamba-2 layer -- batch 256, 128 heads, headdim 64, state 128
(4 MiB fp32 state per sequence), 8 groups, buffer length 16, fp32 read path -- with synthetic
seeded inputs already resident in HBM. One timed step = one replayssm_step over the batch (replay
and append; every 16th step also folds the buffer in the same launch), i.e. one decode step of the
layer. value = batch * steps / timed seconds = tokens/s/layer.

Prints ONE JSON line (rank 0) with the metric, the dominant kernel's roofline (algorithmic bytes
per launch / its mean duration from HIP events on the launch stream), the same-run conventional
read-update-write step, and the float64 CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--read-prec fp32|bf16|fp8|mxfp4]
                  [--master-prec fp32|fp16|fp16_sr|fp8|fp8_sr] [--no-cpu-baseline] [--kernels-only]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))


def measured_traffic(key):
    """HBM bytes per non-flush replay launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs (profiles/traffic_counters.json), or None when the kernel sources changed since."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_counters.json")))
        csrc = os.path.join(ROOT, "hybrid_mamba_decode_amd", "csrc")
        h = hashlib.sha256(open(os.path.join(csrc, "kernels.hip"), "rb").read() +
                           open(os.path.join(csrc, "device.h"), "rb").read()).hexdigest()[:16]
        if h != rec["kernel_source_sha256_16"] or key not in rec["kernels"]:
            return None
        k = rec["kernels"][key]
        return {"bytes_per_launch": k["read_bytes_per_launch"] + k["write_bytes_per_launch"],
                "over_algorithmic": k["traffic_over_alg"]}
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--read-prec", default="fp32", choices=["fp32", "bf16", "fp8", "mxfp4"])
    ap.add_argument("--master-prec", default="fp32", choices=["fp32", "fp16", "fp16_sr", "fp8", "fp8_sr"],
                    help="checkpoint precision: fp16 / fp8 (E4M3 codes with a per-head scale; reads "
                         "then come from it) round to nearest even at each flush, the _sr forms "
                         "stochastically")
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--buffer-len", type=int, default=16)
    ap.add_argument("--pool", type=int, default=32, help="distinct input sets cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--kernels-only", action="store_true",
                    help="only the replay steps (for profiler runs)")
    ap.add_argument("--workload", default="serving", choices=["serving", "spec", "sweep", "gdn", "mixer", "ceilings"],
                    help="serving: the headline line; spec: batch 512, T=4 verify+rollback vs "
                         "per-draft snapshots; sweep: batch x L over a 10-layer stack; gdn: a Gated "
                         "DeltaNet layer (--read-prec fp32|bf16|fp8|mxfp4); mixer: the step with the Mamba-2 "
                         "mixer edges fused; ceilings: read / copy / read-modify-write bandwidth of plain "
                         "PyTorch kernels")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB read + 1 GiB write elementwise kernel (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode step "
              "needs no communication: sequences or head groups shard across GPUs with no collective "
              "inside the step, so one GPU's share at its real shape is the measurement).", file=sys.stderr)
        sys.exit(2)

    import torch
    import hybrid_mamba_decode_amd as rs
    from hybrid_mamba_decode_amd import traffic
    import workload

    torch.cuda.set_device(0)
    if args.workload != "serving":
        import bench_workloads
        bench_workloads.run(args)
        return
    H, P, N, G = 128, 64, 128, 8
    Bt, L = args.batch, args.buffer_len
    prec = args.read_prec
    mprec = args.master_prec
    mstore = mprec.split("_")[0]                       # the master's storage: fp32, fp16 or fp8
    src = traffic.read_source(prec, mstore)            # precision the replay reads the state in
    tkey = prec if mprec == "fp32" else f"{prec}+master_{mprec}"
    seed = workload.config_seed(1)
    A, D = workload.layer_params(seed, H)
    S0 = workload.initial_state(seed, Bt, H, P, N)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    A_d, D_d = dev(A), dev(D)
    S0_d = dev(S0)
    host_pool = [workload.step_inputs(seed, t, Bt, H, P, N, G) for t in range(args.pool)]
    pool = [tuple(dev(a) for a in tok) for tok in host_pool]
    y = torch.empty(Bt, H, P, device="cuda")

    lay = rs.ReplaySSM(Bt, H, P, N, G, A_d, D_d, buffer_len=L, read_prec=prec, master_prec=mprec,
                       sr_seed=seed & 0x7FFFFFFF)
    lay.load_state(S0_d)
    stream = torch.cuda.current_stream()

    # warmup (also compiles nothing: kernels are prebuilt)
    for k in range(args.warmup):
        x, B, C, dt = pool[k % len(pool)]
        lay.step(x, B, C, dt, y)
    # restart from a window boundary so the timed steps cover whole windows
    lay.load_state(S0_d)
    torch.cuda.synchronize()

    K = args.steps
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    t0 = time.perf_counter()
    for k in range(K):
        x, B, C, dt = pool[k % len(pool)]
        ev0[k].record(stream)
        lay.step(x, B, C, dt, y)
        ev1[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert lay.check() == rs.RSSM_OK
    assert torch.isfinite(y).all().item()
    # kept for the CPU-baseline leg, whose float64 oracle run starts with these same K tokens
    timed_y = y.clone()
    timed_state = lay.materialize_state() if not args.kernels_only else None

    # The same K steps again without the per-launch timing events (each event adds a short gap
    # between launches); reported beside `value`, which keeps the instrumented timed region.
    lay.load_state(S0_d)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(K):
        x, B, C, dt = pool[k % len(pool)]
        lay.step(x, B, C, dt, y)
    torch.cuda.synchronize()
    wall_plain = time.perf_counter() - t1
    assert lay.check() == rs.RSSM_OK

    durs = np.array([ev0[k].elapsed_time(ev1[k]) * 1e-3 for k in range(K)])   # seconds
    ks = np.array([(k % L) + 1 for k in range(K)])      # records in the window incl. this token
    is_flush = ks == L
    bytes_nf = np.array([traffic.replay_nonflush(H, P, N, G, int(kk), src) * Bt for kk in ks])
    bytes_fl = traffic.replay_flush_step(H, P, N, G, L, prec, mstore) * Bt
    nf = ~is_flush
    nf_gbps = bytes_nf[nf].sum() / durs[nf].sum() / 1e9
    fl_gbps = (bytes_fl * is_flush.sum()) / durs[is_flush].sum() / 1e9 if is_flush.any() else None
    amort_bytes = traffic.replay_window_amortized(H, P, N, G, L, prec, master=mstore) * Bt
    value = Bt * K / wall
    # one whole window from the per-launch event means (k = 1 .. L-1 replayed, then the flush
    # step): independent of how K falls on window boundaries
    window_us = None
    if all((ks == kk).any() for kk in range(1, L + 1)):
        window_us = sum(float(durs[ks == kk].mean()) for kk in range(1, L + 1)) * 1e6

    result = {
        "metric": "SSM decode tokens/s/layer at batch 256 + achieved HBM GB/s (% of peak)",
        "value": round(value, 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "fp16": "f16", "fp8": "fp8 e4m3"}[mstore]
                 + (" master" if prec != "fp32" or mprec != "fp32" else "")
                 + ("" if prec == "fp32" else f" + {prec} read copy"),
        "data": "synthetic (seeded; value distributions of the layer definition)",
        "config": {"workload": f"one Mamba-2 layer decode step, batch {Bt}, 128 heads, headdim 64, "
                               f"state 128 (4 MiB fp32/sequence), 8 groups, buffer length {L}, "
                               f"{prec} read path" + ("" if mprec == "fp32" else f", {mprec} master"),
                   "batch": Bt, "buffer_len": L, "read_prec": prec, "master_prec": mprec},
        "roofline": {
            "kernel": "replay step, non-flush (step_kernel<prec, L bucket 16, rows, 0>; narrow_step_kernel for fp8 / MXFP4"
                      " reads, an fp8 master's included)",
            "bound": "hbm",
            "achieved": round(nf_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(nf_gbps / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(tkey),
            "mean_launch_us": round(float(durs[nf].mean()) * 1e6, 2),
            "alg_bytes_per_launch": int(bytes_nf[nf].mean()),
        },
        "tokens_per_s_without_launch_events": round(Bt * K / wall_plain, 1),
        "tokens_per_s_window_amortized": round(Bt * L / (window_us * 1e-6), 1) if window_us else None,
        "hbm_gbps_all_steps": round((bytes_nf[nf].sum() + bytes_fl * is_flush.sum()) / durs.sum() / 1e9, 1),
        "alg_bytes_per_step_amortized": int(amort_bytes),
        "nonflush_us_by_k": {int(kk): round(float(durs[ks == kk].mean()) * 1e6, 1) for kk in range(1, L)
                             if (ks == kk).any()},
        "flush_step": {"mean_launch_us": round(float(durs[is_flush].mean()) * 1e6, 2) if is_flush.any() else None,
                       "gbps": round(fl_gbps, 1) if fl_gbps else None,
                       "alg_bytes_per_launch": int(bytes_fl)},
    }

    if args.calib_copy:
        a = torch.ones(1 << 28, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    if not args.kernels_only:
        # conventional read-update-write step on the same shapes, same stream, same inputs
        cfg = rs.make_config(Bt, H, P, N, G)
        state = S0_d.clone()
        for k in range(min(args.warmup, 8)):
            x, B, C, dt = pool[k % len(pool)]
            rs.conventional_step(cfg, state, x, B, C, dt, A_d, D_d, y)
        torch.cuda.synchronize()
        Kc = max(16, K // 4)
        c0 = [torch.cuda.Event(enable_timing=True) for _ in range(Kc)]
        c1 = [torch.cuda.Event(enable_timing=True) for _ in range(Kc)]
        tc = time.perf_counter()
        for k in range(Kc):
            x, B, C, dt = pool[k % len(pool)]
            c0[k].record(stream)
            rs.conventional_step(cfg, state, x, B, C, dt, A_d, D_d, y)
            c1[k].record(stream)
        torch.cuda.synchronize()
        wall_c = time.perf_counter() - tc
        dc = np.array([c0[k].elapsed_time(c1[k]) * 1e-3 for k in range(Kc)])
        conv_bytes = traffic.conventional(H, P, N, G) * Bt
        conv_tps = Bt * Kc / wall_c
        result["conventional"] = {
            "tokens_per_s_layer": round(conv_tps, 1),
            "mean_launch_us": round(float(dc.mean()) * 1e6, 2),
            "gbps": round(conv_bytes / dc.mean() / 1e9, 1),
            "frac": round(conv_bytes / dc.mean() / 1e9 / HBM_PEAK_GBPS, 4),
        }
        result["speedup_vs_conventional"] = round(value / conv_tps, 3)
        del state

    if not args.no_cpu_baseline and not args.kernels_only:
        result["cpu_baseline"] = cpu_baseline(args, host_pool, Bt, A, D, S0, K, timed_y.cpu().numpy(),
                                              timed_state.cpu().numpy())

    print(json.dumps(result), flush=True)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, host_pool, Bt, A, D, S0, K, timed_y, timed_state):
    """The float64 stepwise oracle on the host cores: the full batch of the same layer, decode
    steps cycling through the same pool of seeded token sets as the GPU leg, until about
    --cpu-seconds of oracle time have run, on the oracle's OpenMP threads; then the same on one
    thread for a third of that time. Only the oracle calls are timed.

    The first K of those steps are exactly the GPU's timed run (same start state, same tokens), so
    the leg also reports the normwise error (max |diff| / max |ref|) of the timed run's last
    outputs and of the GPU state after it against the oracle's, over the whole batch."""
    import oracle
    pool = host_pool[:32]
    parity = {}

    def timed(budget, check):
        S = S0.astype(np.float64)
        steps, el = 0, 0.0
        while (el < budget or (check and steps < K)) and steps < 100000:
            tok = pool[steps % len(pool)]
            t0 = time.perf_counter()
            y = oracle.step(S, *tok, A, D)
            el += time.perf_counter() - t0
            steps += 1
            if check and steps == K:
                err = lambda a, r: float(np.max(np.abs(a - r)) / np.max(np.abs(r)))
                parity.update({"last_step_output_err": err(timed_y, y), "final_state_err": err(timed_state, S),
                               "steps": K, "sequences": "all"})
        return steps, el

    threads = oracle.threads()    # OMP_NUM_THREADS, else every core the process may use
    steps, el = timed(args.cpu_seconds, check=len(pool) == len(host_pool) or K <= len(pool))
    oracle.set_threads(1)
    steps1, el1 = timed(args.cpu_seconds / 3, check=False)
    oracle.set_threads(threads)
    return {"value": round(Bt * steps / el, 1), "unit": "tokens/s/layer",
            "cores": threads, "kind": "oracle", "cpu_model": _cpu_model(),
            "one_thread": {"value": round(Bt * steps1 / el1, 1), "steps": steps1, "seconds": round(el1, 1)},
            "timed_run_parity": parity or None,
            "sample": f"full batch {Bt} of the same layer, {steps} decode steps over a pool of "
                      f"{len(pool)} token sets, float64 stepwise recurrence (OpenMP over sequence x "
                      f"head, {threads} threads), {el:.1f} s; then {steps1} steps on 1 thread, {el1:.1f} s"}


if __name__ == "__main__":
    main()
