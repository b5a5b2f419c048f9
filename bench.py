#!/usr/bin/env python3
"""Batch-1 greedy decode throughput of the persistent megakernel on one MI355X.

One bench step = one decode token: the whole hot path (RMSNorm, QKV/O/gate-up/down GEMVs, RoPE,
KV append, split-KV GQA attention, LM head, greedy argmax) for every layer.  After a real GPU
prefill of the workload's random prompt (untimed), W warm-up steps run, the position is rewound,
and exactly K steps are timed as ONE persistent-kernel launch, bracketed by device syncs and HIP
events on the launch stream; this is repeated (default 3 launches, rewinding to the same
position) and the median launch gives the value.

Prints one JSON line: tokens/s, ms per token, the HBM roofline block of the persistent kernel
(algorithmic weight + KV bytes per launch over its duration), the oracle's CPU baseline on a
bounded sample (teacher-forced from synthetic KV, which doubles as a parity check), and the
hipGraph-of-per-op-kernels baseline on the same steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E spec
METRIC = "batch-1 decode tokens/s on 1 GPU; % of HBM roofline (bytes/token ÷ peak BW)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("kernels.hip", "pmk_device.h", "schedule.cpp", "pmk_abi.cpp"):
        with open(os.path.join(ROOT, "persistent_megakernel_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, bytes_per_launch_steps: int):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_persistent_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_hash") != kernel_source_hash() or d.get("steps") != bytes_per_launch_steps:
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed decode steps (default: the workload's)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="8b")
    ap.add_argument("--mode", default="megakernel", choices=["megakernel", "graph", "per_op"])
    ap.add_argument("--sync", default="flags", choices=["flags", "counters"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--no-tune", dest="tune", action="store_false",
                    help="keep the even GEMV row split (default: before the timed launch, pmk_tune twice re-splits the "
                         "gate/up rows by the streaming rate each CU measured in traced warm-up steps and keeps a "
                         "re-split only if those steps then run faster)")
    ap.add_argument("--repeat", type=int, default=3,
                    help="timed launches of K steps each (from the same position); value is the median one")
    ap.add_argument("--kernel-only", action="store_true",
                    help="profiling: start from synthetic KV instead of a prefill and skip every leg but the timed launches")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (counter scale calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures the single-GPU decode path only; --gpus {args.gpus} is not supported "
              "(the path shards as independent replicas; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synthgen
    import persistent_megakernel_02_amd as pmk

    w = synthgen.WORKLOADS[args.workload]
    K = args.steps if args.steps is not None else w.steps
    W = args.warmup
    P = w.prompt
    if P + max(K, W) > w.max_seq:
        w = w.with_(steps=max(K, W))
    dev = torch.device("cuda", 0)
    t_setup = time.time()
    log(f"[bench] workload {w.name}: generating weights")
    wts = synthgen.make_weights(w)
    log(f"[bench] weights generated in {time.time() - t_setup:.1f}s; uploading")
    sync_mode = pmk.PMK_SYNC_COUNTERS if args.sync == "counters" else pmk.PMK_SYNC_FLAGS
    trace_steps = 0 if args.no_trace and not args.tune else 8
    dec = pmk.Decoder(pmk.model_config(w), 0, pmk.schedule_config(sync_mode=sync_mode, trace_steps=trace_steps))
    dw = pmk.DeviceWeights(wts)
    dec.load_weights(dw)
    torch.cuda.synchronize()
    del dw
    torch.cuda.empty_cache()
    mode = {"megakernel": pmk.PMK_MODE_MEGAKERNEL, "graph": pmk.PMK_MODE_GRAPH, "per_op": pmk.PMK_MODE_PER_OP}[args.mode]
    dec.set_mode(mode)
    # ---- prefill (untimed in the decode metric; its own rate is reported) ----
    prompt = torch.from_numpy(synthgen.make_prompt(w)).to(dev)
    kv_scales = None
    if w.kvdtype == "fp8":
        # static per (layer, kv head, K|V) scale: 8 maps to 448 (k, v of these models have unit-order spread)
        kv_scales = torch.full((w.layers, w.n_kv, 2), 8.0 / 448.0, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    t0 = time.time()
    if args.kernel_only:
        log(f"[bench] synthetic KV of {P} positions")
        k, v, sc = synthgen.make_kv(w, P)
        nxt = int(synthgen.make_prompt(w, 1)[0])
        dec.load_kv(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), P, nxt,
                    torch.from_numpy(sc).to(dev) if sc is not None else None)
        del k, v
        first = torch.tensor([nxt], dtype=torch.int32, device=dev)
    else:
        log(f"[bench] prefill {P} tokens")
        first = dec.prefill(prompt, kv_scales)
    torch.cuda.synchronize()
    prefill_s = time.time() - t0
    first_tok = first.clone()
    if args.copy_calib:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    out_tokens = torch.empty(max(K, W), dtype=torch.int32, device=dev)
    n_done = torch.zeros(1, dtype=torch.int32, device=dev)
    # ---- warm-up, speed-weighted row split (untimed), rewind, timed launch ----
    if W > 0:
        dec.decode(W, out_tokens=out_tokens, n_done=n_done)
        torch.cuda.synchronize()
        dec.rewind(P, first_tok)
    tune_kept = 0
    if args.tune:
        t_tune = time.time()
        for _ in range(2):
            tune_kept += int(dec.tune(trace_steps))
        torch.cuda.synchronize()
        log(f"[bench] tuned the GEMV row split in {time.time() - t_tune:.2f}s: {tune_kept} of 2 re-splits kept "
            f"(schedule {dec.schedule_info().hash:#018x})")
    stream = torch.cuda.current_stream()
    times = []
    for r in range(max(1, args.repeat)):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        dec.decode(K, out_tokens=out_tokens, n_done=n_done)
        ev1.record(stream)
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / 1e3)
        err = dec.poll_error()
        if err.code:
            raise RuntimeError(f"device error {err.code} (cu {err.cu} task {err.task})")
        dec.rewind(P, first_tok)
    elapsed = sorted(times)[len(times) // 2]  # the median launch
    ms_per_step = elapsed * 1e3 / K
    tokens_per_s = K / elapsed
    bytes_launch = sum(w.weight_bytes() + w.kv_bytes_read(i) for i in range(K))
    achieved = bytes_launch / elapsed / 1e9
    log(f"[bench] {K} steps in {elapsed * 1e3:.2f} ms: {tokens_per_s:.1f} tok/s, {achieved:.0f} GB/s "
        f"({100 * achieved / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f} GB/s)")
    extra = {"timed_launches_s": [round(t, 6) for t in times]}
    if not args.kernel_only:
        extra["prefill_tokens_per_s"] = round(P / prefill_s, 1)

    # ---- sync share from the per-task trace (separate, untimed call) ----
    if trace_steps and not args.no_trace and not args.kernel_only:
        dec.set_trace(True)
        dec.decode(trace_steps, out_tokens=out_tokens, n_done=n_done)
        torch.cuda.synchronize()
        share, step_us = dec.trace_stats()
        dec.set_trace(False)
        dec.rewind(P, first_tok)
        extra["sync_wait_share"] = round(share, 4)
        extra["traced_step_us"] = round(step_us, 2)
        log(f"[bench] traced: wait share {share:.3f}, step {step_us:.1f} us")

    # ---- hipGraph-of-per-op-kernels baseline on the same steps ----
    if not args.no_graph_baseline and not args.kernel_only and mode == pmk.PMK_MODE_MEGAKERNEL:
        dec.set_mode(pmk.PMK_MODE_GRAPH)
        dec.decode(4, out_tokens=out_tokens, n_done=n_done)  # capture + warm
        torch.cuda.synchronize()
        dec.rewind(P, first_tok)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dec.decode(K, out_tokens=out_tokens, n_done=n_done)
        e1.record(stream)
        torch.cuda.synchronize()
        g = e0.elapsed_time(e1) / 1e3
        extra["graph_baseline_tokens_per_s"] = round(K / g, 2)
        extra["megakernel_speedup_vs_graph"] = round(g / elapsed, 3)
        log(f"[bench] hipGraph per-op baseline: {K / g:.1f} tok/s")
        dec.set_mode(mode)
        dec.rewind(P, first_tok)

    # ---- oracle CPU baseline on a bounded sample (+ parity of those steps) ----
    cpu = None
    if not args.no_cpu_baseline and not args.kernel_only:
        import oracle
        from tests.parity import check, gpu_run, oracle_teacher_forced
        sample = 2 if w.hidden >= 4096 else 4
        k, v, sc = synthgen.make_kv(w, P)
        nxt = int(synthgen.make_prompt(w, 1)[0])
        run = gpu_run(w, wts, sample, kv=(k, v, P), next_token=nxt, kv_scales=sc, dec=dec)
        t0 = time.time()
        ref, _ = oracle_teacher_forced(w, wts, run, kv=(k, v, P), kv_scales=sc)
        osecs = time.time() - t0
        md = check(w, run, ref, True, f"bench/{w.name}")
        cpu = {"value": round(sample / osecs, 4), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{sample} teacher-forced decode steps of the full {w.name} model from {P} synthetic KV "
                         f"positions (including the oracle's KV load), fp32 accumulation"}
        extra["parity_max_abs_logit_diff"] = float(f"{md:.3e}")
        extra["parity"] = "pass"

    traffic = traffic_from_profile(w.name, K)
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f16": "f16", "bf16": "bf16", "fp8": "fp8-e4m3 (fp32 accumulate)"}[w.wdtype],
        "data": "synthetic (seeded N(0,0.02) weights, random prompt)",
        "config": {"workload": w.name, "layers": w.layers, "hidden": w.hidden, "heads": [w.n_q, w.n_kv],
                   "head_dim": w.head_dim, "ffn": w.ffn, "vocab": w.vocab, "prompt": P, "decode_steps": K,
                   "batch": 1, "mode": args.mode, "sync": args.sync, "parallelism": "single GPU",
                   "row_split": ("tuned (gate/up)" if tune_kept else "even (tuned split measured slower)")
                   if args.tune else "even"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "roofline_detail": {"bytes_per_token_mean": round(bytes_launch / K), "t_min_us": round(
            bytes_launch / K / (PEAK_HBM_GBS * 1e3), 2), "us_per_token": round(ms_per_step * 1e3, 2)},
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    dec.close()


if __name__ == "__main__":
    main()
