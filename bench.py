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


def traffic_from_profile(workload: str, algorithmic_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary (calibrated FETCH_SIZE +
    WRITE_SIZE of a profiled launch, over that launch's algorithmic bytes), scaled to this launch's
    algorithmic bytes; None if the summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_persistent_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_hash") != kernel_source_hash():
        return None
    return round(d["hbm_bytes_per_launch"] / d["algorithmic_bytes_per_launch"] * algorithmic_bytes)


def cpu_baseline(w, wts, dec, P):
    """The oracle as it stands on the host's cores, on a bounded sample of the same workload:
    teacher-forced decode steps from the synthetic KV of the bench's prompt length (timed without
    loading the KV), a prefill of a few prompt tokens, and 1-thread decode figures for the tiny and
    ~1B workloads.  The decode steps also give the bench line a parity check against the GPU."""
    import numpy as np
    import oracle
    import synthgen
    from tests.parity import check, gpu_run
    sample = 2 if w.hidden >= 4096 else 4
    k, v, sc = synthgen.make_kv(w, P)
    nxt = int(synthgen.make_prompt(w, 1)[0])
    run = gpu_run(w, wts, sample, kv=(k, v, P), next_token=nxt, kv_scales=sc, dec=dec)
    om = oracle.OracleModel(wts)
    if sc is not None:
        om.set_kv_scales(sc)
    om.load_kv(k, v, P)
    del k, v
    ref, inp = [], run.first
    t0 = time.time()
    for i in range(sample):
        _, lg = om.step(inp)
        ref.append(lg)
        inp = int(run.tokens[i])
    dsecs = time.time() - t0
    md = check(w, run, np.stack(ref), True, f"bench/{w.name}")
    npre = 16 if w.hidden >= 4096 else 64
    om2 = oracle.OracleModel(wts, max_seq=npre)
    if sc is not None:
        om2.set_kv_scales(sc)
    t0 = time.time()
    om2.prefill(synthgen.make_prompt(w, npre), want_logits=False)
    psecs = time.time() - t0
    del om, om2
    threads = oracle.num_threads()
    one = {}
    oracle.set_num_threads(1)
    try:
        for name, n in (("tiny", 8), ("1b", 2)):
            ws = synthgen.WORKLOADS[name]
            wt = wts if name == w.name else synthgen.make_weights(ws)
            m = oracle.OracleModel(wt)
            m.prefill(synthgen.make_prompt(ws), want_logits=False)
            t0 = time.time()
            tok = 0
            for _ in range(n):
                tok, _ = m.step(tok, want_logits=False)
            one[name] = round(n / (time.time() - t0), 3)
            del m, wt
    finally:
        oracle.set_num_threads(threads)
    cpu = {"value": round(sample / dsecs, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{sample} teacher-forced decode steps of the full {w.name} model from {P} synthetic KV "
                     f"positions (KV load not timed); prefill of {npre} prompt tokens timed apart; 1-thread decode of "
                     f"the tiny and ~1B workloads after their stated prompts; fp32 accumulation",
           "prefill_tokens_per_s": round(npre / psecs, 3), "one_thread_tokens_per_s": one}
    return cpu, md


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
                    help="keep the default schedule (default: before the timed launch, pmk_tune searches the schedule "
                         "knobs and speed-weighted row shares, keeping a change only if it passes the correctness gate "
                         "and runs faster)")
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
    if args.kernel_only:
        trace_steps = 0  # profiled runs time only the launches
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
    tune = None
    if args.tune:
        t_tune = time.time()
        r = dec.tune(32)
        torch.cuda.synchronize()
        tune = {"kept": r.desc.decode(), "candidates": r.tried, "accepted": r.kept, "gate_rejected": r.gate_rejected,
                "invalid": r.invalid, "us_per_step_default": round(r.us_before, 2),
                "us_per_step_tuned": round(r.us_after, 2), "gain": round(r.us_before / r.us_after, 4),
                "attn_splits": r.chosen.attn_splits, "combine_parts": r.chosen.combine_parts,
                "combine_o_share": r.chosen.combine_o_share}
        log(f"[bench] tuning search in {time.time() - t_tune:.1f}s: {r.tried} candidates, kept [{tune['kept']}], "
            f"{r.us_before:.1f} -> {r.us_after:.1f} us/step (schedule {dec.schedule_info().hash:#018x})")
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
        cpu, md = cpu_baseline(w, wts, dec, P)
        extra["parity_max_abs_logit_diff"] = float(f"{md:.3e}")
        extra["parity"] = "pass"

    traffic = traffic_from_profile(w.name, bytes_launch)
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
        "dtype": {"f16": "f16", "bf16": "bf16", "fp8": "fp8-e4m3 (fp32 accumulate)",
                  "int8": "int8 weights, f16 activations (fp32 accumulate)",
                  "int4": "int4 weights, f16 activations (fp32 accumulate)"}[w.wdtype],
        "data": "synthetic (seeded N(0,0.02) weights, random prompt)",
        "config": {"workload": w.name, "layers": w.layers, "hidden": w.hidden, "heads": [w.n_q, w.n_kv],
                   "head_dim": w.head_dim, "ffn": w.ffn, "vocab": w.vocab, "prompt": P, "decode_steps": K,
                   "batch": 1, "mode": args.mode, "sync": args.sync, "parallelism": "single GPU",
                   "tuning": tune if tune else "off (default schedule)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "roofline_detail": {"bytes_per_token_mean": round(bytes_launch / K), "t_min_us": round(
            bytes_launch / K / (PEAK_HBM_GBS * 1e3), 2), "us_per_token": round(ms_per_step * 1e3, 2)},
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    # release the device buffers and the context before the interpreter exits
    dec.close()
    del dec, out_tokens, n_done, first, first_tok, prompt
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
