#!/usr/bin/env python3
"""Draft-and-verify throughput of the EAGLE hot path on one MI355X.

One "step" is one full round on resident inputs: tree init, gamma draft steps
(fc, decoder layer with tree-masked attention, LM head + softmax/top-k), the
tree expand/rerank after each, and greedy verification against synthetic
target logits (workloads with a target model run the target's own pass over
the tree instead; --verify sample verifies by speculative sampling).  The
metric is draft-tree nodes per second (nodes of the verify tree, root
excluded, summed over the batch).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--verify greedy|sample] [--no-cpu] [--no-breakdown]

Prints one JSON line.  Besides the contract fields it carries
  roofline      the dominant kernel (the LM head with its fused top-k):
                algorithmic bytes per launch / mean launch time from HIP events
                recorded on the launch stream inside the timed region
  cpu_baseline  the CPU oracle timed on this host on whole rounds of the same
                workload (a bounded sample of ~15 s)
  breakdown     per kernel family: launches per round, mean us, GB/s, TFLOP/s
                and the per-launch roofline (max of bytes / 8 TB/s and flops /
                MFMA peak) summed over the round (a separate profiled pass,
                outside the timed region)
  extra_workloads  (default workload only) the 8B EAGLE-2 tree (B 8) and the
                EAGLE-3 chain (B 32): nodes/s, ms per round and the fraction of
                their per-launch roofline the round reaches
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
EVENT_EVERY = 8               # rounds between the timed region's LM-head event samples

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {"lmhead": ["eagle_feature_space_amd/csrc/lmhead.hip",
                             "eagle_feature_space_amd/csrc/stream.h",
                             "eagle_feature_space_amd/csrc/common.h"]}


def source_hash(family):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(family, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the kernel source as it is now."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        e = t[workload][family]
    except (OSError, KeyError, ValueError):
        return None
    if e.get("source_sha256_16") != source_hash(family):
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(cfg, weights, inp, target, seconds):
    import numpy as np
    from threadpoolctl import threadpool_info

    from eagle_feature_space_amd import synth
    from oracle.head import DraftHead
    from oracle.round import run_round

    head = DraftHead(cfg.head, {k: synth.f32(v) for k, v in weights.items()})
    kw = dict(n=inp.n, t_root=inp.t_root, target=synth.f32(target))
    if inp.k_ctx is not None:
        kw.update(k_ctx=synth.f32(inp.k_ctx), v_ctx=synth.f32(inp.v_ctx))
    if inp.f_root is not None:
        kw.update(f_root=synth.f32(inp.f_root))
    if inp.lmh is not None:
        kw.update(lmh=synth.f32(inp.lmh), ctx_tokens=inp.ctx_tokens, n_new=inp.n_new)
    rounds = 0
    t0 = time.perf_counter()
    while True:
        run_round(cfg, head, **kw)
        rounds += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    nodes = cfg.B * cfg.n_final
    return {"value": nodes * rounds / el, "unit": "nodes/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rounds} full rounds of {cfg.name} (numpy fp32, {nodes} nodes each) in {el:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def family_breakdown(E, R):
    """Per kernel family over the last R profiled rounds: launches, time,
    algorithmic bytes and flops, and the per-launch roofline time
    max(bytes / 8 TB/s, flops / MFMA peak) summed over the family's launches."""
    out = {}
    tot_ms = tot_bytes = tot_roof = 0.0
    for fam in E.PROF_FAMILIES:
        p = E.eagle_profile_read(fam)
        if p["launches"] == 0:
            continue
        ms = p["ms"] * p["launches"] / max(1, p["timed"])
        tot_ms += ms
        tot_bytes += p["bytes"]
        tot_roof += p["roof_ms"]
        out[fam] = {"launches_per_round": p["launches"] / R,
                    "us_per_round": round(ms * 1e3 / R, 2),
                    "GB_per_round": round(p["bytes"] / R / 1e9, 4),
                    "GBps": round(p["bytes"] / (ms * 1e-3) / 1e9, 1) if ms > 0 and p["bytes"] else None,
                    "TFLOPps": round(p["flops"] / (ms * 1e-3) / 1e12, 2) if ms > 0 and p["flops"] else None,
                    "roofline_us_per_round": round(p["roof_ms"] * 1e3 / R, 2),
                    "roofline_frac": round(p["roof_ms"] / ms, 4) if ms > 0 and p["roof_ms"] else None}
    out["kernels_us_per_round"] = round(tot_ms * 1e3 / R, 2)
    out["round_bytes_GB"] = round(tot_bytes / R / 1e9, 4)
    out["round_hbm_roofline_us"] = round(tot_bytes / R / (HBM_PEAK_GBS * 1e9) * 1e6, 2)
    # each launch bound by HBM or by the MFMA peak, whichever takes longer
    out["round_roofline_us"] = round(tot_roof * 1e3 / R, 2)
    return out


def extra_workload(name, steps, warmup):
    """Throughput of another workload (no CPU baseline): nodes/s, ms per round
    and the fraction of its per-launch roofline the round reaches."""
    import torch

    from eagle_feature_space_amd import binding as E
    from eagle_feature_space_amd import configs as C
    from eagle_feature_space_amd import synth
    from eagle_feature_space_amd.runner import GpuRound, to_dev

    cfg = C.ALL_CONFIGS[name]
    print(f"[bench] extra {name}: generating inputs", file=sys.stderr, flush=True)
    gr = GpuRound(cfg, synth.head_weights(cfg.head, cfg.seed_w), synth.round_inputs(cfg))
    tgt = to_dev(synth.target_logits(cfg), gr.dev)
    # warm-up of at least half a second: after the seconds of host-side input
    # generation a few rounds leave the GPU below its working clocks
    tw = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - tw < 0.5:
        gr.run(target=tgt, attend=cfg.tree_attend)
        torch.cuda.synchronize()
        n_warm += 1
    t0 = time.perf_counter()
    for _ in range(steps):
        gr.run(target=tgt, attend=cfg.tree_attend)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    R = 5
    E.eagle_profile_reset()
    E.eagle_profile_enable(True)
    for _ in range(R):
        gr.run(target=tgt, attend=cfg.tree_attend)
    torch.cuda.synchronize()
    E.eagle_profile_enable(False)
    fb = family_breakdown(E, R)
    ms = el * 1e3 / steps
    nodes = cfg.B * cfg.n_final
    res = {"value": round(nodes * steps / el, 2), "unit": "nodes/s", "ms_per_step": round(ms, 4),
           "steps": steps, "warmup": n_warm, "nodes_per_round": nodes,
           "round_roofline_us": fb["round_roofline_us"],
           "round_roofline_frac": round(fb["round_roofline_us"] / (ms * 1e3), 4),
           "families_us_per_round": {k: v["us_per_round"] for k, v in fb.items() if isinstance(v, dict)}}
    del gr, tgt
    torch.cuda.empty_cache()
    return res


LIB_GEMM_SHAPES = (("lm_head_512", 512, 128256, 8192), ("gate_up_512", 512, 57344, 8192),
                   ("down_512", 512, 8192, 28672), ("qkv_512", 512, 10240, 8192),
                   ("lm_head_80", 80, 128256, 4096), ("gate_up_80", 80, 28672, 4096))


def lib_gemm():
    """Reference only: the vendor GEMM (torch.nn.functional.linear, bf16 in and
    out, hipBLASLt on ROCm) at the head's tiled-GEMM shapes, cold weights
    (rotating copies beyond the 256 MB cache), median of 16 timed launches.
    One JSON line per shape."""
    import torch
    for name, M, N, K in LIB_GEMM_SHAPES:
        x = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        ws = [torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
              for _ in range(2 if N * K * 2 > (1 << 30) else 4)]
        ts = []
        for it in range(20):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.nn.functional.linear(x, ws[it % len(ws)])
            e1.record()
            e1.synchronize()
            if it >= 4:
                ts.append(e0.elapsed_time(e1) * 1e3)
        us = sorted(ts)[len(ts) // 2]
        print(json.dumps({"gemm": name, "M": M, "N": N, "K": K, "us": round(us, 1),
                          "tflops": round(2 * M * N * K / us / 1e6, 1),
                          "weight_tbps": round(N * K * 2 / us / 1e6, 3)}), flush=True)
        del ws, x
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c1_8b_static")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--verify", choices=("greedy", "sample"), default="greedy",
                    help="greedy verification (default) or lossless speculative sampling "
                         "(inverse temperature 1, seeded uniforms)")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extra workloads (8B EAGLE-2 tree, EAGLE-3 chain) the default "
                         "run reports beside the headline")
    ap.add_argument("--lib-gemm", action="store_true",
                    help="instead of the benchmark: time the vendor GEMM (torch / hipBLASLt) at the "
                         "tiled-GEMM shapes, for reference")
    ap.add_argument("--copy-probe", action="store_true",
                    help="one 1 GiB device-to-device copy before warm-up (a known-size kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requests shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.lib_gemm:
        if not torch.cuda.is_available():
            print("--lib-gemm needs a GPU", file=sys.stderr)
            sys.exit(3)
        lib_gemm()
        return

    from eagle_feature_space_amd import binding as E
    from eagle_feature_space_amd import configs as C
    from eagle_feature_space_amd import synth
    from eagle_feature_space_amd.runner import GpuRound, to_dev

    if not os.path.exists(E.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no CPU fallback)", file=sys.stderr)
        sys.exit(3)

    cfg = C.ALL_CONFIGS[args.workload]
    print(f"[bench] {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    weights = synth.head_weights(cfg.head, cfg.seed_w)
    inp = synth.round_inputs(cfg)
    target = synth.target_logits(cfg)
    gr = GpuRound(cfg, weights, inp)
    tgt = to_dev(target, gr.dev)
    torch.cuda.synchronize()

    sample = None
    if args.verify == "sample":
        sample = (1.0, to_dev(synth.verify_draws(cfg, tgt.shape[1]), gr.dev))
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=gr.dev).fill_(7)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        gr.run(target=tgt, attend=cfg.tree_attend, sample=sample)
    torch.cuda.synchronize()

    # ---- timed region: K rounds; HIP events bracket the LM-head launches of
    # every EVENT_EVERY-th round only (an event pair costs ~9 us of the round's
    # time; one round in eight keeps that under 0.5% while still sampling the
    # launches inside the timed region)
    E.eagle_profile_reset()
    lm_mask = 1 << E.PROF_FAMILIES["lmhead"]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        timed = i % EVENT_EVERY == 0
        if timed:
            E.eagle_profile_enable(lm_mask)
        gr.run(target=tgt, attend=cfg.tree_attend, sample=sample)
        if timed:
            E.eagle_profile_enable(False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    lm = E.eagle_profile_read("lmhead")

    nodes = cfg.B * cfg.n_final
    ms_per_step = elapsed * 1e3 / args.steps
    value = nodes * args.steps / elapsed
    avg_ms = lm["ms"] / max(1, lm["timed"])
    bytes_per_launch = lm["bytes"] / max(1, lm["launches"])
    flops_per_launch = lm["flops"] / max(1, lm["launches"])
    traffic = measured_traffic("lmhead", cfg.name)
    peak_tf = BF16_PEAK_TFLOPS if cfg.head.dtype == C.DTYPE_BF16 else FP32_PEAK_TFLOPS
    # the binding resource of the launch: HBM bytes or MFMA flops, whichever
    # takes longer at the datasheet peak
    if flops_per_launch / (peak_tf * 1e12) > bytes_per_launch / (HBM_PEAK_GBS * 1e9):
        achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_tf,
                    "unit": "TFLOP/s", "frac": round(achieved / peak_tf, 4)}
    else:
        achieved = bytes_per_launch / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roofline = {"kernel": "LM head + fused softmax/top-k partials", **roofline,
                "traffic": traffic, "bytes_per_launch": bytes_per_launch,
                "flops_per_launch": flops_per_launch,
                "mean_launch_us": round(avg_ms * 1e3, 2), "launches_timed": lm["timed"]}

    # ---- per-family breakdown (separate profiled pass)
    breakdown = None
    if not args.no_breakdown:
        R = max(5, min(20, args.steps))
        E.eagle_profile_reset()
        E.eagle_profile_enable(True)
        for _ in range(R):
            gr.run(target=tgt, attend=cfg.tree_attend, sample=sample)
        torch.cuda.synchronize()
        E.eagle_profile_enable(False)
        breakdown = family_breakdown(E, R)
        breakdown["round_roofline_frac_of_timed_round"] = round(
            breakdown["round_roofline_us"] / (ms_per_step * 1e3), 4)

    # ---- per-round distribution (separate pass, events at round start, end of
    # drafting and end of verify; the events add a few µs to each round)
    round_stats = None
    if not args.no_breakdown:
        R = max(20, min(50, args.steps))
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(R)]
        for r in range(R):
            ev[r][0].record()
            gr.init()
            for st in range(cfg.gamma):
                gr.step(st)
                gr.expand(st)
            if cfg.tree_attend:
                gr.attend()
            ev[r][1].record()
            vt = gr.target_logits() if gr.target is not None else tgt
            if sample is None:
                gr.verify(vt)
            else:
                gr.verify_sample(vt, *sample)
            ev[r][2].record()
        torch.cuda.synchronize()
        tot = sorted(e[0].elapsed_time(e[2]) * 1e3 for e in ev)
        drf = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in ev)
        ver = sorted(e[1].elapsed_time(e[2]) * 1e3 for e in ev)
        q = lambda v, f: round(v[min(len(v) - 1, int(f * len(v)))], 2)
        round_stats = {"rounds": R, "round_us_p10": q(tot, 0.1), "round_us_p50": q(tot, 0.5),
                       "round_us_p90": q(tot, 0.9), "draft_us_p50": q(drf, 0.5),
                       "verify_us_p50": q(ver, 0.5)}
        if gr.target is not None:
            round_stats["verify_includes"] = "the target's pass over the tree"

    extras = None
    if args.workload == "c1_8b_static" and not args.no_extras:
        del gr, tgt
        torch.cuda.empty_cache()
        extras = {w: extra_workload(w, 20, 3) for w in ("c2_8b_dynamic", "c3_8b_eagle3")}

    cpu = None
    if not args.no_cpu and cfg.target_layers > 0:
        cpu = {"value": None, "skipped": "the oracle's target pass at this size is not a bounded sample"}
    elif not args.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, weights, inp, target, args.cpu_seconds)

    h = cfg.head
    out = {
        "metric": "draft-tree nodes/sec (draft+verify) at d=4096,|V|=128256; % MFMA/HBM roofline",
        "value": round(value, 2), "unit": "nodes/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if h.dtype == C.DTYPE_BF16 else "f32",
        "data": "synthetic: seeded random-init head weights, inputs and target logits",
        "config": {"workload": cfg.name, "B": cfg.B, "d": h.d, "vocab": h.vocab,
                   "heads": f"{h.n_q}q/{h.n_kv}kv x {h.head_dim}", "ffn": h.ffn,
                   "n": int(inp.n.max()), "tree": {0: "chain", 1: "static", 2: "dynamic"}[cfg.tree],
                   "gamma": cfg.gamma, "top_k": cfg.top_k, "top_m": cfg.top_m,
                   "nodes_per_round": nodes, "verify": args.verify},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "breakdown": breakdown,
        "round_stats": round_stats,
        "extra_workloads": extras,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
