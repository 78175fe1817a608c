"""Throughput of the fp8 paged MQA indexer (logits + top-2048) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 1..5] [--no-cpu-baseline]

One step = mqa_paged_logits + mqa_topk over one batch of the named synthetic
workload (inputs already resident in HBM). The timed region is exactly K steps
bracketed by torch.cuda.synchronize(); value = indexed KV tokens (sum of context
lengths) per second. Steps rotate over enough copies of the inputs that every step
reads buffers evicted from the 256 MB Infinity Cache by the steps in between.

Prints one JSON line with, besides the headline value:
  roofline      the logits kernel (the dominant one) against HBM: algorithmic bytes
                per launch / its mean launch time, the latter from HIP events around
                each launch in a separate instrumented pass of K steps;
  cpu_baseline  the CPU oracle (float64, numpy) on the same workload, timed on this
                host's cores; a reported baseline, not a target.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0
METRIC = "indexed KV tokens/s (logits+top-2048) and % HBM peak, H=64 D=128 fp8"
ROW_BYTES = 132
LOGITS_SRC = os.path.join(ROOT, "fp8_paged_mqa_amd", "csrc", "logits.hip")
TOPK_SRC = os.path.join(ROOT, "fp8_paged_mqa_amd", "csrc", "topk.hip")


def algorithmic_bytes(w):
    """Bytes the logits and top-k launches must move at minimum (each input read
    once, each output written once)."""
    sum_ctx = w.sum_ctx
    rows = w.rows
    nv = w.visible().astype(np.int64)
    logits = (ROW_BYTES * sum_ctx            # key rows + scales
              + 4 * sum_ctx                  # block-table entries
              + w.q.nbytes + w.weights.nbytes + 4 * w.batch
              + 4 * rows * w.max_model_len)  # every logit slot, -inf tail included
    topk = 4 * int(nv[nv > w.k].sum()) + 4 * rows * w.k + 4 * w.batch
    return int(logits), int(topk)


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel, workload_tag, digest):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if one exists for
    this kernel source; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_tag}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source sha256\[:16\]:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(r"hbm bytes per launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_bytes or m_src.group(1) != digest:
        return None
    return float(m_bytes.group(1))


def cpu_baseline(w, min_seconds=10.0):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    runs, t0 = 0, time.perf_counter()
    while True:
        o = oracle.paged_mqa_logits(w.q, w.kv_cache, w.weights, w.context_lens, w.block_tables,
                                    w.max_model_len)
        oracle.topk(o, w.context_lens, w.next_n, w.k, w.max_model_len)
        runs += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or runs >= 20:
            break
    return {"value": w.sum_ctx * runs / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"the whole workload (logits + top-{w.k}), {runs} run(s), {el:.1f} s, float64 numpy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    sys.path.insert(0, ROOT)
    from fp8_paged_mqa_amd import mqa, workloads

    w = workloads.make_config(args.config, poison_unused=False)
    print(f"[bench] {w.name}: sum_ctx={w.sum_ctx} pool={w.num_blocks}", file=sys.stderr, flush=True)
    dev = "cuda"
    shape = mqa.make_shape(w.batch, w.next_n, w.heads, w.num_blocks, w.block_tables.shape[1])
    L, k = w.max_model_len, w.k
    copies = []
    for _ in range(max(1, args.copies)):
        copies.append(dict(
            q=torch.from_numpy(w.q).to(dev), kv=torch.from_numpy(w.kv_cache).to(dev),
            w=torch.from_numpy(w.weights).to(dev),
            ctx=torch.from_numpy(w.context_lens.astype(np.int32)).to(dev),
            bt=torch.from_numpy(w.block_tables.astype(np.int32)).to(dev),
            out=torch.empty((w.rows, L), dtype=torch.float32, device=dev),
            idx=torch.empty((w.rows, k), dtype=torch.int32, device=dev),
            ws=torch.empty(max(1, mqa.mqa_topk_workspace_bytes(shape, L, k)), dtype=torch.uint8, device=dev)))

    def logits(c):
        mqa.mqa_paged_logits(c["q"], c["kv"], c["w"], c["ctx"], c["bt"], L, c["out"], shape)

    def topk(c):
        mqa.mqa_topk(c["out"], c["ctx"], L, k, c["idx"], shape, c["ws"])

    for i in range(args.warmup):
        c = copies[i % len(copies)]
        logits(c)
        topk(c)
    torch.cuda.synchronize()

    # Timed region: exactly K steps.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        c = copies[i % len(copies)]
        logits(c)
        topk(c)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Instrumented pass: HIP events around each launch on the launch stream.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        c = copies[i % len(copies)]
        ev[i][0].record()
        logits(c)
        ev[i][1].record()
        topk(c)
        ev[i][2].record()
    torch.cuda.synchronize()
    t_logits = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    t_topk = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3

    bytes_logits, bytes_topk = algorithmic_bytes(w)
    achieved = bytes_logits / t_logits / 1e9
    tag = f"config{args.config}"
    traffic = traffic_from_profile("logits", tag, source_digest(LOGITS_SRC))
    value = w.sum_ctx / (ms_per_step * 1e-3)
    step_gbps = (bytes_logits + bytes_topk) / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3fn-mfma/f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "next_n": w.next_n, "heads": w.heads,
                   "head_dim": 128, "block_size": 1, "max_model_len": L, "k": k,
                   "sum_ctx": w.sum_ctx, "pool_rows": w.num_blocks, "input_copies": len(copies)},
        "hbm_frac_step": step_gbps / HBM_PEAK_GBPS,
        "kernels_us": {"logits": t_logits * 1e6, "topk": t_topk * 1e6},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "kernel": "paged_logits_kernel",
                     "algorithmic_bytes": bytes_logits,
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        wc = workloads.make_config(args.config, poison_unused=False)
        result["cpu_baseline"] = cpu_baseline(wc)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
