"""Throughput of the fp8 paged MQA indexer (logits + top-2048) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--block-size S] [--no-cpu-baseline]
    python bench.py --op kwrite [--tokens T]   (the K-cache write alone; not the default line)
    python bench.py --op prefill [--m M --n N --heads H]   (non-paged logits; not the default line)
    python bench.py --op mla   (sparse MLA decode over the selected positions; not the default line)

One step = mqa_paged_logits + mqa_topk over one batch of the named synthetic workload,
inputs already resident in HBM. Steps are captured into a HIP graph and replayed (the
indexer runs once per layer per decode step, so serving stacks replay it from graphs;
eager launches from Python cost more host time than the GPU work). Consecutive steps
rotate over `--copies` copies of the inputs and outputs, so every step reads buffers
that the steps in between have evicted from the 256 MB Infinity Cache.

Timed region: exactly K steps (graph replays), bracketed by torch.cuda.synchronize().
value = indexed KV tokens (sum of context lengths) per second of that region.

The JSON line also carries:
  roofline      the logits kernel (the dominant one) against HBM: algorithmic bytes per
                launch / its mean launch time, from HIP events on the launch stream around
                graphs of back-to-back logits launches (same rotation);
  traffic       measured HBM bytes per logits launch (rocprofv3 FETCH_SIZE + WRITE_SIZE,
                scaled by the copy calibration) from the committed profile summary, when
                that summary was taken on the current kernel source;
  cpu_baseline  the CPU oracle (float64 numpy) on the same workload on this host's cores;
                a reported baseline, not a target.
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


def algorithmic_bytes(w):
    """Bytes each launch must move at minimum: every input read once, every output
    written once."""
    sum_ctx = w.sum_ctx
    rows = w.rows
    nv = w.visible().astype(np.int64)
    blocks = int(((w.context_lens.astype(np.int64) + w.block_size - 1) // w.block_size).sum())
    logits = (ROW_BYTES * sum_ctx            # key rows + scales
              + 4 * blocks                   # block-table entries (one per block)
              + w.q.nbytes + w.weights.nbytes + 4 * w.batch
              + 4 * rows * w.max_model_len)  # every logit slot, -inf tail included
    topk = 4 * int(nv[nv > w.k].sum()) + 4 * rows * w.k + 4 * w.batch
    return int(logits), int(topk)


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel, workload_tag, digest):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary taken on this kernel
    source; None otherwise."""
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
        if el >= min_seconds or runs >= 1000:
            break
    return {"value": w.sum_ctx * runs / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"the whole workload (logits + top-{w.k}, float64 numpy), {runs} run(s) in {el:.1f} s"}


MFMA_F16_PEAK_TFLOPS = 2500.0


def bench_prefill(args):
    """Non-paged logits: M query rows (causal: row i sees keys [0, N - M + i]) over N keys,
    8 rotating input/output copies, graph replays. Bound by the f16 matrix cores it uses."""
    import torch
    sys.path.insert(0, ROOT)
    from fp8_paged_mqa_amd import mqa, workloads
    M, N, H, C = args.m, args.n, args.heads, max(1, min(args.copies, 4))
    rng = np.random.Generator(np.random.PCG64(11))
    ks = np.zeros(M, np.int32)
    ke = (np.arange(M) + (N - M) + 1).astype(np.int32)
    copies = []
    for _ in range(C):
        q = torch.from_numpy(workloads.to_e4m3fn_bytes(rng.standard_normal((M, H, 128), dtype=np.float32))).cuda()
        k = torch.from_numpy(workloads.to_e4m3fn_bytes(rng.standard_normal((N, 128), dtype=np.float32))).cuda()
        sc = torch.from_numpy(rng.lognormal(0, 0.5, size=N).astype(np.float32)).cuda()
        w = torch.from_numpy(rng.standard_normal((M, H), dtype=np.float32)).cuda()
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        copies.append((q, k, sc, w, torch.from_numpy(ks).cuda(), torch.from_numpy(ke).cuda(), out))
    def run(c):
        mqa.mqa_logits(*c)
    for i in range(3):
        run(copies[i % C])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(C):
            run(copies[i])
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // (4 * C))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * C)
    visible = int(np.clip(ke - ks, 0, N).astype(np.int64).sum())
    flops = 2.0 * H * 128 * visible
    nbytes = M * H * 128 + N * 132 + 4 * M * H + 8 * M + 4 * M * N
    tflops = flops / (us * 1e-6) / 1e12
    print(json.dumps({
        "metric": "non-paged (prefill) indexer logits, TFLOP/s of the contraction",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": reps * C, "us_per_call": us,
        "higher_is_better": True, "dtype": "fp8e4m3fn->f16 mfma, f32 accumulate", "data": "synthetic",
        "config": {"workload": f"M={M} query rows, N={N} keys, H={H}, causal windows", "m": M, "n": N, "heads": H},
        "hbm_gbps_algorithmic": nbytes / (us * 1e-6) / 1e9,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_F16_PEAK_TFLOPS, "kernel": "prefill_logits_kernel",
                     "algorithmic_flops": flops, "traffic": None}}), flush=True)


def bench_kwrite(args):
    """Tokens/s of mqa_indexer_k_write: T bf16 key rows quantised into a 600k-row cache at
    permuted slots (8 rotating copies, graph replays)."""
    import torch
    sys.path.insert(0, ROOT)
    from fp8_paged_mqa_amd import mqa
    T, nslots, C = args.tokens, 600_000, max(1, args.copies)
    rng = np.random.Generator(np.random.PCG64(7))
    copies = []
    for _ in range(C):
        k = torch.from_numpy((rng.standard_normal((T, 128), dtype=np.float32)
                              * rng.lognormal(0, 1, size=(T, 1)).astype(np.float32))).to(torch.bfloat16).cuda()
        slots = torch.from_numpy(rng.permutation(nslots)[:T].astype(np.int64)).cuda()
        kv = torch.zeros((nslots, 132), dtype=torch.uint8, device="cuda")
        copies.append((k, slots, kv))
    def run(c):
        mqa.mqa_indexer_k_write(*c)
    for i in range(4):
        run(copies[i % C])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(C):
            run(copies[i])
    for _ in range(max(1, args.warmup // C)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // C)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * C)
    nbytes = T * (256 + 8 + 132)  # bf16 keys + slot read, row written
    achieved = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "indexer K-cache write tokens/s (bf16 keys -> e4m3fn + fp32 scale rows)",
        "value": T / (us * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": reps * C, "warmup": args.warmup,
        "us_per_call": us, "higher_is_better": True, "dtype": "bf16->fp8e4m3fn", "data": "synthetic",
        "config": {"workload": f"{T} tokens into a {nslots}-row cache at permuted slots", "tokens": T},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "kernel": "k_write_kernel<true>",
                     "algorithmic_bytes": nbytes, "traffic": None}}), flush=True)


def bench_mla(args):
    """Attended positions/s of mqa_sparse_mla_decode on the decode workload behind the
    indexer's headline shape: 64 requests, N = 1, each row attending its min(2048, ctx)
    selected positions (ctx ~ U{1..8192}) of a 600 000-row latent cache (576-byte rows,
    one token per block, random permutation), 16 heads. Graph replays over rotating copies."""
    import torch
    sys.path.insert(0, ROOT)
    from fp8_paged_mqa_amd import mqa, workloads
    case = workloads.make_mla_workload(poison_unused=False)
    C = max(1, args.copies)
    dev = "cuda"
    q_h, kv_h = torch.from_numpy(case.q), torch.from_numpy(case.kv_cache)
    idx_h, bt_h = torch.from_numpy(case.indices), torch.from_numpy(case.block_tables)
    copies = []
    for _ in range(C):
        q, kv, idx, bt = q_h.to(dev), kv_h.to(dev), idx_h.to(dev), bt_h.to(dev)
        shape = mqa.mla_shape_of(q, kv, bt, idx, case.next_n)
        nbytes = mqa.mqa_sparse_mla_workspace_bytes(shape)
        copies.append(dict(q=q, kv=kv, idx=idx, bt=bt, shape=shape,
                           ws=torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev),
                           out=torch.empty((case.rows, 16, 512), dtype=torch.float32, device=dev),
                           lse=torch.empty((case.rows, 16), dtype=torch.float32, device=dev)))
    def run(c):
        mqa.mqa_sparse_mla_decode(c["q"], case.q_scale, c["kv"], case.kv_scale, c["idx"], c["bt"], case.sm_scale,
                                  c["out"], c["lse"], shape=c["shape"], workspace=c["ws"])
    for i in range(4):
        run(copies[i % C])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(C):
            run(copies[i])
    for _ in range(max(1, args.warmup // C)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // C)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * C)
    listed, rows, topk = case.listed, case.rows, case.topk
    # Algorithmic bytes: each listed row once, the index list, one table entry per listed
    # position, the queries, the outputs and lse. The splits' partial states are extra.
    nbytes = 576 * listed + 4 * rows * topk + 4 * listed + rows * 16 * 576 + rows * 16 * 512 * 4 + rows * 16 * 4
    ws_bytes = mqa.mqa_sparse_mla_workspace_bytes(copies[0]["shape"])
    achieved = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "sparse MLA decode: attended positions/s (16 heads, 576-dim fp8 latent rows)",
        "value": listed / (us * 1e-6), "unit": "positions/s", "n_gpus": 1, "steps": reps * C,
        "warmup": args.warmup, "us_per_call": us, "higher_is_better": True,
        "dtype": "fp8e4m3fn->f16 mfma, f32 softmax", "data": "synthetic",
        "config": {"workload": "64 requests, N=1, min(2048, ctx) positions per row, ctx~U{1..8192}, "
                               "600000-row latent cache, permuted", "rows": rows, "topk": topk, "listed": listed,
                   "input_copies": C},
        "partial_state_bytes": 2 * ws_bytes,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "kernel": "sparse_mla_kernel + sparse_mla_combine_kernel",
                     "algorithmic_bytes": nbytes, "traffic": None}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=None,
                    help="named decode workload for the indexer step (default decode_b64_ctx8192)")
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--block-size", type=int, default=1,
                    help="tokens per KV block (1: the pages' layout; the default line uses 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", default="step", choices=["step", "kwrite", "prefill", "mla"])
    ap.add_argument("--m", type=int, default=4096, help="query rows for --op prefill")
    ap.add_argument("--n", type=int, default=8192, help="keys for --op prefill")
    ap.add_argument("--heads", type=int, default=32, help="heads for --op prefill")
    ap.add_argument("--tokens", type=int, default=65536, help="tokens per call for --op kwrite")
    ap.add_argument("--calibrate-copy-mib", type=int, default=256,
                    help="size of the plain device copy run once for counter calibration (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if args.op == "kwrite":
        bench_kwrite(args)
        return
    if args.op == "prefill":
        bench_prefill(args)
        return
    if args.op == "mla":
        bench_mla(args)
        return

    import torch
    sys.path.insert(0, ROOT)
    from fp8_paged_mqa_amd import mqa, workloads

    w = workloads.make_named(args.workload or workloads.DEFAULT_WORKLOAD, poison_unused=False,
                             block_size=args.block_size)
    print(f"[bench] {w.name}: sum_ctx={w.sum_ctx} pool={w.num_blocks}", file=sys.stderr, flush=True)
    dev = "cuda"
    shape = mqa.make_shape(w.batch, w.next_n, w.heads, w.num_blocks, w.block_tables.shape[1],
                           block_size=w.block_size)
    L, k = w.max_model_len, w.k
    C = max(1, args.copies)
    ws_bytes = max(1, mqa.mqa_topk_workspace_bytes(shape, L, k))
    copies = []
    for _ in range(C):
        copies.append(dict(
            q=torch.from_numpy(w.q).to(dev), kv=torch.from_numpy(w.kv_cache).to(dev),
            w=torch.from_numpy(w.weights).to(dev),
            ctx=torch.from_numpy(w.context_lens.astype(np.int32)).to(dev),
            bt=torch.from_numpy(w.block_tables.astype(np.int32)).to(dev),
            out=torch.empty((w.rows, L), dtype=torch.float32, device=dev),
            idx=torch.empty((w.rows, k), dtype=torch.int32, device=dev),
            ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev)))

    def logits(c):
        mqa.mqa_paged_logits(c["q"], c["kv"], c["w"], c["ctx"], c["bt"], L, c["out"], shape)

    def topk(c):
        mqa.mqa_topk(c["out"], c["ctx"], L, k, c["idx"], shape, c["ws"])

    def step(c):
        logits(c)
        topk(c)

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(copies[i % C])
        return g

    # Eager warmup (also loads the code objects), then the graphs.
    for i in range(4):
        step(copies[i % C])
    torch.cuda.synchronize()
    g_steps = capture(step, C)                 # C steps, one per input copy
    rem = args.steps % C
    g_rem = capture(step, rem) if rem else None
    for _ in range(max(1, args.warmup // C)):
        g_steps.replay()
    torch.cuda.synchronize()

    # Timed region: exactly K steps.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps // C):
        g_steps.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Per-kernel mean launch time: HIP events on the launch stream around graphs of
    # back-to-back launches of one kernel.
    def per_launch_us(fn, reps=8):
        g = capture(fn, C)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * C)

    t_logits = per_launch_us(logits)
    t_topk = per_launch_us(topk)

    # Host-launched steps (no graph), for reference.
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_eager = min(args.steps, 50)
    for i in range(n_eager):
        step(copies[i % C])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t1) * 1e3 / n_eager

    if args.calibrate_copy_mib > 0:  # a plain copy of known size, for counter calibration
        nbytes = args.calibrate_copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    bytes_logits, bytes_topk = algorithmic_bytes(w)
    achieved = bytes_logits / (t_logits * 1e-6) / 1e9
    tag = w.name.split(":")[0] + (f"_bs{w.block_size}" if w.block_size > 1 else "")
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
        "dtype": "fp8e4m3fn->f16 mfma, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "next_n": w.next_n, "heads": w.heads,
                   "head_dim": 128, "block_size": w.block_size, "max_model_len": L, "k": k,
                   "sum_ctx": w.sum_ctx, "pool_rows": w.num_blocks, "input_copies": C,
                   "timing": "HIP graph replay of the step"},
        "hbm_frac_step": step_gbps / HBM_PEAK_GBPS,
        "kernels_us": {"logits": t_logits, "topk": t_topk},
        "eager_ms_per_step": eager_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "kernel": "paged_logits_kernel",
                     "algorithmic_bytes": bytes_logits, "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
