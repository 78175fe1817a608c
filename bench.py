"""Throughput of the fp8 paged MQA indexer (logits + top-2048) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--block-size S]
                    [--no-cpu-baseline] [--no-workloads]
    python bench.py --op gather [--workload NAME]   (gather ceiling of the logits' row reads)
    python bench.py --op kwrite [--tokens T]   (the K-cache write alone; not the default line)
    python bench.py --op prefill [--m M --n N --heads H]   (non-paged logits; not the default line)
    python bench.py --op mla   (sparse MLA decode over the selected positions; not the default line)

One step = mqa_paged_logits + mqa_topk over one batch of the named synthetic workload,
inputs already resident in HBM. Steps are captured into a HIP graph and replayed (the
indexer runs once per layer per decode step, so serving stacks replay it from graphs;
eager launches from Python cost more host time than the GPU work). Consecutive steps
rotate over copies of the inputs and outputs (up to `--copies`, at least enough that
~768 MB pass between two uses of one copy), so every step reads buffers that the steps
in between have evicted from the 256 MB Infinity Cache.

Timed region: exactly K steps (graph replays), bracketed by torch.cuda.synchronize().
value = indexed KV tokens (sum of context lengths) per second of that region.

The JSON line also carries:
  step_us       median, p10 and p90 of the mean step time of 24 replays of the rotating
                steps (HIP events around each replay);
  roofline      the logits kernel (the dominant one) against HBM: algorithmic bytes per
                launch / its mean launch time, from HIP events on the launch stream around
                graphs of back-to-back logits launches (same rotation);
  traffic       measured HBM bytes per logits launch (rocprofv3 FETCH_SIZE + WRITE_SIZE,
                scaled by the copy calibration) from the committed profile summary, when
                that summary was taken on the current kernel source;
  gather_ceiling  the measurement probe's pure gather of the same rows in the same order
                (include/mqa_probe.h) and the logits kernel's time as a fraction of it;
  workloads     the same protocol on every named workload (the five serving shapes and
                the context-parallel shard) at the run's block size: step time (mean of the timed region, and
                p50/p10/p90), tokens/s, per-launch logits and top-k times, the logits
                roofline fraction (algorithmic, and measured-traffic when a profile of the
                current source exists);
  cpu_baseline  the CPU oracle (float64 numpy) on the same workload on this host's cores,
                with the host CPU model; a reported baseline, not a target.
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
        qf = rng.standard_normal((M, H, 128), dtype=np.float32)
        kf = rng.standard_normal((N, 128), dtype=np.float32)
        if args.prefill_data == "zero":  # same work on operands that do not switch
            qf[:] = 0.0
            kf[:] = 0.0
        q = torch.from_numpy(workloads.to_e4m3fn_bytes(qf)).cuda()
        k = torch.from_numpy(workloads.to_e4m3fn_bytes(kf)).cuda()
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
        "config": {"workload": f"M={M} query rows, N={N} keys, H={H}, causal windows", "m": M, "n": N, "heads": H,
                   "operands": args.prefill_data},
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
                           ws=torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev),
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def input_copies(w, requested):
    """Enough rotating copies that a step never finds its inputs and outputs in the 256 MB
    Infinity Cache (at least ~768 MB between two uses of one copy), at most `requested`."""
    per_step = w.kv_cache.nbytes + 4 * w.rows * w.max_model_len + w.block_tables.nbytes
    return int(max(2, min(requested, -(-(768 << 20) // max(per_step, 1)))))


class Step:
    """Device copies of one workload and the captured graphs of its step."""

    def __init__(self, w, copies):
        import torch
        from fp8_paged_mqa_amd import mqa
        self.torch, self.mqa, self.w = torch, mqa, w
        dev = "cuda"
        self.shape = mqa.make_shape(w.batch, w.next_n, w.heads, w.num_blocks, w.block_tables.shape[1],
                                    block_size=w.block_size)
        self.L, self.k, self.C = w.max_model_len, w.k, copies
        ws_bytes = max(16, mqa.mqa_topk_workspace_bytes(self.shape, self.L, self.k))  # zero-filled once
        host = dict(q=torch.from_numpy(w.q), kv=torch.from_numpy(w.kv_cache), w=torch.from_numpy(w.weights),
                    ctx=torch.from_numpy(w.context_lens.astype(np.int32)),
                    bt=torch.from_numpy(w.block_tables.astype(np.int32)))
        self.copies = []
        for _ in range(copies):
            c = {key: t.to(dev) for key, t in host.items()}
            c["out"] = torch.empty((w.rows, self.L), dtype=torch.float32, device=dev)
            c["idx"] = torch.empty((w.rows, self.k), dtype=torch.int32, device=dev)
            c["ws"] = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
            self.copies.append(c)

    def logits(self, c):
        self.mqa.mqa_paged_logits(c["q"], c["kv"], c["w"], c["ctx"], c["bt"], self.L, c["out"], self.shape)

    def topk(self, c):
        self.mqa.mqa_topk(c["out"], c["ctx"], self.L, self.k, c["idx"], self.shape, c["ws"])

    def step(self, c):
        self.logits(c)
        self.topk(c)

    def capture(self, fn, n):
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g):
            for i in range(n):
                fn(self.copies[i % self.C])
        return g

    def replay_us(self, g, per_replay, reps):
        """Per-replay mean time of one unit (us), from HIP events on the launch stream around
        each replay, for `reps` back-to-back replays."""
        torch = self.torch
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            g.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 / per_replay for i in range(reps)])


def measure(w, steps, warmup, copies, tag):
    """Timed region of exactly `steps` steps, then per-step and per-launch distributions."""
    import torch
    st = Step(w, input_copies(w, copies))
    C = st.C
    for i in range(4):                 # eager warmup (also loads the code objects)
        st.step(st.copies[i % C])
    torch.cuda.synchronize()
    g_steps = st.capture(st.step, C)   # C steps, one per input copy
    rem = steps % C
    g_rem = st.capture(st.step, rem) if rem else None
    for _ in range(max(1, warmup // C)):
        g_steps.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps // C):
        g_steps.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    # Distribution: each sample is the mean step time of one replay of C rotating steps.
    dist = st.replay_us(g_steps, C, 24)
    t_logits = float(np.mean(st.replay_us(st.capture(st.logits, C), C, 8)))
    t_topk = float(np.mean(st.replay_us(st.capture(st.topk, C), C, 8)))
    bytes_logits, bytes_topk = algorithmic_bytes(w)
    frac = bytes_logits / (t_logits * 1e-6) / 1e9 / HBM_PEAK_GBPS
    traffic = traffic_from_profile("logits", tag, source_digest(LOGITS_SRC))
    med = float(np.median(dist))
    out = {
        "ms_per_step": ms_per_step,
        "step_us_p50": med, "step_us_p10": float(np.percentile(dist, 10)),
        "step_us_p90": float(np.percentile(dist, 90)),
        "tokens_per_s": w.sum_ctx / (ms_per_step * 1e-3),
        "kernels_us": {"logits": t_logits, "topk": t_topk},
        "logits_roofline_frac": frac,
        "logits_algorithmic_bytes": bytes_logits,
        "logits_traffic_bytes": traffic,
        "logits_traffic_frac": None if traffic is None else traffic / (t_logits * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "hbm_frac_step": (bytes_logits + bytes_topk) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "input_copies": C,
    }
    return st, out


def gather_rows(w):
    """Cache rows the logits kernel reads, in the order it visits them (request-major,
    position ascending)."""
    S = w.block_size
    rows = []
    for b in range(w.batch):
        t = np.arange(int(w.context_lens[b]), dtype=np.int64)
        rows.append(w.block_tables[b][t // S].astype(np.int64) * S + t % S)
    return np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)


def gather_ceiling(st):
    """The probe's gather of the rows the logits kernel reads (same copies, same rotation),
    best over 1, 2 and 4 workgroups of 4 waves per CU and 2 or 4 stages in flight with the
    logits kernel's register loads ("GxS"), and over 1 or 2 workgroups per CU and 2 or 3
    stages of direct-to-LDS loads of each row's aligned 144-byte window ("lds_GxS")."""
    torch, mqa, w = st.torch, st.mqa, st.w
    rows = torch.from_numpy(gather_rows(w)).cuda()
    best, tried = None, {}
    forms = [("", mqa.mqa_probe_gather, gpc, depth) for gpc in (1, 2, 4) for depth in (2, 4)]
    forms += [("lds_", mqa.mqa_probe_gather_lds, gpc, depth) for gpc in (1, 2) for depth in (2, 3)]
    for tag, probe, gpc, depth in forms:
        sink = torch.empty(mqa.mqa_probe_gather_sink_words(gpc), dtype=torch.int32, device="cuda")
        fn = lambda c, probe=probe, gpc=gpc, sink=sink, depth=depth: probe(c["kv"], rows, gpc, sink, depth)  # noqa: E731
        us = float(np.mean(st.replay_us(st.capture(fn, st.C), st.C, 8)))
        tried[f"{tag}{gpc}x{depth}"] = us
        if best is None or us < best[0]:
            best = (us, gpc, depth, "lds" if tag else "registers")
    n = int(rows.numel())
    return {"us": best[0], "groups_per_cu": best[1], "stages_in_flight": best[2], "loads": best[3], "rows": n,
            "gbps_algorithmic": (ROW_BYTES + 4) * n / (best[0] * 1e-6) / 1e9,
            "us_by_groups_x_stages": tried}


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
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-workload table (every named workload, same protocol)")
    ap.add_argument("--op", default="step", choices=["step", "kwrite", "prefill", "mla", "gather"])
    ap.add_argument("--m", type=int, default=4096, help="query rows for --op prefill")
    ap.add_argument("--n", type=int, default=8192, help="keys for --op prefill")
    ap.add_argument("--heads", type=int, default=32, help="heads for --op prefill")
    ap.add_argument("--prefill-data", default="random", choices=["random", "zero"],
                    help="operand codes for --op prefill: random (the benchmark) or all zero (the clock the "
                         "chip holds when the operands do not switch; same instructions and cycles)")
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
    from fp8_paged_mqa_amd import workloads

    name = args.workload or workloads.DEFAULT_WORKLOAD
    w = workloads.make_named(name, poison_unused=False, block_size=args.block_size)
    print(f"[bench] {w.name}: sum_ctx={w.sum_ctx} pool={w.num_blocks}", file=sys.stderr, flush=True)
    tag = w.name.split(":")[0] + (f"_bs{w.block_size}" if w.block_size > 1 else "")
    st, m = measure(w, args.steps, args.warmup, args.copies, tag)
    ceiling = gather_ceiling(st)
    if args.op == "gather":
        print(json.dumps({
            "metric": "gather ceiling: 132-byte cache rows the paged logits kernel reads, in its order",
            "value": ceiling["gbps_algorithmic"], "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
            "data": "synthetic", "config": {"workload": w.name, "block_size": w.block_size},
            "gather": ceiling, "logits_us": m["kernels_us"]["logits"],
            "logits_frac_of_ceiling": ceiling["us"] / m["kernels_us"]["logits"]}), flush=True)
        return

    # Host-launched steps (no graph), for reference.
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_eager = min(args.steps, 50)
    for i in range(n_eager):
        st.step(st.copies[i % st.C])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t1) * 1e3 / n_eager

    if args.calibrate_copy_mib > 0:  # a plain copy of known size, for counter calibration
        nbytes = args.calibrate_copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    bytes_logits = m["logits_algorithmic_bytes"]
    t_logits = m["kernels_us"]["logits"]
    achieved = bytes_logits / (t_logits * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3fn->f16 mfma, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "next_n": w.next_n, "heads": w.heads,
                   "head_dim": 128, "block_size": w.block_size, "max_model_len": st.L, "k": st.k,
                   "sum_ctx": w.sum_ctx, "pool_rows": w.num_blocks, "input_copies": st.C,
                   "timing": "HIP graph replay of the step"},
        "step_us": {"p50": m["step_us_p50"], "p10": m["step_us_p10"], "p90": m["step_us_p90"],
                    "sample": f"24 replays of {st.C} rotating steps, HIP events per replay"},
        "hbm_frac_step": m["hbm_frac_step"],
        "kernels_us": m["kernels_us"],
        "eager_ms_per_step": eager_ms,
        "gather_ceiling": {**ceiling, "logits_frac_of_ceiling": ceiling["us"] / t_logits},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "kernel": "paged_logits_kernel",
                     "algorithmic_bytes": bytes_logits, "traffic": m["logits_traffic_bytes"]},
    }
    del st
    torch.cuda.empty_cache()
    if not args.no_workloads:
        table = {}
        for other in workloads.WORKLOADS:
            wo = w if other == name else workloads.make_named(other, poison_unused=False, block_size=args.block_size)
            print(f"[bench] workload {other}: sum_ctx={wo.sum_ctx}", file=sys.stderr, flush=True)
            st_o, mo = measure(wo, args.steps, args.warmup, args.copies,
                               other + (f"_bs{wo.block_size}" if wo.block_size > 1 else ""))
            table[other] = {k: v for k, v in mo.items() if k != "logits_algorithmic_bytes"}
            table[other]["block_size"] = wo.block_size
            del st_o
            torch.cuda.empty_cache()
        result["workloads"] = table
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
        result["cpu_baseline"]["cpu_model"] = cpu_model()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
