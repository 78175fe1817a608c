"""HIP path vs the CPU oracle, element by element (needs an MI355X)."""
import json
import os
import struct

import numpy as np
import pytest

import oracle
from fp8_paged_mqa_amd import workloads as wl
from gpu_helpers import check_logits, check_topk, oracle_logits, run_gpu, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Context lengths straddling 2048 (where the page reports a kernel's top-k collapsing)
# and the other power-of-two tile sizes, plus the primes 127 and 131.
SWEEP_SMALL = [1, 2, 3, 4, 5, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 131, 255, 256,
               257, 511, 512, 513, 1023, 1024, 1025, 2047, 2048, 2049, 3000, 4095, 4096, 4097,
               8191, 8192, 8193]
SWEEP_LARGE = [16383, 16384, 16385, 65535, 65536, 65537, 131071, 131072, 131073, 202751, 202752]


def _parity(case, k=None, what=""):
    say(f"[gpu] {what}: B={case.batch} N={case.next_n} H={case.heads} L={case.max_model_len} "
        f"sum_ctx={case.sum_ctx}")
    g, idx = run_gpu(case, k=k)
    o = oracle_logits(case)
    err = check_logits(g, o, what)
    ties = check_topk(idx, g, o, case, k=k, what=what)
    say(f"[gpu] {what}: max |err| {err:.2e}, near-ties {ties}")


def test_fp8_format_one_hot_all_code_pairs():
    """logit = relu(dec(a) * dec(b)) for every pair of e4m3fn codes: pins the OCP (fn)
    decode and subnormals on the matrix cores (an 8-bit significand product is exact)."""
    codes = np.arange(256, dtype=np.uint8)
    B = 256
    q = np.zeros((B, 1, 16, 128), np.uint8)
    q[:, 0, 0, 0] = codes
    kv = np.zeros((256, 132), np.uint8)
    kv[:, 0] = codes
    kv[:, 128:] = np.frombuffer(struct.pack("<f", 1.0), np.uint8)
    w = np.zeros((B, 16), np.float32)
    w[:, 0] = 1.0
    case = wl.Workload("one-hot", q, kv, w, np.full(B, 256, np.int32),
                       np.tile(np.arange(256, dtype=np.int32), (B, 1)), 256, 1, k=16)
    g, _ = run_gpu(case, k=16)
    dec = oracle.E4M3FN_VALUES
    expect = np.maximum(np.outer(dec, dec), 0.0)   # NaN propagates through the product and relu
    nan = np.isnan(expect)
    assert np.array_equal(np.isnan(g), nan)
    assert np.array_equal(g[~nan].astype(np.float64), expect[~nan])


def test_closed_forms_on_gpu():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["single_token"]
    for c in cases:
        H = max(16, c["heads"])       # the kernel needs H % 16 == 0: pad with zero heads
        q = np.zeros((1, 1, H, 128), np.uint8)
        kv = np.zeros((1, 132), np.uint8)
        if "q_fill" in c:
            q[0, 0, :c["heads"]] = int(c["q_fill"], 16)
        for h, d, code in c.get("q", []):
            q[0, 0, h, d] = int(code, 16)
        if "k_fill" in c:
            kv[0, :128] = int(c["k_fill"], 16)
        for d, code in c.get("k", []):
            kv[0, d] = int(code, 16)
        kv[0, 128:] = np.frombuffer(struct.pack("<f", c["scale"]), np.uint8)
        w = np.zeros((1, H), np.float32)
        w[0, :c["heads"]] = c["w"]
        case = wl.Workload(c["name"], q, kv, w, np.array([1], np.int32), np.array([[0, -1]], np.int32), 2, 1, k=1)
        g, idx = run_gpu(case, k=1)
        assert abs(g[0, 0] - c["expected"]) <= 1e-6 * max(1.0, abs(c["expected"])), (c["name"], g[0, 0])
        assert g[0, 1] == -np.inf and idx[0, 0] == 0


@pytest.mark.parametrize("heads", [32, 64])
@pytest.mark.parametrize("next_n", [1, 2, 4])
def test_boundary_sweep_small(next_n, heads):
    ctx = [c for c in SWEEP_SMALL if c >= 1]
    case = wl.make_case(batch=len(ctx), next_n=next_n, heads=heads, ctx=ctx, max_model_len=8200,
                        seed=1000 + 10 * next_n + heads)
    _parity(case, what=f"sweep<=8193 N={next_n} H={heads}")


@pytest.mark.parametrize("heads", [32, 64])
@pytest.mark.parametrize("next_n", [1, 2, 4])
def test_boundary_sweep_large(next_n, heads):
    case = wl.make_case(batch=len(SWEEP_LARGE), next_n=next_n, heads=heads, ctx=SWEEP_LARGE,
                        max_model_len=202752, seed=2000 + 10 * next_n + heads)
    _parity(case, what=f"sweep>=16383 N={next_n} H={heads}")


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_named_workload(name):
    case = wl.make_named(name)
    _parity(case, what=name)


@pytest.mark.parametrize("heads,next_n", [(16, 1), (48, 3), (80, 1), (96, 2), (112, 1), (128, 4),
                                           (32, 3), (64, 3), (80, 3), (128, 3)])
def test_other_head_counts(heads, next_n):
    case = wl.make_case(batch=5, next_n=next_n, heads=heads, ctx=[1, 70, 2049, 300, 4100],
                        max_model_len=4200, seed=3000 + heads + next_n)
    _parity(case, what=f"H={heads} N={next_n}")


@pytest.mark.parametrize("heads,next_n", [(16, 2), (16, 3), (16, 4), (48, 2), (32, 3), (64, 4), (48, 3)])
def test_half_stage_instances(heads, next_n):
    """Every half-stage kernel (a wave holds several decode rows of a request, pages under
    64 tokens) in a call too large for the small-call form: 40 requests; the last two shapes
    split each request's rows over two row groups."""
    ctx = [1, 70, 2049, 300, 4100, 64, 65, 2048, 4095, 1000] * 4
    case = wl.make_case(batch=len(ctx), next_n=next_n, heads=heads, ctx=ctx, max_model_len=4200,
                        seed=3100 + heads + next_n)
    _parity(case, what=f"half-stage H={heads} N={next_n}")


@pytest.mark.parametrize("batch,max_ctx", [(64, 400), (65, 400), (300, 400), (5500, 40), (8192, 24)])
def test_request_counts(batch, max_ctx):
    """Up to 64 requests each wave scans the context lengths itself (one per lane); above,
    the workgroup shares one scan in LDS (at 300 requests two per thread; at 5500 and at
    the largest batch the call accepts, 8192, 22 and 32 per thread and more than 64 KB of
    LDS). Empty contexts included."""
    rng = np.random.default_rng(6000 + batch)
    ctx = rng.integers(0, max_ctx, batch)
    ctx[0], ctx[-1], ctx[batch // 2] = 0, max_ctx - 15, min(64, max_ctx - 1)
    case = wl.make_case(batch=batch, next_n=2, heads=32, ctx=ctx.tolist(), max_model_len=max_ctx,
                        seed=6000 + batch)
    _parity(case, what=f"B={batch}")


# Small calls (at most 64 requests, one row group, and a grid of no more than one workgroup
# per CU holding a wave for every stage of every request at its largest context) take the
# form where each wave's stage is fixed by its index. Shapes on both sides of the size limit
# (64 requests, H = 16, L = 960 fits exactly; L = 1024 does not), empty and full contexts,
# a context filling every stage with no tail, several decode rows per wave, 16-token pages.
@pytest.mark.parametrize("batch,next_n,heads,L,ctx,block_size", [
    (64, 1, 16, 960, "random", 1),
    (64, 1, 16, 1024, "random", 1),
    (1, 1, 64, 192, [192], 1),
    (3, 1, 64, 4096, [0, 64, 4096], 1),
    (4, 4, 16, 2048, [1, 100, 2048, 1000], 1),
    (16, 2, 32, 2048, "random", 1),
    (5, 1, 32, 2048, [17, 2048, 1, 640, 1999], 16),
])
def test_small_calls(batch, next_n, heads, L, ctx, block_size):
    if ctx == "random":
        rng = np.random.default_rng(7000 + batch + L)
        ctx = rng.integers(0, L + 1, batch)
        ctx[0], ctx[-1] = L, 0
        ctx = ctx.tolist()
    nblk = sum((c + block_size - 1) // block_size for c in ctx)
    case = wl.make_case(batch=batch, next_n=next_n, heads=heads, ctx=ctx, max_model_len=L,
                        seed=7100 + batch + L, block_size=block_size, pool=nblk + 5)
    _parity(case, what=f"small B={batch} N={next_n} H={heads} L={L} S={block_size}")


@pytest.mark.parametrize("k", [1, 7, 100, 2047, 2048])
def test_k_values(k):
    case = wl.make_case(batch=6, next_n=2, heads=32, ctx=[1, 2, 100, 2048, 2050, 9000],
                        max_model_len=9000, seed=4000 + k, k=k)
    _parity(case, k=k, what=f"k={k}")


# block_size > 1: token t is slot t % S of block table[t // S] (the page's reference walks
# blocks; the page lists 16, 64 and 256 as the block sizes tried). Context lengths that
# end mid-block, a permuted block pool and one interleaved across requests.
@pytest.mark.parametrize("block_size,table", [(2, "permuted"), (16, "permuted"), (64, "interleaved"),
                                              (256, "permuted")])
@pytest.mark.parametrize("next_n,heads", [(1, 64), (2, 32), (4, 32)])
def test_block_sizes(block_size, table, next_n, heads):
    ctx = [1, 15, 16, 17, 63, 64, 65, 255, 257, 2049, 4100]
    nblk = sum((c + block_size - 1) // block_size for c in ctx)
    case = wl.make_case(batch=len(ctx), next_n=next_n, heads=heads, ctx=ctx, max_model_len=4160,
                        seed=5000 + block_size + 10 * next_n, table=table, block_size=block_size,
                        pool=nblk + 7)
    assert case.block_size == block_size
    _parity(case, what=f"S={block_size} {table} N={next_n} H={heads}")


@pytest.mark.parametrize("block_size", [8192, 65536])
def test_largest_block_sizes(block_size):
    """Pages of 8192 tokens and of 65536, the largest size the call accepts: contexts that
    end just before, at and just after a page boundary, and rows past 32768 positions
    (the chunked top-k)."""
    ctx = [1, 8191, 8192, 8193, 65535, 65536, 65537, 70000]
    nblk = sum((c + block_size - 1) // block_size for c in ctx)
    case = wl.make_case(batch=len(ctx), next_n=1, heads=64, ctx=ctx, max_model_len=70016,
                        seed=5100 + block_size % 1000, block_size=block_size, pool=nblk + 3)
    assert case.block_size == block_size
    _parity(case, what=f"S={block_size}")
