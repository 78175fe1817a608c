"""Seeded synthetic inputs for the paged MQA indexer (logits + top-k).

This module only draws and lays out inputs: it holds none of the method's
arithmetic (no decode, no dot product, no selection). Values are drawn in
float32 and encoded to e4m3fn bytes with torch's CPU cast (round to nearest
even); everything downstream sees bytes. Tests, the benchmark and the smoke
check all build their inputs here, so the HIP path and the CPU oracle always
see identical bytes.

Layouts (the calling convention of the paged indexer in the stepcodex.com
issue "[Bug] aiter ops triton attention pa_mqa_logits", section "Minimal
reproduction"):
  q             uint8 [B, N, H, 128]   e4m3fn
  kv_cache      uint8 [num_blocks, 132] 128 e4m3fn key bytes + fp32 scale (LE)
                      ([num_blocks, block_size, 132] for block_size > 1)
  weights       f32   [B*N, H]
  context_lens  i32   [B]
  block_tables  i32   [B, W]           block of token t: entry t // block_size;
                                       entries past the last block hold -1
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 128
ROW_BYTES = HEAD_DIM + 4
TOPK = 2048


@dataclass
class Workload:
    name: str
    q: np.ndarray
    kv_cache: np.ndarray
    weights: np.ndarray
    context_lens: np.ndarray
    block_tables: np.ndarray
    max_model_len: int
    next_n: int
    k: int = TOPK
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def heads(self) -> int:
        return int(self.q.shape[2])

    @property
    def rows(self) -> int:
        return self.batch * self.next_n

    @property
    def num_blocks(self) -> int:
        return int(self.kv_cache.shape[0])

    @property
    def block_size(self) -> int:
        return 1 if self.kv_cache.ndim == 2 else int(self.kv_cache.shape[1])

    @property
    def sum_ctx(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    def visible(self) -> np.ndarray:
        """Visible positions per row: max(0, min(ctx - N + j + 1, L))."""
        ctx = np.repeat(self.context_lens.astype(np.int64), self.next_n)
        j = np.tile(np.arange(self.next_n), self.batch)
        return np.clip(ctx - self.next_n + j + 1, 0, self.max_model_len)


def to_e4m3fn_bytes(x: np.ndarray) -> np.ndarray:
    """float32 -> e4m3fn bytes via torch's CPU cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _kv_rows(key_bytes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    rows = np.empty((key_bytes.shape[0], ROW_BYTES), dtype=np.uint8)
    rows[:, :HEAD_DIM] = key_bytes
    rows[:, HEAD_DIM:] = np.ascontiguousarray(scales, dtype="<f4").view(np.uint8).reshape(-1, 4)
    return rows


def _poison_rows(kv: np.ndarray, used: np.ndarray) -> None:
    """Unreferenced rows become NaN keys (0x7F) with a NaN scale, so that a
    gather from a wrong row cannot go unnoticed."""
    unused = np.ones(kv.shape[0], dtype=bool)
    unused[used] = False
    kv[unused, :HEAD_DIM] = 0x7F
    kv[unused, HEAD_DIM:] = np.frombuffer(np.float32(np.nan).tobytes(), dtype=np.uint8)


def _tables_from_assignment(ctx: np.ndarray, width: int, assign) -> np.ndarray:
    bt = np.full((ctx.size, width), -1, dtype=np.int32)
    for b, c in enumerate(ctx.tolist()):
        bt[b, :c] = assign(b, c)
    return bt


def build(name, rng, *, batch, next_n, heads, ctx, max_model_len, pool, table,
          table_width=None, outlier_frac=0.0, poison_unused=True, k=TOPK,
          key_fn=None, scale_fn=None, q_fn=None, w_fn=None, block_size=1) -> Workload:
    """Draws a workload in the fixed order ctx -> tables -> q -> K -> scales ->
    outliers -> weights. ``ctx`` is an int array already drawn by the caller.

    table: "identity"  request b reads blocks [0, n_b) (every request the same)
           "permuted"  one permutation of the pool, sliced per request in order
           "interleaved" one permutation, dealt out block by block across the
                       requests still running (for i, for b with n_b > i)
    where n_b = ceil(ctx_b / block_size) and the pool counts blocks. With
    block_size > 1 the cache is [pool, block_size, 132] and ``table_width``
    counts blocks.
    """
    ctx = np.asarray(ctx, dtype=np.int32)
    bs = int(block_size)
    if bs > 1:
        return _build_blocked(name, rng, batch=batch, next_n=next_n, heads=heads, ctx=ctx,
                              max_model_len=max_model_len, pool=pool, table=table,
                              table_width=table_width, poison_unused=poison_unused, k=k, bs=bs)
    width = int(table_width or max(1, int(ctx.max(initial=1))))
    if table == "identity":
        bt = _tables_from_assignment(ctx, width, lambda b, c: np.arange(c))
    elif table == "permuted":
        perm = rng.permutation(pool).astype(np.int32)
        offs = np.concatenate([[0], np.cumsum(ctx.astype(np.int64))])
        assert offs[-1] <= pool, "pool smaller than the sum of context lengths"
        bt = _tables_from_assignment(ctx, width, lambda b, c: perm[offs[b]:offs[b] + c])
    elif table == "interleaved":
        perm = rng.permutation(pool).astype(np.int32)
        b_idx = np.repeat(np.arange(ctx.size), ctx)
        t_idx = np.concatenate([np.arange(c) for c in ctx.tolist()]) if ctx.size else np.zeros(0, int)
        order = np.lexsort((b_idx, t_idx))            # token-major, then request
        assert order.size <= pool
        bt = np.full((ctx.size, width), -1, dtype=np.int32)
        bt[b_idx[order], t_idx[order]] = perm[:order.size]
    else:
        raise ValueError(table)

    rows = batch * next_n
    q_f = q_fn(rng, (batch, next_n, heads, HEAD_DIM)) if q_fn else \
        rng.standard_normal((batch, next_n, heads, HEAD_DIM), dtype=np.float32)
    k_f = key_fn(rng, (pool, HEAD_DIM)) if key_fn else \
        rng.standard_normal((pool, HEAD_DIM), dtype=np.float32)
    scales = scale_fn(rng, pool) if scale_fn else \
        rng.lognormal(0.0, 0.5, size=pool).astype(np.float32)
    if outlier_frac > 0:
        hot = rng.random(pool) < outlier_frac
        k_f[hot] *= 8.0
    weights = w_fn(rng, (rows, heads)) if w_fn else \
        rng.standard_normal((rows, heads), dtype=np.float32)

    kv = _kv_rows(to_e4m3fn_bytes(k_f), scales)
    if poison_unused:
        used = bt[bt >= 0]
        _poison_rows(kv, used)
    return Workload(name=name, q=to_e4m3fn_bytes(q_f), kv_cache=kv,
                    weights=np.ascontiguousarray(weights, dtype=np.float32),
                    context_lens=ctx, block_tables=bt, max_model_len=int(max_model_len),
                    next_n=int(next_n), k=int(k),
                    meta={"table": table, "pool": int(pool)})


def _build_blocked(name, rng, *, batch, next_n, heads, ctx, max_model_len, pool, table,
                   table_width, poison_unused, k, bs) -> Workload:
    """build() for block_size > 1: tables of block ids, cache [pool, bs, 132]."""
    nblk = (ctx.astype(np.int64) + bs - 1) // bs
    width = int(table_width or max(1, int(nblk.max(initial=1))))
    if table == "identity":
        bt = _tables_from_assignment(nblk, width, lambda b, n: np.arange(n))
    elif table == "permuted":
        perm = rng.permutation(pool).astype(np.int32)
        offs = np.concatenate([[0], np.cumsum(nblk)])
        assert offs[-1] <= pool, "pool smaller than the blocks in use"
        bt = _tables_from_assignment(nblk, width, lambda b, n: perm[offs[b]:offs[b] + n])
    elif table == "interleaved":
        perm = rng.permutation(pool).astype(np.int32)
        b_idx = np.repeat(np.arange(nblk.size), nblk)
        i_idx = np.concatenate([np.arange(n) for n in nblk.tolist()]) if nblk.size else np.zeros(0, int)
        order = np.lexsort((b_idx, i_idx))
        assert order.size <= pool
        bt = np.full((nblk.size, width), -1, dtype=np.int32)
        bt[b_idx[order], i_idx[order]] = perm[:order.size]
    else:
        raise ValueError(table)
    rows = batch * next_n
    q_f = rng.standard_normal((batch, next_n, heads, HEAD_DIM), dtype=np.float32)
    k_f = rng.standard_normal((pool * bs, HEAD_DIM), dtype=np.float32)
    scales = rng.lognormal(0.0, 0.5, size=pool * bs).astype(np.float32)
    weights = rng.standard_normal((rows, heads), dtype=np.float32)
    kv = _kv_rows(to_e4m3fn_bytes(k_f), scales)
    if poison_unused:  # every row that no token t < ctx reads
        used = np.concatenate([bt[b, np.arange(c) // bs].astype(np.int64) * bs + np.arange(c) % bs
                               for b, c in enumerate(ctx.tolist())] + [np.zeros(0, np.int64)])
        _poison_rows(kv, used)
    return Workload(name=name, q=to_e4m3fn_bytes(q_f), kv_cache=kv.reshape(pool, bs, ROW_BYTES),
                    weights=np.ascontiguousarray(weights, dtype=np.float32),
                    context_lens=ctx, block_tables=bt, max_model_len=int(max_model_len),
                    next_n=int(next_n), k=int(k),
                    meta={"table": table, "pool": int(pool), "block_size": bs})


# ---------------------------------------------------------------------------
# The five named workloads, keyed by a short name that says what each one is.
# ---------------------------------------------------------------------------
WORKLOADS = {
    "decode_b1_ctx2049": "decode bs=1 N=1 H=32 ctx=2049 L=4096 identity table (reproducer shape)",
    "decode_b64_ctx8192": "decode bs=64 N=1 H=64 ctx~U[1,8192] L=8192 permuted 600k-row pool",
    "mtp_b32_n2_ctx32k": "MTP verify bs=32 N=2 H=64 ctx~U[2048,32768] L=32768 permuted pool",
    "long_b4_ctx202752": "long context bs=4 N=1 H=64 ctx={65536,131071,131072,202752} L=202752 540k pool, 1% x8 keys",
    "mixed_b128_n4": "mixed serving bs=128 N=4 H=32 ctx~lognormal(6000,1.2) L=202752 interleaved pool",
    # one GPU's share when the long-context requests are split across 8 GPUs by token
    # range (each GPU then selects a local top-k that one all-gather merges)
    "long_b4_cp8_shard": "context-parallel shard: long context bs=4 ctx/8={8192,16384,16384,25344} L=25344 67.5k pool, 1% x8 keys",
}
DEFAULT_WORKLOAD = "decode_b64_ctx8192"


def make_named(workload: str, *, poison_unused: bool = True, seed: int | None = None,
               block_size: int = 1) -> Workload:
    """The named workload (a key of WORKLOADS). With block_size S > 1 the same context
    lengths are laid out in blocks of S tokens: the pool becomes ceil(rows / S) blocks
    (at least the blocks in use) and the table kind is kept; keys and scales are drawn
    afresh."""
    if workload not in WORKLOADS:
        raise ValueError(f"unknown workload {workload!r}; one of {list(WORKLOADS)}")
    n = list(WORKLOADS).index(workload) + 1  # selects the recipe below and the default seed
    rng = np.random.Generator(np.random.PCG64(42 + (n - 1) if seed is None else seed))
    name = f"{workload}: {WORKLOADS[workload]}"
    if block_size > 1:
        return _make_named_blocked(n, rng, name, poison_unused, int(block_size))
    if n == 1:
        ctx = np.array([2049])
        return build(name, rng, batch=1, next_n=1, heads=32, ctx=ctx, max_model_len=4096,
                     pool=2065, table="identity", table_width=2065, poison_unused=poison_unused)
    if n == 2:
        ctx = rng.integers(1, 8192, size=64, endpoint=True)
        ctx[:5] = [2047, 2048, 2049, 4096, 4097]
        return build(name, rng, batch=64, next_n=1, heads=64, ctx=ctx, max_model_len=8192,
                     pool=600_000, table="permuted", table_width=8192,
                     poison_unused=poison_unused)
    if n == 3:
        ctx = rng.integers(2048, 32768, size=32, endpoint=True)
        return build(name, rng, batch=32, next_n=2, heads=64, ctx=ctx, max_model_len=32768,
                     pool=int(ctx.sum()), table="permuted", table_width=32768,
                     poison_unused=poison_unused)
    if n == 4:
        ctx = np.array([65536, 131071, 131072, 202752])
        return build(name, rng, batch=4, next_n=1, heads=64, ctx=ctx, max_model_len=202752,
                     pool=540_000, table="permuted", table_width=202752, outlier_frac=0.01,
                     poison_unused=poison_unused)
    if n == 6:
        ctx = np.array([8192, 16384, 16384, 25344])
        return build(name, rng, batch=4, next_n=1, heads=64, ctx=ctx, max_model_len=25344,
                     pool=67_500, table="permuted", table_width=25344, outlier_frac=0.01,
                     poison_unused=poison_unused)
    if n == 5:
        ctx = np.clip(np.round(np.exp(rng.normal(np.log(6000.0), 1.2, size=128))), 4, 202752)
        ctx = ctx.astype(np.int64)
        return build(name, rng, batch=128, next_n=4, heads=32, ctx=ctx, max_model_len=202752,
                     pool=int(ctx.sum()), table="interleaved", table_width=int(ctx.max()),
                     poison_unused=poison_unused)
    raise ValueError(n)


def _make_named_blocked(n, rng, name, poison_unused, bs) -> Workload:
    # Same context-length draws as make_named's block_size 1 path.
    if n == 1:
        ctx, kw = np.array([2049]), dict(batch=1, next_n=1, heads=32, max_model_len=4096, rows=2065,
                                         table="identity")
    elif n == 2:
        ctx = rng.integers(1, 8192, size=64, endpoint=True)
        ctx[:5] = [2047, 2048, 2049, 4096, 4097]
        kw = dict(batch=64, next_n=1, heads=64, max_model_len=8192, rows=600_000, table="permuted")
    elif n == 3:
        ctx = rng.integers(2048, 32768, size=32, endpoint=True)
        kw = dict(batch=32, next_n=2, heads=64, max_model_len=32768, rows=int(ctx.sum()), table="permuted")
    elif n == 4:
        ctx = np.array([65536, 131071, 131072, 202752])
        kw = dict(batch=4, next_n=1, heads=64, max_model_len=202752, rows=540_000, table="permuted")
    elif n == 6:
        ctx = np.array([8192, 16384, 16384, 25344])
        kw = dict(batch=4, next_n=1, heads=64, max_model_len=25344, rows=67_500, table="permuted")
    elif n == 5:
        ctx = np.clip(np.round(np.exp(rng.normal(np.log(6000.0), 1.2, size=128))), 4, 202752).astype(np.int64)
        kw = dict(batch=128, next_n=4, heads=32, max_model_len=202752, rows=int(ctx.sum()), table="interleaved")
    else:
        raise ValueError(n)
    rows = kw.pop("rows")
    need = int(((np.asarray(ctx, dtype=np.int64) + bs - 1) // bs).sum())
    pool = max(need, (rows + bs - 1) // bs)
    return build(f"{name}, block_size {bs}", rng, ctx=ctx, pool=pool, poison_unused=poison_unused,
                 block_size=bs, **kw)


def make_case(*, batch, next_n, heads, ctx, max_model_len=None, seed=0, table="permuted",
              pool=None, table_width=None, poison_unused=True, k=TOPK, block_size=1, **kw) -> Workload:
    """A small seeded case (for sweeps and edge cases). ``pool`` counts blocks."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = np.broadcast_to(np.asarray(ctx, dtype=np.int64), (batch,)).copy()
    L = int(max_model_len or max(1, int(ctx.max(initial=1))))
    if pool is None:
        nblk = (ctx + block_size - 1) // block_size
        pool = int(nblk.max(initial=1)) if table == "identity" else max(1, int(nblk.sum()))
    if block_size > 1:
        kw["block_size"] = block_size
    return build(f"case b{batch} n{next_n} h{heads} seed{seed}", rng, batch=batch,
                 next_n=next_n, heads=heads, ctx=ctx, max_model_len=L, pool=pool, table=table,
                 table_width=table_width, poison_unused=poison_unused, k=k, **kw)


def page_random_bytes_case(ctx_len: int, seed: int = 42, heads: int = 32,
                           max_model_len: int = 202752) -> Workload:
    """The reproducer's own recipe: every cache byte uniform random (so keys
    include NaN codes and the scales are arbitrary fp32 bit patterns), q ~ N(0,1)
    cast to e4m3fn, weights ~ N(0,1), identity table of ctx + 16 blocks."""
    rng = np.random.Generator(np.random.PCG64(seed))
    blocks = ctx_len + 16
    kv = rng.integers(0, 256, size=(blocks, ROW_BYTES), dtype=np.uint8)
    q = to_e4m3fn_bytes(rng.standard_normal((1, 1, heads, HEAD_DIM), dtype=np.float32))
    w = rng.standard_normal((1, heads), dtype=np.float32)
    bt = np.arange(blocks, dtype=np.int32)[None, :]
    return Workload(name=f"random-bytes ctx={ctx_len}", q=q, kv_cache=kv, weights=w,
                    context_lens=np.array([ctx_len], dtype=np.int32), block_tables=bt,
                    max_model_len=max_model_len, next_n=1)


# ---------------------------------------------------------------------------
# Sparse MLA decode inputs: latent rows of 576 e4m3fn codes (512 compressed + 64 rotary
# dims), 16 query heads per row, per-tensor fp32 scales, and per-row position lists of
# the shape the indexer's top-k emits (min(topk, visible) distinct positions in any
# order, then -1 padding).

MLA_KV_DIM = 576
MLA_HEADS = 16
MLA_SM_SCALE = float(np.float32(1.0 / np.sqrt(192.0)))  # 1/sqrt(128 + 64): DeepSeek-V3 head dims
MLA_Q_SCALE = 0.75
MLA_KV_SCALE = 1.25


@dataclass
class MlaCase:
    name: str
    next_n: int
    q: np.ndarray             # uint8 [B*N, 16, 576]
    kv_cache: np.ndarray      # uint8 [num_slots, 576] or [num_blocks, S, 576]
    block_tables: np.ndarray  # int32 [B, W]
    indices: np.ndarray       # int32 [B*N, topk]
    context_lens: np.ndarray  # int32 [B]
    q_scale: float
    kv_scale: float
    sm_scale: float

    @property
    def batch(self) -> int:
        return int(self.block_tables.shape[0])

    @property
    def rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def topk(self) -> int:
        return int(self.indices.shape[1])

    @property
    def block_size(self) -> int:
        return 1 if self.kv_cache.ndim == 2 else int(self.kv_cache.shape[1])

    @property
    def num_blocks(self) -> int:
        return int(self.kv_cache.shape[0])

    @property
    def listed(self) -> int:
        return int((self.indices >= 0).sum())


def make_mla_case(*, batch, next_n, ctx, topk=TOPK, block_size=1, seed=0, pool=None, table="permuted",
                  poison_unused=True, q_scale=MLA_Q_SCALE, kv_scale=MLA_KV_SCALE, sm_scale=MLA_SM_SCALE,
                  table_width=None, outlier_rows=0.0) -> MlaCase:
    """Seeded sparse-MLA inputs. ctx counts tokens of each request (the N query tokens
    included); row j of request b lists min(topk, ctx - N + j + 1) distinct positions of
    its visible prefix in random order. ``pool`` counts blocks of ``block_size`` tokens.
    Unreferenced cache rows hold NaN codes when ``poison_unused``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = np.broadcast_to(np.asarray(ctx, dtype=np.int64), (batch,)).copy()
    S = int(block_size)
    nblk = (ctx + S - 1) // S
    W = int(table_width or max(1, int(nblk.max(initial=1))))
    if pool is None:
        pool = max(1, int(nblk.sum()))
    if table == "permuted":
        perm = rng.permutation(pool)
        tables = np.full((batch, W), -1, dtype=np.int64)
        off = 0
        for b in range(batch):
            tables[b, :nblk[b]] = perm[off:off + nblk[b]]
            off += int(nblk[b])
        assert off <= pool, "pool too small"
    elif table == "identity":
        tables = np.tile(np.arange(W, dtype=np.int64), (batch, 1))
        assert W <= pool
    else:
        raise ValueError(table)
    q = to_e4m3fn_bytes(rng.standard_normal((batch * next_n, MLA_HEADS, MLA_KV_DIM), dtype=np.float32))
    vals = rng.standard_normal((pool * S, MLA_KV_DIM), dtype=np.float32)
    if outlier_rows:
        vals[rng.random(pool * S) < outlier_rows] *= 8.0
    rows = to_e4m3fn_bytes(vals)
    idx = np.full((batch * next_n, topk), -1, dtype=np.int64)
    used = np.zeros(pool * S, dtype=bool)
    for b in range(batch):
        for j in range(next_n):
            vis = max(0, int(ctx[b]) - next_n + j + 1)
            n = min(topk, vis)
            pos = rng.choice(vis, size=n, replace=False) if n else np.zeros(0, np.int64)
            idx[b * next_n + j, :n] = pos
            if n:
                used[tables[b][pos // S] * S + pos % S] = True
    if poison_unused:
        rows[~used] = 0x7F
    kv = rows if S == 1 else rows.reshape(pool, S, MLA_KV_DIM)
    return MlaCase(f"mla b{batch} n{next_n} topk{topk} S{S} seed{seed}", next_n, q, kv,
                   tables.astype(np.int32), idx.astype(np.int32), ctx.astype(np.int32),
                   float(np.float32(q_scale)), float(np.float32(kv_scale)), float(np.float32(sm_scale)))


def make_mla_workload(*, poison_unused=False, seed=None) -> MlaCase:
    """Sparse MLA decode behind the indexer's decode workload of 64 requests, N = 1,
    ctx ~ U{1..8192} (2047, 2048, 2049, 4096, 4097 forced): each row attends its
    min(2048, ctx) selected positions, gathered through a random permutation of a
    600 000-row latent cache (one token per block)."""
    rng = np.random.Generator(np.random.PCG64(4242 if seed is None else seed))
    ctx = rng.integers(1, 8193, size=64)
    ctx[:5] = [2047, 2048, 2049, 4096, 4097]
    return make_mla_case(batch=64, next_n=1, ctx=ctx, topk=TOPK, pool=600_000, table_width=8192,
                         seed=int(rng.integers(1 << 31)), poison_unused=poison_unused)
