"""CPU oracle for the fp8 paged MQA logits and the per-row top-k that follows them.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library under ``fp8_paged_mqa_amd/`` and its binding) never calls it,
and this module imports nothing from the product path.

What it computes, and where that is defined
-------------------------------------------
Source page: the stepcodex.com issue mirror "[Bug] aiter ops triton attention
pa_mqa_logits" (stepcodex.com/en/issue/bug-aiter-ops-triton-attention-pa),
section "Minimal reproduction": the torch reference function (``torch_ref``)
and the reproducer's ``test()``.

* The KV cache row of a token holds D fp8-e4m3fn bytes followed by 4 bytes that
  are read as one fp32 dequant scale. The row is dequantised as fp8 value times
  scale before the dot product.
* The cache is [num_blocks, block_size, 1, D+4]; the reference reads block_size
  from that shape and walks a request's blocks: token t is slot t % block_size of
  block block_tables[b][t // block_size]. The reproducer uses block_size 1.
* All H query heads of a decode row are dotted with the same dequantised key
  (MQA: the cache has one key head).
* Decode row j of request b sits at position ctx - N + j, where ctx is the
  request's context length and N = next_n; token t is visible to it iff
  t < ctx and t <= ctx - N + j. Every other slot of the output row is -inf.
* logit = sum over heads of weight[row, h] * relu(score_h), row = b*N + j.
* The reproducer keeps k = min(2048, ctx) positions per row with ``torch.topk``
  and compares the two selections as sets (indices sorted before comparing).

Precision: the page's text calls the reference "bf16", yet its code upcasts to
fp32. This oracle reads the method as its exact mathematical definition and
evaluates it in float64:

* every finite e4m3fn value is an integer multiple of 2**-9 with magnitude
  below 2**18, so a 128-term dot product of two such vectors is a multiple of
  2**-18 below 2**43 in magnitude: exact in float64 whatever the summation
  order (the matmul below is therefore exact);
* the scale product, the relu, the weight product and the head sum are then
  rounded once each in float64.

Top-k: the row's visible positions are ordered by (logit descending, position
ascending), with -0.0 equal to +0.0 (float comparison already treats them as
equal), and the first min(k, visible) positions are kept. The page leaves the
order of equal logits open; lowest-position-first is the reading taken here.

No blocking, fusion or reordering beyond these steps is done.
"""
from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 128          # index_head_dim of the models the page names (D)
ROW_BYTES = HEAD_DIM + 4  # D fp8 bytes, then one little-endian fp32 scale


# ---------------------------------------------------------------------------
# Step 1: e4m3fn decode.
# The page's reference views the cache bytes as torch.float8_e4m3fn. That
# dtype is the OCP 8-bit floating point E4M3 format: 1 sign bit, 4 exponent
# bits (bias 7), 3 mantissa bits, no infinities, S.1111.111 is NaN, exponent
# field 0 encodes subnormals m * 2**-9.
# ---------------------------------------------------------------------------
def decode_e4m3fn(code: int) -> float:
    """Value of one e4m3fn byte, from the format definition."""
    code = int(code) & 0xFF
    sign = -1.0 if (code >> 7) else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return math.nan
    if exponent == 0:
        return sign * mantissa * 2.0 ** -9          # (m / 8) * 2**(1 - 7)
    return sign * (8 + mantissa) * 2.0 ** (exponent - 10)  # (1 + m/8) * 2**(e - 7)


E4M3FN_VALUES = np.array([decode_e4m3fn(c) for c in range(256)], dtype=np.float64)


def decode_bytes(codes: np.ndarray) -> np.ndarray:
    """Elementwise e4m3fn decode of a uint8 array into float64."""
    return E4M3FN_VALUES[np.asarray(codes, dtype=np.uint8)]


# ---------------------------------------------------------------------------
# Step 2: the cache row. Bytes [0, D) are fp8 key values, bytes [D, D+4) are
# the per-token fp32 scale, read little-endian (``.view(torch.float32)`` of the
# trailing bytes in the page's reference). A block holds block_size such rows.
# ---------------------------------------------------------------------------
def block_size_of(kv_cache: np.ndarray) -> int:
    """block_size of a cache shaped [num_blocks, D+4] (block_size 1),
    [num_blocks, block_size, D+4] or [num_blocks, block_size, 1, D+4]."""
    kv = np.asarray(kv_cache)
    return 1 if kv.ndim == 2 else int(kv.shape[1])


def split_kv_rows(kv_cache: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Returns (key values [num_blocks * block_size, D] float64, scales [...] float64),
    row blk * block_size + slot."""
    kv = np.asarray(kv_cache, dtype=np.uint8).reshape(-1, ROW_BYTES)
    keys = decode_bytes(kv[:, :HEAD_DIM])
    scales = np.ascontiguousarray(kv[:, HEAD_DIM:ROW_BYTES]).view("<f4")[:, 0]
    return keys, scales.astype(np.float64)


def token_rows(table_row: np.ndarray, ctx: int, block_size: int) -> np.ndarray:
    """Cache row of tokens 0..ctx-1 of one request: slot t % block_size of block
    table_row[t // block_size]."""
    t = np.arange(ctx, dtype=np.int64)
    return np.asarray(table_row)[t // block_size].astype(np.int64) * block_size + t % block_size


def visible_count(ctx: int, next_n: int, j: int, max_model_len: int) -> int:
    """Number of visible positions of decode row j: t <= ctx - N + j (and t < ctx,
    which that already implies), capped by the output row length."""
    return max(0, min(ctx - next_n + j + 1, max_model_len))


def _check_preconditions(context_lens, block_tables, max_model_len, block_size=1):
    for b, ctx in enumerate(np.asarray(context_lens).tolist()):
        if ctx < 0 or ctx > max_model_len or ctx > block_tables.shape[1] * block_size:
            raise ValueError(
                f"request {b}: context length {ctx} outside [0, min(max_model_len, table capacity)]")


# ---------------------------------------------------------------------------
# Steps 3-5: scores, relu, weights, head sum, mask.
# ---------------------------------------------------------------------------
def paged_mqa_logits(q, kv_cache, weights, context_lens, block_tables, max_model_len):
    """Logits [B*N, max_model_len] float64.

    q            uint8 [B, N, H, D]   e4m3fn bytes
    kv_cache     uint8 [num_blocks, (block_size, (1,)) D + 4]
    weights      float [B*N, H]
    context_lens int   [B]
    block_tables int   [B, W]         block of logical token t: entry t // block_size
    """
    q = np.asarray(q, dtype=np.uint8)
    B, N, H, D = q.shape
    assert D == HEAD_DIM
    block_tables = np.asarray(block_tables)
    bs = block_size_of(kv_cache)
    _check_preconditions(context_lens, block_tables, max_model_len, bs)
    keys, scales = split_kv_rows(kv_cache)
    w = np.asarray(weights, dtype=np.float64).reshape(B * N, H)
    qv = decode_bytes(q)                                   # [B, N, H, D]
    out = np.full((B * N, max_model_len), -np.inf, dtype=np.float64)
    for b in range(B):
        ctx = int(context_lens[b])
        if ctx <= 0:
            continue
        phys = token_rows(block_tables[b], ctx, bs)
        k_b = keys[phys]                                   # [ctx, D]  key of token t
        s_b = scales[phys]                                 # [ctx]
        for j in range(N):
            nv = visible_count(ctx, N, j, max_model_len)
            if nv == 0:
                continue
            score = k_b[:nv] @ qv[b, j].T                  # [nv, H]  q_h . k_t, exact
            x = score * s_b[:nv, None]                     # dequant scale on the key
            out[b * N + j, :nv] = np.maximum(x, 0.0) @ w[b * N + j]   # sum_h w_h relu(x_h)
    return out


def paged_mqa_logit_at(q, kv_cache, weights, context_lens, block_tables, max_model_len, row, t):
    """One logit, computed on its own with plain loops (for sampled checks at
    sizes where the whole output is not wanted)."""
    q = np.asarray(q, dtype=np.uint8)
    B, N, H, D = q.shape
    b, j = divmod(int(row), N)
    ctx = int(context_lens[b])
    if t < 0 or t >= visible_count(ctx, N, j, max_model_len):
        return -math.inf
    bs = block_size_of(kv_cache)
    kv = np.asarray(kv_cache, dtype=np.uint8).reshape(-1, ROW_BYTES)
    phys = int(block_tables[b, t // bs]) * bs + t % bs
    key = decode_bytes(kv[phys, :HEAD_DIM])
    scale = float(np.ascontiguousarray(kv[phys, HEAD_DIM:ROW_BYTES]).view("<f4")[0])
    w = np.asarray(weights, dtype=np.float64).reshape(B * N, H)[row]
    total = 0.0
    for h in range(H):
        score = float(np.dot(decode_bytes(q[b, j, h]), key))
        total += float(w[h]) * max(score * scale, 0.0)
    return total


# ---------------------------------------------------------------------------
# Step 6: per-row top-k.
# ---------------------------------------------------------------------------
def topk_row(values: np.ndarray, k: int) -> np.ndarray:
    """Positions of the k largest entries of ``values`` (all of them if fewer),
    ties broken by lowest position, returned sorted ascending."""
    values = np.asarray(values, dtype=np.float64)
    order = np.lexsort((np.arange(values.size), -values))   # last key is primary
    return np.sort(order[:min(k, values.size)])


def topk(logits, context_lens, next_n, k, max_model_len=None):
    """Indices [B*N, k] int32. Row r keeps min(k, visible_r) positions of its
    visible prefix (ascending), then -1 padding."""
    logits = np.asarray(logits)
    rows, L = logits.shape
    if max_model_len is None:
        max_model_len = L
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        b, j = divmod(r, next_n)
        nv = visible_count(int(context_lens[b]), next_n, j, max_model_len)
        sel = topk_row(logits[r, :nv], k)
        out[r, :sel.size] = sel
    return out


# ---------------------------------------------------------------------------
# Upstream of the op: writing the indexer's keys into the cache.
#
# The page's reference reads a token's row as 128 e4m3fn codes times one fp32
# scale (bytes [D, D+4) of the row). The page does not say how the writer picks
# that scale; the reading taken here is the per-token absolute maximum mapped
# onto the largest finite e4m3fn value: scale = amax / 448 in fp32, codes =
# e4m3fn(x / scale) with x / scale computed in fp32 and rounded to nearest even.
# A row of zeros gets scale 1 and the codes of its zeros (-0.0 is code 0x80, as
# everywhere else). NaN inputs give NaN codes and
# scale; an input of infinite magnitude gives an infinite scale.
# ---------------------------------------------------------------------------
E4M3FN_MAX = 448.0


def encode_e4m3fn(x) -> np.ndarray:
    """Round each float64 value to the nearest e4m3fn code, ties to the even code
    (OCP FP8 E4M3 with the fn convention: no infinities, S.1111.111 is NaN).
    Magnitudes that round above 448 become NaN, as in a non-saturating
    conversion: 464, halfway between 448 and the next step 480, ties to 448
    (even mantissa); anything larger overflows. Returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    finite_codes = np.arange(0x7F, dtype=np.uint8)          # 0x00 .. 0x7E: +0 .. 448
    mags = E4M3FN_VALUES[finite_codes]                      # increasing
    ax = np.abs(x)
    hi = np.searchsorted(mags, ax, side="left")             # first code with value >= |x|
    hi_c = np.minimum(hi, 0x7E)
    lo_c = np.maximum(hi_c - 1, 0)
    d_lo = ax - mags[lo_c]
    d_hi = mags[hi_c] - ax
    exact = mags[hi_c] == ax
    take_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    code = np.where(take_hi, hi_c, lo_c).astype(np.uint8)
    # beyond 448: above the tie at 464 the value rounds to 480, which has no code
    code = np.where(ax > 464.0, np.uint8(0x7F), code)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    sign = (np.signbit(x) & ~np.isnan(x)).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def quantize_k_row(k_row) -> tuple[np.ndarray, np.float32]:
    """One token's 128 keys (float32 values) -> (128 e4m3fn codes, fp32 scale)."""
    k32 = np.asarray(k_row, dtype=np.float32)
    amax = np.float32(np.max(np.abs(k32))) if not np.isnan(k32).any() else np.float32(np.nan)
    if amax == 0:  # scale 1: the codes of the zeros themselves (-0.0 keeps its sign)
        return encode_e4m3fn(k32.astype(np.float64)), np.float32(1.0)
    scale = np.float32(amax / np.float32(E4M3FN_MAX))       # fp32 division
    scaled = (k32 / scale).astype(np.float32)                # fp32 division per element
    return encode_e4m3fn(scaled.astype(np.float64)), scale


def write_k_cache(k, slot_mapping, kv_cache):
    """Returns a copy of ``kv_cache`` (uint8, [num_slots, D+4] or [num_blocks,
    block_size, (1,) D+4]) with token i's row written at slot slot_mapping[i]
    (row blk * block_size + offset); slots outside [0, num_slots) are skipped.
    k is [T, D] float values (bf16 inputs are passed as their float32 values)."""
    out = np.array(kv_cache, dtype=np.uint8, copy=True)
    rows = out.reshape(-1, ROW_BYTES)
    k = np.asarray(k, dtype=np.float32)
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0 or slot >= rows.shape[0]:
            continue
        codes, scale = quantize_k_row(k[i])
        rows[slot, :HEAD_DIM] = codes
        rows[slot, HEAD_DIM:ROW_BYTES] = np.frombuffer(np.float32(scale).astype("<f4").tobytes(), dtype=np.uint8)
    return out


# ---------------------------------------------------------------------------
# The non-paged (prefill) form of the same logits. The page names the prefill
# indexer kernel (aiter's fp8_mqa_logits) in "Observations while narrowing it
# down" as computing the same quantity over contiguous keys for M query rows, but
# gives no signature. Reading taken: keys are contiguous (codes [N, D] plus one
# fp32 scale per key), query row m sees keys n with ks[m] <= n < ke[m] (ranges
# clamped to [0, N]; an empty range leaves the row -inf), and
#   logit[m, n] = sum_h w[m, h] * relu(scale_n * (q[m, h, :] . k[n, :])).
# ---------------------------------------------------------------------------
def mqa_logits(q, k, k_scale, weights, ks, ke):
    """Logits [M, N] float64.

    q        uint8 [M, H, D]  e4m3fn bytes
    k        uint8 [N, D]     e4m3fn bytes
    k_scale  float [N]
    weights  float [M, H]
    ks, ke   int   [M]        query row m sees keys [ks[m], ke[m])
    """
    q = np.asarray(q, dtype=np.uint8)
    M, H, D = q.shape
    assert D == HEAD_DIM
    keys = decode_bytes(np.asarray(k, dtype=np.uint8))             # [N, D]
    N = keys.shape[0]
    scales = np.asarray(k_scale, dtype=np.float32).astype(np.float64)
    w = np.asarray(weights, dtype=np.float64).reshape(M, H)
    qv = decode_bytes(q)                                            # [M, H, D]
    out = np.full((M, N), -np.inf, dtype=np.float64)
    for m in range(M):
        lo = min(max(int(ks[m]), 0), N)
        hi = min(max(int(ke[m]), 0), N)
        if hi <= lo:
            continue
        score = keys[lo:hi] @ qv[m].T                               # [n, H], exact
        x = score * scales[lo:hi, None]
        out[m, lo:hi] = np.maximum(x, 0.0) @ w[m]
    return out
