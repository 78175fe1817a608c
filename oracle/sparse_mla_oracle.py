"""CPU oracle for sparse MLA decode over the indexer's selected positions.

TEST INFRASTRUCTURE, like ``mqa_oracle``: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; it imports nothing from
the product path.

What it computes, and where that is defined
-------------------------------------------
* The stepcodex.com issue "[Bug] aiter ops triton attention pa_mqa_logits", section
  "Downstream impact": the positions the indexer's top-k keeps are the ones the
  sparse attention of the next step attends to.
* The chat-gpts.plus summary (post 69330) of the aiter MLA decode issue, sections
  "问题场景" and "环境排查": MLA decode with fp8 queries and an fp8 KV cache, 16 query
  heads sharing one latent KV head (gqa ratio 16), 1 to 4 query tokens per request
  (speculative depth 3), correctness judged by the cosine difference of the output
  against a reference.
* vLLM pull request 31282, "The Bug": the MLA cache used with that kernel holds one
  token per page (block_size 1), reached through a block table.

The pages do not fix the MLA dimensions, the placement of the fp8 scales or the form
of the index list. Readings taken (each listed with the others in the design notes):

* latent rows of 576 dims (a 512-dim compressed KV part followed by a 64-dim rotary
  part, the published DeepSeek-V3 sizes); a query head is also 576 dims; the value
  of a token is the first 512 dims of its row;
* q and the cache hold e4m3fn codes with one fp32 scale each for the whole tensor
  (``q_scale``, ``kv_scale``); the softmax scale is an argument;
* for decode row r = b*N + j, ``indices[r]`` lists positions of request b; a negative
  entry is padding and attends nothing; a position is listed once per attended copy
  (duplicates are attended as often as they are listed); the row of position t is
  slot t % S of block ``block_tables[b][t // S]`` (S from the cache shape);
* score(h, t) = sm_scale * q_scale * kv_scale * (q[r, h, :] . k_t), with q and k_t the
  decoded codes; p = softmax over the row's listed positions;
  out[r, h, :] = kv_scale * sum_t p(h, t) * k_t[:512];
  lse[r, h] = log(sum_t exp(score(h, t))) (natural log);
* a row with no listed position has out = 0 and lse = -inf.

Precision: the 576-term dot products of decoded e4m3fn values are exact in float64
(each product is a multiple of 2**-18 below 2**17.6 in magnitude, so the sums stay
below 2**27.2 on a 2**-18 grid: 46 bits). Everything after that (scale product,
exponentials, sums, the value contraction) is float64 with the usual rounding.
"""
from __future__ import annotations

import numpy as np

from .mqa_oracle import decode_bytes

MLA_KV_DIM = 576   # compressed KV (512) + rotary (64) dims of a latent row
MLA_V_DIM = 512    # value dims: the compressed part of the row
MLA_HEADS = 16     # query heads per latent KV head (gqa ratio 16)


def mla_block_size_of(kv_cache: np.ndarray) -> int:
    """Cache shape [num_slots, 576] (one token per block) or [num_blocks, S, (1,) 576]."""
    kv = np.asarray(kv_cache)
    return 1 if kv.ndim == 2 else int(kv.shape[1])


def mla_rows_of(positions: np.ndarray, table_row: np.ndarray, block_size: int) -> np.ndarray:
    """Cache row (in units of 576-byte rows) of each listed position of one request."""
    t = np.asarray(positions, dtype=np.int64)
    entries = np.asarray(table_row, dtype=np.int64)[t // block_size]
    return entries * block_size + t % block_size


def sparse_mla_decode(q, q_scale, kv_cache, kv_scale, indices, block_tables, next_n, sm_scale):
    """(out [R, H, 512] float64, lse [R, H] float64).

    q            uint8 [R, H, 576] (or [B, N, H, 576]) e4m3fn codes
    kv_cache     uint8 [num_slots, 576] or [num_blocks, S, (1,) 576] e4m3fn codes
    indices      int   [R, topk] positions, negative = padding
    block_tables int   [B, W]
    """
    qb = np.asarray(q, dtype=np.uint8)
    qb = qb.reshape(-1, qb.shape[-2], qb.shape[-1])
    R, H, D = qb.shape
    assert D == MLA_KV_DIM
    S = mla_block_size_of(kv_cache)
    rows_all = np.asarray(kv_cache, dtype=np.uint8).reshape(-1, MLA_KV_DIM)
    num_blocks = rows_all.shape[0] // S
    tables = np.asarray(block_tables, dtype=np.int64)
    idx = np.asarray(indices, dtype=np.int64).reshape(R, -1)
    W = tables.shape[1]
    qv = decode_bytes(qb)                                           # [R, H, 576]
    c = float(np.float32(sm_scale)) * float(np.float32(q_scale)) * float(np.float32(kv_scale))
    vs = float(np.float32(kv_scale))
    out = np.zeros((R, H, MLA_V_DIM), dtype=np.float64)
    lse = np.full((R, H), -np.inf, dtype=np.float64)
    for r in range(R):
        b = r // next_n
        pos = idx[r][idx[r] >= 0]
        if pos.size == 0:
            continue
        if pos.max() >= W * S:
            raise ValueError(f"row {r}: position {pos.max()} beyond the block table ({W} x {S})")
        entries = tables[b][pos // S]
        if entries.min() < 0 or entries.max() >= num_blocks:
            raise ValueError(f"row {r}: block table entry outside the cache")
        keys = decode_bytes(rows_all[mla_rows_of(pos, tables[b], S)])   # [n, 576]
        score = (keys @ qv[r].T) * c                                # [n, H]; dot exact
        m = score.max(axis=0)
        e = np.exp(score - m)
        l = e.sum(axis=0)
        p = e / l
        out[r] = vs * (p.T @ keys[:, :MLA_V_DIM])
        lse[r] = m + np.log(l)
    return out, lse


def sparse_mla_error_bound(q, q_scale, kv_cache, kv_scale, indices, block_tables, next_n, sm_scale):
    """Per output element, kv_scale * sum_t p(h, t) * |k_t[c]| (float64, [R, H, 512]):
    the magnitude a relative error in the probabilities is measured against. By the
    triangle inequality it bounds |out| and equals it where the listed values of a column
    share one sign; with one listed position it is kv_scale * |k_t|, with a zero query
    kv_scale times the mean of |k_t| over the list."""
    qb = np.asarray(q, dtype=np.uint8)
    qb = qb.reshape(-1, qb.shape[-2], qb.shape[-1])
    R, H, _ = qb.shape
    S = mla_block_size_of(kv_cache)
    rows_all = np.asarray(kv_cache, dtype=np.uint8).reshape(-1, MLA_KV_DIM)
    tables = np.asarray(block_tables, dtype=np.int64)
    idx = np.asarray(indices, dtype=np.int64).reshape(R, -1)
    qv = decode_bytes(qb)
    c = float(np.float32(sm_scale)) * float(np.float32(q_scale)) * float(np.float32(kv_scale))
    bound = np.zeros((R, H, MLA_V_DIM), dtype=np.float64)
    for r in range(R):
        pos = idx[r][idx[r] >= 0]
        if pos.size == 0:
            continue
        keys = decode_bytes(rows_all[mla_rows_of(pos, tables[r // next_n], S)])
        score = (keys @ qv[r].T) * c
        e = np.exp(score - score.max(axis=0))
        p = e / e.sum(axis=0)
        bound[r] = float(np.float32(kv_scale)) * (p.T @ np.abs(keys[:, :MLA_V_DIM]))
    return bound
