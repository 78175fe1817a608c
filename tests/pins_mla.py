"""Checks that pin the sparse-MLA oracle to facts outside itself.

Each ``pin_*`` takes the oracle module ``oracle.sparse_mla_oracle`` (or a mutant
copy of it) and raises when it disagrees. Independent sources:
  * torch's float8_e4m3fn upcast for every decoded value;
  * torch.nn.functional.scaled_dot_product_attention and torch.logsumexp in
    float64 on rows gathered with plain loops from the block rule;
  * closed forms: one listed position (the output is that row's value), a zero
    query (the output is the mean of the listed values), a listed-twice position
    (its weight doubles), a dominating score (the softmax saturates exactly);
  * exact rational dot products (fractions.Fraction) for the scores;
  * invariants of the definition: order of the list and padding do not matter, the
    block layout does not matter.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

from fp8_paged_mqa_amd import workloads as wl

D, DV, H = 576, 512, 16


def _torch_decode(codes) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _row_of(case, b, t):
    S = case.block_size
    rows = case.kv_cache.reshape(-1, D)
    return rows[int(case.block_tables[b][t // S]) * S + t % S]


def _run(mla, case):
    return mla.sparse_mla_decode(case.q, case.q_scale, case.kv_cache, case.kv_scale, case.indices,
                                 case.block_tables, case.next_n, case.sm_scale)


def _close(a, b, rel=1e-12):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return a.shape == b.shape and np.allclose(a, b, rtol=rel, atol=rel * max(1.0, float(np.abs(b).max(initial=0))))


def pin_mla_matches_torch_sdpa(mla):
    """Every row equals torch's scaled_dot_product_attention (float64) over the rows its
    positions name, with scale = sm_scale*q_scale*kv_scale and values kv_scale * the
    first 512 dims; lse equals torch.logsumexp of the scores."""
    for S, N in ((1, 2), (4, 3)):
        case = wl.make_mla_case(batch=3, next_n=N, ctx=[37, 70, 5], topk=24, block_size=S, seed=11 + S)
        out, lse = _run(mla, case)
        c = case.sm_scale * case.q_scale * case.kv_scale
        for r in range(case.rows):
            b = r // N
            pos = [int(t) for t in case.indices[r] if t >= 0]
            keys = torch.from_numpy(_torch_decode(np.stack([_row_of(case, b, t) for t in pos])))
            qv = torch.from_numpy(_torch_decode(case.q[r]))
            ref = torch.nn.functional.scaled_dot_product_attention(qv, keys, keys[:, :DV] * case.kv_scale, scale=c)
            assert _close(out[r], ref.numpy()), (S, r)
            ref_lse = torch.logsumexp((qv @ keys.T) * c, dim=1)
            assert _close(lse[r], ref_lse.numpy()), (S, r)


def pin_mla_single_position(mla):
    """One listed position: p = 1, so the output is kv_scale times that row's first 512
    decoded values, and lse is its score (dot product by exact rationals)."""
    case = wl.make_mla_case(batch=2, next_n=1, ctx=[50, 9], topk=8, seed=21)
    case.indices[:, 1:] = -1
    out, lse = _run(mla, case)
    c = case.sm_scale * case.q_scale * case.kv_scale
    for r in range(2):
        t = int(case.indices[r, 0])
        row = _row_of(case, r, t)
        kv = _torch_decode(row)
        assert np.array_equal(out[r], np.broadcast_to(case.kv_scale * kv[:DV], (H, DV))), r
        qv = _torch_decode(case.q[r])
        for h in range(H):
            dot = sum(Fraction(float(qv[h, i])) * Fraction(float(kv[i])) for i in range(D))
            assert math.isclose(lse[r, h], float(dot) * c, rel_tol=1e-14, abs_tol=1e-300), (r, h)


def pin_mla_zero_query_is_mean(mla):
    """q = 0: every score is 0, so p is uniform over the listed entries (a position
    listed twice counts twice) and lse = log(number listed)."""
    case = wl.make_mla_case(batch=2, next_n=2, ctx=[30, 12], topk=10, seed=22)
    case.q[:] = 0
    case.indices[1, 3] = case.indices[1, 0]          # a duplicate entry
    out, lse = _run(mla, case)
    for r in range(case.rows):
        pos = [int(t) for t in case.indices[r] if t >= 0]
        vals = np.stack([_torch_decode(_row_of(case, r // 2, t))[:DV] for t in pos])
        mean = torch.from_numpy(vals).mean(dim=0).numpy() * case.kv_scale
        assert _close(out[r], np.broadcast_to(mean, (H, DV))), r
        assert np.allclose(lse[r], math.log(len(pos)), rtol=1e-14), r


def pin_mla_duplicate_weight(mla):
    """Positions [a, a, b]: with x = e^{s_a}, y = e^{s_b}, the output is
    kv_scale * (2x v_a + y v_b) / (2x + y) per head (plain Python exponentials)."""
    case = wl.make_mla_case(batch=1, next_n=1, ctx=[40], topk=3, seed=23)
    a, bb = int(case.indices[0, 0]), int(case.indices[0, 1])
    case.indices[0] = [a, bb, a]
    out, _ = _run(mla, case)
    ka, kb = _torch_decode(_row_of(case, 0, a)), _torch_decode(_row_of(case, 0, bb))
    qv = _torch_decode(case.q[0])
    c = case.sm_scale * case.q_scale * case.kv_scale
    for h in range(H):
        sa = sum(float(qv[h, i]) * float(ka[i]) for i in range(D)) * c
        sb = sum(float(qv[h, i]) * float(kb[i]) for i in range(D)) * c
        mx = max(sa, sb)
        x, y = math.exp(sa - mx), math.exp(sb - mx)
        want = case.kv_scale * (2 * x * ka[:DV] + y * kb[:DV]) / (2 * x + y)
        assert _close(out[0, h], want, rel=1e-11), h


def pin_mla_saturated_softmax(mla):
    """Scores that differ by ~1e7: the softmax saturates, so the output is exactly the
    dominating row's values and lse its score (no overflow: the maximum is subtracted)."""
    case = wl.make_mla_case(batch=1, next_n=1, ctx=[6], topk=6, table="identity", seed=24)
    case.q[:] = 0x7E                                  # +448 in every dim and head
    rows = case.kv_cache.reshape(-1, D)
    order = [int(t) for t in case.indices[0]]
    for i, t in enumerate(order):
        rows[t] = 0x00
        rows[t, :DV] = 0x30 + i                       # small positive values, growing with i
    top = order[-1]
    rows[top] = 0x7E                                  # the dominating row: +448 everywhere
    out, lse = _run(mla, case)
    kv = _torch_decode(rows[top])
    assert np.array_equal(out[0], np.broadcast_to(case.kv_scale * kv[:DV], (H, DV)))
    c = case.sm_scale * case.q_scale * case.kv_scale
    assert np.allclose(lse[0], D * 448.0 * 448.0 * c, rtol=1e-15)


def pin_mla_padding_order_and_empty(mla):
    """Shuffling a row's list and interleaving -1 entries change nothing; a row listing
    nothing is 0 with lse -inf."""
    case = wl.make_mla_case(batch=2, next_n=1, ctx=[64, 3], topk=16, seed=25)
    out, lse = _run(mla, case)
    rng = np.random.default_rng(5)
    alt = wl.MlaCase(**{**case.__dict__})
    wide = np.full((2, 40), -1, dtype=np.int32)
    for r in range(2):
        pos = [int(t) for t in case.indices[r] if t >= 0]
        slots = np.sort(rng.choice(40, size=len(pos), replace=False))
        wide[r, slots] = rng.permutation(pos)
    alt.indices = wide
    out2, lse2 = _run(mla, alt)
    assert _close(out2, out, rel=1e-13) and _close(lse2, lse, rel=1e-13)
    alt.indices = np.full((2, 5), -1, dtype=np.int32)
    out3, lse3 = _run(mla, alt)
    assert np.array_equal(out3, np.zeros_like(out3)) and np.all(lse3 == -np.inf)


def pin_mla_block_size_identity(mla):
    """The same rows in 8-token blocks behind a permuted block table give exactly the
    per-token layout's result."""
    case = wl.make_mla_case(batch=2, next_n=2, ctx=[45, 20], topk=12, seed=26)
    S = 8
    nblk = [(int(c) + S - 1) // S for c in case.context_lens]
    perm = np.random.default_rng(6).permutation(sum(nblk) + 3)
    rows = case.kv_cache.reshape(-1, D)
    blocked = np.full((perm.size, S, D), 0x7F, dtype=np.uint8)
    tables = np.full((2, max(nblk)), -1, dtype=np.int32)
    off = 0
    for b in range(2):
        for i in range(nblk[b]):
            tables[b, i] = perm[off]
            for s in range(S):
                t = i * S + s
                if t < case.context_lens[b]:
                    blocked[perm[off], s] = rows[case.block_tables[b][t]]
            off += 1
    out, lse = _run(mla, case)
    out2, lse2 = mla.sparse_mla_decode(case.q, case.q_scale, blocked, case.kv_scale, case.indices, tables,
                                       case.next_n, case.sm_scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def _bound(mla, case):
    return mla.sparse_mla_error_bound(case.q, case.q_scale, case.kv_cache, case.kv_scale, case.indices,
                                      case.block_tables, case.next_n, case.sm_scale)


def pin_mla_bound_closed_forms(mla):
    """The tolerance scale B[r, h, c] = kv_scale * sum_t p(h, t) * |v_t[c]| in closed forms:
    one listed position gives kv_scale * |v_t|; a zero query gives kv_scale times the mean
    of |v_t| over the list (a duplicate counted twice); positions [a, b, a] give
    kv_scale * (2x|v_a| + y|v_b|) / (2x + y) with x = e^(s_a - m), y = e^(s_b - m) from
    plain Python loops; a saturated softmax gives kv_scale * |v_top|. Values decoded by
    torch, absolute values taken here."""
    # one position per row
    case = wl.make_mla_case(batch=2, next_n=1, ctx=[50, 9], topk=8, seed=31)
    case.indices[:, 1:] = -1
    bnd = _bound(mla, case)
    for r in range(2):
        v = _torch_decode(_row_of(case, r, int(case.indices[r, 0])))[:DV]
        assert np.array_equal(bnd[r], np.broadcast_to(case.kv_scale * np.abs(v), (H, DV))), r
    # zero query: uniform weights over the listed entries
    case = wl.make_mla_case(batch=2, next_n=2, ctx=[30, 12], topk=10, seed=32)
    case.q[:] = 0
    case.indices[3, 4] = case.indices[3, 1]
    bnd = _bound(mla, case)
    for r in range(case.rows):
        pos = [int(t) for t in case.indices[r] if t >= 0]
        mags = [np.abs(_torch_decode(_row_of(case, r // 2, t))[:DV]) for t in pos]
        want = case.kv_scale * sum(mags) / len(pos)
        assert _close(bnd[r], np.broadcast_to(want, (H, DV)), rel=1e-13), r
    # [a, b, a] with plain exponentials
    case = wl.make_mla_case(batch=1, next_n=1, ctx=[40], topk=3, seed=33)
    a, bb = int(case.indices[0, 0]), int(case.indices[0, 1])
    case.indices[0] = [a, bb, a]
    bnd = _bound(mla, case)
    ka, kb = _torch_decode(_row_of(case, 0, a)), _torch_decode(_row_of(case, 0, bb))
    qv = _torch_decode(case.q[0])
    c = case.sm_scale * case.q_scale * case.kv_scale
    for h in range(H):
        sa = sum(float(qv[h, i]) * float(ka[i]) for i in range(D)) * c
        sb = sum(float(qv[h, i]) * float(kb[i]) for i in range(D)) * c
        mx = max(sa, sb)
        x, y = math.exp(sa - mx), math.exp(sb - mx)
        want = [case.kv_scale * (2 * x * abs(float(ka[i])) + y * abs(float(kb[i]))) / (2 * x + y) for i in range(DV)]
        assert _close(bnd[0, h], np.array(want), rel=1e-11), h
    # saturated softmax: scores ~1e7 apart
    case = wl.make_mla_case(batch=1, next_n=1, ctx=[6], topk=6, table="identity", seed=34)
    case.q[:] = 0x7E
    rows = case.kv_cache.reshape(-1, D)
    order = [int(t) for t in case.indices[0]]
    for i, t in enumerate(order):
        rows[t] = 0x00
        rows[t, :DV] = 0x30 + i
    rows[order[-1]] = 0x7E
    rows[order[-1], 1:DV:2] = 0xFE                    # -448 in the odd value dims
    bnd = _bound(mla, case)
    assert np.array_equal(bnd[0], np.full((H, DV), case.kv_scale * 448.0))


def pin_mla_bound_dominates_output(mla):
    """Triangle inequality: |out| <= B in every element, with equality (to rounding) in
    the value columns whose listed entries all share one sign; B is the bound of the
    rows the row's own request lists (rows of request b read table row b)."""
    case = wl.make_mla_case(batch=3, next_n=2, ctx=[60, 33, 90], topk=4, block_size=4, seed=35)
    out, _ = _run(mla, case)
    bnd = _bound(mla, case)
    assert np.all(np.abs(out) <= bnd * (1 + 1e-12) + 1e-300)
    for r in range(case.rows):
        pos = [int(t) for t in case.indices[r] if t >= 0]
        vals = np.stack([_torch_decode(_row_of(case, r // 2, t))[:DV] for t in pos])
        same = np.all(vals >= 0, axis=0) | np.all(vals <= 0, axis=0)
        assert same.any(), r
        assert np.allclose(np.abs(out[r][:, same]), bnd[r][:, same], rtol=1e-12, atol=0), r


MLA_PINS = [
    pin_mla_matches_torch_sdpa,
    pin_mla_single_position,
    pin_mla_zero_query_is_mean,
    pin_mla_duplicate_weight,
    pin_mla_saturated_softmax,
    pin_mla_padding_order_and_empty,
    pin_mla_block_size_identity,
    pin_mla_bound_closed_forms,
    pin_mla_bound_dominates_output,
]
