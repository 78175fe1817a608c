"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with the fact it checks. ``test_oracle_pins.py`` runs them
against the oracle; ``test_oracle_mutations.py`` runs them against copies of
the oracle with planted mistakes and requires every mistake to be caught.

Independent sources used here (none of them is the oracle's own code):
  * torch's float8_e4m3fn upcast (a separate decoder implementation);
  * the OCP E4M3 spot values and the hand-derived closed forms under golden/;
  * exact rational arithmetic (fractions.Fraction) on tiny inputs, with the
    torch decoder, and masking written from the page's rule with plain loops;
  * invariants the definition implies (paging identity, batch and length
    invariance, the -inf prefix);
  * a special case (all operands non-negative) in which relu is the identity
    and the logits reduce to torch float64 matrix products;
  * the top-k counting definition, by brute force.
"""
from __future__ import annotations

import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import torch

from fp8_paged_mqa_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def torch_decode_table() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


TORCH_E4M3 = torch_decode_table()


def _same(a, b) -> bool:
    a, b = float(a), float(b)
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------
def pin_decode_matches_torch(orc):
    for c in range(256):
        assert _same(orc.decode_e4m3fn(c), TORCH_E4M3[c]), f"code {c:#04x}"
        assert _same(orc.E4M3FN_VALUES[c], TORCH_E4M3[c]), f"table code {c:#04x}"


def pin_decode_golden_spot_values(orc):
    with open(os.path.join(GOLDEN, "e4m3fn_spot_values.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            code, value = line.split()[:2]
            assert _same(orc.decode_e4m3fn(int(code, 16)), float(value)), line


def pin_decode_structure(orc):
    vals = np.array([orc.decode_e4m3fn(c) for c in range(256)])
    nan_codes = [c for c in range(256) if math.isnan(vals[c])]
    assert nan_codes == [0x7F, 0xFF]
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase strictly"
    for c in range(0x7F):
        assert vals[c | 0x80] == -vals[c], "sign symmetry"
    finite = vals[np.isfinite(vals)]
    scaled = finite * 2 ** 9
    assert np.all(scaled == np.round(scaled)) and np.abs(scaled).max() < 2 ** 18


# ---------------------------------------------------------------------------
# Closed forms (hand-derived, golden/closed_forms.json)
# ---------------------------------------------------------------------------
def _load_closed_forms():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        return json.load(f)


def _scale_bytes(s):
    return np.frombuffer(struct.pack("<f", s), dtype=np.uint8)


def pin_closed_forms_single_token(orc):
    for case in _load_closed_forms()["single_token"]:
        H = case["heads"]
        q = np.zeros((1, 1, H, 128), np.uint8)
        kv = np.zeros((1, 132), np.uint8)
        if "q_fill" in case:
            q[...] = int(case["q_fill"], 16)
        for h, d, code in case.get("q", []):
            q[0, 0, h, d] = int(code, 16)
        if "k_fill" in case:
            kv[0, :128] = int(case["k_fill"], 16)
        for d, code in case.get("k", []):
            kv[0, d] = int(code, 16)
        kv[0, 128:] = _scale_bytes(case["scale"])
        w = np.array([case["w"]], np.float32)
        out = orc.paged_mqa_logits(q, kv, w, np.array([1]), np.array([[0, -1]]), 2)
        assert out[0, 0] == case["expected"], (case["name"], out[0, 0])
        assert out[0, 1] == -np.inf, case["name"]
        one = orc.paged_mqa_logit_at(q, kv, w, np.array([1]), np.array([[0, -1]]), 2, 0, 0)
        assert one == case["expected"], (case["name"], "single-logit path", one)


def pin_closed_forms_paged(orc):
    for case in _load_closed_forms()["paged"]:
        H, N, ctx, L = case["heads"], case["next_n"], case["ctx"], case["max_model_len"]
        q = np.full((1, N, H, 128), int(case["q_fill"], 16), np.uint8)
        rows = case["kv_rows_dim0"]
        kv = np.zeros((len(rows), 132), np.uint8)
        for i, code in enumerate(rows):
            kv[i, 0] = int(code, 16)
            kv[i, 128:] = _scale_bytes(case["scale"])
        w = np.array(case["w"], np.float32)
        bt = np.array([case["block_table"]])
        out = orc.paged_mqa_logits(q, kv, w, np.array([ctx]), bt, L)
        exp = np.array([[float(v) for v in r] for r in case["expected"]])
        assert np.array_equal(out, exp), (case["name"], out)
        for r in range(N):
            for t in range(L):
                one = orc.paged_mqa_logit_at(q, kv, w, np.array([ctx]), bt, L, r, t)
                assert one == exp[r, t], (case["name"], r, t, one)


# ---------------------------------------------------------------------------
# Exact rationals on tiny inputs
# ---------------------------------------------------------------------------
def _exact_logits(case):
    """Fraction brute force: torch decode, struct scale, page mask, plain loops."""
    B, N, H, D = case.q.shape
    L = case.max_model_len
    out = [[None] * L for _ in range(B * N)]
    for b in range(B):
        ctx = int(case.context_lens[b])
        for j in range(N):
            r = b * N + j
            for t in range(L):
                if not (t < ctx and t <= ctx - N + j):
                    continue
                bs = case.block_size  # token t: slot t % bs of block table[t // bs]
                row = case.kv_cache.reshape(-1, 132)[int(case.block_tables[b, t // bs]) * bs + t % bs]
                scale = Fraction(struct.unpack("<f", row[128:132].tobytes())[0])
                total = Fraction(0)
                terms = Fraction(0)
                for h in range(H):
                    dot = sum(Fraction(TORCH_E4M3[case.q[b, j, h, i]]) * Fraction(TORCH_E4M3[row[i]])
                              for i in range(D))
                    x = dot * scale
                    term = Fraction(float(case.weights[r, h])) * (x if x > 0 else Fraction(0))
                    total += term
                    terms += abs(term)
                out[r][t] = (total, terms)
    return out


def pin_exact_rationals(orc):
    for seed, (B, N, H, ctxs, bs) in enumerate([(1, 1, 1, [5], 1), (2, 2, 3, [4, 6], 1), (2, 1, 4, [1, 3], 1),
                                                (1, 3, 2, [6], 1), (2, 2, 2, [1, 5], 1), (2, 2, 2, [5, 3], 2),
                                                (1, 2, 3, [7], 4)]):
        case = wl.make_case(batch=B, next_n=N, heads=H, ctx=ctxs, max_model_len=7, seed=100 + seed,
                            block_size=bs, pool=8 if bs > 1 else None)
        got = orc.paged_mqa_logits(case.q, case.kv_cache, case.weights, case.context_lens,
                                   case.block_tables, case.max_model_len)
        exact = _exact_logits(case)
        for r in range(B * N):
            for t in range(case.max_model_len):
                if exact[r][t] is None:
                    assert got[r, t] == -np.inf, (seed, r, t)
                    continue
                total, terms = exact[r][t]
                bound = 8 * H * 2.0 ** -53 * float(terms) + 1e-300
                assert abs(got[r, t] - float(total)) <= bound, (seed, r, t, got[r, t], float(total))


# ---------------------------------------------------------------------------
# Special case: every operand non-negative, so relu is the identity and the
# logits are s_t * (sum_h w_h q_h) . k_t, computed here with torch float64.
# ---------------------------------------------------------------------------
def pin_nonnegative_reduces_to_matmul(orc):
    nonneg = lambda rng, shape: np.abs(rng.standard_normal(shape, dtype=np.float32))  # noqa: E731
    case = wl.make_case(batch=3, next_n=2, heads=32, ctx=[40, 17, 64], max_model_len=80, seed=7,
                        q_fn=nonneg, key_fn=nonneg)
    got = orc.paged_mqa_logits(case.q, case.kv_cache, case.weights, case.context_lens,
                               case.block_tables, case.max_model_len)
    dec = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).to(torch.float64)  # noqa: E731
    qd = dec(case.q)                                        # [B, N, H, D]
    kd = dec(np.ascontiguousarray(case.kv_cache[:, :128]))  # [rows, D]
    sd = torch.from_numpy(np.ascontiguousarray(case.kv_cache[:, 128:]).view("<f4")[:, 0].astype(np.float64))
    wd = torch.from_numpy(case.weights.astype(np.float64))
    for b in range(case.batch):
        ctx = int(case.context_lens[b])
        for j in range(case.next_n):
            r = b * case.next_n + j
            nv = ctx - case.next_n + j + 1
            phys = torch.from_numpy(case.block_tables[b, :nv].astype(np.int64))
            wq = wd[r] @ qd[b, j]                           # [D]
            ref = (kd[phys] @ wq) * sd[phys]
            ref_terms = (kd[phys] @ (wd[r].abs() @ qd[b, j])) * sd[phys]
            assert np.all(np.abs(got[r, :nv] - ref.numpy()) <= 1e-13 * ref_terms.numpy() + 1e-300), (b, j)
            assert np.all(got[r, nv:] == -np.inf)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------
def pin_mask_is_visible_prefix(orc):
    for seed, (N, ctxs) in enumerate([(1, [0, 1, 2, 9]), (2, [1, 2, 3, 9]), (3, [2, 3, 4, 9]),
                                      (4, [0, 3, 4, 5, 9])]):
        case = wl.make_case(batch=len(ctxs), next_n=N, heads=16, ctx=ctxs, max_model_len=12,
                            seed=200 + seed)
        out = orc.paged_mqa_logits(case.q, case.kv_cache, case.weights, case.context_lens,
                                   case.block_tables, case.max_model_len)
        for b, ctx in enumerate(ctxs):
            for j in range(N):
                row = out[b * N + j]
                finite = np.isfinite(row)
                # row j's query is token ctx - N + j; it sees itself and everything before it
                expect = max(0, ctx - N + j + 1)
                assert finite.sum() == expect, (N, ctx, j)
                assert finite[:expect].all() and (row[expect:] == -np.inf).all()


def pin_paging_identity(orc):
    """A permuted table over scattered rows equals the same tokens stored in
    logical order behind an identity-style table."""
    case = wl.make_case(batch=3, next_n=2, heads=32, ctx=[33, 5, 70], max_model_len=80, seed=11,
                        table="permuted", pool=200)
    out = orc.paged_mqa_logits(case.q, case.kv_cache, case.weights, case.context_lens,
                               case.block_tables, case.max_model_len)
    ctx = case.context_lens
    order = np.concatenate([case.block_tables[b, :ctx[b]] for b in range(case.batch)])
    kv2 = case.kv_cache[order]
    offs = np.concatenate([[0], np.cumsum(ctx)])
    bt2 = np.full_like(case.block_tables, -1)
    for b in range(case.batch):
        bt2[b, :ctx[b]] = np.arange(offs[b], offs[b + 1])
    out2 = orc.paged_mqa_logits(case.q, kv2, case.weights, ctx, bt2, case.max_model_len)
    assert np.array_equal(out, out2)


def pin_block_size_identity(orc):
    """The same tokens stored in blocks of 16 (permuted blocks, a partly filled last
    block per request) give exactly the logits of a block_size 1 cache holding each
    token's row behind a per-token table."""
    case = wl.make_case(batch=3, next_n=2, heads=32, ctx=[33, 5, 70], max_model_len=80, seed=13,
                        block_size=16, pool=12)
    assert case.kv_cache.shape[1] == 16
    out = orc.paged_mqa_logits(case.q, case.kv_cache, case.weights, case.context_lens,
                               case.block_tables, case.max_model_len)
    rows = case.kv_cache.reshape(-1, 132)
    bt1 = np.full((case.batch, 80), -1, dtype=np.int32)
    for b in range(case.batch):
        for t in range(int(case.context_lens[b])):
            bt1[b, t] = int(case.block_tables[b, t // 16]) * 16 + t % 16
    out1 = orc.paged_mqa_logits(case.q, rows, case.weights, case.context_lens, bt1, case.max_model_len)
    assert np.array_equal(out, out1)
    assert np.isfinite(out).sum() == sum(max(0, int(c) - 2 + j + 1) for c in case.context_lens for j in range(2))


def pin_batch_and_length_invariance(orc):
    case = wl.make_case(batch=4, next_n=2, heads=32, ctx=[12, 30, 3, 25], max_model_len=32, seed=12)
    full = orc.paged_mqa_logits(case.q, case.kv_cache, case.weights, case.context_lens,
                                case.block_tables, case.max_model_len)
    N = case.next_n
    for b in range(case.batch):
        alone = orc.paged_mqa_logits(case.q[b:b + 1], case.kv_cache, case.weights[b * N:(b + 1) * N],
                                     case.context_lens[b:b + 1], case.block_tables[b:b + 1], 40)
        assert np.array_equal(alone[:, :32], full[b * N:(b + 1) * N]), b
        assert np.all(alone[:, 32:] == -np.inf)


# ---------------------------------------------------------------------------
# Top-k
# ---------------------------------------------------------------------------
def _topk_by_counting(values, k):
    """p is kept iff (#strictly larger) + (#equal at a lower position) < k."""
    keep = []
    for p, v in enumerate(values):
        larger = sum(1 for u in values if u > v)
        earlier_equal = sum(1 for t, u in enumerate(values[:p]) if u == v)
        if larger + earlier_equal < k:
            keep.append(p)
    return keep


def pin_topk_counting_definition(orc):
    rng = np.random.default_rng(5)
    for trial in range(40):
        n = int(rng.integers(1, 60))
        k = int(rng.integers(1, 70))
        vals = rng.integers(-4, 5, size=n).astype(np.float64) * 0.5   # many exact ties
        if trial % 5 == 0:
            vals[rng.random(n) < 0.3] = -0.0
        got = orc.topk_row(vals, k).tolist()
        assert got == _topk_by_counting(vals.tolist(), k), (trial, n, k)


def pin_topk_rows_and_padding(orc):
    logits = np.array([[3.0, 1.0, 2.0, -np.inf, -np.inf],
                       [5.0, 5.0, 5.0, 5.0, -np.inf],
                       [0.0, -np.inf, -np.inf, -np.inf, -np.inf],
                       [-np.inf] * 5])
    ctx = np.array([3, 4, 1, 0])
    got = orc.topk(logits, ctx, 1, 2)
    assert got.tolist() == [[0, 2], [0, 1], [0, -1], [-1, -1]]
    # next_n = 2: rows of one request see ctx-2+j+1 positions
    got2 = orc.topk(np.array([[1.0, 9.0, 4.0, 7.0], [1.0, 9.0, 4.0, 7.0]]), np.array([4]), 2, 3)
    assert got2.tolist() == [[0, 1, 2], [1, 2, 3]]


def pin_topk_ctx_k_plus_one_drops_argmin(orc):
    rng = np.random.default_rng(9)
    for trial in range(10):
        n = 33
        vals = rng.standard_normal(n)
        if trial % 2:
            vals[rng.integers(0, n, size=3)] = vals.min()   # tied minima
        sel = orc.topk_row(vals, n - 1)
        dropped = sorted(set(range(n)) - set(sel.tolist()))
        minima = np.flatnonzero(vals == vals.min())
        assert dropped == [int(minima.max())], (trial, dropped)


# ---------------------------------------------------------------------------
# K-cache write (quantisation upstream of the op)
# ---------------------------------------------------------------------------
def _encode_probe_values():
    rng = np.random.default_rng(5)
    vals = TORCH_E4M3[np.isfinite(TORCH_E4M3)]
    mids = (np.sort(vals)[1:] + np.sort(vals)[:-1]) / 2
    return np.concatenate([rng.standard_normal(20000) * 40, np.linspace(-470, 470, 9401), vals, mids,
                           [0.0, -0.0, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 1e-30, 463.99, 464.0, 464.01,
                            np.nan, np.inf, -np.inf]]).astype(np.float32)


def pin_encode_matches_torch(orc):
    """Round to nearest even e4m3fn, checked against torch's independent cast on random
    values, a fine grid over the whole range, every code value, every midpoint between
    neighbouring codes, the top-of-range tie at 464, and NaN / inf."""
    x = _encode_probe_values()
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.encode_e4m3fn(x.astype(np.float64))
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (bad.size, x[bad][:5], got[bad][:5], ref[bad][:5])


def pin_quantize_round_trip(orc):
    """Dequantising a written row the way the page's reference reads the cache (code
    value times the row's fp32 scale) returns each key to within half an e4m3 step,
    and the row's largest magnitude lands exactly on +-448."""
    rng = np.random.default_rng(6)
    for trial in range(40):
        k = (rng.standard_normal(128) * rng.lognormal(0, 3)).astype(np.float32)
        if trial % 7 == 0:
            k[rng.integers(0, 128, 5)] = 0.0
        codes, scale = orc.quantize_k_row(k)
        assert np.float32(scale) == np.float32(np.abs(k).max() / np.float32(448.0))
        deq = TORCH_E4M3[codes] * float(scale)
        y = k.astype(np.float64) / float(scale)                  # position on the e4m3 grid
        # half a step: 2^-4 relative in the normal range, 2^-10 absolute (times scale) below 2^-6
        bound = np.where(np.abs(y) >= 2.0 ** -6, np.abs(k) * 2.0 ** -4, 2.0 ** -10 * float(scale)) * (1 + 1e-6)
        assert np.all(np.abs(deq - k) <= bound + 1e-30), trial
        i = int(np.argmax(np.abs(k)))
        assert TORCH_E4M3[codes[i]] == (448.0 if k[i] > 0 else -448.0)
    codes, scale = orc.quantize_k_row(np.zeros(128, np.float32))
    assert np.all(codes == 0) and scale == np.float32(1.0)
    # signed zeros keep their sign through scale 1, as torch's own cast does
    z = np.where(np.arange(128) % 3 == 0, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    codes, scale = orc.quantize_k_row(z)
    want = torch.from_numpy(z).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert scale == np.float32(1.0) and np.array_equal(codes, want) and want[0] == 0x80


def pin_write_slots_and_logits(orc):
    """write_k_cache puts token i at slot_mapping[i] (row blk * S + offset for a blocked
    cache), skips slots outside the cache, leaves every other byte alone; the logits of
    the written cache equal a float64 evaluation on the dequantised keys."""
    rng = np.random.default_rng(7)
    T, S, nblk = 10, 4, 6
    k = (rng.standard_normal((T, 128)) * 3).astype(np.float32)
    cache = rng.integers(0, 256, size=(nblk, S, 132), dtype=np.uint8)
    slots = np.array([5, 0, 23, -1, 9, 24, 11, 2, 17, 8])     # -1 and 24 lie outside
    out = orc.write_k_cache(k, slots, cache)
    rows_in, rows_out = cache.reshape(-1, 132), out.reshape(-1, 132)
    written = {int(s_): i for i, s_ in enumerate(slots) if 0 <= s_ < nblk * S}
    for r in range(nblk * S):
        if r not in written:
            assert np.array_equal(rows_out[r], rows_in[r]), r
            continue
        kk = k[written[r]]
        scale = struct.unpack("<f", rows_out[r, 128:132].tobytes())[0]
        assert scale == float(np.float32(np.abs(kk).max() / np.float32(448.0)))
        ref_codes = torch.from_numpy((kk / np.float32(scale)).astype(np.float32)).to(torch.float8_e4m3fn)
        assert np.array_equal(rows_out[r, :128], ref_codes.view(torch.uint8).numpy()), r
    # logits over the written rows: request 0 reads tokens 0, 1, 2 (slots 5, 0, 23)
    q = rng.integers(0, 256, size=(1, 1, 16, 128), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38                                # no NaN query codes
    w = rng.standard_normal((1, 16)).astype(np.float32)
    bt = np.array([[1, 0, 5]])                                  # blocks: slot 5 = blk 1 off 1, ...
    # tokens t=0..2 -> rows bt[t//4]*4 + t%4 = 4, 5, 6; write those slots with tokens 0..2
    out2 = orc.write_k_cache(k[:3], np.array([4, 5, 6]), cache)
    got = orc.paged_mqa_logits(q, out2, w, np.array([3]), bt, 3)
    for t in range(3):
        row = out2.reshape(-1, 132)[4 + t]
        scale = struct.unpack("<f", row[128:132].tobytes())[0]
        key = TORCH_E4M3[row[:128]] * scale
        want = sum(float(w[0, h]) * max(float(np.dot(TORCH_E4M3[q[0, 0, h]], key)), 0.0) for h in range(16))
        assert abs(got[0, t] - want) <= 1e-9 * (1 + abs(want)), (t, got[0, t], want)


# ---------------------------------------------------------------------------
# Non-paged (prefill) logits
# ---------------------------------------------------------------------------
def _split_rows(kv):
    rows = np.asarray(kv, dtype=np.uint8).reshape(-1, 132)
    return rows[:, :128].copy(), np.ascontiguousarray(rows[:, 128:132]).view("<f4")[:, 0].copy()


def pin_prefill_exact_rationals(orc):
    """Fraction brute force of the prefill form on tiny shapes with arbitrary windows
    (empty, clipped at both ends, reversed)."""
    rng = np.random.default_rng(8)
    for trial, (M, H, N) in enumerate([(3, 2, 6), (4, 1, 5), (2, 3, 7)]):
        case = wl.make_case(batch=1, next_n=1, heads=H, ctx=[N], seed=300 + trial, table="identity")
        k, sc = _split_rows(case.kv_cache[:N])
        q = rng.integers(0, 256, size=(M, H, 128), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x38
        w = rng.standard_normal((M, H)).astype(np.float32)
        ks = rng.integers(-2, N + 1, size=M)
        ke = rng.integers(-1, N + 3, size=M)
        ks[0], ke[0] = 0, N
        got = orc.mqa_logits(q, k, sc, w, ks, ke)
        for m in range(M):
            for n in range(N):
                if not (max(ks[m], 0) <= n < min(ke[m], N)):
                    assert got[m, n] == -np.inf, (trial, m, n)
                    continue
                total, terms = Fraction(0), Fraction(0)
                for h in range(H):
                    dot = sum(Fraction(TORCH_E4M3[q[m, h, i]]) * Fraction(TORCH_E4M3[k[n, i]]) for i in range(128))
                    x = dot * Fraction(float(sc[n]))
                    term = Fraction(float(w[m, h])) * (x if x > 0 else Fraction(0))
                    total += term
                    terms += abs(term)
                assert abs(got[m, n] - float(total)) <= 8 * H * 2.0 ** -53 * float(terms) + 1e-300, (trial, m, n)


def pin_prefill_matches_decode_rows(orc):
    """Decode rows are prefill rows over the request's keys: with ks = 0 and ke = the
    row's visible count, the prefill form over the request's rows in logical order
    reproduces the paged logits exactly (a separately pinned path)."""
    case = wl.make_case(batch=2, next_n=3, heads=32, ctx=[40, 17], max_model_len=48, seed=301, table="permuted")
    paged = orc.paged_mqa_logits(case.q, case.kv_cache, case.weights, case.context_lens, case.block_tables, 48)
    for b in range(2):
        ctx = int(case.context_lens[b])
        k, sc = _split_rows(case.kv_cache[case.block_tables[b, :ctx]])
        N = case.next_n
        q = case.q[b]                                                # [N, H, D]
        w = case.weights[b * N:(b + 1) * N]
        ke = np.array([ctx - N + j + 1 for j in range(N)])
        got = orc.mqa_logits(q, k, sc, w, np.zeros(N, int), ke)
        assert np.array_equal(got, paged[b * N:(b + 1) * N, :ctx]), b


PINS = [
    pin_block_size_identity,
    pin_decode_matches_torch,
    pin_decode_golden_spot_values,
    pin_decode_structure,
    pin_closed_forms_single_token,
    pin_closed_forms_paged,
    pin_exact_rationals,
    pin_nonnegative_reduces_to_matmul,
    pin_mask_is_visible_prefix,
    pin_paging_identity,
    pin_batch_and_length_invariance,
    pin_topk_counting_definition,
    pin_topk_rows_and_padding,
    pin_topk_ctx_k_plus_one_drops_argmin,
    pin_encode_matches_torch,
    pin_quantize_round_trip,
    pin_write_slots_and_logits,
    pin_prefill_exact_rationals,
    pin_prefill_matches_decode_rows,
]
