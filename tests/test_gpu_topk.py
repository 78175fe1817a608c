"""mqa_topk on crafted logit rows, one call per path (every row fits one workgroup when
max_model_len <= 8192 or <= 32768, with the fewest of 4, 8, 16 or 32 values per thread
that hold the row; beyond, rows longer than 32768 take the chunked path inside the same
launch as the whole rows), compared as sets with the oracle's selection (larger first,
ties by lower position, -0.0 equal to +0.0). The lengths include both sides of every
boundary between those forms (4096, 8192, 16384, 32768).

The rows are chosen to reach each branch of the selection: spread values (linear bins),
few distinct values (a threshold bin of thousands of elements, refined by radix digits;
beyond 8192 candidates the chunked path refines from the row itself), a constant row (a single
bin), signed zeros, infinities and a spread that overflows (top-key bins), a narrow
band around 1e6, a log-uniform spread over 60 decades, subnormals, and rows holding
NaNs. The oracle orders NaN below everything; the header fixes the kernel's order for
NaN as that of the bit patterns (positive NaN above +inf, negative NaN below -inf),
so NaN rows are checked against that order instead.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_mqa_amd import mqa
from gpu_helpers import say

pytestmark = pytest.mark.gpu

KINDS = ["normal", "few", "const", "zeros", "inf", "overflow", "narrow", "wide", "subnormal", "nan", "two_inf"]


def crafted_row(kind, n, rng):
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "few":
        return rng.integers(0, 4, n).astype(np.float32)
    if kind == "const":
        return np.full(n, 2.5, np.float32)
    if kind == "zeros":
        return rng.choice(np.array([-0.0, 0.0, -1.0, 1.0], np.float32), n, p=[0.45, 0.45, 0.05, 0.05])
    if kind == "inf":
        x = rng.standard_normal(n).astype(np.float32)
        x[rng.random(n) < 0.01] = np.inf
        x[rng.random(n) < 0.01] = -np.inf
        return x
    if kind == "overflow":
        return (rng.uniform(-1.0, 1.0, n) * 3e38).astype(np.float32)
    if kind == "narrow":
        return (np.float32(1e6) + rng.integers(0, 64, n).astype(np.float32) * np.float32(0.0625)).astype(np.float32)
    if kind == "wide":
        return (rng.choice([-1.0, 1.0], n) * 10.0 ** rng.uniform(-30, 30, n)).astype(np.float32)
    if kind == "subnormal":
        return (rng.integers(-1000, 1000, n) * np.float32(1e-42)).astype(np.float32)
    if kind == "two_inf":  # key bins (an infinity) holding ~n/2 ties each
        x = rng.integers(0, 2, n).astype(np.float32)
        x[rng.integers(0, n)] = np.inf
        return x
    if kind == "nan":
        x = rng.standard_normal(n).astype(np.float32)
        bits = x.view(np.uint32)
        pos = rng.random(n) < 0.02
        neg = rng.random(n) < 0.02
        bits[pos] = 0x7FC00000 | rng.integers(0, 1 << 22, int(pos.sum())).astype(np.uint32)
        bits[neg] = 0xFFC00000 | rng.integers(0, 1 << 22, int(neg.sum())).astype(np.uint32)
        x[rng.random(n) < 0.01] = np.inf
        return x
    raise ValueError(kind)


def bit_order_topk(vals, k):
    """The k positions first in the header's order for NaN-holding rows: the fp32 bit
    pattern mapped onto an unsigned order (-0.0 folded onto +0.0), ties by position."""
    u = vals.view(np.uint32).astype(np.int64)
    u = np.where(u == 0x80000000, 0, u)
    key = np.where(u >= 0x80000000, 0xFFFFFFFF - u, u + 0x80000000)
    order = np.lexsort((np.arange(u.size), -key))
    return np.sort(order[:min(k, u.size)])


def run_case(L, k, specs, seed, ws=None):
    """specs: list of (kind, nv). One call to mqa_topk over all rows (with the given
    workspace, else a fresh zero-filled one)."""
    rng = np.random.default_rng(seed)
    rows = len(specs)
    logits = np.full((rows, L), np.nan, np.float32)  # beyond nv: never read as a value
    for r, (kind, nv) in enumerate(specs):
        logits[r, :nv] = crafted_row(kind, nv, rng)
    ctx = np.array([nv for _, nv in specs], np.int32)
    shape = mqa.make_shape(rows, 1, 64, L, L)
    d_logits = torch.from_numpy(logits).cuda()
    d_ctx = torch.from_numpy(ctx).cuda()
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    nbytes = mqa.mqa_topk_workspace_bytes(shape, L, k)
    if ws is None:
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")  # zero before first use
    assert ws.numel() >= nbytes
    mqa.mqa_topk(d_logits, d_ctx, L, k, idx, shape, ws)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r, (kind, nv) in enumerate(specs):
        vals = logits[r, :nv]
        want = bit_order_topk(vals, k) if kind == "nan" else oracle.topk_row(vals.astype(np.float64), k)
        m = min(k, nv)
        assert np.all(got[r, m:] == -1), f"{kind} nv={nv} k={k}: padding"
        sel = np.sort(got[r, :m])
        assert np.array_equal(sel, want), (
            f"{kind} nv={nv} k={k}: {np.setdiff1d(sel, want).size} positions differ from the expected set")


@pytest.mark.parametrize("k", [2048, 1, 100, 1023])
def test_topk_short_rows(k):
    """max_model_len = 4096: 4 or 8 values per thread (one 1024-thread workgroup per row)."""
    nvs = sorted({1, 1024, 1025, 2048, 2049, 3000, 4096} | {k + 1})
    specs = [(kind, nv) for kind in KINDS for nv in nvs if nv <= 4096]
    say(f"[gpu] topk crafted rows L=4096 k={k} rows={len(specs)}")
    run_case(4096, k, specs, seed=6900 + k)


@pytest.mark.parametrize("k", [2048, 1, 100, 2047])
def test_topk_rows_fit_one_workgroup(k):
    nvs = sorted({1, 2048, 2049, 3000, 4096, 4097, 8192} | {k + 1})
    specs = [(kind, nv) for kind in KINDS for nv in nvs if nv <= 8192]
    say(f"[gpu] topk crafted rows L=8192 k={k} rows={len(specs)}")
    run_case(8192, k, specs, seed=7000 + k)


@pytest.mark.parametrize("k", [2048, 1, 777])
def test_topk_wide_rows(k):
    """Rows up to 32768 in one workgroup each; constant, few-valued and two-valued rows
    put more than 8192 elements in the threshold bin (the refinement over the row)."""
    nvs = [1, 2049, 4096, 4097, 8192, 8193, 16384, 16385, 20000, 32768]
    specs = [(kind, nv) for kind in KINDS for nv in nvs]
    say(f"[gpu] topk crafted rows L=32768 k={k} rows={len(specs)}")
    run_case(32768, k, specs, seed=7200 + k)


@pytest.mark.parametrize("k", [2048, 300])
def test_topk_long_rows(k):
    nvs = [5, 2049, 4096, 4097, 8192, 8193, 16384, 16385, 20000, 32768, 32769, 40000]
    specs = [(kind, nv) for kind in KINDS for nv in nvs]
    say(f"[gpu] topk crafted rows L=40000 k={k} rows={len(specs)}")
    run_case(40000, k, specs, seed=7100 + k)


def test_topk_workspace_reused_and_left_zero():
    """One workspace serves a sequence of calls of different shapes (its layout moves with
    the row count): chunked rows of every kind, whole threshold bins, refinement over the
    row, trivial rows. Every call is checked, and after each the workspace holds zeros
    again, as the next call requires."""
    seq = [
        (40000, 2048, [(kind, nv) for kind in KINDS for nv in (5, 8193, 40000)], 7300),
        (52000, 100, [(kind, 52000) for kind in KINDS], 7301),
        (202752, 2048, [("normal", 202752), ("const", 150000), ("few", 99999), ("zeros", 3)], 7302),
        (33000, 2048, [(kind, nv) for kind in KINDS for nv in (2049, 32769, 33000)], 7303),
    ]
    need = max(mqa.mqa_topk_workspace_bytes(mqa.make_shape(len(sp), 1, 64, L, L), L, k) for L, k, sp, _ in seq)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for L, k, specs, seed in seq:
        say(f"[gpu] topk reused workspace L={L} k={k} rows={len(specs)}")
        run_case(L, k, specs, seed, ws=ws)
        nz = int(torch.count_nonzero(ws).item())
        assert nz == 0, f"L={L} k={k}: {nz} workspace bytes left nonzero"


def test_topk_chunked_mode_more_rows_than_a_workgroup_scans():
    """The chunked launch with more rows than one workgroup holds (1300 > 1024): the items
    are numbered over several blocks of rows, and the whole rows of all four cost classes,
    the trivial rows and a chunked row every hundred are dealt over many rounds."""
    nvs = [5, 2048, 2049, 3000, 4096, 4097, 6000, 8192, 8193, 12000, 16384, 16385, 25000, 32768]
    kinds = ["normal", "few", "narrow", "zeros", "inf"]
    specs = []
    for r in range(1300):
        nv = (32769, 36000, 40000)[(r // 100) % 3] if r % 100 == 57 else nvs[r % len(nvs)]
        specs.append((kinds[r % len(kinds)], nv))
    say(f"[gpu] topk chunked mode, {len(specs)} rows, L=40000")
    run_case(40000, 2048, specs, seed=7400)
