"""Invariances, exact-tie cases and edge cases of the HIP path (needs an MI355X)."""
import numpy as np
import pytest

import oracle
from fp8_paged_mqa_amd import workloads as wl
from gpu_helpers import check_logits, check_topk, oracle_logits, run_gpu, say

pytestmark = pytest.mark.gpu


def test_paging_identity_bitwise():
    """A permuted table over scattered rows gives bit-identical logits to the same
    tokens stored contiguously behind an identity-style table: the arithmetic of a
    logit depends only on its own key row."""
    case = wl.make_case(batch=6, next_n=2, heads=64, ctx=[5, 300, 2049, 4097, 1, 9000],
                        max_model_len=9000, seed=51, table="permuted", pool=40000)
    g1, i1 = run_gpu(case)
    ctx = case.context_lens
    order = np.concatenate([case.block_tables[b, :ctx[b]] for b in range(case.batch)])
    offs = np.concatenate([[0], np.cumsum(ctx)])
    bt2 = np.full_like(case.block_tables, -1)
    for b in range(case.batch):
        bt2[b, :ctx[b]] = np.arange(offs[b], offs[b + 1])
    case2 = wl.Workload("contiguous", case.q, case.kv_cache[order], case.weights, ctx, bt2,
                        case.max_model_len, case.next_n)
    g2, i2 = run_gpu(case2)
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))
    assert np.array_equal(np.sort(i1, axis=1), np.sort(i2, axis=1))


def test_batch_composition_and_length_bitwise():
    """A request's rows are bit-identical alone, inside a batch, and for a longer L."""
    case = wl.make_case(batch=5, next_n=4, heads=32, ctx=[7, 3000, 2048, 12000, 100],
                        max_model_len=12000, seed=52)
    full, _ = run_gpu(case)
    N = case.next_n
    for b in [1, 3]:
        alone = wl.Workload("alone", case.q[b:b + 1], case.kv_cache, case.weights[b * N:(b + 1) * N],
                            case.context_lens[b:b + 1], case.block_tables[b:b + 1], 12345, N)
        g, _ = run_gpu(alone)
        assert np.array_equal(g[:, :12000].view(np.uint32), full[b * N:(b + 1) * N].view(np.uint32))
        assert np.all(g[:, 12000:] == -np.inf)


def test_small_call_rows_match_large_call_bitwise():
    """A request alone in a small call (each wave's stage fixed by its index) gives the same
    bits as inside a batch large enough for the scheduled form."""
    ctx = [1, 63, 64, 65, 2049, 4096, 700, 3000] * 5
    case = wl.make_case(batch=len(ctx), next_n=1, heads=64, ctx=ctx, max_model_len=8192, seed=54)
    full, _ = run_gpu(case)
    for b in [0, 2, 3, 4, 5]:
        alone = wl.Workload("alone", case.q[b:b + 1], case.kv_cache, case.weights[b:b + 1],
                            case.context_lens[b:b + 1], case.block_tables[b:b + 1], 4096, 1)
        g, _ = run_gpu(alone)
        assert np.array_equal(g[0].view(np.uint32), full[b, :4096].view(np.uint32)), b
        assert np.all(full[b, 4096:] == -np.inf)


def test_two_workgroup_small_call_rows_match_scheduled_rows_bitwise():
    """Twelve requests of at most 8192 positions: with max_model_len 8192 two workgroups per
    CU hold a wave for each of their stages (the small-call form, waves past 1024 too); with
    max_model_len 65536 the call runs in scheduled whole stages. Same bits on the first 8192
    positions, -inf after."""
    ctx = [1, 63, 64, 65, 2047, 2048, 2049, 4097, 8192, 5000, 700, 33]
    case = wl.make_case(batch=len(ctx), next_n=1, heads=64, ctx=ctx, max_model_len=8192, seed=55)
    half, ih = run_gpu(case)
    bt = np.full((case.batch, 65536), -1, dtype=np.int32)  # a table as wide as the rows
    bt[:, :case.block_tables.shape[1]] = case.block_tables
    longer = wl.Workload("longer", case.q, case.kv_cache, case.weights, case.context_lens, bt, 65536, 1)
    whole, iw = run_gpu(longer)
    assert np.array_equal(half.view(np.uint32), whole[:, :8192].view(np.uint32))
    assert np.all(whole[:, 8192:] == -np.inf)
    assert np.array_equal(np.sort(ih, axis=1), np.sort(iw, axis=1))


def test_repeatable():
    case = wl.make_named("mtp_b32_n2_ctx32k")
    g1, i1 = run_gpu(case)
    g2, i2 = run_gpu(case)
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))
    assert np.array_equal(np.sort(i1, axis=1), np.sort(i2, axis=1))


@pytest.mark.parametrize("ctx", [2049, 8193, 202752])
def test_exact_ties_take_lowest_positions(ctx):
    """Every key row identical: each row's logits are all equal, so the selection is
    exactly the first k visible positions (ties go to the lowest position)."""
    case = wl.make_case(batch=2, next_n=2, heads=64, ctx=[ctx, 40], max_model_len=ctx, seed=53,
                        pool=ctx + 40)
    case.kv_cache[:] = case.kv_cache[0]
    g, idx = run_gpu(case)
    nv = case.visible()
    for r in range(case.rows):
        vals = g[r, :nv[r]]
        assert np.all(vals == vals[0]), r
        m = min(case.k, int(nv[r]))
        assert np.array_equal(np.sort(idx[r, :m]), np.arange(m)), r
        assert np.all(idx[r, m:] == -1)


def test_all_zero_logits():
    """q = 0: every visible logit is exactly 0 (and never -0 in the order)."""
    case = wl.make_case(batch=3, next_n=1, heads=32, ctx=[3000, 9000, 2048], max_model_len=9000, seed=54)
    case.q[:] = 0
    g, idx = run_gpu(case)
    o = oracle_logits(case)
    check_logits(g, o, "zero q")
    assert np.all(g[np.isfinite(g)] == 0)
    check_topk(idx, g, o, case, what="zero q")
    assert np.array_equal(np.sort(idx[0]), np.arange(2048))


def test_negative_scales():
    """Scales of both signs: relu applies to scale * score, not to the score."""
    neg = lambda rng, n: (rng.lognormal(0, 0.5, n) * np.where(rng.random(n) < 0.5, -1, 1)).astype(np.float32)  # noqa: E731
    case = wl.make_case(batch=4, next_n=2, heads=64, ctx=[100, 2049, 5000, 17], max_model_len=5000,
                        seed=55, scale_fn=neg)
    g, idx = run_gpu(case)
    o = oracle_logits(case)
    check_logits(g, o, "negative scales")
    check_topk(idx, g, o, case, what="negative scales")


@pytest.mark.parametrize("ctx", [1024, 2048, 2049, 3000, 4096, 8192])
def test_page_random_bytes_recipe(ctx):
    """The reproducer's own inputs: every cache byte random (NaN key codes, arbitrary
    fp32 scales), identity table of ctx + 16 blocks, L = 202752. Compared where the
    oracle is finite and below 1e30, with the bound scaled by sum_h |w_h relu(x_h)|
    (cancellation among huge terms), as the page compares finite entries only."""
    case = wl.page_random_bytes_case(ctx)
    g, idx = run_gpu(case)
    o = oracle_logits(case)
    wabs = wl.Workload(case.name, case.q, case.kv_cache, np.abs(case.weights), case.context_lens,
                       case.block_tables, case.max_model_len, 1)
    s = oracle_logits(wabs)
    nv = int(case.visible()[0])
    assert np.all(g[:, nv:] == -np.inf) and np.all(o[:, nv:] == -np.inf)   # the mask is positional
    ok = np.isfinite(o) & (np.abs(o) < 1e30) & np.isfinite(s) & (s < 1e30)
    err = np.abs(g[ok].astype(np.float64) - o[ok])
    assert np.all(err <= 5e-3 + 1e-3 * s[ok]), err.max()
    nan_rows = np.isnan(g).any(axis=1)
    say(f"[gpu] random bytes ctx={ctx}: compared {ok.sum()} of {np.isfinite(o).sum()} finite, "
        f"rows with NaN {nan_rows.sum()}")
    if not nan_rows[0]:
        exact = oracle.topk(g.astype(np.float64), case.context_lens, 1, case.k, case.max_model_len)
        m = min(case.k, ctx)
        assert np.array_equal(np.sort(idx[0, :m]), exact[0, :m])


def test_degenerate_contexts():
    """ctx = 0, ctx < next_n, ctx = 1, and a full-length row."""
    case = wl.make_case(batch=5, next_n=4, heads=32, ctx=[0, 1, 3, 4, 64], max_model_len=64, seed=56)
    g, idx = run_gpu(case)
    o = oracle_logits(case)
    check_logits(g, o, "degenerate ctx")
    check_topk(idx, g, o, case, what="degenerate ctx")
    assert np.all(idx[:4] == -1) and np.all(g[:4] == -np.inf)   # request 0: ctx 0


def test_out_of_range_device_values_are_contained():
    """Device-side values the host cannot check: table entries outside [0, num_blocks)
    give NaN logits at exactly those positions; ctx beyond the table width is read as
    the table width. No access leaves the buffers (the kernel clamps)."""
    case = wl.make_case(batch=3, next_n=1, heads=32, ctx=[100, 50, 80], max_model_len=120, seed=57,
                        table_width=100, poison_unused=False)
    bad = {(0, 7): -1, (0, 99): case.num_blocks, (2, 0): 1 << 30}
    for (b, t), v in bad.items():
        case.block_tables[b, t] = v
    ctx_dev = case.context_lens.copy()
    ctx_dev[1] = 100000          # beyond the table width (100): read as 100
    bt_full = case.block_tables.copy()
    bt_full[1, 50:] = np.arange(50) # make the clamped tail of request 1 well defined
    dev = wl.Workload("bad", case.q, case.kv_cache, case.weights, ctx_dev, bt_full, 120, 1)
    g, idx = run_gpu(dev)
    for (b, t) in bad:
        assert np.isnan(g[b, t]), (b, t)
    ref_bt = bt_full.copy()
    for (b, t) in bad:
        ref_bt[b, t] = 0
    ref = wl.Workload("ref", case.q, case.kv_cache, case.weights, np.array([100, 100, 80]), ref_bt, 120, 1)
    o = oracle_logits(ref)
    mask = np.ones_like(o, dtype=bool)
    for (b, t) in bad:
        mask[b, t] = False
    g2, o2 = np.where(mask, g, 0.0), np.where(mask, o, 0.0)
    check_logits(g2.astype(np.float32), o2, "contained")


def test_graph_replay_matches_eager():
    """The calls allocate nothing and never synchronise, so a step captures into a HIP
    graph. Replays, with eager work and host syncs in between, must equal the eager
    result every time (long rows: the four-kernel top-k path)."""
    import torch
    from fp8_paged_mqa_amd import mqa
    from gpu_helpers import device_inputs, shape_of
    case = wl.make_case(batch=4, next_n=2, heads=64, ctx=[40000, 9000, 100, 3000],
                        max_model_len=40000, seed=58)
    d = device_inputs(case)
    shape = shape_of(case)
    L, k = case.max_model_len, case.k
    out = torch.empty((case.rows, L), dtype=torch.float32, device="cuda")
    idx = torch.empty((case.rows, k), dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(1, mqa.mqa_topk_workspace_bytes(shape, L, k)), dtype=torch.uint8, device="cuda")

    def step():
        mqa.mqa_paged_logits(d["q"], d["kv"], d["w"], d["ctx"], d["bt"], L, out, shape)
        mqa.mqa_topk(out, d["ctx"], L, k, idx, shape, ws)

    step()
    torch.cuda.synchronize()
    ref_logits = out.clone()
    ref_idx = torch.sort(idx, dim=1).values
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        out.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref_logits.view(torch.int32)), rep
        assert torch.equal(torch.sort(idx, dim=1).values, ref_idx), rep
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("next_n,heads", [(2, 64), (4, 32)])
@pytest.mark.parametrize("block_size", [16, 64])
def test_block_size_identity_bitwise(block_size, next_n, heads):
    """A cache in blocks of S (permuted blocks) gives bit-identical logits and the same
    selections as a block_size 1 cache holding each token's row behind a per-token table.
    With S = 64 the decode rows are split over row groups in whole stages; with S = 16 and
    S = 1 one wave holds all of them, in half stages."""
    case = wl.make_case(batch=4, next_n=next_n, heads=heads, ctx=[5, 1000, 2049, 4097], max_model_len=4100,
                        seed=61 + block_size + next_n, block_size=block_size, pool=600)
    gS, iS = run_gpu(case)
    rows = case.kv_cache.reshape(-1, 132)
    bt1 = np.full((case.batch, 4100), -1, dtype=np.int32)
    for b in range(case.batch):
        t = np.arange(int(case.context_lens[b]))
        bt1[b, :t.size] = case.block_tables[b, t // block_size] * block_size + t % block_size
    case1 = wl.Workload("per-token", case.q, rows, case.weights, case.context_lens, bt1,
                        case.max_model_len, case.next_n)
    g1, i1 = run_gpu(case1)
    assert np.array_equal(gS.view(np.uint32), g1.view(np.uint32))
    assert np.array_equal(np.sort(iS, axis=1), np.sort(i1, axis=1))
