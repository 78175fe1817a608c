"""Seeded random call shapes, each checked against the oracle like the named workloads
(needs an MI355X).

The shapes are drawn once, from a fixed seed, over the whole supported domain: batch,
next_n 1..4, heads 16..128, block sizes 1..64, permuted and interleaved tables, k from 1
to 2048, max_model_len up to 12 000 (and 210 000 in the second set), and context lengths that mix uniform draws with the
boundaries where a kernel changes form (k and k + 1, multiples of 64 and their
neighbours, 0, max_model_len). They reach every launch form of the logits kernel (small
call, scheduled whole stages at one or two workgroups per CU, half stages, row groups) and
every top-k kernel without being chosen for any of them, which is the point: a shape no
hand-written case thought of. A second set draws max_model_len from 8193 to 210 000, so that
the whole-row selects with 16 and 32 values per thread and the chunked kernel get the same.
"""
import numpy as np
import pytest

from fp8_paged_mqa_amd import workloads as wl
from gpu_helpers import check_logits, check_topk, oracle_logits, run_gpu, say

pytestmark = pytest.mark.gpu

N_SHAPES = 30
N_LONG = 16
WORK_CAP = 2.5e7  # sum(ctx) * next_n * heads: keeps each oracle call to about a second


def _draw_shapes(n=N_SHAPES, seed=20261202, l_lo=1, l_hi=12000, cap=WORK_CAP):
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        batch = int(rng.choice([1, 2, 3, 5, 16, 33, 64, 65, 100]))
        next_n = int(rng.integers(1, 5))
        heads = int(rng.choice([16, 32, 48, 64, 80, 128]))
        block_size = int(rng.choice([1, 1, 1, 2, 16, 64]))
        k = int(rng.choice([1, 7, 100, 2048, 2048]))
        L = int(rng.integers(l_lo, l_hi + 1))
        special = [0, 1, k, k + 1, 63, 64, 65, 2047, 2048, 2049, 4096, 8192, 8193, 32768, 32769, L - 1, L]
        ctx = rng.integers(0, L + 1, batch)
        pick = rng.random(batch) < 0.4
        ctx[pick] = rng.choice(special, int(pick.sum()))
        ctx = np.clip(ctx, 0, L).astype(np.int64)
        if ctx.sum() * next_n * heads > cap:
            continue
        table = str(rng.choice(["permuted", "interleaved"]))
        shapes.append(dict(batch=batch, next_n=next_n, heads=heads, block_size=block_size, k=k,
                           L=L, ctx=ctx.tolist(), table=table, seed=int(rng.integers(1 << 30))))
    return shapes


SHAPES = _draw_shapes()
# max_model_len past 8192 and past 32768: rows the top-k selects whole with 16 or 32 values
# per thread, and the chunked kernel's long rows beside its whole rows.
LONG_SHAPES = _draw_shapes(N_LONG, seed=20261204, l_lo=8193, l_hi=210000, cap=6e7)


def _run_shape(s, i):
    case = wl.make_case(batch=s["batch"], next_n=s["next_n"], heads=s["heads"], ctx=s["ctx"],
                        max_model_len=s["L"], seed=s["seed"], table=s["table"], k=s["k"],
                        block_size=s["block_size"])
    what = (f"shape {i}: B={s['batch']} N={s['next_n']} H={s['heads']} S={s['block_size']} "
            f"L={s['L']} k={s['k']} {s['table']}")
    say(f"[gpu] {what}")
    g, idx = run_gpu(case)
    o = oracle_logits(case)
    check_logits(g, o, what)
    check_topk(idx, g, o, case, what=what)


@pytest.mark.parametrize("i", range(N_SHAPES))
def test_random_shape(i):
    _run_shape(SHAPES[i], i)


@pytest.mark.parametrize("i", range(N_LONG))
def test_random_long_shape(i):
    _run_shape(LONG_SHAPES[i], f"long {i}")
