"""Non-paged (prefill) logits on the HIP path vs the oracle, element by element."""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_mqa_amd import mqa
from fp8_paged_mqa_amd import workloads as wl
from gpu_helpers import check_logits, say

pytestmark = pytest.mark.gpu


def _inputs(M, N, H, seed, neg_scales=False):
    rng = np.random.default_rng(seed)
    q = wl.to_e4m3fn_bytes(rng.standard_normal((M, H, 128), dtype=np.float32))
    k = wl.to_e4m3fn_bytes(rng.standard_normal((N, 128), dtype=np.float32))
    sc = rng.lognormal(0.0, 0.5, size=N).astype(np.float32)
    if neg_scales:
        sc[rng.random(N) < 0.3] *= -1
    w = rng.standard_normal((M, H), dtype=np.float32)
    return q, k, sc, w


def _run(q, k, sc, w, ks, ke, stride=None):
    M, H, _ = q.shape
    N = k.shape[0]
    stride = stride or N
    out = torch.full((M, stride), float("nan"), dtype=torch.float32, device="cuda")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    mqa.mqa_logits(d(q), d(k), d(sc), d(w), d(ks.astype(np.int32)), d(ke.astype(np.int32)), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("H", [16, 32, 48, 64])
def test_prefill_causal(H):
    M, N = 300, 777                      # neither a multiple of a workgroup's rows nor of 64 keys
    q, k, sc, w = _inputs(M, N, H, seed=80 + H)
    ks = np.zeros(M, int)
    ke = np.arange(M) + (N - M) + 1      # query i sits at position N - M + i and sees itself
    say(f"[gpu] prefill causal M={M} N={N} H={H}")
    g = _run(q, k, sc, w, ks, ke)
    check_logits(g, oracle.mqa_logits(q, k, sc, w, ks, ke), f"prefill causal H={H}")


def test_prefill_arbitrary_windows_and_stride():
    M, N, H = 257, 1030, 32
    q, k, sc, w = _inputs(M, N, H, seed=90, neg_scales=True)
    rng = np.random.default_rng(91)
    ks = rng.integers(-50, N + 50, size=M)
    ke = rng.integers(-50, N + 50, size=M)
    ks[:5], ke[:5] = [0, 10, 500, -3, 1029], [N, 10, 499, 2000, 1030]   # full, empty, reversed, clipped, one
    say(f"[gpu] prefill windows M={M} N={N}")
    g = _run(q, k, sc, w, ks, ke, stride=1040)
    check_logits(g[:, :N], oracle.mqa_logits(q, k, sc, w, ks, ke), "prefill windows")
    assert np.all(np.isnan(g[:, N:])), "columns past N must stay untouched"


def test_prefill_large_sampled():
    """The shape the page's prefill reproducer reaches (M = 4096, N = 8192, 32 heads),
    causal. Every one of the 4096 rows must hold finite values exactly inside its window
    [0, N - M + m + 1) and -inf everywhere else (the windows need no oracle); 24 rows
    spread over M are compared with the oracle element by element."""
    M, N, H = 4096, 8192, 32
    q, k, sc, w = _inputs(M, N, H, seed=92)
    ks = np.zeros(M, int)
    ke = np.arange(M) + (N - M) + 1
    say(f"[gpu] prefill M={M} N={N} H={H}")
    g = _run(q, k, sc, w, ks, ke)
    col = np.arange(N)[None, :]
    inside = (col >= ks[:, None]) & (col < ke[:, None])
    assert np.array_equal(np.isneginf(g), ~inside), "-inf pattern of the full output"
    assert np.all(np.isfinite(g[inside])), "a slot inside a window is not finite"
    rows = np.unique(np.r_[0, 1, 15, 16, 17, 255, 1000, 2047, 2048, 4095, np.random.default_rng(93).integers(0, M, 14)])
    o = oracle.mqa_logits(q[rows], k, sc, w[rows], ks[rows], ke[rows])
    check_logits(g[rows], o, "prefill large (sampled rows)")


def _draw_prefill_shapes(n=12):
    """Seeded random prefill calls: M and N off every tile multiple, every supported head
    count, windows mixing causal, arbitrary (empty, reversed, clipped) and full ones, and
    an output row stride at or past N."""
    rng = np.random.default_rng(20261203)
    shapes = []
    for _ in range(n):
        M = int(rng.integers(1, 400))
        N = int(rng.integers(1, 3000))
        H = int(rng.choice([16, 32, 48, 64]))
        kind = rng.choice(["causal", "random", "mixed"])
        if kind == "causal":
            ks = np.zeros(M, np.int64)
            ke = np.arange(M) + (N - M) + 1
        else:
            ks = rng.integers(-40, N + 40, size=M)
            ke = rng.integers(-40, N + 40, size=M)
            if kind == "mixed":
                full = rng.random(M) < 0.5
                ks[full], ke[full] = 0, N
        stride = N + int(rng.choice([0, 0, 1, 3, 37]))
        shapes.append((M, N, H, ks, ke, stride, bool(rng.random() < 0.5), int(rng.integers(1 << 30))))
    return shapes


@pytest.mark.parametrize("i", range(12))
def test_prefill_random_shapes(i):
    M, N, H, ks, ke, stride, neg, seed = _draw_prefill_shapes()[i]
    q, k, sc, w = _inputs(M, N, H, seed=seed, neg_scales=neg)
    say(f"[gpu] prefill random shape {i}: M={M} N={N} H={H} stride={stride}")
    g = _run(q, k, sc, w, ks, ke, stride=stride)
    check_logits(g[:, :N], oracle.mqa_logits(q, k, sc, w, ks, ke), f"prefill random shape {i}")
    assert np.all(np.isnan(g[:, N:])), "columns past N must stay untouched"
