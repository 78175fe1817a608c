"""mqa_topk_noalloc (the library's static device scratch) against mqa_topk (a caller
workspace), through the C ABI: identical indices on two calls in a row, the second
smaller, both on rows longer than 32768 (the chunked passes that use scratch), and on a
call whose rows need no scratch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from fp8_paged_mqa_amd import mqa
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _logits(rows, L, seed):
    """Seeded logits with exact ties (a run of equal values) and signed zeros."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, L)) * 30).astype(np.float32)
    x[:, 100:400] = np.float32(12.5)
    x[:, 500:520] = np.float32(-0.0)
    x[:, 520:540] = np.float32(0.0)
    return x


def _call(fn, logits, ctx, L, k, idx, shape, *extra):
    st = fn(ctypes.c_void_p(logits.data_ptr()), ctypes.c_void_p(ctx.data_ptr()), L, k,
            ctypes.c_void_p(idx.data_ptr()), ctypes.byref(shape), *extra,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == mqa.MQA_OK, mqa.mqa_status_string(st)


@pytest.mark.parametrize("calls", [
    # (batch, next_n, L, contexts): the second call of each sequence is smaller
    [(4, 2, 202752, [202752, 131071, 65537, 40000]), (2, 1, 70000, [69999, 33000])],
    [(3, 1, 8192, [8192, 3000, 2049]), (1, 1, 4096, [2049])],
])
def test_noalloc_matches_workspace_entry_point(calls):
    k = 2048
    for n, (B, N, L, ctx) in enumerate(calls):
        say(f"[gpu] topk_noalloc call {n}: B={B} N={N} L={L}")
        rows = B * N
        host = _logits(rows, L, seed=700 + n)
        logits = torch.from_numpy(host).cuda()
        ctx_d = torch.tensor(ctx, dtype=torch.int32, device="cuda")
        shape = mqa.make_shape(B, N, 64, 1, L)
        want = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
        got = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
        nbytes = mqa.mqa_topk_workspace_bytes(shape, L, k)
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        _call(mqa._lib.mqa_topk_noalloc, logits, ctx_d, L, k, got, shape)
        _call(mqa._lib.mqa_topk, logits, ctx_d, L, k, want, shape, ctypes.c_void_p(ws.data_ptr()),
              ctypes.c_size_t(ws.numel()))
        torch.cuda.synchronize()
        g, w = got.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(np.sort(g, axis=1), np.sort(w, axis=1)), f"call {n}: sets differ"
        ref = oracle.topk(host.astype(np.float64), np.array(ctx), N, k, L)
        assert np.array_equal(np.sort(g, axis=1), np.sort(ref, axis=1)), f"call {n}: not the oracle's top-k"
