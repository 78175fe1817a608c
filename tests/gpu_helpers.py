"""Shared pieces of the GPU parity tests: run a workload through the C-ABI and
compare with the CPU oracle.

Acceptance (the tolerance the target states: 1e-3 relative, 5e-3 absolute near 0):
  logits  identical -inf pattern; finite wherever the oracle is finite;
          |gpu - oracle| <= 5e-3 + 1e-3 * |oracle| on every finite slot.
  top-k   (exact)  the GPU set equals the oracle's top-k evaluated on the GPU's own
                   logits (both decide in fp32 values, lowest position first on ties);
          (oracle) same number of -1 pads as the oracle on its own logits, and every
                   position in the symmetric difference lies within the logit tolerance
                   of the oracle's k-th value (a near-tie).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from fp8_paged_mqa_amd import mqa

ABS_TOL = 5e-3
REL_TOL = 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(wl):
    dev = "cuda"
    return dict(
        q=torch.from_numpy(np.ascontiguousarray(wl.q)).to(dev),
        kv=torch.from_numpy(np.ascontiguousarray(wl.kv_cache)).to(dev),
        w=torch.from_numpy(np.ascontiguousarray(wl.weights)).to(dev),
        ctx=torch.from_numpy(np.ascontiguousarray(wl.context_lens, dtype=np.int32)).to(dev),
        bt=torch.from_numpy(np.ascontiguousarray(wl.block_tables, dtype=np.int32)).to(dev),
    )


def shape_of(wl):
    return mqa.make_shape(wl.batch, wl.next_n, wl.heads, wl.num_blocks, wl.block_tables.shape[1],
                          block_size=wl.block_size)


def run_gpu(wl, k=None, poison=True):
    """Logits [rows, L] float32 and indices [rows, k] int32 from the HIP path. Outputs
    are pre-filled with NaN / a sentinel so that an unwritten slot cannot pass."""
    k = wl.k if k is None else k
    d = device_inputs(wl)
    shape = shape_of(wl)
    L = wl.max_model_len
    out = torch.full((wl.rows, L), float("nan") if poison else 0.0, dtype=torch.float32, device="cuda")
    idx = torch.full((wl.rows, k), -7, dtype=torch.int32, device="cuda")
    nbytes = mqa.mqa_topk_workspace_bytes(shape, L, k)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")  # zero before first use
    mqa.mqa_paged_logits(d["q"], d["kv"], d["w"], d["ctx"], d["bt"], L, out, shape)
    mqa.mqa_topk(out, d["ctx"], L, k, idx, shape, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


def oracle_logits(wl):
    return oracle.paged_mqa_logits(wl.q, wl.kv_cache, wl.weights, wl.context_lens,
                                   wl.block_tables, wl.max_model_len)


def check_logits(g, o, what=""):
    assert g.shape == o.shape
    o_ninf = o == -np.inf
    g_ninf = g == -np.inf
    bad = np.flatnonzero((o_ninf != g_ninf).ravel())
    assert bad.size == 0, f"{what}: -inf pattern differs at {bad.size} slots, first {np.unravel_index(bad[0], o.shape)}"
    fin = np.isfinite(o)
    nonfin = np.flatnonzero((fin & ~np.isfinite(g)).ravel())
    assert nonfin.size == 0, f"{what}: GPU not finite at {nonfin.size} slots, first {np.unravel_index(nonfin[0], o.shape)}"
    err = np.abs(g[fin].astype(np.float64) - o[fin])
    lim = ABS_TOL + REL_TOL * np.abs(o[fin])
    worst = int(np.argmax(err - lim)) if err.size else 0
    assert err.size == 0 or np.all(err <= lim), (
        f"{what}: {(err > lim).sum()} slots out of tolerance; worst err {err[worst]:.3e} at |o|={abs(o[fin][worst]):.3e}")
    return float(err.max()) if err.size else 0.0


def check_topk(idx_g, g, o, wl, k=None, what=""):
    k = wl.k if k is None else k
    L = wl.max_model_len
    nv = wl.visible()
    assert idx_g.shape == (wl.rows, k)
    exact = oracle.topk(g.astype(np.float64), wl.context_lens, wl.next_n, k, L)
    ref = oracle.topk(o, wl.context_lens, wl.next_n, k, L)
    near_ties = 0
    for r in range(wl.rows):
        m = min(k, int(nv[r]))
        row = idx_g[r]
        assert np.all(row[m:] == -1), f"{what}: row {r} padding"
        sel = np.sort(row[:m])
        assert np.all(sel >= 0) and np.unique(sel).size == m, f"{what}: row {r} has duplicates or pads inside"
        assert np.array_equal(sel, exact[r, :m]), f"{what}: row {r} is not the top-{k} of the GPU logits"
        if int(nv[r]) > k:
            gs, os_ = set(sel.tolist()), set(ref[r, :m].tolist())
            vk = o[r, ref[r, :m]].min()
            for p in gs ^ os_:
                assert abs(o[r, p] - vk) <= ABS_TOL + REL_TOL * abs(vk), (
                    f"{what}: row {r} position {p} differs from the oracle's set and is not a near-tie "
                    f"(o={o[r, p]:.6f}, k-th={vk:.6f})")
                near_ties += 1
    return near_ties
