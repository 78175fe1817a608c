"""The K-cache write (quantise keys into 132-byte rows) on the HIP path vs the oracle:
the written bytes must be identical (codes and scale are integer/bit decisions taken
in fp32 on both sides), rows of skipped slots untouched."""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_mqa_amd import mqa
from fp8_paged_mqa_amd import workloads as wl
from gpu_helpers import check_logits, oracle_logits, run_gpu, say

pytestmark = pytest.mark.gpu


def _keys(rng, T, dtype):
    mag = rng.lognormal(0.0, 2.0, size=(T, 1)).astype(np.float32)
    k = (rng.standard_normal((T, 128)).astype(np.float32) * mag)
    special = [np.zeros(128), np.r_[np.zeros(127), [3.0]], np.full(128, -2.5), np.linspace(-1e-30, 1e-30, 128),
               np.linspace(-1e30, 1e30, 128), (np.arange(128) % 9 - 4) * 2.0 ** -12,
               # rows the hardware conversion must not take: a NaN key, infinite keys, and
               # a largest magnitude so small that amax / 448 underflows to zero
               np.r_[[np.nan], np.linspace(-3, 3, 127)], np.r_[[np.inf], np.ones(127)],
               np.r_[np.ones(127), [-np.inf]], np.r_[[1.4e-45, -1.4e-45], np.zeros(126)],
               # a subnormal largest magnitude with a nonzero (subnormal) scale
               np.linspace(-1e-40, 1e-40, 128)]
    for i, row in enumerate(special):
        k[i] = row
    t = torch.from_numpy(k)
    if dtype == torch.bfloat16:
        t = t.to(torch.bfloat16)
    return t


def _run(k, slots, cache_np):
    kv = torch.from_numpy(cache_np.copy()).cuda()
    mqa.mqa_indexer_k_write(k.cuda(), torch.from_numpy(slots).cuda(), kv)
    torch.cuda.synchronize()
    return kv.cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_k_write_bitwise(dtype):
    rng = np.random.default_rng(71)
    T, nslots = 3000, 5000
    k = _keys(rng, T, dtype)
    slots = rng.permutation(nslots)[:T].astype(np.int64)
    slots[::97] = -1
    slots[5::211] = nslots + 3                                # outside: skipped
    cache = rng.integers(0, 256, size=(nslots, 132), dtype=np.uint8)
    say(f"[gpu] k write {dtype} T={T}")
    got = _run(k, slots, cache)
    want = oracle.write_k_cache(k.float().numpy(), slots, cache)
    diff = np.flatnonzero((got != want).any(axis=1))
    assert diff.size == 0, f"{diff.size} rows differ, first {diff[:5]}"


def test_k_write_blocked_cache_and_logits():
    """Keys written into a 64-token-block cache through slot = block * 64 + offset, then
    read back by the paged logits: identical bytes and oracle parity."""
    rng = np.random.default_rng(72)
    S, nblk = 64, 40
    case = wl.make_case(batch=3, next_n=2, heads=64, ctx=[100, 1000, 700], max_model_len=1024,
                        seed=73, block_size=S, pool=nblk, poison_unused=False)
    T = int(case.context_lens.sum())
    k = torch.from_numpy((rng.standard_normal((T, 128)) * 2).astype(np.float32)).to(torch.bfloat16)
    slots = np.concatenate([case.block_tables[b, np.arange(c) // S].astype(np.int64) * S + np.arange(c) % S
                            for b, c in enumerate(case.context_lens.tolist())])
    got = _run(k, slots, case.kv_cache)
    want = oracle.write_k_cache(k.float().numpy(), slots, case.kv_cache)
    assert np.array_equal(got, want)
    written = wl.Workload("written", case.q, got, case.weights, case.context_lens, case.block_tables,
                          case.max_model_len, case.next_n)
    g, _ = run_gpu(written)
    check_logits(g, oracle_logits(written), "logits of written cache")


def test_k_write_benchmark_size():
    """The call `bench.py --op kwrite` times: 65 536 bf16 tokens (normal keys times a
    lognormal magnitude per token) into permuted slots of a 600 000-row cache, in one
    launch. Every written row is compared with the oracle's quantisation of its token, and
    every other row must still be zero."""
    rng = np.random.Generator(np.random.PCG64(7))
    T, nslots = 65536, 600_000
    k32 = (rng.standard_normal((T, 128), dtype=np.float32)
           * rng.lognormal(0, 1, size=(T, 1)).astype(np.float32))
    k = torch.from_numpy(k32).to(torch.bfloat16)
    slots = rng.permutation(nslots)[:T].astype(np.int64)
    say(f"[gpu] k write benchmark size T={T} slots={nslots}")
    kv = torch.zeros((nslots, 132), dtype=torch.uint8, device="cuda")
    mqa.mqa_indexer_k_write(k.cuda(), torch.from_numpy(slots).cuda(), kv)
    torch.cuda.synchronize()
    got = kv.cpu().numpy()
    keys = k.float().numpy()
    want = np.zeros((T, 132), np.uint8)
    for i in range(T):
        codes, scale = oracle.quantize_k_row(keys[i])
        want[i, :128] = codes
        want[i, 128:] = np.frombuffer(np.float32(scale).astype("<f4").tobytes(), dtype=np.uint8)
    diff = np.flatnonzero((got[slots] != want).any(axis=1))
    assert diff.size == 0, f"{diff.size} of {T} rows differ, first tokens {diff[:5]}"
    untouched = np.ones(nslots, bool)
    untouched[slots] = False
    assert not got[untouched].any(), "a row outside the slot mapping was written"
