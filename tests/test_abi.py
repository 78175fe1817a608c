"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from fp8_paged_mqa_amd import mqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mqa.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(mqa_\w+)\s*\(", text, flags=re.M)))


def all_headers():
    inc = os.path.join(ROOT, "include")
    return sorted(os.path.join(inc, f) for f in os.listdir(inc) if f.endswith(".h"))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(mqa.EXPORTS)
    probe = os.path.join(ROOT, "include", "mqa_probe.h")
    assert declared_functions(probe) == sorted(mqa.PROBE_EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", mqa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    names = [n for h in all_headers() for n in declared_functions(h)]
    assert len(names) == len(mqa.EXPORTS) + len(mqa.PROBE_EXPORTS)
    for name in names:
        assert name in exported, name
        assert hasattr(mqa._lib, name)


def test_probe_host_checks():
    # rejected before any HIP call
    sink = ctypes.c_void_p(0x10000)
    probe = mqa._lib.mqa_probe_gather
    assert probe(FAKE, 10, FAKE, -1, 2, 2, sink, 1 << 20, None) == 2
    assert probe(FAKE, 0, FAKE, 5, 2, 2, sink, 1 << 20, None) == 2
    assert probe(FAKE, 10, FAKE, 5, 0, 2, sink, 1 << 20, None) == 3
    assert probe(FAKE, 10, FAKE, 5, 9, 2, sink, 1 << 20, None) == 3
    assert probe(FAKE, 10, FAKE, 5, 2, 3, sink, 1 << 20, None) == 3
    assert probe(None, 10, FAKE, 5, 2, 2, sink, 1 << 20, None) == 1
    assert probe(ctypes.c_void_p(0x10002), 10, FAKE, 5, 2, 2, sink, 1 << 20, None) == 3
    assert probe(FAKE, 10, FAKE, 0, 2, 2, sink, 0, None) == 0
    lds = mqa._lib.mqa_probe_gather_lds
    assert lds(FAKE, 10, FAKE, -1, 2, 2, sink, 1 << 20, None) == 2
    assert lds(FAKE, 10, FAKE, 5, 2, 4, sink, 1 << 20, None) == 3    # 2 or 3 stages
    assert lds(FAKE, 10, FAKE, 5, 9, 2, sink, 1 << 20, None) == 3
    assert lds(None, 10, FAKE, 5, 2, 3, sink, 1 << 20, None) == 1
    assert lds(ctypes.c_void_p(0x10004), 10, FAKE, 5, 2, 3, sink, 1 << 20, None) == 3  # cache 16-byte aligned
    assert lds(FAKE, 10, FAKE, 0, 2, 3, sink, 0, None) == 0


def test_status_strings():
    for st in range(7):
        assert mqa.mqa_status_string(st)
    assert mqa.mqa_status_string(0) == "ok"
    assert "unknown" in mqa.mqa_status_string(99)


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every case below is rejected first


def call_logits(shape, L=100, ptrs=(FAKE,) * 6):
    q, kv, w, ctx, bt, out = ptrs
    return mqa._lib.mqa_paged_logits(q, kv, w, ctx, bt, L, out,
                                     ctypes.byref(shape) if shape is not None else None, None)


def call_topk(shape, L=100, k=2048, ws=None, ws_bytes=0, ptrs=(FAKE,) * 3):
    logits, ctx, idx = ptrs
    return mqa._lib.mqa_topk(logits, ctx, L, k, idx,
                             ctypes.byref(shape) if shape is not None else None, ws, ws_bytes, None)


def good_shape(**kw):
    d = dict(batch=2, next_n=2, heads=64, num_blocks=1000, block_table_stride=100)
    d.update(kw)
    return mqa.make_shape(**d)


@pytest.mark.parametrize("kw,L,status", [
    (dict(batch=-1), 100, mqa.MQA_ERR_SHAPE),
    (dict(next_n=0), 100, mqa.MQA_ERR_SHAPE),
    (dict(heads=0), 100, mqa.MQA_ERR_SHAPE),
    (dict(num_blocks=0), 100, mqa.MQA_ERR_SHAPE),
    (dict(block_table_stride=0), 100, mqa.MQA_ERR_SHAPE),
    ({}, 0, mqa.MQA_ERR_SHAPE),
    (dict(head_dim=64), 100, mqa.MQA_ERR_UNSUPPORTED),
    (dict(block_size=0), 100, mqa.MQA_ERR_SHAPE),
    (dict(block_size=3), 100, mqa.MQA_ERR_UNSUPPORTED),    # not a power of two
    (dict(block_size=48), 100, mqa.MQA_ERR_UNSUPPORTED),
    (dict(block_size=1 << 17), 100, mqa.MQA_ERR_UNSUPPORTED),
    (dict(block_size=64, block_table_stride=1 << 25), 100, mqa.MQA_ERR_UNSUPPORTED),  # W*S >= 2^31
    (dict(block_size=64, num_blocks=1 << 25), 100, mqa.MQA_ERR_UNSUPPORTED),          # rows >= 2^31
    (dict(heads=24), 100, mqa.MQA_ERR_UNSUPPORTED),
    (dict(heads=144), 100, mqa.MQA_ERR_UNSUPPORTED),
    (dict(next_n=5), 100, mqa.MQA_ERR_UNSUPPORTED),
    ({}, (1 << 30) + 1, mqa.MQA_ERR_UNSUPPORTED),
])
def test_logits_rejects_bad_shapes(kw, L, status):
    assert call_logits(good_shape(**kw), L=L) == status
    assert call_topk(good_shape(**kw), L=L) == status


def test_null_pointers():
    assert call_logits(None) == mqa.MQA_ERR_NULL
    assert call_topk(None) == mqa.MQA_ERR_NULL
    for i in range(6):
        ptrs = [FAKE] * 6
        ptrs[i] = None
        assert call_logits(good_shape(), ptrs=tuple(ptrs)) == mqa.MQA_ERR_NULL, i
    for i in range(3):
        ptrs = [FAKE] * 3
        ptrs[i] = None
        assert call_topk(good_shape(), ptrs=tuple(ptrs)) == mqa.MQA_ERR_NULL, i


def test_misaligned_pointers():
    odd = ctypes.c_void_p(0x10002)
    for i in range(6):
        ptrs = [FAKE] * 6
        ptrs[i] = odd
        assert call_logits(good_shape(), ptrs=tuple(ptrs)) == mqa.MQA_ERR_UNSUPPORTED, i
    q_off = ctypes.c_void_p(0x10004)   # 4-byte aligned but not 16: q and weights need 16
    assert call_logits(good_shape(), ptrs=(q_off,) + (FAKE,) * 5) == mqa.MQA_ERR_UNSUPPORTED
    assert call_logits(good_shape(), ptrs=(FAKE, FAKE, q_off) + (FAKE,) * 3) == mqa.MQA_ERR_UNSUPPORTED


def test_logits_batch_limit():
    assert call_logits(good_shape(batch=8193)) == mqa.MQA_ERR_UNSUPPORTED
    assert call_topk(good_shape(batch=8193)) != mqa.MQA_ERR_UNSUPPORTED


def test_logits_work_count_limit():
    # stages and -inf chunks are counted in 32 bits: B * N * (ceil(L / 64) + 1) < 2^31
    assert call_logits(good_shape(batch=8192, next_n=4), L=1 << 30) == mqa.MQA_ERR_UNSUPPORTED
    assert call_logits(good_shape(batch=1024, next_n=4), L=1 << 25) == mqa.MQA_ERR_UNSUPPORTED  # 4096 * (2^19 + 1)


def test_topk_k_range():
    assert call_topk(good_shape(), k=0) == mqa.MQA_ERR_SHAPE
    assert call_topk(good_shape(), k=2049) == mqa.MQA_ERR_UNSUPPORTED


def test_empty_batch_is_a_no_op():
    # batch 0 enqueues nothing, so null data pointers are fine and no GPU is touched
    assert call_logits(good_shape(batch=0), ptrs=(None,) * 6) == mqa.MQA_OK
    assert call_topk(good_shape(batch=0), ptrs=(None,) * 3) == mqa.MQA_OK


def test_topk_workspace_alignment_and_size():
    # max_model_len above 32768 needs the workspace: missing, short or not 16-byte aligned
    # are all MQA_ERR_WORKSPACE, checked before any pointer is used
    shape = good_shape(block_table_stride=40000)
    need = mqa.mqa_topk_workspace_bytes(shape, 40000, 2048)
    assert need > 0
    assert call_topk(shape, L=40000) == mqa.MQA_ERR_WORKSPACE
    assert call_topk(shape, L=40000, ws=ctypes.c_void_p(0x10000), ws_bytes=need - 1) == mqa.MQA_ERR_WORKSPACE
    assert call_topk(shape, L=40000, ws=ctypes.c_void_p(0x10008), ws_bytes=need) == mqa.MQA_ERR_WORKSPACE
    assert mqa.mqa_topk_workspace_bytes(shape, 32768, 2048) == 0
    assert mqa.mqa_topk_workspace_bytes(shape, 32769, 2048) > 0


def call_topk_noalloc(shape, L=100, k=2048, ptrs=(FAKE,) * 3):
    logits, ctx, idx = ptrs
    return mqa._lib.mqa_topk_noalloc(logits, ctx, L, k, idx,
                                     ctypes.byref(shape) if shape is not None else None, None)


def test_topk_noalloc_host_checks():
    # the same shape checks as mqa_topk, then the static scratch limit (64 MiB), all
    # before any HIP call
    assert call_topk_noalloc(None) == mqa.MQA_ERR_NULL
    assert call_topk_noalloc(good_shape(block_size=3)) == mqa.MQA_ERR_UNSUPPORTED
    assert call_topk_noalloc(good_shape(), k=0) == mqa.MQA_ERR_SHAPE
    assert call_topk_noalloc(good_shape(), k=2049) == mqa.MQA_ERR_UNSUPPORTED
    big = good_shape(batch=1024, next_n=1, block_table_stride=202752)
    assert mqa.mqa_topk_workspace_bytes(big, 202752, 2048) > 64 << 20
    assert call_topk_noalloc(big, L=202752) == mqa.MQA_ERR_SCRATCH
    ok = good_shape(batch=128, next_n=4, block_table_stride=202752)
    assert 0 < mqa.mqa_topk_workspace_bytes(ok, 202752, 2048) <= 64 << 20
    assert call_topk_noalloc(ok, L=202752, ptrs=(None,) * 3) == mqa.MQA_ERR_NULL
    assert call_topk_noalloc(good_shape(batch=0), ptrs=(None,) * 3) == mqa.MQA_OK
    odd = ctypes.c_void_p(0x10002)
    for i in range(3):
        ptrs = [FAKE] * 3
        ptrs[i] = odd
        assert call_topk_noalloc(good_shape(), ptrs=tuple(ptrs)) == mqa.MQA_ERR_UNSUPPORTED, i


def test_workspace_size_query():
    assert mqa.mqa_topk_workspace_bytes(good_shape(), 100, 2048) >= 0
    assert mqa.mqa_topk_workspace_bytes(good_shape(block_size=3), 100, 2048) == 0
    assert mqa.mqa_topk_workspace_bytes(good_shape(), 100, 0) == 0


def call_kwrite(dtype=0, T=4, nslots=100, ptrs=(FAKE,) * 3):
    k, slots, kv = ptrs
    return mqa._lib.mqa_indexer_k_write(k, dtype, T, slots, kv, nslots, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), mqa.MQA_ERR_SHAPE),
    (dict(nslots=0), mqa.MQA_ERR_SHAPE),
    (dict(dtype=2), mqa.MQA_ERR_UNSUPPORTED),
    (dict(dtype=-1), mqa.MQA_ERR_UNSUPPORTED),
    (dict(ptrs=(None, FAKE, FAKE)), mqa.MQA_ERR_NULL),
    (dict(ptrs=(FAKE, None, FAKE)), mqa.MQA_ERR_NULL),
    (dict(ptrs=(FAKE, FAKE, None)), mqa.MQA_ERR_NULL),
    (dict(ptrs=(ctypes.c_void_p(0x10008), FAKE, FAKE)), mqa.MQA_ERR_UNSUPPORTED),      # keys need 16 B
    (dict(dtype=1, ptrs=(ctypes.c_void_p(0x10004), FAKE, FAKE)), mqa.MQA_ERR_UNSUPPORTED),
    (dict(ptrs=(FAKE, ctypes.c_void_p(0x10004), FAKE)), mqa.MQA_ERR_UNSUPPORTED),      # int64 slots need 8 B
    (dict(ptrs=(FAKE, FAKE, ctypes.c_void_p(0x10002))), mqa.MQA_ERR_UNSUPPORTED),
])
def test_k_write_rejects(kw, status):
    assert call_kwrite(**kw) == status


def test_k_write_zero_tokens_is_a_no_op():
    assert call_kwrite(T=0, ptrs=(None,) * 3) == mqa.MQA_OK


def call_prefill(m=4, n=64, heads=32, stride=64, ptrs=(FAKE,) * 7):
    q, k, sc, w, ks, ke, out = ptrs
    return mqa._lib.mqa_logits(q, k, sc, w, ks, ke, out, stride, m, n, heads, None)


@pytest.mark.parametrize("kw,status", [
    (dict(m=-1), mqa.MQA_ERR_SHAPE),
    (dict(n=0), mqa.MQA_ERR_SHAPE),
    (dict(heads=0), mqa.MQA_ERR_SHAPE),
    (dict(stride=63), mqa.MQA_ERR_SHAPE),
    (dict(heads=24), mqa.MQA_ERR_UNSUPPORTED),
    (dict(heads=80), mqa.MQA_ERR_UNSUPPORTED),
    (dict(n=(1 << 29) + 1, stride=(1 << 29) + 1), mqa.MQA_ERR_UNSUPPORTED),
    (dict(ptrs=(None,) + (FAKE,) * 6), mqa.MQA_ERR_NULL),
    (dict(ptrs=(FAKE,) * 6 + (None,)), mqa.MQA_ERR_NULL),
    (dict(ptrs=(ctypes.c_void_p(0x10008),) + (FAKE,) * 6), mqa.MQA_ERR_UNSUPPORTED),
    (dict(ptrs=(FAKE, ctypes.c_void_p(0x10004)) + (FAKE,) * 5), mqa.MQA_ERR_UNSUPPORTED),
    (dict(ptrs=(FAKE,) * 3 + (ctypes.c_void_p(0x10004),) + (FAKE,) * 3), mqa.MQA_ERR_UNSUPPORTED),
])
def test_prefill_logits_rejects(kw, status):
    assert call_prefill(**kw) == status


def test_prefill_zero_rows_is_a_no_op():
    assert call_prefill(m=0, ptrs=(None,) * 7) == mqa.MQA_OK


def mla_shape(**kw):
    base = dict(batch=2, next_n=2, heads=16, head_dim=576, v_dim=512, block_size=1, block_table_stride=100,
                topk=64, num_blocks=1000)
    base.update(kw)
    return mqa.mqa_mla_shape(*(base[f] for f, _ in mqa.mqa_mla_shape._fields_))


def call_mla(shape=None, ptrs=None, lse=None, ws=None, ws_bytes=0):
    q, kv, idx, bt, out = ptrs if ptrs is not None else (FAKE,) * 5
    shp = None if shape is None else ctypes.byref(shape)
    return mqa._lib.mqa_sparse_mla_decode(q, 1.0, kv, 1.0, idx, bt, 0.07, out, lse, shp, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), mqa.MQA_ERR_SHAPE),
    (dict(next_n=0), mqa.MQA_ERR_SHAPE),
    (dict(topk=0), mqa.MQA_ERR_SHAPE),
    (dict(block_size=0), mqa.MQA_ERR_SHAPE),
    (dict(block_table_stride=0), mqa.MQA_ERR_SHAPE),
    (dict(num_blocks=0), mqa.MQA_ERR_SHAPE),
    (dict(heads=32), mqa.MQA_ERR_UNSUPPORTED),
    (dict(head_dim=512), mqa.MQA_ERR_UNSUPPORTED),
    (dict(v_dim=576), mqa.MQA_ERR_UNSUPPORTED),
    (dict(block_size=3), mqa.MQA_ERR_UNSUPPORTED),
    (dict(block_size=1 << 17), mqa.MQA_ERR_UNSUPPORTED),
    (dict(block_size=64, block_table_stride=1 << 25), mqa.MQA_ERR_UNSUPPORTED),
    (dict(block_size=64, num_blocks=1 << 25), mqa.MQA_ERR_UNSUPPORTED),
    (dict(batch=65536, next_n=1), mqa.MQA_ERR_UNSUPPORTED),
    (dict(topk=(1 << 20) + 1), mqa.MQA_ERR_UNSUPPORTED),
])
def test_sparse_mla_rejects_shapes(kw, status):
    assert call_mla(mla_shape(**kw)) == status


def test_sparse_mla_rejects_pointers():
    assert call_mla(None) == mqa.MQA_ERR_NULL
    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = None
        assert call_mla(mla_shape(), tuple(ptrs)) == mqa.MQA_ERR_NULL, i
    for i in (0, 1, 4):  # q, kv_cache, out: 16-byte alignment
        ptrs = [FAKE] * 5
        ptrs[i] = ctypes.c_void_p(0x10008)
        assert call_mla(mla_shape(), tuple(ptrs)) == mqa.MQA_ERR_UNSUPPORTED, i
    for i in (2, 3):  # indices, block_tables: 4-byte alignment
        ptrs = [FAKE] * 5
        ptrs[i] = ctypes.c_void_p(0x10002)
        assert call_mla(mla_shape(), tuple(ptrs)) == mqa.MQA_ERR_UNSUPPORTED, i
    assert call_mla(mla_shape(), lse=ctypes.c_void_p(0x10002)) == mqa.MQA_ERR_UNSUPPORTED


def test_sparse_mla_zero_rows_is_a_no_op():
    assert call_mla(mla_shape(batch=0), (None,) * 5) == mqa.MQA_OK


def test_sparse_mla_workspace():
    big = mla_shape(batch=64, next_n=1, topk=2048)
    need = mqa.mqa_sparse_mla_workspace_bytes(big)
    assert need > 0 and need % (2 * 16 * 512 + 4 * 2 * 16) == 0  # per split: f16 mean, f32 max and sum
    assert call_mla(big) == mqa.MQA_ERR_WORKSPACE
    assert call_mla(big, ws=FAKE, ws_bytes=need - 1) == mqa.MQA_ERR_WORKSPACE
    assert mqa.mqa_sparse_mla_workspace_bytes(mla_shape(batch=1, next_n=1, topk=64)) == 0
    assert mqa.mqa_sparse_mla_workspace_bytes(mla_shape(heads=8)) == 0


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it says so and exits non-zero before it
    touches a device (runs here, without a GPU)."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
