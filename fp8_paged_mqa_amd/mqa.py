"""ctypes binding of libmqa's C ABI (include/mqa.h), same entry-point names.

Argument marshalling only: tensors are passed as device pointers, shapes as an
``mqa_shape`` struct, and the current torch stream as the HIP stream. Every step
of the computation runs in libmqa's kernels. Importing this module loads the
library and raises if it has not been built (``python -m fp8_paged_mqa_amd.build``);
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmqa.so")

MQA_OK, MQA_ERR_NULL, MQA_ERR_SHAPE, MQA_ERR_UNSUPPORTED, MQA_ERR_WORKSPACE, MQA_ERR_HIP, MQA_ERR_SCRATCH = range(7)

EXPORTS = ("mqa_paged_logits", "mqa_topk", "mqa_topk_noalloc", "mqa_topk_workspace_bytes", "mqa_status_string",
           "mqa_indexer_k_write", "mqa_logits", "mqa_sparse_mla_decode", "mqa_sparse_mla_workspace_bytes")
MQA_DTYPE_BF16, MQA_DTYPE_F32 = 0, 1
# The measurement probe (include/mqa_probe.h): not part of the operation.
PROBE_EXPORTS = ("mqa_probe_gather", "mqa_probe_gather_lds", "mqa_probe_gather_sink_words")


class mqa_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("next_n", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("block_table_stride", ctypes.c_int32), ("num_blocks", ctypes.c_int64)]


class mqa_mla_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("next_n", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("block_table_stride", ctypes.c_int32), ("topk", ctypes.c_int32), ("num_blocks", ctypes.c_int64)]


class MqaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({mqa_status_string(status)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m fp8_paged_mqa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    shp = ctypes.POINTER(mqa_shape)
    lib.mqa_paged_logits.argtypes = [vp, vp, vp, vp, vp, i32, vp, shp, vp]
    lib.mqa_paged_logits.restype = ctypes.c_int
    lib.mqa_topk.argtypes = [vp, vp, i32, i32, vp, shp, vp, sz, vp]
    lib.mqa_topk.restype = ctypes.c_int
    lib.mqa_topk_noalloc.argtypes = [vp, vp, i32, i32, vp, shp, vp]
    lib.mqa_topk_noalloc.restype = ctypes.c_int
    lib.mqa_topk_workspace_bytes.argtypes = [shp, i32, i32]
    lib.mqa_topk_workspace_bytes.restype = sz
    lib.mqa_status_string.argtypes = [ctypes.c_int]
    lib.mqa_status_string.restype = ctypes.c_char_p
    i64 = ctypes.c_int64
    lib.mqa_indexer_k_write.argtypes = [vp, i32, i64, vp, vp, i64, vp]
    lib.mqa_indexer_k_write.restype = ctypes.c_int
    lib.mqa_logits.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, vp]
    lib.mqa_logits.restype = ctypes.c_int
    f32 = ctypes.c_float
    mshp = ctypes.POINTER(mqa_mla_shape)
    lib.mqa_sparse_mla_decode.argtypes = [vp, f32, vp, f32, vp, vp, f32, vp, vp, mshp, vp, sz, vp]
    lib.mqa_sparse_mla_decode.restype = ctypes.c_int
    lib.mqa_sparse_mla_workspace_bytes.argtypes = [mshp]
    lib.mqa_sparse_mla_workspace_bytes.restype = sz
    lib.mqa_probe_gather_sink_words.argtypes = [i32]
    lib.mqa_probe_gather_sink_words.restype = sz
    lib.mqa_probe_gather.argtypes = [vp, i64, vp, i64, i32, i32, vp, sz, vp]
    lib.mqa_probe_gather.restype = ctypes.c_int
    lib.mqa_probe_gather_lds.argtypes = [vp, i64, vp, i64, i32, i32, vp, sz, vp]
    lib.mqa_probe_gather_lds.restype = ctypes.c_int
    return lib


_lib = _load()


def make_shape(batch, next_n, heads, num_blocks, block_table_stride, head_dim=128, block_size=1):
    return mqa_shape(int(batch), int(next_n), int(heads), int(head_dim), int(block_size),
                     int(block_table_stride), int(num_blocks))


def shape_of(q: torch.Tensor, kv_cache: torch.Tensor, block_tables: torch.Tensor) -> mqa_shape:
    """Shape struct from tensors laid out as the header describes: q [B,N,H,D],
    kv_cache [num_blocks, D+4] (block_size 1) or [num_blocks, block_size, (1,) D+4],
    block_tables [B, W]."""
    B, N, H, D = q.shape
    return make_shape(B, N, H, kv_cache.shape[0], block_tables.shape[1], head_dim=D,
                      block_size=kv_cache.shape[1] if kv_cache.dim() >= 3 else 1)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def mqa_status_string(status: int) -> str:
    return _lib.mqa_status_string(int(status)).decode()


def mqa_paged_logits(q, kv_cache, weights, context_lens, block_tables, max_model_len, out,
                     shape: mqa_shape | None = None, stream=None, check: bool = True) -> int:
    """out[B*N, L] <- indexer logits. Tensors must be contiguous device tensors:
    q uint8 [B,N,H,128], kv_cache uint8 [num_blocks,132], weights f32 [B*N,H],
    context_lens i32 [B], block_tables i32 [B,W], out f32 [B*N,L]."""
    if shape is None:
        shape = shape_of(q, kv_cache, block_tables)
    st = _lib.mqa_paged_logits(_ptr(q), _ptr(kv_cache), _ptr(weights), _ptr(context_lens),
                               _ptr(block_tables), int(max_model_len), _ptr(out),
                               ctypes.byref(shape), _stream(stream))
    if check and st != MQA_OK:
        raise MqaError(st, "mqa_paged_logits")
    return st


def mqa_topk_workspace_bytes(shape: mqa_shape, max_model_len: int, k: int) -> int:
    return int(_lib.mqa_topk_workspace_bytes(ctypes.byref(shape), int(max_model_len), int(k)))


def mqa_topk(logits, context_lens, max_model_len, k, idx, shape: mqa_shape, workspace=None,
             stream=None, check: bool = True) -> int:
    """idx[B*N, k] <- per-row top-k positions (a set per row, -1 padded)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.mqa_topk(_ptr(logits), _ptr(context_lens), int(max_model_len), int(k), _ptr(idx),
                       ctypes.byref(shape), _ptr(workspace), ws_bytes, _stream(stream))
    if check and st != MQA_OK:
        raise MqaError(st, "mqa_topk")
    return st


def mqa_topk_noalloc(logits, context_lens, max_model_len, k, idx, shape: mqa_shape, stream=None,
                     check: bool = True) -> int:
    """As mqa_topk, with the library's static device scratch instead of a workspace."""
    st = _lib.mqa_topk_noalloc(_ptr(logits), _ptr(context_lens), int(max_model_len), int(k), _ptr(idx),
                               ctypes.byref(shape), _stream(stream))
    if check and st != MQA_OK:
        raise MqaError(st, "mqa_topk_noalloc")
    return st


def mqa_logits(q, k, k_scale, weights, ks, ke, out, stream=None, check: bool = True) -> int:
    """out[M, >= N] <- non-paged logits: q uint8 [M,H,128], k uint8 [N,128], k_scale f32 [N],
    weights f32 [M,H], ks/ke i32 [M] (row i sees keys [ks[i], ke[i]))."""
    M, H, _ = q.shape
    N = k.shape[0]
    st = _lib.mqa_logits(_ptr(q), _ptr(k), _ptr(k_scale), _ptr(weights), _ptr(ks), _ptr(ke), _ptr(out),
                         int(out.stride(0)), int(M), int(N), int(H), _stream(stream))
    if check and st != MQA_OK:
        raise MqaError(st, "mqa_logits")
    return st


def mqa_indexer_k_write(k, slot_mapping, kv_cache, stream=None, check: bool = True) -> int:
    """Quantise k [T, 128] (bf16 or fp32) into the cache rows slot_mapping (int64 [T])
    of kv_cache (uint8 [num_slots, 132] or [num_blocks, block_size, (1,) 132])."""
    if k.dtype == torch.bfloat16:
        dtype = MQA_DTYPE_BF16
    elif k.dtype == torch.float32:
        dtype = MQA_DTYPE_F32
    else:
        dtype = -1  # rejected by the library
    num_slots = kv_cache.numel() // 132
    st = _lib.mqa_indexer_k_write(_ptr(k), dtype, int(k.shape[0]), _ptr(slot_mapping), _ptr(kv_cache),
                                  int(num_slots), _stream(stream))
    if check and st != MQA_OK:
        raise MqaError(st, "mqa_indexer_k_write")
    return st


def mla_shape_of(q, kv_cache, block_tables, indices, next_n=1) -> mqa_mla_shape:
    """Shape struct from tensors laid out as the header describes: q [B*N, 16, 576],
    kv_cache [num_slots, 576] (block_size 1) or [num_blocks, S, (1,) 576], block_tables
    [B, W], indices [B*N, topk]."""
    rows, heads, dim = q.shape
    bs = kv_cache.shape[1] if kv_cache.dim() >= 3 else 1
    return mqa_mla_shape(int(block_tables.shape[0]), int(next_n), int(heads), int(dim), 512, int(bs),
                         int(block_tables.shape[1]), int(indices.shape[1]), int(kv_cache.shape[0]))


def mqa_sparse_mla_workspace_bytes(shape: mqa_mla_shape) -> int:
    return int(_lib.mqa_sparse_mla_workspace_bytes(ctypes.byref(shape)))


def mqa_sparse_mla_decode(q, q_scale, kv_cache, kv_scale, indices, block_tables, sm_scale, out, lse=None,
                          shape: mqa_mla_shape | None = None, workspace=None, next_n=1, stream=None,
                          check: bool = True) -> int:
    """out[B*N, 16, 512] (and lse[B*N, 16]) <- attention of each row over its listed
    positions. q uint8 [B*N,16,576], kv_cache uint8 (576-byte rows), indices int32
    [B*N, topk], block_tables int32 [B, W]; out / lse float32."""
    if shape is None:
        shape = mla_shape_of(q, kv_cache, block_tables, indices, next_n)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.mqa_sparse_mla_decode(_ptr(q), float(q_scale), _ptr(kv_cache), float(kv_scale), _ptr(indices),
                                    _ptr(block_tables), float(sm_scale), _ptr(out), _ptr(lse), ctypes.byref(shape),
                                    _ptr(workspace), ws_bytes, _stream(stream))
    if check and st != MQA_OK:
        raise MqaError(st, "mqa_sparse_mla_decode")
    return st


def mqa_probe_gather_sink_words(groups_per_cu: int) -> int:
    return int(_lib.mqa_probe_gather_sink_words(int(groups_per_cu)))


def mqa_probe_gather(kv_cache, rows, groups_per_cu, sink, stages_in_flight=2, stream=None, check: bool = True) -> int:
    """Measurement probe: gathers the 132-byte cache rows listed in rows (int32 [n]) the
    way the paged logits kernel reads them, folding them into sink (int32)."""
    st = _lib.mqa_probe_gather(_ptr(kv_cache), int(kv_cache.numel() // 132), _ptr(rows), int(rows.numel()),
                               int(groups_per_cu), int(stages_in_flight), _ptr(sink), int(sink.numel()),
                               _stream(stream))
    if check and st != 0:
        raise RuntimeError(f"mqa_probe_gather: status {st}")
    return st


def mqa_probe_gather_lds(kv_cache, rows, groups_per_cu, sink, stages_in_flight=2, stream=None,
                         check: bool = True) -> int:
    """The probe's direct-to-LDS form: each listed row's 16-byte-aligned 144-byte window
    gathered into LDS (stages_in_flight 2 or 3)."""
    st = _lib.mqa_probe_gather_lds(_ptr(kv_cache), int(kv_cache.numel() // 132), _ptr(rows), int(rows.numel()),
                                   int(groups_per_cu), int(stages_in_flight), _ptr(sink), int(sink.numel()),
                                   _stream(stream))
    if check and st != 0:
        raise RuntimeError(f"mqa_probe_gather_lds: status {st}")
    return st


class Indexer:
    """Holds the device buffers of one problem shape (output, indices, top-k
    workspace) so that repeated calls allocate nothing."""

    def __init__(self, batch, next_n, heads, num_blocks, block_table_stride, max_model_len,
                 k=2048, device="cuda"):
        self.shape = make_shape(batch, next_n, heads, num_blocks, block_table_stride)
        self.max_model_len = int(max_model_len)
        self.k = int(k)
        rows = batch * next_n
        self.logits = torch.empty((rows, self.max_model_len), dtype=torch.float32, device=device)
        self.idx = torch.empty((rows, self.k), dtype=torch.int32, device=device)
        nbytes = mqa_topk_workspace_bytes(self.shape, self.max_model_len, self.k)
        self.workspace = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)  # zero before first use

    def __call__(self, q, kv_cache, weights, context_lens, block_tables, stream=None):
        mqa_paged_logits(q, kv_cache, weights, context_lens, block_tables, self.max_model_len,
                         self.logits, self.shape, stream)
        mqa_topk(self.logits, context_lens, self.max_model_len, self.k, self.idx, self.shape,
                 self.workspace, stream)
        return self.logits, self.idx
