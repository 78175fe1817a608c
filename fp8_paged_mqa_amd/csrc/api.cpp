// C ABI of libmqa: argument validation on the host, then kernel launches on the
// caller's stream. Declarations and the contract of each entry point: include/mqa.h.
#include "mqa.h"

#include <stdint.h>

#include "launch.h"

namespace {

constexpr int32_t kHeadDim = 128;
constexpr int32_t kMaxTopk = 2048;
constexpr int32_t kMaxModelLen = 1 << 30;
constexpr int32_t kMaxBatch = 8192;  // the logits schedule keeps 3 ints per request in LDS
constexpr int32_t kMaxBlockSize = 1 << 16;

int32_t log2_exact(int32_t v) {
  int32_t s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape checks shared by both entry points. Sizes that cannot describe a problem are
// MQA_ERR_SHAPE; well-formed shapes the kernels do not implement are MQA_ERR_UNSUPPORTED.
int check_shape(const mqa_shape* s, int32_t max_model_len) {
  if (s == nullptr) return MQA_ERR_NULL;
  if (s->batch < 0 || s->next_n < 1 || s->heads < 1 || s->head_dim < 1 || s->block_size < 1 ||
      s->block_table_stride < 1 || s->num_blocks < 1 || max_model_len < 1)
    return MQA_ERR_SHAPE;
  if ((int64_t)s->batch * s->next_n > INT32_MAX) return MQA_ERR_SHAPE;
  if (s->head_dim != kHeadDim) return MQA_ERR_UNSUPPORTED;
  if (s->block_size > kMaxBlockSize || (s->block_size & (s->block_size - 1)) != 0) return MQA_ERR_UNSUPPORTED;
  if ((int64_t)s->block_table_stride * s->block_size > INT32_MAX) return MQA_ERR_UNSUPPORTED;
  if (s->block_size > 1 && s->num_blocks > INT32_MAX / s->block_size) return MQA_ERR_UNSUPPORTED;
  if (s->heads % 16 != 0 || s->heads > 128) return MQA_ERR_UNSUPPORTED;
  if (s->next_n > 4) return MQA_ERR_UNSUPPORTED;
  if (max_model_len > kMaxModelLen) return MQA_ERR_UNSUPPORTED;
  return MQA_OK;
}

constexpr int32_t kMlaHeads = 16, kMlaDim = 576, kMlaVDim = 512;
constexpr int32_t kMlaMaxRows = 65535;   // grid dimension of the row index
constexpr int32_t kMlaMaxTopk = 1 << 20;

int check_mla_shape(const mqa_mla_shape* s) {
  if (s == nullptr) return MQA_ERR_NULL;
  if (s->batch < 0 || s->next_n < 1 || s->topk < 1 || s->block_size < 1 || s->block_table_stride < 1 ||
      s->num_blocks < 1 || s->heads < 1 || s->head_dim < 1 || s->v_dim < 1)
    return MQA_ERR_SHAPE;
  if (s->heads != kMlaHeads || s->head_dim != kMlaDim || s->v_dim != kMlaVDim) return MQA_ERR_UNSUPPORTED;
  if (s->block_size > kMaxBlockSize || (s->block_size & (s->block_size - 1)) != 0) return MQA_ERR_UNSUPPORTED;
  if ((int64_t)s->block_table_stride * s->block_size > INT32_MAX) return MQA_ERR_UNSUPPORTED;
  if (s->num_blocks > INT32_MAX / s->block_size) return MQA_ERR_UNSUPPORTED;
  if ((int64_t)s->batch * s->next_n > kMlaMaxRows || s->topk > kMlaMaxTopk) return MQA_ERR_UNSUPPORTED;
  return MQA_OK;
}

// Checks shared by both top-k entry points that do not involve the workspace.
int check_topk(const mqa_shape* shape, int32_t max_model_len, int32_t k) {
  const int st = check_shape(shape, max_model_len);
  if (st != MQA_OK) return st;
  if (k < 1) return MQA_ERR_SHAPE;
  if (k > kMaxTopk) return MQA_ERR_UNSUPPORTED;
  return MQA_OK;
}

int check_topk_data(const float* logits, const int32_t* context_lens, const int32_t* idx) {
  if (!logits || !context_lens || !idx) return MQA_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(context_lens, 4) || !aligned(idx, 4)) return MQA_ERR_UNSUPPORTED;
  return MQA_OK;
}

int launch_topk_checked(const float* logits, const int32_t* context_lens, int32_t max_model_len, int32_t k,
                        int32_t* idx, const mqa_shape* shape, void* workspace, hipStream_t stream) {
  mqa::TopkLaunch a;
  a.logits = logits;
  a.ctx_lens = context_lens;
  a.idx = idx;
  a.workspace = workspace;
  a.batch = shape->batch;
  a.next_n = shape->next_n;
  a.token_capacity = shape->block_table_stride * shape->block_size;
  a.max_model_len = max_model_len;
  a.k = k;
  return mqa::launch_topk(a, stream) == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* mqa_status_string(int status) {
  switch (status) {
    case MQA_OK: return "ok";
    case MQA_ERR_NULL: return "a required pointer is NULL";
    case MQA_ERR_SHAPE: return "invalid shape or size";
    case MQA_ERR_UNSUPPORTED:
      return "unsupported: needs head_dim 128, block_size a power of two up to 65536 (with "
             "block_table_stride * block_size and, for block_size > 1, num_blocks * block_size "
             "below 2^31), heads a multiple of 16 up to 128, "
             "next_n 1..4, max_model_len <= 2^30, batch <= 8192 and batch * next_n * (ceil(max_model_len / 64) + 1) < 2^31 for the logits, k 1..2048, non-paged n <= 2^29, 16-byte aligned q and weights, "
             "4-byte aligned kv_cache, logits, idx and integer arrays, 16-byte aligned top-k workspace; sparse MLA decode: heads 16, "
             "head_dim 576, v_dim 512, rows <= 65535, topk <= 2^20, 16-byte aligned q, kv_cache, out and workspace";
    case MQA_ERR_WORKSPACE: return "workspace missing or too small";
    case MQA_ERR_HIP: return "HIP launch error";
    case MQA_ERR_SCRATCH:
      return "the problem needs more device scratch than the library's static buffer holds (64 MiB per device)";
    default: return "unknown status";
  }
}

int mqa_paged_logits(const uint8_t* q, const uint8_t* kv_cache, const float* weights,
                     const int32_t* context_lens, const int32_t* block_tables,
                     int32_t max_model_len, float* out, const mqa_shape* shape,
                     hipStream_t stream) {
  const int st = check_shape(shape, max_model_len);
  if (st != MQA_OK) return st;
  if (shape->batch > kMaxBatch) return MQA_ERR_UNSUPPORTED;
  // The kernel counts key stages (64 tokens, plus one unit per request) and -inf tail
  // chunks in 32-bit prefix sums.
  if ((int64_t)shape->batch * shape->next_n * ((max_model_len + 63) / 64 + 1) > INT32_MAX)
    return MQA_ERR_UNSUPPORTED;
  if (shape->batch == 0) return MQA_OK;
  if (!q || !kv_cache || !weights || !context_lens || !block_tables || !out) return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(weights, 16) || !aligned(kv_cache, 4) || !aligned(out, 4) ||
      !aligned(context_lens, 4) || !aligned(block_tables, 4))
    return MQA_ERR_UNSUPPORTED;
  mqa::LogitsLaunch a;
  a.q = q;
  a.kv = kv_cache;
  a.w = weights;
  a.ctx_lens = context_lens;
  a.bt = block_tables;
  a.out = out;
  a.num_blocks = shape->num_blocks;
  a.batch = shape->batch;
  a.next_n = shape->next_n;
  a.heads = shape->heads;
  a.bt_stride = shape->block_table_stride;
  a.max_model_len = max_model_len;
  a.block_shift = log2_exact(shape->block_size);
  return mqa::launch_logits(a, stream) == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

size_t mqa_topk_workspace_bytes(const mqa_shape* shape, int32_t max_model_len, int32_t k) {
  if (check_shape(shape, max_model_len) != MQA_OK || k < 1 || k > kMaxTopk) return 0;
  return mqa::topk_workspace_bytes((int64_t)shape->batch * shape->next_n, max_model_len);
}


int mqa_topk(const float* logits, const int32_t* context_lens, int32_t max_model_len, int32_t k,
             int32_t* idx, const mqa_shape* shape, void* workspace, size_t workspace_bytes,
             hipStream_t stream) {
  int st = check_topk(shape, max_model_len, k);
  if (st != MQA_OK) return st;
  const size_t need = mqa_topk_workspace_bytes(shape, max_model_len, k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return MQA_ERR_WORKSPACE;
  if (shape->batch == 0) return MQA_OK;
  if ((st = check_topk_data(logits, context_lens, idx)) != MQA_OK) return st;
  return launch_topk_checked(logits, context_lens, max_model_len, k, idx, shape, workspace, stream);
}

int mqa_topk_noalloc(const float* logits, const int32_t* context_lens, int32_t max_model_len, int32_t k,
                     int32_t* idx, const mqa_shape* shape, hipStream_t stream) {
  int st = check_topk(shape, max_model_len, k);
  if (st != MQA_OK) return st;
  const size_t need = mqa_topk_workspace_bytes(shape, max_model_len, k);
  if (need > mqa::topk_static_scratch_bytes()) return MQA_ERR_SCRATCH;
  if (shape->batch == 0) return MQA_OK;
  if ((st = check_topk_data(logits, context_lens, idx)) != MQA_OK) return st;
  void* ws = nullptr;
  if (need > 0 && mqa::topk_static_scratch(&ws) != hipSuccess) return MQA_ERR_HIP;
  return launch_topk_checked(logits, context_lens, max_model_len, k, idx, shape, ws, stream);
}

int mqa_logits(const uint8_t* q, const uint8_t* k, const float* k_scale, const float* weights,
               const int32_t* ks, const int32_t* ke, float* out, int64_t out_stride, int32_t m, int32_t n,
               int32_t heads, hipStream_t stream) {
  if (m < 0 || n < 1 || heads < 1 || out_stride < n) return MQA_ERR_SHAPE;
  if (heads % 16 != 0 || heads > 64) return MQA_ERR_UNSUPPORTED;
  if (n > (1 << 29)) return MQA_ERR_UNSUPPORTED;  // byte offsets of a row stay below 2^31
  if (m == 0) return MQA_OK;
  if (!q || !k || !k_scale || !weights || !ks || !ke || !out) return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(weights, 16) || !aligned(k_scale, 4) || !aligned(ks, 4) ||
      !aligned(ke, 4) || !aligned(out, 4))
    return MQA_ERR_UNSUPPORTED;
  mqa::PrefillLaunch a;
  a.q = q;
  a.k = k;
  a.k_scale = k_scale;
  a.w = weights;
  a.ks = ks;
  a.ke = ke;
  a.out = out;
  a.out_stride = out_stride;
  a.m = m;
  a.n = n;
  a.heads = heads;
  return mqa::launch_prefill(a, stream) == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

int mqa_indexer_k_write(const void* k, int32_t k_dtype, int64_t num_tokens, const int64_t* slot_mapping,
                        uint8_t* kv_cache, int64_t num_slots, hipStream_t stream) {
  if (num_tokens < 0 || num_slots < 1) return MQA_ERR_SHAPE;
  if (k_dtype != MQA_DTYPE_BF16 && k_dtype != MQA_DTYPE_F32) return MQA_ERR_UNSUPPORTED;
  if (num_slots > INT64_MAX / 132) return MQA_ERR_SHAPE;
  if (num_tokens == 0) return MQA_OK;
  if (!k || !slot_mapping || !kv_cache) return MQA_ERR_NULL;
  if (!aligned(k, 16) || !aligned(slot_mapping, 8) || !aligned(kv_cache, 4))
    return MQA_ERR_UNSUPPORTED;
  mqa::KWriteLaunch a;
  a.k = k;
  a.slots = slot_mapping;
  a.kv = kv_cache;
  a.num_tokens = num_tokens;
  a.num_slots = num_slots;
  a.bf16 = k_dtype == MQA_DTYPE_BF16;
  return mqa::launch_k_write(a, stream) == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

size_t mqa_sparse_mla_workspace_bytes(const mqa_mla_shape* shape) {
  if (check_mla_shape(shape) != MQA_OK) return 0;
  return mqa::sparse_mla_plan((int64_t)shape->batch * shape->next_n, shape->topk).workspace_bytes;
}

int mqa_sparse_mla_decode(const uint8_t* q, float q_scale, const uint8_t* kv_cache, float kv_scale,
                          const int32_t* indices, const int32_t* block_tables, float sm_scale, float* out,
                          float* lse, const mqa_mla_shape* shape, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  const int st = check_mla_shape(shape);
  if (st != MQA_OK) return st;
  const int64_t rows = (int64_t)shape->batch * shape->next_n;
  if (rows == 0) return MQA_OK;
  if (!q || !kv_cache || !indices || !block_tables || !out) return MQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(indices, 4) ||
      !aligned(block_tables, 4) || (lse && !aligned(lse, 4)) || (workspace && !aligned(workspace, 16)))
    return MQA_ERR_UNSUPPORTED;
  const mqa::SparseMlaPlan plan = mqa::sparse_mla_plan(rows, shape->topk);
  if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
    return MQA_ERR_WORKSPACE;
  mqa::SparseMlaLaunch a;
  a.q = q;
  a.kv = kv_cache;
  a.indices = indices;
  a.bt = block_tables;
  a.out = out;
  a.lse = lse;
  a.workspace = workspace;
  a.q_scale = q_scale;
  a.kv_scale = kv_scale;
  a.sm_scale = sm_scale;
  a.rows = rows;
  a.num_blocks = shape->num_blocks;
  a.next_n = shape->next_n;
  a.topk = shape->topk;
  a.bt_stride = shape->block_table_stride;
  a.block_shift = log2_exact(shape->block_size);
  return mqa::launch_sparse_mla(a, plan, stream) == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

}  // extern "C"
