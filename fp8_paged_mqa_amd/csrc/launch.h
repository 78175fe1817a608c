// Internal interface between the C-ABI layer (api.cpp) and the kernel translation units.
// Validation happens in api.cpp; the launchers assume valid arguments.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace mqa {

struct LogitsLaunch {
  const uint8_t* q;
  const uint8_t* kv;
  const float* w;
  const int32_t* ctx_lens;
  const int32_t* bt;
  float* out;
  int64_t num_blocks;
  int32_t batch, next_n, heads, bt_stride, max_model_len;
  int32_t block_shift;  // log2(block_size)
};

struct TopkLaunch {
  const float* logits;
  const int32_t* ctx_lens;
  int32_t* idx;
  void* workspace;  // topk_workspace_bytes(rows, max_model_len) bytes, 16-byte aligned
  int32_t batch, next_n, max_model_len, k;
  int32_t token_capacity;  // block_table_stride * block_size: tokens a table row can address
};

struct PrefillLaunch {
  const uint8_t* q;       // [m, heads, 128]
  const uint8_t* k;       // [n, 128]
  const float* k_scale;   // [n]
  const float* w;         // [m, heads]
  const int32_t* ks;      // [m]
  const int32_t* ke;      // [m]
  float* out;             // [m, out_stride]
  int64_t out_stride;
  int32_t m, n, heads;
};

// Enqueue the non-paged logits kernel on `stream`.
hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream);

struct KWriteLaunch {
  const void* k;          // [num_tokens, 128] bf16 or fp32
  const int64_t* slots;   // [num_tokens] cache row of each token (outside [0, num_slots): skipped)
  uint8_t* kv;            // [num_slots, 132]
  int64_t num_tokens, num_slots;
  bool bf16;
};

// Enqueue the K-cache write on `stream`.
hipError_t launch_k_write(const KWriteLaunch& a, hipStream_t stream);

struct SparseMlaLaunch {
  const uint8_t* q;        // [rows, 16, 576] e4m3fn
  const uint8_t* kv;       // [num_blocks * block_size, 576] e4m3fn
  const int32_t* indices;  // [rows, topk] positions, negative = padding
  const int32_t* bt;       // [batch, bt_stride]
  float* out;              // [rows, 16, 512]
  float* lse;              // [rows, 16] or null
  void* workspace;         // SparseMlaPlan::workspace_bytes, 16-byte aligned
  float q_scale, kv_scale, sm_scale;
  int64_t rows, num_blocks;
  int32_t next_n, topk, bt_stride, block_shift;
};

struct SparseMlaPlan {
  int32_t splits = 1, tiles_per_split = 1;
  size_t workspace_bytes = 0;
};

// Split of each row's list over workgroups for the current device, and the workspace
// it needs.
SparseMlaPlan sparse_mla_plan(int64_t rows, int32_t topk);

// Enqueue the sparse MLA decode (and the split merge when plan.splits > 1).
hipError_t launch_sparse_mla(const SparseMlaLaunch& a, const SparseMlaPlan& plan, hipStream_t stream);

// Device scratch the top-k launch needs for `rows` rows of length max_model_len
// (0 when every row fits one workgroup).
size_t topk_workspace_bytes(int64_t rows, int32_t max_model_len);

// Enqueue the logits kernel on `stream`; returns the hipError_t of the launch.
hipError_t launch_logits(const LogitsLaunch& a, hipStream_t stream);

// Enqueue the top-k kernel(s) on `stream`.
hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream);

// Size of the library's static device scratch for the no-allocation top-k, and its
// device address on the current device (looked up once per device; no allocation).
size_t topk_static_scratch_bytes();
hipError_t topk_static_scratch(void** ptr);

}  // namespace mqa
