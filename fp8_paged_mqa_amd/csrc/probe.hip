// Measurement probe: a pure gather of 132-byte cache rows, no arithmetic of the method.
//
// It reads exactly the bytes the paged logits kernel reads for a list of cache rows (the
// 128 key bytes and the 4-byte scale of each row, with the same per-lane access pattern:
// lane (g, c) of a 16-row tile loads bytes [16g, 16g+16) and [64+16g, 64+16g+16) of row c
// plus the scale dword) and folds them into one word per lane so that nothing is
// optimised away. Its time is the ceiling a gather of those rows reaches on this GPU; the
// paged logits kernel is measured against it.
#include <hip/hip_runtime.h>

#include "mqa_probe.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kRow = 132;
constexpr int kThreads = 256;
constexpr int kStage = 64;   // rows per wave per stage (4 tiles of 16)

__device__ __forceinline__ i32x4 load16(const uint8_t* p) {
  i32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
  return v;
}

struct Stage {
  i32x4 lo[4], hi[4];
  int scale[4];
};

// Each wave walks a contiguous share of the row list, DEPTH 64-row stages in flight.
template <int DEPTH>
__global__ __launch_bounds__(kThreads) void probe_gather_kernel(const uint8_t* kv, int64_t nrows, const int32_t* rows,
                                                                  int64_t n, int32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nst = (n + kStage - 1) / kStage;
  const int64_t s_lo = wave * nst / nwaves, s_hi = (wave + 1) * nst / nwaves;
  int acc = 0;
  auto issue = [&](int64_t st, Stage& s) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = st * kStage + u * 16 + c;
      const int64_t r = rows[i < n ? i : n - 1];
      const uint8_t* p = kv + (r < 0 || r >= nrows ? 0 : r) * kRow;  // rows outside the cache read row 0
      s.lo[u] = load16(p + 16 * g);
      s.hi[u] = load16(p + 64 + 16 * g);
      s.scale[u] = *reinterpret_cast<const int*>(p + 128);
    }
  };
  auto fold = [&](const Stage& s) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const i32x4 x = s.lo[u] ^ s.hi[u];
      acc += x.x ^ x.y ^ x.z ^ x.w ^ s.scale[u];
    }
  };
  Stage ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (s_lo + d < s_hi) issue(s_lo + d, ring[d]);
  for (int64_t st = s_lo; st < s_hi; st += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (st + d < s_hi) {
        fold(ring[d]);
        if (st + d + DEPTH < s_hi) issue(st + d + DEPTH, ring[d]);
      }
    }
  }
  sink[wave * 64 + lane] = acc;
}

int compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

}  // namespace

extern "C" {

size_t mqa_probe_gather_sink_words(int32_t groups_per_cu) {
  if (groups_per_cu < 1 || groups_per_cu > 8) return 0;
  return (size_t)compute_units() * groups_per_cu * kThreads;
}

int mqa_probe_gather(const uint8_t* kv_cache, int64_t num_rows_in_cache, const int32_t* rows, int64_t n,
                     int32_t groups_per_cu, int32_t stages_in_flight, int32_t* sink, size_t sink_words,
                     hipStream_t stream) {
  if (n < 0 || num_rows_in_cache < 1) return 2;
  if (groups_per_cu < 1 || groups_per_cu > 8 || (stages_in_flight != 2 && stages_in_flight != 4)) return 3;
  if (n == 0) return 0;
  if (!kv_cache || !rows || !sink) return 1;
  if ((reinterpret_cast<uintptr_t>(kv_cache) & 3) != 0 || (reinterpret_cast<uintptr_t>(rows) & 3) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
    return 3;
  const unsigned blocks = (unsigned)(groups_per_cu * compute_units());
  if (sink_words < (size_t)blocks * kThreads) return 4;
  if (stages_in_flight == 2)
    hipLaunchKernelGGL(probe_gather_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, kv_cache, num_rows_in_cache,
                       rows, n, sink);
  else
    hipLaunchKernelGGL(probe_gather_kernel<4>, dim3(blocks), dim3(kThreads), 0, stream, kv_cache, num_rows_in_cache,
                       rows, n, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
