// Measurement probe: a pure gather of 132-byte cache rows, no arithmetic of the method.
//
// It reads exactly the bytes the paged logits kernel reads for a list of cache rows (the
// 128 key bytes and the 4-byte scale of each row, with the same per-lane access pattern:
// lane (g, c) of a 16-row tile loads bytes [16g, 16g+16) and [64+16g, 64+16g+16) of row c
// plus the scale dword) and folds them into one word per lane so that nothing is
// optimised away. Its time is the ceiling a gather of those rows reaches on this GPU; the
// paged logits kernel is measured against it.
//
// A second form gathers the same rows straight into LDS (global_load_lds_dwordx4): each
// row's 16-byte-aligned 144-byte window, which holds its 132 bytes, as nine 16-byte pieces,
// so that loads in flight cost no registers.
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

// Direct-to-LDS form. Per wave: DEPTH stage buffers of 64 windows (9 KB each) and the row
// indices of a batch of kBatch stages, all in the wave's own part of LDS (no wave reads
// another's, so no barrier). The gathers are inline asm (an LDS destination behind a
// vector-memory counter is not something the compiler tracks), so the kernel issues its own
// waits: a batch's row indices are loaded with ordinary loads and drained before its first
// gather, and inside a batch the only vector-memory operations are the gathers.
constexpr int kPieces = 9;                              // 16-byte pieces of a 144-byte window
constexpr int kLdsStage = kStage * kPieces * 16;        // 9216 bytes: one stage of one wave
constexpr int kBatch = 8;                               // stages whose row indices are in LDS
constexpr int kWavesPerGroup = kThreads / 64;

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}

// 16 bytes from src into LDS bytes [m0 + 16*lane, +16).
__device__ __forceinline__ void load_lds16(const uint8_t* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}

template <int DEPTH>
__global__ __launch_bounds__(kThreads) void probe_gather_lds_kernel(const uint8_t* kv, int64_t nrows,
                                                                      const int32_t* rows, int64_t n,
                                                                      int32_t* sink) {
  static_assert(DEPTH >= 2 && DEPTH <= 3, "stages in flight");
  __shared__ __attribute__((aligned(16))) uint8_t buf[kWavesPerGroup][DEPTH][kLdsStage];
  __shared__ int32_t ridx[kWavesPerGroup][kBatch * kStage];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerGroup + w;
  const int64_t nst = (n + kStage - 1) / kStage;
  const int64_t s_lo = wave * nst / nwaves, s_hi = (wave + 1) * nst / nwaves;
  // Last 16-byte-aligned piece start that stays inside the cache.
  const int64_t last_piece = ((nrows * kRow) & ~(int64_t)15) - 16;
  int acc = 0;
  for (int64_t b0 = s_lo; b0 < s_hi; b0 += kBatch) {
    const int nb = (int)(s_hi - b0 < kBatch ? s_hi - b0 : kBatch);
    for (int j = 0; j < nb; ++j) {
      const int64_t i = (b0 + j) * kStage + lane;
      const int32_t r = rows[i < n ? i : n - 1];
      ridx[w][j * kStage + lane] = (r < 0 || r >= nrows) ? 0 : r;  // rows outside the cache read row 0
    }
    __builtin_amdgcn_s_waitcnt(0);  // indices loaded and in LDS; no gather is in flight
    asm volatile("" ::: "memory");
    auto issue = [&](int j, int slot) {
      const uint32_t base = (uint32_t)(uintptr_t)&buf[w][slot][0];
      // Addresses first (the LDS reads of the indices wait once), then the nine gathers
      // back to back.
      const uint8_t* src[kPieces];
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        const int ch = i * 64 + lane;  // piece ch of the stage: window ch / 9, piece ch % 9
        const int rs = ch / kPieces, pc = ch - rs * kPieces;
        const int64_t r = ridx[w][j * kStage + rs];
        int64_t a = ((r * kRow) & ~(int64_t)15) + 16 * pc;
        src[i] = kv + (a < last_piece ? a : last_piece);
      }
#pragma unroll
      for (int i = 0; i < kPieces; ++i)
        load_lds16(src[i], (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + 1024 * i)));
    };
    for (int d = 0; d < DEPTH && d < nb; ++d) issue(d, d);
    for (int j = 0; j < nb; ++j) {
      const int after = (nb - 1 - j < DEPTH - 1) ? nb - 1 - j : DEPTH - 1;  // stages issued after j
      if (after >= 2) wait_vm<2 * kPieces>();
      else if (after == 1) wait_vm<kPieces>();
      else wait_vm<0>();
      const int slot = j % DEPTH;
#pragma unroll
      for (int i = 0; i < kPieces; ++i) acc ^= *reinterpret_cast<const int*>(&buf[w][slot][1024 * i + 16 * lane]);
      wait_lgkm0();  // this slot's reads are done before it is refilled
      if (j + DEPTH < nb) issue(j + DEPTH, slot);
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

int mqa_probe_gather_lds(const uint8_t* kv_cache, int64_t num_rows_in_cache, const int32_t* rows, int64_t n,
                         int32_t groups_per_cu, int32_t stages_in_flight, int32_t* sink, size_t sink_words,
                         hipStream_t stream) {
  if (n < 0 || num_rows_in_cache < 1) return 2;
  if (groups_per_cu < 1 || groups_per_cu > 8 || (stages_in_flight != 2 && stages_in_flight != 3)) return 3;
  if (n == 0) return 0;
  if (!kv_cache || !rows || !sink) return 1;
  if ((reinterpret_cast<uintptr_t>(kv_cache) & 15) != 0 || (reinterpret_cast<uintptr_t>(rows) & 3) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
    return 3;
  const unsigned blocks = (unsigned)(groups_per_cu * compute_units());
  if (sink_words < (size_t)blocks * kThreads) return 4;
  if (stages_in_flight == 2)
    hipLaunchKernelGGL(probe_gather_lds_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, kv_cache,
                       num_rows_in_cache, rows, n, sink);
  else
    hipLaunchKernelGGL(probe_gather_lds_kernel<3>, dim3(blocks), dim3(kThreads), 0, stream, kv_cache,
                       num_rows_in_cache, rows, n, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
