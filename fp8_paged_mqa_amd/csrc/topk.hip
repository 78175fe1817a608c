// Per-row top-k of the indexer logits on gfx950 (radix select).
//
// Row r = b*N + j keeps the k largest logits of its visible prefix [0, nv),
// nv = ctx_b - N + j + 1 (stepcodex.com issue "[Bug] aiter ops triton attention
// pa_mqa_logits", section "Minimal reproduction": top-k with k = min(2048, ctx),
// compared as a set). Equal logits are taken lowest position first.
//
// Selection order as one 64-bit integer per element:
//   e = key(logit) << 32 | (0xFFFFFFFF - position)
// where key() is the order-preserving map of an fp32 onto uint32 (-0 folded onto +0).
// Larger e means "selected earlier", and e is unique per position, so the top k of a
// row is exactly the k largest e: a radix select over e needs no tie rule of its own.
// Digits of e, most significant first: 11, 11, 10 bits of the key, then 11, 11, 10
// bits of the position part (only reached when the k-th key is tied).
//
// One workgroup (16 waves) per row:
//   1. LDS histogram of the top 11 key bits over the row (LDS atomics).
//   2. A block-wide scan from the top finds the bin holding the k-th element.
//   3. A second pass over the row emits every element of a higher bin straight to the
//      output (wave ballot + mbcnt compaction, one LDS atomic per wave) and copies the
//      elements of the threshold bin into an LDS candidate list.
//   4. The remaining digits refine the threshold within the candidates the same way,
//      stopping as soon as the threshold bin is taken whole. If the threshold bin does
//      not fit in LDS (extreme ties, e.g. a constant row), the refinement re-reads the
//      row from global memory instead: slower, same result.
// Rows with nv <= k select every visible position without reading the logits.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace mqa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kCap = 8192;  // LDS candidate slots (64 KB)

struct Params {
  const float* logits;
  const int32_t* ctx_lens;
  int32_t* idx;
  int32_t N, W, L, k;
};

// Digit `level` of the selection key: bit offset and width.
__device__ __forceinline__ int digit_shift(int level) {
  return level == 0 ? 53 : level == 1 ? 42 : level == 2 ? 32 : level == 3 ? 21 : level == 4 ? 10 : 0;
}
__device__ __forceinline__ int digit_width(int level) { return (level == 2 || level == 5) ? 10 : 11; }

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t element(const float* row, int t) {
  return ((uint64_t)order_key(row[t]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
}

__device__ __forceinline__ int position(uint64_t e) { return (int)(0xFFFFFFFFu - (uint32_t)e); }

struct Shared {
  uint32_t hist[kBins];
  uint64_t cand[kCap];
  uint32_t wave_sum[kWaves];
  uint32_t n_out;
  uint32_t n_cand;
  uint32_t bin;
  uint32_t above;
};

// Wave-aggregated append: lanes with `pred` get consecutive slots from *counter.
// Must be called by all 64 lanes of the wave. Returns the slot (or -1).
__device__ __forceinline__ int wave_append(bool pred, uint32_t* counter) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return -1;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
  base = __shfl(base, leader);
  const uint32_t below =
      __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
  return pred ? (int)(base + below) : -1;
}

// Exclusive prefix sum over the 1024 threads in thread order.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, Shared& sh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) sh.wave_sum[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += sh.wave_sum[w];
  __syncthreads();
  return before + incl - v;
}

// Finds the bin B (scanning from the top) with above(B) < rem <= above(B) + hist[B].
// Leaves B in sh.bin and above(B) in sh.above. All threads must call it.
__device__ void find_bin(Shared& sh, uint32_t rem) {
  if (threadIdx.x == 0) {
    sh.bin = 0;
    sh.above = 0;
  }
  const int hi = kBins - 1 - 2 * (int)threadIdx.x;
  const int lo = hi - 1;
  const uint32_t ch = sh.hist[hi], cl = sh.hist[lo];
  const uint32_t excl = block_exclusive_scan(ch + cl, sh);
  if (excl < rem && rem <= excl + ch) {
    sh.bin = (uint32_t)hi;
    sh.above = excl;
  } else if (excl + ch < rem && rem <= excl + ch + cl) {
    sh.bin = (uint32_t)lo;
    sh.above = excl + ch;
  }
  __syncthreads();
}

__device__ __forceinline__ void clear_hist(Shared& sh) {
  for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0;
  __syncthreads();
}

// Refinement over a source of elements: either the LDS candidate list or the full row
// (filtered by the level-0 prefix). `rem` elements are still to be taken from those
// matching `prefix` under `pmask`.
template <bool FromRow>
__device__ void refine(Shared& sh, const float* row, int n, uint64_t prefix, uint64_t pmask,
                       uint32_t rem, int32_t* out, int k) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  auto fetch = [&](int i) -> uint64_t { return FromRow ? element(row, i) : sh.cand[i]; };

  for (int level = 1; level < 6; ++level) {
    const int shift = digit_shift(level);
    const uint64_t dmask = (1ull << digit_width(level)) - 1;
    clear_hist(sh);
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint64_t e = fetch(i);
      if ((e & pmask) == prefix) atomicAdd(&sh.hist[(e >> shift) & dmask], 1u);
    }
    __syncthreads();
    find_bin(sh, rem);
    const uint64_t bin = sh.bin;
    const uint32_t above = sh.above;
    const uint32_t cnt = sh.hist[bin];
    // Emit the elements of higher bins.
    for (int base = wave * 64; base < n; base += kThreads) {
      const int i = base + lane;
      const uint64_t e = i < n ? fetch(i) : 0;
      const bool take = i < n && (e & pmask) == prefix && ((e >> shift) & dmask) > bin;
      const int slot = wave_append(take, &sh.n_out);
      if (slot >= 0 && slot < k) out[slot] = position(e);
    }
    rem -= above;
    prefix |= bin << shift;
    pmask |= dmask << shift;
    __syncthreads();
    if (cnt == rem) {  // the whole threshold bin is selected
      for (int base = wave * 64; base < n; base += kThreads) {
        const int i = base + lane;
        const uint64_t e = i < n ? fetch(i) : 0;
        const int slot = wave_append(i < n && (e & pmask) == prefix, &sh.n_out);
        if (slot >= 0 && slot < k) out[slot] = position(e);
      }
      return;
    }
  }
}

__global__ __launch_bounds__(kThreads) void topk_rows_kernel(Params p) {
  __shared__ Shared sh;
  const int r = blockIdx.x;
  const int b = r / p.N;
  const int j = r - b * p.N;
  int ctx = p.ctx_lens[b];
  ctx = max(0, min(ctx, min(p.W, p.L)));
  const int nv = max(0, min(ctx - p.N + j + 1, p.L));
  const int k = p.k;
  const int m = min(k, nv);
  int32_t* out = p.idx + (int64_t)r * k;

  for (int i = m + threadIdx.x; i < k; i += kThreads) out[i] = -1;
  if (nv <= k) {
    for (int t = threadIdx.x; t < nv; t += kThreads) out[t] = t;
    return;
  }

  const float* row = p.logits + (int64_t)r * p.L;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // Level 0 over the whole row.
  clear_hist(sh);
  if (threadIdx.x == 0) {
    sh.n_out = 0;
    sh.n_cand = 0;
  }
  for (int t = threadIdx.x; t < nv; t += kThreads) atomicAdd(&sh.hist[order_key(row[t]) >> 21], 1u);
  __syncthreads();
  find_bin(sh, (uint32_t)k);
  const uint32_t bin0 = sh.bin;
  const uint32_t rem = (uint32_t)k - sh.above;
  const uint32_t cnt0 = sh.hist[bin0];

  for (int base = wave * 64; base < nv; base += kThreads) {
    const int t = base + lane;
    const bool in = t < nv;
    const uint32_t key = in ? order_key(row[t]) : 0u;
    const uint32_t d = key >> 21;
    const int slot = wave_append(in && d > bin0, &sh.n_out);
    if (slot >= 0 && slot < k) out[slot] = t;
    const bool cand = in && d == bin0 && cnt0 <= (uint32_t)kCap;
    const int cslot = wave_append(cand, &sh.n_cand);
    if (cslot >= 0 && cslot < kCap) sh.cand[cslot] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
  }
  __syncthreads();

  const uint64_t prefix = (uint64_t)bin0 << 53;
  const uint64_t pmask = 0x7FFull << 53;
  if (cnt0 == rem) {  // the threshold bin is taken whole
    if (cnt0 <= (uint32_t)kCap) {
      for (int base = wave * 64; base < (int)cnt0; base += kThreads) {
        const int i = base + lane;
        const int slot = wave_append(i < (int)cnt0, &sh.n_out);
        if (slot >= 0 && slot < k) out[slot] = position(sh.cand[i]);
      }
    } else {
      for (int base = wave * 64; base < nv; base += kThreads) {
        const int t = base + lane;
        const bool in = t < nv && (order_key(t < nv ? row[t] : 0.0f) >> 21) == bin0;
        const int slot = wave_append(in, &sh.n_out);
        if (slot >= 0 && slot < k) out[slot] = t;
      }
    }
    return;
  }
  if (cnt0 <= (uint32_t)kCap)
    refine<false>(sh, row, (int)cnt0, prefix, pmask, rem, out, k);
  else
    refine<true>(sh, row, nv, prefix, pmask, rem, out, k);
}

}  // namespace

hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream) {
  Params p;
  p.logits = a.logits;
  p.ctx_lens = a.ctx_lens;
  p.idx = a.idx;
  p.N = a.next_n;
  p.W = a.bt_stride;
  p.L = a.max_model_len;
  p.k = a.k;
  const int64_t rows = (int64_t)a.batch * a.next_n;
  if (rows > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mqa
