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
// Rows with nv <= k select every visible position without reading the logits.
//
// Rows with k < nv <= kChunk (8192): one workgroup of 1024 threads owns the row. Each
// thread loads its 8 logits in one batch and keeps their keys in registers; an LDS
// histogram of the top 11 key bits and a block scan from the top find the bin of the
// k-th element; one pass over the registers emits every element of a higher bin
// (wave ballot + mbcnt compaction, one LDS atomic per wave) and copies the threshold
// bin into an LDS candidate list, which the remaining digits refine the same way.
//
// Longer rows are split into 8192-element chunks, one workgroup each:
//   hist   each chunk adds its LDS histogram into the row's global histogram;
//   split  each chunk finds the threshold bin from the global histogram, emits its
//          elements above it straight to the output (global atomic slot counter per
//          row) and appends its threshold-bin elements to the row's candidate list;
//   finish one workgroup per row refines the candidates in LDS. If the threshold bin
//          holds more than kCap elements (extreme ties, e.g. a constant row) it
//          refines over the whole row from global memory instead: slower, same result.
// A fill kernel clears the histograms and counters first, in stream order.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace mqa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 8;                     // logits per thread per chunk
constexpr int kChunk = kThreads * kPer;     // 8192
constexpr int kBins = 2048;
constexpr int kCap = 8192;                  // LDS candidate slots (64 KB)

struct Params {
  const float* logits;
  const int32_t* ctx_lens;
  int32_t* idx;
  uint32_t* hist;      // [rows][kBins]
  uint32_t* counters;  // [rows][2]: emitted, candidates
  uint64_t* cand;      // [rows][kCap]
  int32_t N, W, L, k, nchunk;
};

__device__ __forceinline__ int digit_shift(int level) {
  return level == 0 ? 53 : level == 1 ? 42 : level == 2 ? 32 : level == 3 ? 21 : level == 4 ? 10 : 0;
}
__device__ __forceinline__ int digit_width(int level) { return (level == 2 || level == 5) ? 10 : 11; }

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t compose(uint32_t key, int t) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
}

__device__ __forceinline__ int position(uint64_t e) { return (int)(0xFFFFFFFFu - (uint32_t)e); }

// Row geometry shared by all kernels.
struct Row {
  int r, nv, k;
  __device__ Row(const Params& p, int row) : r(row), k(p.k) {
    const int b = row / p.N;
    const int j = row - b * p.N;
    int ctx = p.ctx_lens[b];
    ctx = max(0, min(ctx, min(p.W, p.L)));
    nv = max(0, min(ctx - p.N + j + 1, p.L));
  }
};

struct Core {
  uint32_t hist[kBins];
  uint32_t wave_sum[kWaves];
  uint32_t n_out;
  uint32_t n_cand;
  uint32_t bin;
  uint32_t above;
};

struct Full : Core {
  uint64_t cand[kCap];
};

// Wave-aggregated append: lanes with `pred` get consecutive slots from *counter (LDS or
// global). Must be called by all 64 lanes of the wave. Returns the slot (or -1).
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
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, Core& sh) {
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
__device__ void find_bin(Core& sh, uint32_t rem) {
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

__device__ __forceinline__ void clear_hist(Core& sh) {
  for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0;
  __syncthreads();
}

// Keys of the chunk starting at `base`: element i of thread tid is base + i*1024 + tid.
// All loads are issued before any is used (addresses clamped into the row).
__device__ __forceinline__ void load_chunk(const float* row, int base, int nv, uint32_t (&key)[kPer]) {
  float v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) v[i] = row[min(base + i * kThreads + (int)threadIdx.x, nv - 1)];
#pragma unroll
  for (int i = 0; i < kPer; ++i) key[i] = order_key(v[i]);
}

// Refinement over the LDS candidate list (FromRow = false) or the whole row filtered by
// the level-0 prefix (FromRow = true). `rem` elements are still to be taken from those
// matching `prefix` under `pmask`; emitted positions go to out[sh.n_out++].
template <bool FromRow>
__device__ void refine(Full& sh, const float* row, int n, uint64_t prefix, uint64_t pmask,
                       uint32_t rem, int32_t* out, int k) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  auto fetch = [&](int i) -> uint64_t { return FromRow ? compose(order_key(row[i]), i) : sh.cand[i]; };

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
    for (int base = wave * 64; base < n; base += kThreads) {  // emit the higher bins
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

// Whole select of a row with k < nv <= kChunk by one workgroup.
__device__ void select_short_row(const Params& p, const Row& row_info, Full& sh) {
  const int nv = row_info.nv, k = row_info.k;
  const float* row = p.logits + (int64_t)row_info.r * p.L;
  int32_t* out = p.idx + (int64_t)row_info.r * k;

  uint32_t key[kPer];
  load_chunk(row, 0, nv, key);
  clear_hist(sh);
  if (threadIdx.x == 0) {
    sh.n_out = 0;
    sh.n_cand = 0;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (i * kThreads + (int)threadIdx.x < nv) atomicAdd(&sh.hist[key[i] >> 21], 1u);
  __syncthreads();
  find_bin(sh, (uint32_t)k);
  const uint32_t bin0 = sh.bin;
  const uint32_t rem = (uint32_t)k - sh.above;
  const uint32_t cnt0 = sh.hist[bin0];
  const bool whole = cnt0 == rem;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int t = i * kThreads + (int)threadIdx.x;
    const bool in = t < nv;
    const uint32_t d = key[i] >> 21;
    const int slot = wave_append(in && (d > bin0 || (whole && d == bin0)), &sh.n_out);
    if (slot >= 0 && slot < k) out[slot] = t;
    const int cslot = wave_append(in && !whole && d == bin0, &sh.n_cand);
    if (cslot >= 0 && cslot < kCap) sh.cand[cslot] = compose(key[i], t);
  }
  __syncthreads();
  if (!whole) refine<false>(sh, row, (int)cnt0, (uint64_t)bin0 << 53, 0x7FFull << 53, rem, out, k);
}

// Rows with nv <= k, and rows that fit one chunk, are finished here by chunk 0's workgroup.
// Longer rows: this chunk's histogram is added into the row's global histogram.
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(Params p) {
  __shared__ Full sh;
  const int r = blockIdx.x / p.nchunk;
  const int ch = blockIdx.x - r * p.nchunk;
  const Row ri(p, r);
  const int nv = ri.nv, k = ri.k;
  if (nv <= kChunk || nv <= k) {
    if (ch != 0) return;
    int32_t* out = p.idx + (int64_t)r * k;
    const int m = min(k, nv);
    for (int i = m + threadIdx.x; i < k; i += kThreads) out[i] = -1;
    if (nv <= k) {
      for (int t = threadIdx.x; t < nv; t += kThreads) out[t] = t;
      return;
    }
    select_short_row(p, ri, sh);
    return;
  }
  const int base = ch * kChunk;
  if (base >= nv) return;
  const float* row = p.logits + (int64_t)r * p.L;
  uint32_t key[kPer];
  load_chunk(row, base, nv, key);
  clear_hist(sh);
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (base + i * kThreads + (int)threadIdx.x < nv) atomicAdd(&sh.hist[key[i] >> 21], 1u);
  __syncthreads();
  uint32_t* gh = p.hist + (int64_t)r * kBins;
  for (int i = threadIdx.x; i < kBins; i += kThreads) {
    const uint32_t v = sh.hist[i];
    if (v) atomicAdd(&gh[i], v);
  }
}

// Long rows: threshold bin from the global histogram, emit the elements above it,
// collect the elements in it.
__global__ __launch_bounds__(kThreads) void topk_split_kernel(Params p) {
  __shared__ Core sh;
  const int r = blockIdx.x / p.nchunk;
  const int ch = blockIdx.x - r * p.nchunk;
  const Row ri(p, r);
  const int nv = ri.nv, k = ri.k;
  if (nv <= kChunk || nv <= k) return;
  const int base = ch * kChunk;
  if (base >= nv) return;
  const float* row = p.logits + (int64_t)r * p.L;
  uint32_t key[kPer];
  load_chunk(row, base, nv, key);
  const uint32_t* gh = p.hist + (int64_t)r * kBins;
  for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = gh[i];
  __syncthreads();
  find_bin(sh, (uint32_t)k);
  const uint32_t bin0 = sh.bin;
  const uint32_t rem = (uint32_t)k - sh.above;
  const bool whole = sh.hist[bin0] == rem;
  int32_t* out = p.idx + (int64_t)r * k;
  uint32_t* cnt = p.counters + 2 * (int64_t)r;
  uint64_t* cand = p.cand + (int64_t)r * kCap;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int t = base + i * kThreads + (int)threadIdx.x;
    const bool in = t < nv;
    const uint32_t d = key[i] >> 21;
    const int slot = wave_append(in && (d > bin0 || (whole && d == bin0)), &cnt[0]);
    if (slot >= 0 && slot < k) out[slot] = t;
    const int cslot = wave_append(in && !whole && d == bin0, &cnt[1]);
    if (cslot >= 0 && cslot < kCap) cand[cslot] = compose(key[i], t);
  }
}

// Long rows: refine the threshold-bin candidates.
__global__ __launch_bounds__(kThreads) void topk_finish_kernel(Params p) {
  __shared__ Full sh;
  const int r = blockIdx.x;
  const Row ri(p, r);
  const int nv = ri.nv, k = ri.k;
  if (nv <= kChunk || nv <= k) return;
  const uint32_t* gh = p.hist + (int64_t)r * kBins;
  for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = gh[i];
  __syncthreads();
  find_bin(sh, (uint32_t)k);
  const uint32_t bin0 = sh.bin;
  const uint32_t above = sh.above;
  const uint32_t rem = (uint32_t)k - above;
  const uint32_t cnt0 = sh.hist[bin0];
  if (cnt0 == rem) return;  // the split pass took the whole bin
  const float* row = p.logits + (int64_t)r * p.L;
  int32_t* out = p.idx + (int64_t)r * k;
  if (threadIdx.x == 0) sh.n_out = above;  // the split pass emitted exactly `above`
  if (cnt0 <= (uint32_t)kCap) {
    const uint64_t* cand = p.cand + (int64_t)r * kCap;
    for (int i = threadIdx.x; i < (int)cnt0; i += kThreads) sh.cand[i] = cand[i];
    __syncthreads();
    refine<false>(sh, row, (int)cnt0, (uint64_t)bin0 << 53, 0x7FFull << 53, rem, out, k);
  } else {
    __syncthreads();
    refine<true>(sh, row, nv, (uint64_t)bin0 << 53, 0x7FFull << 53, rem, out, k);
  }
}

__global__ void fill_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

size_t topk_workspace_bytes(int64_t rows, int32_t max_model_len) {
  if (max_model_len <= kChunk) return 0;
  return (size_t)rows * ((size_t)kBins * 4 + 2 * 4 + (size_t)kCap * 8);
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.batch * a.next_n;
  Params p;
  p.logits = a.logits;
  p.ctx_lens = a.ctx_lens;
  p.idx = a.idx;
  p.N = a.next_n;
  p.W = a.bt_stride;
  p.L = a.max_model_len;
  p.k = a.k;
  p.nchunk = (a.max_model_len + kChunk - 1) / kChunk;
  // Workspace: histograms, then counters, then candidates (8-byte aligned).
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  p.hist = reinterpret_cast<uint32_t*>(ws);
  p.counters = reinterpret_cast<uint32_t*>(ws + rows * kBins * 4);
  p.cand = reinterpret_cast<uint64_t*>(ws + rows * (kBins * 4 + 8));
  if (rows * p.nchunk > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (p.nchunk > 1) {
    const int64_t words = rows * (kBins + 2);
    const int64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                       stream, p.hist, words);
  }
  hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)(rows * p.nchunk)), dim3(kThreads), 0, stream, p);
  if (p.nchunk > 1) {
    hipLaunchKernelGGL(topk_split_kernel, dim3((unsigned)(rows * p.nchunk)), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mqa
