// Non-paged (prefill) fp8 MQA logits on gfx950:
//   out[m, n] = sum_h w[m,h] * relu(scale_n * (q[m,h,:] . k[n,:]))   if ks[m] <= n < ke[m]
//               -inf                                                otherwise,
// over contiguous keys (codes [N, 128] e4m3fn, one fp32 scale per key). The quantity is
// the one the paged decode kernel computes; the stepcodex.com issue "[Bug] aiter ops
// triton attention pa_mqa_logits", section "Observations while narrowing it down", names
// the prefill kernel (fp8_mqa_logits) that computes it for M query rows at once.
//
// Mapping onto CDNA4. With many query rows the contraction is dense: the keys of a
// 64-key stage serve every query row of a workgroup, so they are staged once in LDS,
// already converted to f16 (exact) in the B-operand layout of v_mfma_f32_16x16x32_f16,
// and the query rows stay in VGPRs as A operands (same byte-to-k assignment as the
// paged kernel: lane (g, c) owns bytes [16g, 16g+16) and [64+16g, 64+16g+16) of its row).
//   * Workgroup: 8 waves (two per SIMD), each owning QPW query rows (4 MFMA row tiles of
//     16 heads). A grid of query blocks x key splits: splits are added when there are
//     fewer query blocks than CUs. A workgroup computes the 64-key stages of its split
//     that meet the union of its rows' windows and writes -inf over the rest of its
//     split (nontemporal stores).
//   * Stage pipeline: every thread loads 16 key bytes and its key's scale for the next
//     stage into registers while the waves compute the current one from LDS; then the
//     bytes are converted (the scale's sign folded into the fp8 sign bits, exact) and
//     stored to LDS for the next round. Two barriers per stage.
//   * LDS layout per 16-key tile: [k-step 0..3][lane 0..63][8 f16], so each k-step's B
//     operands are one conflict-free 1 KB ds_read_b128 per wave.
//   * Epilogue as in the paged kernel: relu, weights, head sum per lane, two cross-lane
//     swaps, times |scale|, window mask; a row's 64 logits of a stage leave in one
//     256-byte store.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace mqa {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 128;
constexpr int kWave = 64;
constexpr int kWaves = 8;
constexpr int kThreads = kWave * kWaves;
constexpr int kStage = 64;              // keys per stage: 4 MFMA column tiles
constexpr int kTileBytes = 4 * 64 * 16;  // one 16-key tile of f16 B operands (4 KB)

struct Params {
  const uint8_t* q;     // [M, H, 128]
  const uint8_t* k;     // [N, 128]
  const float* ksc;     // [N]
  const float* w;       // [M, H]
  const int32_t* ks;    // [M]
  const int32_t* ke;    // [M]
  float* out;           // [M, ostride]
  int64_t ostride;
  int32_t M, N, H;
  int32_t split_keys;   // keys per split (a multiple of kStage)
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ i32x4 load16(const uint8_t* p) {
  i32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 16), 16);
  return v;
}

__device__ __forceinline__ f16x8 fp8x8_to_f16(int lo, int hi) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)lo, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)lo, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)hi, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)hi, 1.0f, true);
  const f16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const f16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

struct Operand {
  f16x8 k[4];
};

__device__ __forceinline__ float sum_lane_groups(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int TPJ, int QPW>
__global__ __launch_bounds__(kThreads, 1) void prefill_logits_kernel(Params p) {
  constexpr int TILES = TPJ * QPW;
  static_assert(TILES <= 4, "query tile budget");
  __shared__ __attribute__((aligned(16))) uint8_t bops[4 * kTileBytes];  // one stage: 16 KB
  __shared__ float sabs[kStage];
  __shared__ int win[2];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int g = lane >> 4;
  const int c = lane & 15;
  const int M = p.M, N = p.N;
  constexpr int QPG = kWaves * QPW;
  const int m0 = blockIdx.x * QPG;
  const int a = blockIdx.y * p.split_keys;
  const int b = min(N, a + p.split_keys);

  // Window union of the workgroup's rows (rows past M and empty windows contribute none).
  if (threadIdx.x == 0) {
    win[0] = N;
    win[1] = 0;
  }
  __syncthreads();
  if ((int)threadIdx.x < QPG && m0 + (int)threadIdx.x < M) {
    const int m = m0 + threadIdx.x;
    const int lo = min(max(p.ks[m], 0), N), hi = min(max(p.ke[m], 0), N);
    if (lo < hi) {
      atomicMin(&win[0], lo);
      atomicMax(&win[1], hi);
    }
  }
  __syncthreads();
  const int c0 = max(a, (win[0] / kStage) * kStage);  // computed stages: [c0, c1)
  const int c1 = min(b, win[1]);

  // This wave's query rows (rows past M repeat row M-1 and are never stored).
  const int mw = m0 + wave * QPW;
  int lo_r[QPW], hi_r[QPW];
  float* orow[QPW];
  bool live[QPW];
#pragma unroll
  for (int jl = 0; jl < QPW; ++jl) {
    const int m = min(mw + jl, M - 1);
    live[jl] = mw + jl < M;
    lo_r[jl] = min(max(p.ks[m], 0), N);
    hi_r[jl] = min(max(p.ke[m], 0), N);
    orow[jl] = p.out + (int64_t)m * p.ostride;
  }

  // -inf over the parts of this split that no stage computes.
  auto fill = [&](int from, int to) {
    const f32x4 ninf = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
    for (int jl = 0; jl < QPW; ++jl) {
      if (!live[jl]) continue;
      float* row = orow[jl];
      const int head = min(to, (from + 3) & ~3);  // scalar stores up to a 16-byte boundary
      for (int t = from + lane; t < head; t += kWave) row[t] = -__builtin_inff();
      const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
      int t = head + 4 * lane;
      for (; t + 4 <= to; t += 4 * kWave) {
        if (vec)
          __builtin_nontemporal_store(ninf, reinterpret_cast<f32x4*>(row + t));
        else
          for (int i = 0; i < 4; ++i) row[t + i] = -__builtin_inff();
      }
      for (int i = 0; i < 4; ++i)
        if (t + i >= head && t + i < to) row[t + i] = -__builtin_inff();
    }
  };
  if (c0 >= c1) {
    fill(a, b);
    return;
  }
  fill(a, c0);
  fill(c1, b);

  // Query rows as f16 A operands, weights.
  Operand qa[TILES];
  f32x4 wv[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const int jl = t / TPJ, mm = t % TPJ;
    const int m = min(mw + jl, M - 1);
    const uint8_t* qr = p.q + ((int64_t)m * p.H + mm * 16 + c) * kD;
    const i32x4 lo = load16(qr + 16 * g), hi = load16(qr + 64 + 16 * g);
    qa[t].k[0] = fp8x8_to_f16(lo.x, lo.y);
    qa[t].k[1] = fp8x8_to_f16(lo.z, lo.w);
    qa[t].k[2] = fp8x8_to_f16(hi.x, hi.y);
    qa[t].k[3] = fp8x8_to_f16(hi.z, hi.w);
    wv[t] = *reinterpret_cast<const f32x4*>(p.w + (int64_t)m * p.H + mm * 16 + 4 * g);
  }

  // Stage loader: thread t holds bytes [16*(t%8), +16) of key t/8 of the stage.
  const int lk = threadIdx.x >> 3;        // key of the stage, 0..63
  const int lb = (threadIdx.x & 7) * 16;  // byte offset in the key's row
  // Where those 16 bytes go: lane (g', c') = key % 16, k-steps 2*(lb >= 64) + {0, 1}.
  const int dst_lane = ((lb & 63) >> 4) * 16 + (lk & 15);
  const int dst_step = lb >= 64 ? 2 : 0;
  uint8_t* const dst = bops + (lk >> 4) * kTileBytes + dst_step * 1024 + dst_lane * 16;
  auto fetch = [&](int s0, i32x4& raw, float& sc) {
    const int key = min(s0 + lk, N - 1);
    raw = load16(p.k + (int64_t)key * kD + lb);
    sc = p.ksc[key];
  };
  auto stash = [&](i32x4 raw, float sc) {
    if (__float_as_int(sc) < 0) raw ^= (int)0x80808080;  // sign of the scale into the codes
    const f16x8 f0 = fp8x8_to_f16(raw.x, raw.y);
    const f16x8 f1 = fp8x8_to_f16(raw.z, raw.w);
    *reinterpret_cast<f16x8*>(dst) = f0;
    *reinterpret_cast<f16x8*>(dst + 1024) = f1;
    if ((threadIdx.x & 7) == 0) sabs[lk] = __builtin_fabsf(sc);
  };

  i32x4 raw;
  float sc;
  fetch(c0, raw, sc);
  for (int s0 = c0; s0 < c1; s0 += kStage) {
    stash(raw, sc);
    __syncthreads();
    if (s0 + kStage < c1) fetch(s0 + kStage, raw, sc);  // next stage in flight meanwhile
    float keep[QPW];
#pragma unroll
    for (int jl = 0; jl < QPW; ++jl) keep[jl] = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      Operand kb;
#pragma unroll
      for (int st = 0; st < 4; ++st)
        kb.k[st] = *reinterpret_cast<const f16x8*>(bops + u * kTileBytes + st * 1024 + lane * 16);
      const float s = sabs[u * 16 + c];
      f32x4 acc[TILES];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[t].k[0], kb.k[0], f32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int st = 1; st < 4; ++st)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[t].k[st], kb.k[st], acc[t], 0, 0, 0);
      }
#pragma unroll
      for (int jl = 0; jl < QPW; ++jl) {
        float part = 0.0f;
#pragma unroll
        for (int mm = 0; mm < TPJ; ++mm) {
          const int t = jl * TPJ + mm;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            part = __builtin_fmaf(wv[t][v], __builtin_elementwise_maximum(acc[t][v], 0.0f), part);
        }
        part = sum_lane_groups(part) * s;
        if (g == u) keep[jl] = part;
      }
    }
    const int t = s0 + lane;  // lane (g, c) stores key 16g + c of the stage
    if (t < c1) {
#pragma unroll
      for (int jl = 0; jl < QPW; ++jl)
        if (live[jl]) orow[jl][t] = (t >= lo_r[jl] && t < hi_r[jl]) ? keep[jl] : -__builtin_inff();
    }
    __syncthreads();  // every wave is done with this stage's operands
  }
}

using KernelFn = void (*)(Params);
constexpr KernelFn kTable[4] = {prefill_logits_kernel<1, 4>, prefill_logits_kernel<2, 2>,
                                prefill_logits_kernel<3, 1>, prefill_logits_kernel<4, 1>};

}  // namespace

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream) {
  const int tpj = a.heads / 16;
  const int qpw = tpj <= 2 ? 4 / tpj : 1;
  const int qpg = kWaves * qpw;
  const int qblocks = (a.m + qpg - 1) / qpg;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  // Key splits so that there are at least as many workgroups as CUs (each split >= 4 stages).
  const int stages = (a.n + kStage - 1) / kStage;
  int splits = qblocks >= cus ? 1 : (cus + qblocks - 1) / qblocks;
  const int max_splits = (stages + 3) / 4;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  const int split_stages = (stages + splits - 1) / splits;
  splits = (stages + split_stages - 1) / split_stages;
  Params p;
  p.q = a.q;
  p.k = a.k;
  p.ksc = a.k_scale;
  p.w = a.w;
  p.ks = a.ks;
  p.ke = a.ke;
  p.out = a.out;
  p.ostride = a.out_stride;
  p.M = a.m;
  p.N = a.n;
  p.H = a.heads;
  p.split_keys = split_stages * kStage;
  hipLaunchKernelGGL(kTable[tpj - 1], dim3((unsigned)qblocks, (unsigned)splits), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mqa
