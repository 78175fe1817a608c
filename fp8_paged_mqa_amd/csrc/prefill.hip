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
// already converted to f16 (exact) in the B-operand layout of v_mfma_f32_32x32x16_f16,
// and the query rows stay in VGPRs as A operands. That shape is used because it
// sustains about 1.6x the rate of the 16x16x32 f16 shape on gfx950 (a timed MFMA-only
// loop: ~1.85 vs ~1.14 PFLOP/s).
//   * A lane (h, j) of a 32x32 tile holds, for its row or column j, the 64 bytes
//     [64h, 64h+64) of the 128-byte contraction, as eight 16-wide k-steps: the k order
//     is permuted the same way on both operands, which leaves the dot products unchanged.
//     A row tile is 32 heads of one query row (heads past H get weight 0); a wave holds
//     two row tiles (two query rows at H <= 32, one at H = 48, 64).
//   * Workgroup: 8 waves (two per SIMD). A grid of query blocks x key splits: splits are
//     added until there are about four workgroups per CU. A workgroup computes the
//     64-key stages of its split that meet the union of its rows' windows and writes
//     -inf over the rest of its split (nontemporal stores).
//   * Stage pipeline: two LDS buffers. At the start of stage s every thread converts its
//     16 key bytes of stage s+1 (loaded during stage s-1; the scale's sign folded into
//     the fp8 sign bits, exact) into the other buffer and loads its bytes of stage s+2,
//     then the waves compute stage s: the conversion and LDS writes overlap the MFMAs.
//     One barrier per stage.
//   * LDS layout per 32-key tile: [k-step 0..7][slot 0..63][8 f16], lane L's operand of
//     k-step st in slot L ^ (2*(st/2) + 8*(L/32)). Each k-step's B operands are one
//     1 KB ds_read_b128 per wave (the XOR permutes lanes within aligned 16-lane groups,
//     so the read stays conflict-free), and the eight threads that convert one key's
//     16-byte pieces write eight different bank slots (unswizzled, they all hit one).
//   * Epilogue: a lane's 16 results are heads 8q + 4h + r (q, r < 4) of key j; relu,
//     weights and the head sum run in registers, one permlane32 swap adds the two lane
//     halves, then |scale| and the window mask. Each 32-key group's epilogue runs one
//     group late, between the next group's MFMAs (the second group's across the stage
//     barrier), and a stage's 64 logits per row leave as one 256-byte store once its
//     second group is done. The stores are range-checked buffer stores (keys past the
//     computed range are dropped by the hardware), so they need no branch and the
//     compiler's wait counts for the key loads stay exact.
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
constexpr int kStage = 64;               // keys per stage: 2 MFMA column tiles of 32
constexpr int kTileBytes = 8 * 64 * 16;  // one 32-key tile of f16 B operands (8 KB)

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

typedef float f32x16 __attribute__((ext_vector_type(16)));

// The 64 bytes a lane holds for one row (bytes [64h, 64h+64)) as the eight f16x8
// operands of the chained 16-wide k-steps.
struct Operand8 {
  f16x8 k[8];
};

// Query row tiles hold 32 heads (v_mfma_f32_32x32x16_f16): heads past H get weight 0.
template <int T32, int QPW>
__global__ __launch_bounds__(kThreads, 1) void prefill_logits_kernel(Params p) {
  constexpr int TILES = T32 * QPW;  // 32-head row tiles held by one wave
  static_assert(TILES <= 2, "query tile budget");
  __shared__ __attribute__((aligned(16))) uint8_t bops[2][2 * kTileBytes];  // two stages: 32 KB
  __shared__ float sabs[2][kStage];
  __shared__ int win[2];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int h = lane >> 5;   // lane half: k-bytes [64h, 64h+64) of its row; result rows 8q + 4h + r
  const int j = lane & 31;   // head (A) / key (B) within a 32-wide tile
  const int M = p.M, N = p.N, H = p.H;
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

  // Query rows as f16 A operands: lane (h, j) holds bytes [64h, 64h+64) of head j of the
  // tile, as the eight 8-element k-steps. Weights of the result rows 8q + 4h + r.
  Operand8 qa[TILES];
  f32x4 wv[TILES][4];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const int jl = t / T32, mm = t % T32;
    const int m = min(mw + jl, M - 1);
    const int head = min(mm * 32 + j, H - 1);  // heads past H: any row, weight 0
    const uint8_t* qr = p.q + ((int64_t)m * H + head) * kD + 64 * h;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const i32x4 x = load16(qr + 16 * v);
      qa[t].k[2 * v] = fp8x8_to_f16(x.x, x.y);
      qa[t].k[2 * v + 1] = fp8x8_to_f16(x.z, x.w);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r0 = mm * 32 + 8 * q + 4 * h;  // rows r0 .. r0+3 of this lane's results
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[t][q][r] = r0 + r < H ? p.w[(int64_t)m * H + r0 + r] : 0.0f;
    }
  }

  // Stage loader: piece P = t + kThreads*e of a stage is bytes [16*(P%8), +16) of key P/8,
  // i.e. the k-steps 2*(P%4), 2*(P%4)+1 of lane (h, j) = ((P%8)/4, key%32) of tile P/256.
  constexpr int kPieces = kStage * kD / (16 * kThreads);
  static_assert(kPieces * kThreads * 16 == kStage * kD, "a stage is whole 16-byte pieces");
  const int lk = threadIdx.x >> 3;
  const int lb = (threadIdx.x & 7) * 16;
  const int dst_off = ((threadIdx.x & 3) * 2) * 1024 +
                      ((((lb >> 6) * 32 + (lk & 31)) ^ (2 * (threadIdx.x & 3) + 8 * (lb >> 6))) * 16);
  auto fetch = [&](int s0, i32x4 (&raw)[kPieces], float (&sc)[kPieces]) {
#pragma unroll
    for (int e = 0; e < kPieces; ++e) {
      const int key = min(s0 + lk + (kThreads / 8) * e, N - 1);
      raw[e] = load16(p.k + (int64_t)key * kD + lb);
      sc[e] = p.ksc[key];
    }
  };
  auto stash = [&](int buf, const i32x4 (&raw)[kPieces], const float (&sc)[kPieces]) {
#pragma unroll
    for (int e = 0; e < kPieces; ++e) {
      i32x4 x = raw[e];
      if (__float_as_int(sc[e]) < 0) x ^= (int)0x80808080;  // sign of the scale into the codes
      uint8_t* dst = bops[buf] + ((lk + (kThreads / 8) * e) >> 5) * kTileBytes + dst_off;
      *reinterpret_cast<f16x8*>(dst) = fp8x8_to_f16(x.x, x.y);
      *reinterpret_cast<f16x8*>(dst + 1024) = fp8x8_to_f16(x.z, x.w);
      if ((threadIdx.x & 7) == 0) sabs[buf][lk + (kThreads / 8) * e] = __builtin_fabsf(sc[e]);
    }
  };

  // Output rows as range-checked buffer resources: a lane's store of key t lands only if
  // t < c1 (and the row exists), without a branch, so the compiler's wait counts for the
  // key loads stay exact instead of falling back to waiting for every store.
  __amdgpu_buffer_rsrc_t orsrc[QPW];
#pragma unroll
  for (int jl = 0; jl < QPW; ++jl)
    orsrc[jl] = __builtin_amdgcn_make_buffer_rsrc(orow[jl], 0, live[jl] ? c1 * 4 : 0, 0x00020000);

  // Per 32-key tile group u of a stage: MFMAs into one accumulator set, then the epilogue
  // (relu, weights, head sum, |scale|) one group later, so the VALU work of group g runs
  // between the MFMAs of group g+1 - across the stage barrier for the second group, whose
  // epilogue runs during the next stage's first group. Lane (h, j) keeps key 32h + j of
  // a stage (from group h); a stage's logits are stored once its second group is done.
  float keep[QPW];
#pragma unroll
  for (int jl = 0; jl < QPW; ++jl) keep[jl] = 0.0f;
  auto epilogue = [&](const f32x16 (&acc)[TILES], float s, int u) {
#pragma unroll
    for (int jl = 0; jl < QPW; ++jl) {
      float part = 0.0f;
#pragma unroll
      for (int mm = 0; mm < T32; ++mm) {
        const int t = jl * T32 + mm;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          part = __builtin_fmaf(wv[t][v / 4][v % 4], __builtin_elementwise_maximum(acc[t][v], 0.0f), part);
      }
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
      part = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * s;  // both halves: key 32u + j
      if (h == u) keep[jl] = part;
    }
  };
  auto store_stage = [&](int base) {
    const int t = base + lane;
#pragma unroll
    for (int jl = 0; jl < QPW; ++jl) {
      const float v = (t >= lo_r[jl] && t < hi_r[jl]) ? keep[jl] : -__builtin_inff();
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), orsrc[jl], t * 4, 0, 0);  // the bits
    }
  };

  // Double-buffered stages: at the start of stage s every thread converts its key pieces
  // of stage s+1 (loaded during stage s-1) into the other buffer and loads those of stage
  // s+2; one barrier per stage.
  i32x4 raw[kPieces];
  float sc[kPieces];
  fetch(c0, raw, sc);
  stash(0, raw, sc);
  fetch(min(c0 + kStage, c1 - 1), raw, sc);
  __syncthreads();
  f32x16 accP[TILES];  // the group whose epilogue is pending
  float sP = 0.0f;
  int uP = -1;         // its group index (-1: none pending)
  int baseP = 0;       // first key of its stage
  int buf = 0;
  for (int s0 = c0; s0 < c1; s0 += kStage) {
    if (s0 + kStage < c1) stash(buf ^ 1, raw, sc);
    if (s0 + 2 * kStage < c1) fetch(s0 + 2 * kStage, raw, sc);
    const uint8_t* const bop = bops[buf];
    // Slot of this lane's operand in k-step rows 2c and 2c+1.
    int slot[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) slot[c] = (lane ^ (2 * c + 8 * h)) * 16;
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // two 32-key tiles per stage
      Operand8 kb;
#pragma unroll
      for (int st = 0; st < 8; ++st)
        kb.k[st] = *reinterpret_cast<const f16x8*>(bop + u * kTileBytes + st * 1024 + slot[st >> 1]);
      f32x16 accC[TILES];
#pragma unroll
      for (int t = 0; t < TILES; ++t)
        accC[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[t].k[0], kb.k[0], f32x16{}, 0, 0, 0);
#pragma unroll
      for (int st = 1; st < 8; ++st)
#pragma unroll
        for (int t = 0; t < TILES; ++t)
          accC[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[t].k[st], kb.k[st], accC[t], 0, 0, 0);
      const float sC = sabs[buf][u * 32 + j];
      if (uP >= 0) {  // uniform
        epilogue(accP, sP, uP);
        if (uP == 1) store_stage(baseP);
      }
#pragma unroll
      for (int t = 0; t < TILES; ++t) accP[t] = accC[t];
      sP = sC;
      uP = u;
      baseP = s0;
    }
    __syncthreads();
    buf ^= 1;
  }
  if (uP >= 0) {
    epilogue(accP, sP, uP);
    store_stage(baseP);
  }
}

using KernelFn = void (*)(Params);
// [T32 - 1]: 32-head row tiles per query row (H = 16, 32 -> 1; 48, 64 -> 2).
constexpr KernelFn kTable[2] = {prefill_logits_kernel<1, 2>, prefill_logits_kernel<2, 1>};

}  // namespace

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream) {
  const int t32 = (a.heads + 31) / 32;
  const int qpw = t32 == 1 ? 2 : 1;
  const int qpg = kWaves * qpw;
  const int qblocks = (a.m + qpg - 1) / qpg;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  // Key splits so that there are about four workgroups per CU (each split >= 4 stages):
  // windows differ in length from row block to row block (causal prefill: by 2x), and
  // with several workgroups per CU the dispatcher evens the load out.
  const int stages = (a.n + kStage - 1) / kStage;
  const int target = 4 * cus;
  int splits = qblocks >= target ? 1 : (target + qblocks - 1) / qblocks;
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
  hipLaunchKernelGGL(kTable[t32 - 1], dim3((unsigned)qblocks, (unsigned)splits), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mqa
