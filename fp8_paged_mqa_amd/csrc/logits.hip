// fp8 paged MQA logits on gfx950.
//
// Computes, for every decode row r = b*N + j and position t of a [B*N, L] fp32 output,
//   logit = sum_h w[r,h] * relu(scale_t * (q[b,j,h,:] . k_t))   if t <= ctx_b - N + j
//   -inf                                                        otherwise,
// where k_t / scale_t are the 128 e4m3fn bytes and the fp32 of the 132-byte cache row
// that the block table maps t to (block_size 1). Definition: stepcodex.com issue
// "[Bug] aiter ops triton attention pa_mqa_logits", section "Minimal reproduction".
//
// Mapping onto CDNA4
//   * Precision: gfx950's fp8 MFMAs (16x16x128 f8f6f4 and 16x16x32 fp8) round the dot
//     product at about 2^-15.5 of sum|q_i k_i|, measured against exact products; near a
//     cancelling head sum that exceeds the 5e-3 + 1e-3*|logit| budget. So fp8 bytes are
//     converted exactly to f16 (v_cvt_scalef32_pk_f16_fp8, scale 1) and contracted with
//     v_mfma_f32_16x16x32_f16, four chained per 128-wide row: f16 products of e4m3
//     values are exact and the fp32 accumulation is correctly rounded.
//   * One wave owns a group of decode rows (at most 4 MFMA row tiles of 16 heads, so
//     at most 64 query rows for H <= 64) and a contiguous token range. Its query rows stay
//     in VGPRs, already in f16, in the A-operand layout, for the whole range. Decode rows
//     beyond one wave's share go to sibling waves of the workgroup that walk the same
//     tokens (their second read of a key row hits L2).
//   * Keys are gathered straight from HBM into the B-operand slots: lane (g, c),
//     g = lane/16, c = lane%16, owns token c of a 16-token column tile and reads bytes
//     [16g, 16g+16) and [64+16g, 64+16g+16) of that token's row, so each dwordx4 load
//     instruction covers the first (then the second) 64 contiguous bytes of 16 rows. A
//     and B use the same byte-to-k assignment, so the contraction covers all 128 k
//     whatever order the hardware uses internally.
//   * The block table is read 64 tokens at a time (one coalesced dword per lane) and
//     redistributed with ds_bpermute; table reads run two 64-token stages ahead of use,
//     key reads one stage ahead, so a wave keeps ~8 KB of gathers in flight.
//   * Epilogue in registers: the dequant scale's sign is folded into the fp8 key (flip
//     the sign bit of every byte, exact), so relu(scale*s) = |scale| * relu(sign*s) and
//     |scale| multiplies once per token after the head sum. Each lane sums w * relu over
//     its 4 heads per row tile and the row tiles of a decode row, then two xor-shuffles
//     finish the head sum across the 4 lane groups of a column.
//   * Stores: after a 64-token stage each lane group keeps one 16-token column tile, so
//     a row's 64 logits leave in one 256-byte store. Positions past the row's causal
//     limit, and the whole tail up to L, are written with -inf in the same pass.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace mqa {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 128;         // head_dim
constexpr int kRow = kD + 4;    // cache row bytes: keys + fp32 scale
constexpr int kWave = 64;
constexpr int kStage = 64;      // tokens per pipeline stage = 4 MFMA column tiles
constexpr int kTilesPerStage = kStage / 16;

struct Params {
  const uint8_t* q;
  const uint8_t* kv;
  const float* w;
  const int32_t* ctx_lens;
  const int32_t* bt;
  float* out;
  int64_t num_blocks;
  int32_t B, N, H, W, L;
  int32_t groups;        // waves that share one token range, one per group of decode rows
  int32_t slots;         // token ranges per workgroup
  int32_t tok_per_wave;  // multiple of kStage
};

__device__ __forceinline__ i32x4 load16(const uint8_t* p) {
  i32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
  return v;
}

// 8 e4m3fn bytes (two dwords) -> 8 f16 values, exactly (every e4m3fn value, NaN and
// subnormals included, is representable in f16).
__device__ __forceinline__ f16x8 fp8x8_to_f16(int lo, int hi) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)lo, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)lo, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)hi, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)hi, 1.0f, true);
  const f16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const f16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The 32 bytes a lane holds for one row (16 at 16g, 16 at 64+16g) as the four f16x8
// operands of the chained k-steps.
struct Operand {
  f16x8 k[4];
};

__device__ __forceinline__ Operand to_operand(i32x4 lo, i32x4 hi) {
  Operand o;
  o.k[0] = fp8x8_to_f16(lo.x, lo.y);
  o.k[1] = fp8x8_to_f16(lo.z, lo.w);
  o.k[2] = fp8x8_to_f16(hi.x, hi.y);
  o.k[3] = fp8x8_to_f16(hi.z, hi.w);
  return o;
}

// Gathered keys of one 64-token stage, in the lane's B-operand slots.
struct Stage {
  i32x4 lo[kTilesPerStage];
  i32x4 hi[kTilesPerStage];
  float scale[kTilesPerStage];
};

// Up to 4 row tiles fit two waves per SIMD (<= 256 VGPRs); the 5..8-tile variants
// (H > 64) take the whole register file.
template <int TPJ, int JPG>
__global__ __launch_bounds__(256, (TPJ * JPG <= 4) ? 2 : 1) void paged_logits_kernel(Params p) {
  constexpr int TILES = TPJ * JPG;  // MFMA row tiles (16 heads each) held by one wave
  static_assert(TILES >= 1 && TILES <= 8, "query tile budget");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;   // lane group: k-slice for operands, row quad for results
  const int c = lane & 15;   // column (token) / row (head) within a 16-wide tile
  const int group = wave % p.groups;
  const int slot = wave / p.groups;

  const int b = blockIdx.x % p.B;
  const int range = blockIdx.x / p.B;
  const int t0 = (range * p.slots + slot) * p.tok_per_wave;
  if (t0 >= p.L) return;
  const int t_end = min(t0 + p.tok_per_wave, p.L);

  int ctx = p.ctx_lens[b];
  ctx = max(0, min(ctx, min(p.W, p.L)));
  const int t_need = min(t_end, ctx);  // positions whose key is read

  const int j0 = group * JPG;           // first decode row of this wave
  const int jn = min(JPG, p.N - j0);    // decode rows this wave owns
  const int64_t out_row0 = (int64_t)(b * p.N + j0) * p.L;

  // Query tiles (A operand) and the weights of the 4 heads each lane reduces per tile.
  Operand qa[TILES];
  f32x4 wv[TILES];
  {
    const uint8_t* qb = p.q + ((int64_t)b * p.N + j0) * p.H * kD;
    const float* wb = p.w + ((int64_t)b * p.N + j0) * p.H;
#pragma unroll
    for (int m = 0; m < TILES; ++m) {
      const bool live = (m / TPJ) < jn;
      const uint8_t* qr = qb + (m * 16 + c) * kD;
      i32x4 a0 = live ? load16(qr + 16 * g) : i32x4{0, 0, 0, 0};
      i32x4 a1 = live ? load16(qr + 64 + 16 * g) : i32x4{0, 0, 0, 0};
      qa[m] = to_operand(a0, a1);
      wv[m] = live ? *reinterpret_cast<const f32x4*>(wb + m * 16 + 4 * g) : f32x4{0, 0, 0, 0};
    }
  }

  int nv[JPG];  // visible positions of each owned decode row
#pragma unroll
  for (int jl = 0; jl < JPG; ++jl) nv[jl] = min(ctx - p.N + (j0 + jl) + 1, p.L);

  const int32_t* btb = p.bt + (int64_t)b * p.W;

  auto load_table = [&](int tc) -> int {
    const int t = tc + lane;
    return (t < t_need) ? btb[t] : -1;
  };

  auto issue_keys = [&](int tc, int tab, Stage& s) {
#pragma unroll
    for (int u = 0; u < kTilesPerStage; ++u) {
      const int phys = __shfl(tab, u * 16 + c);
      const int t = tc + u * 16 + c;
      const bool in_ctx = t < t_need;
      const bool ok = in_ctx && phys >= 0 && (int64_t)phys < p.num_blocks;
      i32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      float sc = in_ctx ? __builtin_nanf("") : 0.0f;  // bad table entry -> NaN logits
      if (ok) {
        const uint8_t* row = p.kv + (int64_t)phys * kRow;
        lo = load16(row + 16 * g);
        hi = load16(row + 64 + 16 * g);
        sc = *reinterpret_cast<const float*>(row + kD);
      }
      s.lo[u] = lo;
      s.hi[u] = hi;
      s.scale[u] = sc;
    }
  };

  auto compute_store = [&](int tc, const Stage& s) {
    float keep[JPG];
#pragma unroll
    for (int jl = 0; jl < JPG; ++jl) keep[jl] = 0.0f;
    if (tc < t_need) {
#pragma unroll
      for (int u = 0; u < kTilesPerStage; ++u) {
        if (tc + u * 16 >= t_need) break;  // wave-uniform
        const float sc = s.scale[u];
        const int flip = (__float_as_int(sc) < 0) ? (int)0x80808080 : 0;
        const i32x4 lo = {s.lo[u].x ^ flip, s.lo[u].y ^ flip, s.lo[u].z ^ flip, s.lo[u].w ^ flip};
        const i32x4 hi = {s.hi[u].x ^ flip, s.hi[u].y ^ flip, s.hi[u].z ^ flip, s.hi[u].w ^ flip};
        const Operand kb = to_operand(lo, hi);
        const float sabs = __builtin_fabsf(sc);
        f32x4 acc[TILES];
#pragma unroll
        for (int m = 0; m < TILES; ++m) {
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[m].k[0], kb.k[0], f32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int st = 1; st < 4; ++st)
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[m].k[st], kb.k[st], acc[m], 0, 0, 0);
        }
#pragma unroll
        for (int jl = 0; jl < JPG; ++jl) {
          float part = 0.0f;
#pragma unroll
          for (int mm = 0; mm < TPJ; ++mm) {
            const int m = jl * TPJ + mm;
#pragma unroll
            for (int v = 0; v < 4; ++v)
              part = __builtin_fmaf(wv[m][v], __builtin_elementwise_maximum(acc[m][v], 0.0f), part);
          }
          part += __shfl_xor(part, 16);
          part += __shfl_xor(part, 32);
          if (g == u) keep[jl] = part * sabs;
        }
      }
    }
    const int t = tc + lane;  // lane (g, c) stores token 16g + c of the stage
    if (t < t_end) {
#pragma unroll
      for (int jl = 0; jl < JPG; ++jl) {
        if (jl < jn) p.out[out_row0 + (int64_t)jl * p.L + t] = (t < nv[jl]) ? keep[jl] : -__builtin_inff();
      }
    }
  };

  // Software pipeline: table two stages ahead, keys one stage ahead.
  int tc = t0;
  int tab_next = load_table(tc + kStage);
  Stage s0, s1;
  issue_keys(tc, load_table(tc), s0);
  while (tc < t_end) {
    int tab_after = load_table(tc + 2 * kStage);
    issue_keys(tc + kStage, tab_next, s1);
    compute_store(tc, s0);
    tc += kStage;
    if (tc >= t_end) break;
    tab_next = load_table(tc + 2 * kStage);
    issue_keys(tc + kStage, tab_after, s0);
    compute_store(tc, s1);
    tc += kStage;
  }
}

using KernelFn = void (*)(Params);

template <int TPJ, int JPG>
constexpr KernelFn kfn() { return paged_logits_kernel<TPJ, JPG>; }

// [TPJ-1][JPG-1]; TPJ = H/16 in 1..8, JPG = decode rows per wave: min(N, 4/TPJ) for
// H <= 64 (at most 4 row tiles, 64 f16 query VGPRs), 1 above (up to 8 row tiles).
constexpr KernelFn kTable[8][4] = {
    {kfn<1, 1>(), kfn<1, 2>(), kfn<1, 3>(), kfn<1, 4>()},
    {kfn<2, 1>(), kfn<2, 2>(), nullptr, nullptr},
    {kfn<3, 1>(), nullptr, nullptr, nullptr},
    {kfn<4, 1>(), nullptr, nullptr, nullptr},
    {kfn<5, 1>(), nullptr, nullptr, nullptr},
    {kfn<6, 1>(), nullptr, nullptr, nullptr},
    {kfn<7, 1>(), nullptr, nullptr, nullptr},
    {kfn<8, 1>(), nullptr, nullptr, nullptr},
};

}  // namespace

hipError_t launch_logits(const LogitsLaunch& a, hipStream_t stream) {
  const int tpj = a.heads / 16;
  const int per_wave = tpj <= 4 ? 4 / tpj : 1;
  const int jpg = a.next_n < per_wave ? a.next_n : per_wave;
  const int groups = (a.next_n + jpg - 1) / jpg;
  const int slots = groups >= 4 ? 1 : 4 / groups;
  Params p;
  p.q = a.q;
  p.kv = a.kv;
  p.w = a.w;
  p.ctx_lens = a.ctx_lens;
  p.bt = a.bt;
  p.out = a.out;
  p.num_blocks = a.num_blocks;
  p.B = a.batch;
  p.N = a.next_n;
  p.H = a.heads;
  p.W = a.bt_stride;
  p.L = a.max_model_len;
  p.groups = groups;
  p.slots = slots;
  p.tok_per_wave = 2 * kStage;
  const int64_t per_wg = (int64_t)slots * p.tok_per_wave;
  const int64_t ranges = (a.max_model_len + per_wg - 1) / per_wg;
  const int64_t blocks = ranges * a.batch;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  KernelFn fn = kTable[tpj - 1][jpg - 1];
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(groups * slots * kWave), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mqa
