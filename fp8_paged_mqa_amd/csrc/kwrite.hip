// Indexer K-cache write on gfx950: quantise each token's 128 keys to e4m3fn with one
// fp32 scale and store them as the 132-byte cache row the paged logits read.
//
// Row format: the stepcodex.com issue "[Bug] aiter ops triton attention pa_mqa_logits",
// section "Minimal reproduction" - the reference reads bytes [0, 128) of a token's row
// as e4m3fn codes and bytes [128, 132) as one fp32 scale, and dequantises code * scale.
// The page does not say how a writer chooses the scale. The rule implemented here maps
// the row's largest magnitude onto the largest finite code: scale = amax / 448 (fp32,
// correctly rounded), code = e4m3fn(x / scale) with x / scale correctly rounded in fp32
// and then rounded to the nearest code, ties to even; a row of zeros gets scale 1.
//
// Mapping: four tokens at a time per wave, one per row of 16 lanes; lane c of a row holds
// keys [8c, 8c+8) (one 16-byte load of bf16, two of fp32), loaded together with the
// token's slot, and a wave loads two such groups before converting either. Four DPP row rotations (ror 8, 4, 2, 1) with a NaN-propagating max leave the
// row's amax in all 16 lanes - no LDS traffic. Each lane stores its 8 codes as one
// 8-byte store, so a row's 16 lanes write the 128 code bytes contiguously, and lane 0
// of the row adds the scale. A grid of ceil(T / 32) four-wave workgroups (a stride loop
// only past 2^20 workgroups). Tokens whose slot lies outside the cache are skipped
// (negative slots mark padding).
#include <hip/hip_runtime.h>

#include "launch.h"

namespace mqa {
namespace {

constexpr int kD = 128;
constexpr int kRow = kD + 4;
constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kUnroll = 2;  // groups of 4 tokens per wave and pass (4 and 8 measured no faster)

// Round |y| (finite or not) to the nearest e4m3fn code, ties to even; magnitudes above
// the tie at 464 (halfway between 448 and 480, which has no code) give NaN, as do NaNs.
__device__ __forceinline__ uint32_t encode_e4m3fn(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float ax = __builtin_fabsf(y);
  if (!(ax <= 464.0f)) return __builtin_isnan(y) ? 0x7Fu : (sign | 0x7Fu);
  uint32_t code;
  if (ax >= 0.015625f) {  // normal e4m3fn range: 2^-6 .. 448
    const uint32_t ua = __float_as_uint(ax);
    const uint32_t exp = (ua >> 23) - 127u + 7u;  // 1 .. 15
    const uint32_t keep = (ua >> 20) & 7u;         // top 3 mantissa bits
    const uint32_t rest = ua & 0xFFFFFu;
    code = (exp << 3) | keep;
    code += (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ? 1u : 0u;  // may carry into exp
  } else {  // subnormal codes: multiples of 2^-9 (exact scaling, then round to even)
    code = (uint32_t)__builtin_rintf(ax * 512.0f);  // 0 .. 8 (8 is 2^-6, the first normal)
  }
  return sign | code;
}

template <int Ctrl>
__device__ __forceinline__ float row_rot_max(float v) {
  return __builtin_elementwise_maximum(
      v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xf, 0xf, false)));
}

// NaN-propagating maximum over a row of 16 lanes; every lane of the row gets it.
__device__ __forceinline__ float row_max(float v) {
  v = row_rot_max<0x128>(v);  // row_ror:8
  v = row_rot_max<0x124>(v);  // row_ror:4
  v = row_rot_max<0x122>(v);  // row_ror:2
  v = row_rot_max<0x121>(v);  // row_ror:1
  return v;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_write_kernel(const void* __restrict__ k, const int64_t* slots,
                                                           uint8_t* __restrict__ kv, int64_t T, int64_t nslots) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane >> 4;  // token of this lane within the wave
  const int c = lane & 15;  // keys [8c, 8c+8)
  const int64_t first = ((int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave)) * 4 * kUnroll;
  const int64_t stride = (int64_t)gridDim.x * kWaves * 4 * kUnroll;
  for (int64_t base0 = first; base0 < T; base0 += stride) {
    // kUnroll groups of 4 tokens: every group's slot and keys are loaded before any is
    // converted, so a wave has all of its loads in flight at once.
    int64_t slot_u[kUnroll];
    float x_u[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t bu = base0 + 4 * u;
      const int64_t i = bu + r < T ? bu + r : T - 1;  // rows past T repeat the last (not stored)
      slot_u[u] = slots[i];
      float* x = x_u[u];
      if (BF16) {
        const uint4 v = reinterpret_cast<const uint4*>(k)[i * (kD / 8) + c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = __uint_as_float(w[j] << 16);
          x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
      } else {
        const float4 v0 = reinterpret_cast<const float4*>(k)[i * (kD / 4) + 2 * c];
        const float4 v1 = reinterpret_cast<const float4*>(k)[i * (kD / 4) + 2 * c + 1];
        x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
        x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
    const int64_t base = base0 + 4 * u;
    const int64_t slot = slot_u[u];
    const float* x = x_u[u];
    float m = __builtin_fabsf(x[0]);
#pragma unroll
    for (int j = 1; j < 8; ++j) m = __builtin_elementwise_maximum(m, __builtin_fabsf(x[j]));
    const float amax = row_max(m);
    const float scale = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
    uint32_t lo = 0, hi = 0;
    if (__builtin_isfinite(amax) && scale > 0.0f) {
      // Every quotient is finite (|x / scale| <= 448 up to rounding): gfx950's packed
      // conversion rounds to the nearest code, ties to even, and overflows past the 464
      // tie to NaN keeping the sign, which is the rule above (checked against the
      // encoder on every code, every midpoint and their float neighbours, subnormal
      // quotients included). Only a NaN quotient would differ (it returns 0xFF), and
      // none occurs here.
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = __fdiv_rn(x[j], scale);
      lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false), true);
      hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false), true);
    } else {  // a non-finite key, or a scale that underflows to zero
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo |= encode_e4m3fn(__fdiv_rn(x[j], scale)) << (8 * j);
        hi |= encode_e4m3fn(__fdiv_rn(x[4 + j], scale)) << (8 * j);
      }
    }
    if (base + r < T && slot >= 0 && slot < nslots) {
      uint8_t* row = kv + slot * kRow;
      // rows are 4-byte aligned: two dword stores
      reinterpret_cast<uint32_t*>(row)[2 * c] = lo;
      reinterpret_cast<uint32_t*>(row)[2 * c + 1] = hi;
      // A NaN scale (a NaN key) is written as the canonical quiet NaN.
      if (c == 0) *reinterpret_cast<float*>(row + kD) = __builtin_isnan(scale) ? __builtin_nanf("") : scale;
    }
    }
  }
}

}  // namespace

hipError_t launch_k_write(const KWriteLaunch& a, hipStream_t stream) {
  const int64_t want = (a.num_tokens + 4 * kWaves * kUnroll - 1) / (4 * kWaves * kUnroll);
  const int64_t cap = (int64_t)1 << 20;
  const unsigned blocks = (unsigned)(want < cap ? want : cap);
  if (a.bf16)
    hipLaunchKernelGGL(k_write_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, a.k, a.slots, a.kv,
                       a.num_tokens, a.num_slots);
  else
    hipLaunchKernelGGL(k_write_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, a.k, a.slots, a.kv,
                       a.num_tokens, a.num_slots);
  return hipGetLastError();
}

}  // namespace mqa
