// Sparse MLA decode over the indexer's selected positions on gfx950.
//
// For decode row r = b*N + j, 16 query heads of 576 e4m3fn codes attend the cache rows
// of the positions listed in indices[r] (negative entries are padding):
//   score(h, t) = sm_scale * q_scale * kv_scale * (q[r,h,:] . k_t)
//   out[r,h,:]  = kv_scale * sum_t softmax_t(score(h, .)) * k_t[0:512]
//   lse[r,h]    = log sum_t exp(score(h, t))
// with k_t the 576 codes of position t's latent row: slot t % S of block
// block_tables[b][t / S]. Where the pieces come from: the stepcodex.com issue "[Bug]
// aiter ops triton attention pa_mqa_logits", section "Downstream impact" (the top-k
// positions feed the sparse attention); the chat-gpts.plus summary (post 69330) of the
// aiter MLA decode issue, sections "问题场景" and "环境排查" (fp8 q and KV, 16 heads per
// latent KV head, 1-4 query tokens per request); vLLM pull request 31282, "The Bug"
// (one token per page). The 576/512 split of a latent row is DeepSeek-V3's
// (512 compressed dims + 64 rotary dims; the value is the compressed part).
//
// Mapping onto CDNA4
//   * Grid: (split, row). A workgroup of 4 waves takes up to 8 tiles of 64 listed
//     positions of one row; a row's list is cut into as many splits as keep the chip
//     busy, and a second kernel merges the splits' partial softmax states.
//   * Gather: a tile's 64 latent rows go straight from HBM into LDS with 16-byte
//     direct-to-LDS loads (global_load_lds_dwordx4), no registers in between, into
//     one of 4 LDS buffers: three tiles stay in flight while one is computed. LDS rows
//     are 592 bytes apart, which makes both read patterns below conflict-free. Every
//     row index is resolved (index list -> block table -> row) before the loop, so
//     the loop issues no other memory reads and waits on explicit vmcnt values.
//   * Scores: wave w computes S^T = K Q^T for tokens 16w..16w+15 of the tile with
//     v_mfma_f32_16x16x32_f16 (18 k-steps over 576 dims; fp8 codes converted exactly
//     to f16, so the products are exact). In the C layout a lane holds 4 tokens of one
//     head, which is the layout the probabilities need as the B operand of O^T = V^T P^T.
//   * Softmax: online, in the log2 domain; the workgroup shares per-wave maxima and the
//     scores through LDS (two barriers per tile); probabilities are scaled by 2^15
//     before rounding to f16, so none falls into the f16 subnormal range.
//   * Values: wave w owns output columns [128w, 128w+128). Its V^T operands come from
//     the row-major tile with ds_read_b64_tr_b8, whose lane pattern delivers to lane
//     (g, i) the byte of column i of 8 consecutive rows (the rows its address group
//     names), i.e. 8 tokens of one column: the A operand of a 32-token k-step.
//     Padding tokens have their value bytes zeroed before the conversion (their
//     probability is 0, and 0 * NaN would not be).
//   * Bound: HBM. Algorithmic bytes = 576 per listed position + the indices, table
//     entries, queries, outputs and the splits' partial states.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace mqa {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 576;                      // latent row: codes per token and per query head
constexpr int kDV = 512;                     // value dims
constexpr int kH = 16;                       // query heads per row
constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kTile = 64;                    // listed positions per tile
constexpr int kRowStride = 592;              // LDS bytes per gathered row
constexpr int kTileBytes = kTile * kRowStride;  // 37888 = 37 KB
constexpr int kBlocks = kTileBytes / 1024;   // 1 KB direct-to-LDS wave loads per tile
constexpr int kNBuf = 4;
constexpr int kMaxTiles = 8;                 // tiles per split
constexpr int kLoads = 9;                    // loads per tile of waves 1..3 (wave 0: 10)
constexpr int kSStride = 68;                 // floats per head in the score exchange
constexpr float kPScale = 32768.0f;          // probabilities are kept as p * 2^15
constexpr float kLn2 = 0.69314718055994531f;
static_assert(kTileBytes % 1024 == 0, "tile = whole 1 KB wave loads");


struct Params {
  const uint8_t* q;      // [R, 16, 576]
  const uint8_t* kv;     // [num_blocks * S, 576]
  const int32_t* idx;    // [R, topk]
  const int32_t* bt;     // [B, W]
  float* out;            // [R, 16, 512]
  float* lse;            // [R, 16] or null
  uint8_t* ws;           // [R, splits] partial states of kPartialBytes (splits > 1)
  float c2;              // sm_scale * q_scale * kv_scale * log2(e)
  float vscale;          // kv_scale (O and l both carry the 2^15 of the probabilities)
  int32_t R, N, topk, W, bshift, splits, tps;
  uint32_t nblk;         // blocks in the cache (clamped to 2^31 - 1)
};

// Partial state of a split: O / l per head and column as f16 (the weighted mean of value
// codes, |O / l| <= 448, so f16 holds it to 2^-11), then m and l per head as f32.
constexpr int kPartialBytes = kH * kDV * 2 + 2 * kH * 4;

struct Smem {
  uint8_t tile[kNBuf][kTileBytes];
  float s[kH * kSStride];        // scores of the tile, [head][token]
  float wmax[kWaves][kH];
  int32_t rows[kMaxTiles][kTile];  // row to load for each token of each list tile
  uint64_t padm[kMaxTiles];        // bit u: token u of the tile is padding
  uint64_t badm[kMaxTiles];        // bit u: token u names a position outside the cache
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ f16x8 fp8x8_to_f16(int lo, int hi) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)lo, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)lo, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)hi, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)hi, 1.0f, true);
  const f16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const f16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Sum / max over the 4 lane groups (lanes i, i+16, i+32, i+48); every lane gets it.
__device__ __forceinline__ float groups_sum(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float groups_max(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Bits 0..3 of m as the bytes 0x00 / 0xFF of a dword.
__device__ __forceinline__ uint32_t bytes_of_bits(uint32_t m) {
  m &= 0xFu;
  m = (m | (m << 7) | (m << 14) | (m << 21)) & 0x01010101u;
  return m * 0xFFu;
}

// s_waitcnt vmcnt(n) (n <= 63), no wait on the other counters.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Barrier without a memory fence (the fence would drain every outstanding
// direct-to-LDS load); the asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct-to-LDS load: 16 bytes from src into LDS bytes [m0 + 16*lane, +16).
// Written as asm so that the compiler does not see an LDS write behind a vector-memory
// counter: it would otherwise wait for every outstanding tile before reading LDS through
// ds_read_b64_tr_b8. Completion is tracked here with explicit vmcnt waits, and LDS
// ordering across waves with the barriers.
__device__ __forceinline__ void load_lds16(const uint8_t* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory");
}

// Issues this wave's direct-to-LDS loads of live tile `lt` into buffer `buf`: blocks
// w, w+4, ... of the tile's 37 KB, lane l filling bytes [16l, 16l+16) of each block.
__device__ __forceinline__ void issue_tile(const Params& p, Smem& sm, int lt, int buf, int wave, int lane) {
  int rowsel[kLoads + 1];
#pragma unroll
  for (int k = 0; k <= kLoads; ++k) {
    const int b = wave + kWaves * k;
    const int o = 1024 * min(b, kBlocks - 1) + 16 * lane;
    const int u = o / kRowStride;
    rowsel[k] = sm.rows[lt][u];
  }
#pragma unroll
  for (int k = 0; k <= kLoads; ++k) {
    const int b = wave + kWaves * k;
    if (b >= kBlocks) break;  // wave-uniform: only wave 0 has a 10th block
    const int o = 1024 * b + 16 * lane;
    const int u = o / kRowStride;
    int cb = o - u * kRowStride;
    if (cb >= kD) cb -= kD;  // the 16-byte pad after a row: reload its first chunk
    const uint8_t* src = p.kv + (uint64_t)(uint32_t)rowsel[k] * kD + cb;
    load_lds16(src, (uint32_t)uniform((int)(uintptr_t)(sm.tile[buf] + 1024 * b)));
  }
}

__global__ __launch_bounds__(kThreads, 1) void sparse_mla_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int G = lane >> 4;
  const int i = lane & 15;
  const int split = blockIdx.x;
  const int r = blockIdx.y;
  const int b = r / p.N;
  const int e0 = split * p.tps * kTile;
  const int ntiles = min(p.tps, (p.topk - e0 + kTile - 1) / kTile);

  // Resolve every listed position of this split to a cache row. Wave w takes list tiles
  // w and w+4: both index loads, then both table loads, so two round trips in all.
  static_assert(kMaxTiles == 2 * kWaves, "two list tiles per wave");
  const uint32_t cap = (uint32_t)p.W << p.bshift;
  const int smask = (1 << p.bshift) - 1;
  int pos[2], ent[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = e0 + (wave + kWaves * h) * kTile + lane;
    pos[h] = (wave + kWaves * h < ntiles && e < p.topk) ? p.idx[(int64_t)r * p.topk + e] : -1;
  }
  // Query rows, loaded behind the index loads (so the table lookups wait for the indices
  // only), as B operands of S^T = K Q^T: lane (G, i) holds dims [32s + 8G, +8) of
  // head i for the 18 k-steps s.
  f16x8 qb[kD / 32];
  {
    const uint8_t* qr = p.q + ((int64_t)r * kH + i) * kD + 8 * G;
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) {
      i32x2 x;
      __builtin_memcpy(&x, __builtin_assume_aligned(qr + 32 * s, 8), 8);
      qb[s] = fp8x8_to_f16(x.x, x.y);
    }
  }

#pragma unroll
  for (int h = 0; h < 2; ++h)
    ent[h] = (pos[h] >= 0 && (uint32_t)pos[h] < cap) ? p.bt[(int64_t)b * p.W + (pos[h] >> p.bshift)] : -1;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = wave + kWaves * h;
    if (t < ntiles) {
      const bool pad = pos[h] < 0;
      const bool ok = !pad && (uint32_t)pos[h] < cap && ent[h] >= 0 && (uint32_t)ent[h] < p.nblk;
      const int row = ok ? (ent[h] << p.bshift) | (pos[h] & smask) : 0;
      // Padding and bad positions load the first valid row of the tile (or row 0).
      const uint64_t okm = __ballot(ok);
      const uint64_t padm = __ballot(pad);
      const uint64_t badm = __ballot(!pad && !ok);
      const int sub = __shfl(row, okm ? __ffsll((unsigned long long)okm) - 1 : 0);
      sm.rows[t][lane] = ok ? row : sub;
      if (lane == 0) {
        sm.padm[t] = padm;
        sm.badm[t] = badm;
      }
    }
  }
  __syncthreads();
  // Live tiles (not all padding): every wave takes the list from one ballot over the
  // tiles' padding masks and keeps it in scalar registers; the loop reaches a live tile's
  // resolved rows through it, so nothing is moved.
  const uint64_t livem = __ballot(lane < ntiles && sm.padm[lane < kMaxTiles ? lane : 0] != ~0ull);
  const int nlive = __popcll(livem);
  auto live_tile = [&](int k) {  // list tile of the k-th live tile
    uint64_t m = livem;
    for (int j = 0; j < k; ++j) m &= m - 1;
    return (int)__builtin_ctzll(m);
  };

  // The query conversion (and its waits on the query loads) must not sink below the
  // prefetch: a wait on a query load would then also wait for the tiles behind it.
#pragma unroll
  for (int s = 0; s < kD / 32; ++s) asm volatile("" ::"v"(qb[s]));
  // Prefetch: live tiles 0..2.
  for (int k = 0; k < min(nlive, kNBuf - 1); ++k) issue_tile(p, sm, live_tile(k), k, wave, lane);

  f32x4 o[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) o[ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -__builtin_inff();  // running maximum (log2 domain) of head i
  float l_run = 0.0f;               // running sum of p * 2^15 of head i

  for (int k = 0; k < nlive; ++k) {
    const int buf = k & (kNBuf - 1);
    const int ahead = min(nlive - 1 - k, kNBuf - 2);  // live tiles issued after this one
    if (ahead >= 2) wait_vm<2 * kLoads>();
    else if (ahead == 1) wait_vm<kLoads>();
    else wait_vm<0>();
    barrier();  // tile k is in LDS, and every wave is done with tile k-1
    if (k + kNBuf - 1 < nlive) issue_tile(p, sm, live_tile(k + kNBuf - 1), (k + kNBuf - 1) & (kNBuf - 1), wave, lane);
    const uint8_t* const tb = sm.tile[buf];

    const int tk = live_tile(k);
    const uint64_t padm = ((uint64_t)(uint32_t)uniform((int)(uint32_t)sm.padm[tk])) |
                          ((uint64_t)(uint32_t)uniform((int)(uint32_t)(sm.padm[tk] >> 32)) << 32);
    const uint64_t badm = ((uint64_t)(uint32_t)uniform((int)(uint32_t)sm.badm[tk])) |
                          ((uint64_t)(uint32_t)uniform((int)(uint32_t)(sm.badm[tk] >> 32)) << 32);

    // Every LDS read of the tile first: the key operands of the scores (lane (G, i): dims
    // [32s + 8G, +8) of token 16*wave + i) and the value operands (transposed reads,
    // independent of the softmax).
    i32x2 kx[kD / 32];
    {
      const uint8_t* kr = tb + (16 * wave + i) * kRowStride + 8 * G;
#pragma unroll
      for (int s = 0; s < kD / 32; ++s) kx[s] = *reinterpret_cast<const i32x2*>(kr + 32 * s);
    }
    i32x2 vx[2][8];
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      const uint8_t* vr = tb + (32 * sg + 8 * G + (i >> 1)) * kRowStride + 128 * wave + 8 * (i & 1);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        vx[sg][ct] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(vr + 16 * ct));
    }

    // S^T for tokens 16*wave + (0..15).
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < kD / 32; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8_to_f16(kx[s].x, kx[s].y), qb[s], acc, 0, 0, 0);
    // acc[v]: token 16*wave + 4G + v, head i.
    float sc[4];
    float mx = -__builtin_inff();
    const int u0 = 16 * wave + 4 * G;
    const uint32_t padv = (uint32_t)(padm >> u0) & 0xFu, badv = (uint32_t)(badm >> u0) & 0xFu;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sc[v] = (padv >> v) & 1u ? -__builtin_inff() : ((badv >> v) & 1u ? __builtin_nanf("") : acc[v] * p.c2);
      mx = __builtin_fmaxf(mx, sc[v]);
    }
    mx = groups_max(mx);
    *reinterpret_cast<f32x4*>(&sm.s[i * kSStride + 16 * wave + 4 * G]) = f32x4{sc[0], sc[1], sc[2], sc[3]};
    if (G == 0) sm.wmax[wave][i] = mx;
    wait_lgkm0();
    barrier();

    // Online softmax state of head i.
    float mt = sm.wmax[0][i];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mt = __builtin_fmaxf(mt, sm.wmax[w][i]);
    const float m_new = __builtin_fmaxf(m_run, mt);
    const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    // Probabilities as B operands: lane (G, i) holds tokens 32*sg + 8G + (0..7), head i.
    f16x8 pb[2];
    float lsum = 0.0f;
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(&sm.s[i * kSStride + 32 * sg + 8 * G]);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(&sm.s[i * kSStride + 32 * sg + 8 * G + 4]);
      const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const _Float16 h = (_Float16)(__builtin_amdgcn_exp2f(sv[e] - m_use) * kPScale);
        pb[sg][e] = h;
        lsum += (float)h;
      }
    }
    l_run = l_run * alpha + groups_sum(lsum);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) o[ct] *= alpha;

    // O^T[cols, heads] += V^T P^T over the tile's 64 tokens, columns 128*wave + 16*ct.
    // Value bytes of padding tokens (token 32*sg + 8G + j is byte j) are zeroed.
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      const uint32_t pm = (uint32_t)(padm >> (32 * sg + 8 * G)) & 0xFFu;
      const uint32_t keep_lo = ~bytes_of_bits(pm), keep_hi = ~bytes_of_bits(pm >> 4);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int lo = vx[sg][ct].x & (int)keep_lo, hi = vx[sg][ct].y & (int)keep_hi;
        o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8_to_f16(lo, hi), pb[sg], o[ct], 0, 0, 0);
      }
    }
  }

  // o[ct][v]: column 128*wave + 16*ct + 4G + v, head i.
  if (p.splits == 1) {
    const float f = l_run == 0.0f ? 0.0f : p.vscale / l_run;  // NaN (a bad position) stays NaN
    float* orow = p.out + ((int64_t)r * kH + i) * kDV + 128 * wave + 4 * G;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) *reinterpret_cast<f32x4*>(orow + 16 * ct) = o[ct] * f;
    if (p.lse && wave == 0 && G == 0)
      p.lse[(int64_t)r * kH + i] =
          l_run > 0.0f ? (m_run + __builtin_amdgcn_logf(l_run) - 15.0f) * kLn2 : (l_run == 0.0f ? -__builtin_inff() : l_run);
  } else {
    uint8_t* part = p.ws + ((int64_t)r * p.splits + split) * kPartialBytes;
    _Float16* orow = reinterpret_cast<_Float16*>(part) + i * kDV + 128 * wave + 4 * G;
    // A split that saw nothing stores 0 (its weight in the merge is 0); NaN stays NaN.
    const float inv = l_run > 0.0f ? 1.0f / l_run : (l_run == 0.0f ? 0.0f : l_run);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const f32x4 v = o[ct] * inv;
      *reinterpret_cast<f16x4*>(orow + 16 * ct) = f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    }
    if (wave == 0 && G == 0) {
      float* ml = reinterpret_cast<float*>(part + kH * kDV * 2);
      ml[i] = m_run;
      ml[kH + i] = l_run;
    }
  }
}

// Merges the splits' partial states (grid (16 heads, rows), 128 threads, four columns per
// thread) in one pass with a running maximum: per split, M' = max(M, m_s),
// acc = acc * 2^(M - M') + 2^(m_s - M') * l_s * (O_s / l_s), L = L * 2^(M - M') + 2^(m_s - M') * l_s;
// out = kv_scale * acc / L.
// Splits are taken eight at a time: the eight states' loads are issued together (split
// indices past the last repeat it and merge with weight 0), then merged in split order, so
// a row of up to eight splits costs one memory round trip.
__global__ __launch_bounds__(128) void sparse_mla_combine_kernel(Params p) {
  constexpr int kBatch = 8;
  const int h = blockIdx.x;
  const int r = blockIdx.y;
  const uint8_t* base = p.ws + (int64_t)r * p.splits * kPartialBytes;
  float M = -__builtin_inff();
  float L = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < p.splits; s0 += kBatch) {
    // Lane t of each wave loads split s0 + t's maximum and sum (vector loads, issued with
    // the outputs' loads rather than as scalar loads the compiler would space out), then
    // every lane reads them from lanes 0..7.
    const float* mine = reinterpret_cast<const float*>(
        base + (int64_t)min(s0 + (int)(threadIdx.x & (kBatch - 1)), p.splits - 1) * kPartialBytes + kH * kDV * 2);
    const float m_t = mine[h];
    const float l_t = mine[kH + h];
    f16x4 oh[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const uint8_t* part = base + (int64_t)min(s0 + i, p.splits - 1) * kPartialBytes;
      oh[i] = *reinterpret_cast<const f16x4*>(part + (h * kDV + 4 * threadIdx.x) * 2);
    }
    float ms[kBatch], ls[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      ms[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_t), i));
      ls[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_t), i));
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      // A repeated index merges as a split that saw nothing (factor 1, weight 0). Branch-free,
      // so that the compiler does not move the loads into the branches one by one.
      const bool ok = s0 + i < p.splits;
      const float msi = ok ? ms[i] : -__builtin_inff();
      const float lsi = ok ? ls[i] : 0.0f;
      const f32x4 os = {(float)oh[i][0], (float)oh[i][1], (float)oh[i][2], (float)oh[i][3]};  // O_s / l_s
      const float mn = __builtin_fmaxf(M, msi);
      const float mu = mn == -__builtin_inff() ? 0.0f : mn;
      const float a = __builtin_amdgcn_exp2f(M - mu);  // 0 while nothing has been seen
      const float w = __builtin_amdgcn_exp2f(msi - mu) * lsi;  // 0 for a split that saw nothing
      acc = acc * a + os * w;
      L = L * a + w;
      M = mn;
    }
  }
  const float f = L == 0.0f ? 0.0f : p.vscale / L;
  // The output is not read again here: nontemporal stores (measured ~1% faster per call).
  __builtin_nontemporal_store(acc * f, reinterpret_cast<f32x4*>(p.out + ((int64_t)r * kH + h) * kDV + 4 * threadIdx.x));
  if (p.lse && threadIdx.x == 0)
    p.lse[(int64_t)r * kH + h] = L > 0.0f ? (M + __builtin_amdgcn_logf(L) - 15.0f) * kLn2 : (L == 0.0f ? -__builtin_inff() : L);
}

int compute_units_of_device() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 256;
  return cus;
}

}  // namespace

SparseMlaPlan sparse_mla_plan(int64_t rows, int32_t topk) {
  SparseMlaPlan plan;
  const int64_t tiles = (topk + kTile - 1) / kTile;
  const int64_t cus = compute_units_of_device();
  int64_t tps = (tiles * rows + cus - 1) / cus;
  tps = tps < 1 ? 1 : (tps > kMaxTiles ? kMaxTiles : tps);
  plan.tiles_per_split = (int32_t)tps;
  plan.splits = (int32_t)((tiles + tps - 1) / tps);
  plan.workspace_bytes = plan.splits > 1 ? (size_t)rows * plan.splits * kPartialBytes : 0;
  return plan;
}

hipError_t launch_sparse_mla(const SparseMlaLaunch& a, const SparseMlaPlan& plan, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  Params p;
  p.q = a.q;
  p.kv = a.kv;
  p.idx = a.indices;
  p.bt = a.bt;
  p.out = a.out;
  p.lse = a.lse;
  p.ws = static_cast<uint8_t*>(a.workspace);
  p.c2 = a.sm_scale * a.q_scale * a.kv_scale * 1.4426950408889634f;
  p.vscale = a.kv_scale;
  p.R = (int32_t)a.rows;
  p.N = a.next_n;
  p.topk = a.topk;
  p.W = a.bt_stride;
  p.bshift = a.block_shift;
  p.splits = plan.splits;
  p.tps = plan.tiles_per_split;
  p.nblk = a.num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)a.num_blocks;
  hipLaunchKernelGGL(sparse_mla_kernel, dim3((unsigned)plan.splits, (unsigned)a.rows), dim3(kThreads), 0, stream, p);
  if (plan.splits > 1)
    hipLaunchKernelGGL(sparse_mla_combine_kernel, dim3(kH, (unsigned)a.rows), dim3(kDV / 4), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mqa
