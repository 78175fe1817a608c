// fp8 paged MQA logits on gfx950.
//
// Computes, for every decode row r = b*N + j and position t of a [B*N, L] fp32 output,
//   logit = sum_h w[r,h] * relu(scale_t * (q[b,j,h,:] . k_t))   if t <= ctx_b - N + j
//   -inf                                                        otherwise,
// where k_t / scale_t are the 128 e4m3fn bytes and the fp32 of the 132-byte cache row
// of token t: slot t % S of block block_tables[b][t / S], S = block_size (a power of
// two). Definition: stepcodex.com issue "[Bug] aiter ops triton attention
// pa_mqa_logits", section "Minimal reproduction".
//
// Mapping onto CDNA4
//   * Precision: gfx950's fp8 MFMAs (16x16x128 f8f6f4 and 16x16x32 fp8) round the dot
//     product at about 2^-15.5 of sum|q_i k_i|, measured against exact products; near a
//     cancelling head sum that exceeds the 5e-3 + 1e-3*|logit| budget. So fp8 bytes are
//     converted exactly to f16 (v_cvt_scalef32_pk_f16_fp8, scale 1) and contracted with
//     v_mfma_f32_16x16x32_f16, four chained per 128-wide row: f16 products of e4m3
//     values are exact and the fp32 accumulation is correctly rounded.
//   * Schedule: one round of persistent workgroups (one or two per CU), so no workgroup
//     waits for a slot. Each wave scans context_lens into prefix sums (for up to 64 requests
//     in its own registers, one request per lane, no barrier or LDS; beyond that in LDS,
//     one copy per workgroup, DPP wave scans and one barrier); every
//     wave then takes an equal contiguous share of the work units of all requests -
//     each 64-token key stage one unit, and each request's start one more, the cost of
//     loading another request's table entries and query rows - split at request
//     boundaries into segments, and afterwards an equal share of the 1 KB chunks of
//     -inf tail that lie past each request's last stage.
//     The balance does not depend on how context lengths are distributed, and nothing
//     is read from the device by the host.
//   * Small calls (a grid of at most two workgroups per CU that already holds a wave for
//     every stage of every request at its largest context, up to 64 requests, one row
//     group) skip the shares: wave gw owns stage gw / B of request gw % B, and loads that
//     stage's table entries and its query rows together with the context lengths, so the
//     first gathers wait for one round trip instead of two.
//   * One wave owns a group of decode rows (at most 8 MFMA row tiles of 16 heads, 4 with
//     64-token pages). Its query rows stay in VGPRs, already in f16, in the A-operand
//     layout, for a whole segment. Decode rows beyond one wave's share are other row
//     groups: other waves walk the same stages for them (their second read of a key row
//     hits L2).
//   * Keys are gathered straight from HBM into the B-operand slots: lane (g, c),
//     g = lane/16, c = lane%16, owns token c of a 16-token column tile and reads bytes
//     [16g, 16g+16) and [64+16g, 64+16g+16) of that token's row, so each dwordx4 load
//     instruction covers the first (then the second) 64 contiguous bytes of 16 rows. A
//     and B use the same byte-to-k assignment, so the contraction covers all 128 k
//     whatever order the hardware uses internally.
//   * The block table is read 64 tokens at a time (lane l reads the entry of token
//     t0 + l: one coalesced dword per lane for S = 1, a broadcast for S >= 64) and
//     redistributed with ds_bpermute; the row is entry * S + t % S. A wave keeps the keys of two 64-token stages in
//     flight (~17 KB), the table entries two stages ahead of their use, and issues its
//     first two stages before converting its query rows. Every gather is issued
//     unconditionally (a dead stage or a table entry outside the cache reads row 0
//     instead), and the prologue issues in the loop's order, so the loop is
//     straight-line code and each compute waits only for its own stage's loads.
//   * Half-stage form (pages under 64 tokens, a wave holding several decode rows or more
//     than 64 heads): the two 32-token halves of the next stage are in flight (~8.4 KB)
//     while a stage is computed, the weights sit in LDS, and one tile's operands and
//     accumulators are live at a time, so even 8 row tiles fit 256 VGPRs and two
//     workgroups share a CU: the same bytes in flight per CU, spread over twice the waves.
//   * Epilogue in registers: the dequant scale's sign is folded into the fp8 key (flip
//     the sign bit of every byte, exact; skipped when no scale of the tile is negative),
//     so relu(scale*s) = |scale| * relu(sign*s) and |scale| multiplies once per token
//     after the head sum. Each lane sums w * relu over its 4 heads per row tile and the
//     row tiles of a decode row; two cross-lane swaps (v_permlane32_swap, then
//     v_permlane16_swap) finish the sum across the 4 lane groups of a column.
//   * Stores: after a 64-token stage each lane group keeps one 16-token column tile, so
//     a row's 64 logits leave in one 256-byte store; positions past a row's causal limit
//     inside its last stage are written with -inf there. The -inf tail past the last
//     stage (most of the output when L >> ctx) is streamed with nontemporal 16-byte
//     stores: nothing reads it back soon, and the write rate rises from ~4.0 to ~5.5 TB/s.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launch.h"

namespace mqa {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 128;          // head_dim
constexpr int kRow = kD + 4;     // cache row bytes: keys + fp32 scale
constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;  // waves per workgroup
constexpr int kThreads = kWave * kWavesPerGroup;
constexpr int kStage = 64;       // tokens per pipeline stage = 4 MFMA column tiles
constexpr int kTilesPerStage = kStage / 16;
constexpr int kTailChunk = 4 * kWave;  // floats per tail chunk: one float4 per lane
// Work units a request's start costs on top of its stages when the key stages are shared
// out: a wave whose share enters another request loads that request's table entries and
// query rows before its next gathers, which measured about one stage of time.
constexpr int kStartUnits = 1;
// Tail chunks one key stage is counted as when the -inf tail is shared out (a stage
// gathers ~17 KB of cache lines, a chunk stores 1 KB; 4, 8 and 16 measured alike).
constexpr int kStageChunks = 8;

struct Params {
  const uint8_t* q;
  const uint8_t* kv;
  const float* w;
  const int32_t* ctx_lens;
  const int32_t* bt;
  float* out;
  uint32_t nblk;      // valid block ids are [0, nblk) (num_blocks capped at 2^31 - 1)
  int32_t B, N, H, W, L;  // W: block-table row length, in blocks
  int32_t bshift;     // log2(block_size)
  int32_t Wt;         // W << bshift: tokens a table row can address
  int32_t groups;     // row groups: waves that walk the same stages for different rows
  int32_t vec_store;  // rows of `out` are 16-byte aligned (L % 4 == 0, aligned base)
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

// Gathered keys of NT consecutive 16-token column tiles (a whole stage, NT = 4, or half
// of one, NT = 2), in the lane's B-operand slots.
template <int NT>
struct Keys {
  i32x4 lo[NT];
  i32x4 hi[NT];
  float scale[NT];
  int bad;  // bit u: tile u's table entry is outside the cache (its row 0 was read)
};

// x summed over the four lane groups {c, c+16, c+32, c+48}; every lane gets the sum
// ((x0 + x2) + (x1 + x3), the same order in every lane).
__device__ __forceinline__ float sum_lane_groups(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then row broadcasts).
__device__ __forceinline__ uint32_t wave_scan_add(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive prefix sums of two values per thread over the workgroup (thread order),
// through red[2 * kWavesPerGroup]. One barrier.
__device__ __forceinline__ void block_scan2(uint32_t v0, uint32_t v1, uint32_t& e0, uint32_t& e1, uint32_t* red) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint32_t i0 = wave_scan_add(v0), i1 = wave_scan_add(v1);
  if (lane == kWave - 1) {
    red[wave] = i0;
    red[kWavesPerGroup + wave] = i1;
  }
  __syncthreads();
  uint32_t b0 = 0, b1 = 0;
#pragma unroll
  for (int w = 0; w < kWavesPerGroup; ++w) {
    b0 += w < wave ? red[w] : 0u;
    b1 += w < wave ? red[kWavesPerGroup + w] : 0u;
  }
  e0 = b0 + i0 - v0;
  e1 = b1 + i1 - v1;
}

// Largest index i in [0, n) with a[i] <= x (a nondecreasing, a[0] <= x).
__device__ __forceinline__ int locate(const int* a, int n, int x) {
  int lo = 0, hi = n;  // invariant: a[lo] <= x, answer < hi
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Up to 4 row tiles fit two waves per SIMD (<= 256 VGPRs); so do up to 8 in the half-stage
// form (HALF: half a stage of keys per pipeline slot, weights in LDS). The whole-stage
// 5..8-tile variants (64-token pages with H > 64) take the whole register file.
template <int TPJ, int JPG, bool SMALL, bool HALF>
__global__ __launch_bounds__(kThreads, (TPJ * JPG <= 4 || HALF) ? 2 : 1) void paged_logits_kernel(Params p) {
  constexpr int TILES = TPJ * JPG;  // MFMA row tiles (16 heads each) held by one wave
  static_assert(TILES >= 1 && TILES <= 8, "query tile budget");
  static_assert(!(SMALL && HALF), "one form per instance");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // More than 64 requests: LDS holds the clamped ctx per request, the work-unit prefix,
  // the tail-chunk prefix and scan scratch. Up to 64, every wave keeps them in registers
  // (one request per lane, no barrier) and LDS is not used.
  extern __shared__ int lds[];
  __shared__ f32x4 wsh[HALF ? kWavesPerGroup : 1][HALF ? TILES : 1][4];  // half form: weights per wave
  const int B = p.B;
  const bool per_wave = B <= kWave;
  int* ctx_s = lds;                     // [B]
  int* stage_pref = ctx_s + B;          // [B+1] work units: stages + kStartUnits each
  int* tail_pref = stage_pref + B + 1;  // [B+1]
  int* scan_tmp = tail_pref + B + 1;    // [2 * kWavesPerGroup]
  const int g = lane >> 4;   // lane group: k-slice for operands, row quad for results
  const int c = lane & 15;   // column (token) / row (head) within a 16-wide tile
  const int L = p.L;
  const int nwaves = gridDim.x * kWavesPerGroup;
  const int gw = blockIdx.x * kWavesPerGroup + wave;

  // Small calls (one row group, at most 64 requests, and a wave for every stage of every
  // request at its largest context): wave gw owns stage gw / B of request gw % B. Its table
  // entries and query rows are loaded at once, beside the context lengths, so no schedule
  // stands between the start and the first gathers.
  const int sb = SMALL ? gw % B : 0;
  const int ss = SMALL ? gw / B : 0;
  int tab_s = 0;
  i32x4 qraw_s[SMALL ? TILES : 1][2];
  f32x4 wv_s[SMALL ? TILES : 1];
  if constexpr (SMALL) {
    tab_s = p.bt[(int64_t)sb * p.W + min((ss * kStage + lane) >> p.bshift, p.W - 1)];
    const int jn_s = min(JPG, p.N);
    const uint8_t* qb = p.q + (int64_t)sb * p.N * p.H * kD;
    const float* wb = p.w + (int64_t)sb * p.N * p.H;
#pragma unroll
    for (int m = 0; m < TILES; ++m) {
      const int mr = min(m / TPJ, jn_s - 1) * TPJ + m % TPJ;
      const uint8_t* qr = qb + (mr * 16 + c) * kD;
      qraw_s[m][0] = load16(qr + 16 * g);
      qraw_s[m][1] = load16(qr + 64 + 16 * g);
      wv_s[m] = *reinterpret_cast<const f32x4*>(wb + mr * 16 + 4 * g);
    }
  }

  // ---- Schedule: per request, the number of 64-token key stages and of tail chunks.
  // Up to 64 requests they stay in registers, lane b holding request b (read back with
  // readlane at a wave-uniform index); beyond, in LDS.
  int r_ctx = 0, r_pref = 0, r_tail = 0, tot_pref = 0, tot_tail = 0;
  int v_all = 0, v_below = 0;  // small calls: stages that exist, and those of the waves below gw
  if (per_wave) {
    int nu = 0, nc = 0, va = 0, vb = 0;
    if (lane < B) {
      r_ctx = max(0, min(p.ctx_lens[lane], min(p.Wt, L)));
      const int ns = (r_ctx + kStage - 1) / kStage;
      const int tail0 = ns * kStage;
      nc = tail0 < L ? p.N * ((L - tail0 + kTailChunk - 1) / kTailChunk) : 0;
      nu = ns > 0 ? ns + kStartUnits : 0;
      if (SMALL) {  // request `lane`'s stages belong to waves lane, lane + B, ...
        va = ns;
        vb = min(ns, gw > lane ? (gw - 1 - lane) / B + 1 : 0);
      }
    }
    const int iu = (int)wave_scan_add((uint32_t)nu), ic = (int)wave_scan_add((uint32_t)nc);
    r_pref = iu - nu;
    r_tail = ic - nc;
    tot_pref = __builtin_amdgcn_readlane(iu, kWave - 1);  // lanes past B add nothing
    tot_tail = __builtin_amdgcn_readlane(ic, kWave - 1);
    if (SMALL) {
      v_all = __builtin_amdgcn_readlane((int)wave_scan_add((uint32_t)va), kWave - 1);
      v_below = __builtin_amdgcn_readlane((int)wave_scan_add((uint32_t)vb), kWave - 1);
    }
  } else {
    const int per = (B + kThreads - 1) / kThreads;  // requests per thread, consecutive
    const int r0 = threadIdx.x * per;
    int stages = 0, chunks = 0;
    for (int i = 0; i < per; ++i) {
      const int b = r0 + i;
      if (b < B) {
        const int ctx = max(0, min(p.ctx_lens[b], min(p.Wt, L)));
        const int ns = (ctx + kStage - 1) / kStage;
        const int tail0 = ns * kStage;
        const int nc = tail0 < L ? p.N * ((L - tail0 + kTailChunk - 1) / kTailChunk) : 0;
        const int nu = ns > 0 ? ns + kStartUnits : 0;
        ctx_s[b] = ctx;
        stage_pref[b] = nu;  // counts for now
        tail_pref[b] = nc;
        stages += nu;
        chunks += nc;
      }
    }
    uint32_t s_excl, c_excl;
    block_scan2((uint32_t)stages, (uint32_t)chunks, s_excl, c_excl, reinterpret_cast<uint32_t*>(scan_tmp));
    int s_run = (int)s_excl, c_run = (int)c_excl;
    for (int i = 0; i < per; ++i) {
      const int b = r0 + i;
      if (b < B) {
        const int nu = stage_pref[b], nc = tail_pref[b];
        stage_pref[b] = s_run;
        tail_pref[b] = c_run;
        s_run += nu;
        c_run += nc;
      }
    }
    if (threadIdx.x == kThreads - 1) {
      stage_pref[B] = s_run;
      tail_pref[B] = c_run;
    }
    __syncthreads();
  }

  // Clamped ctx, work-unit prefix and tail-chunk prefix of request i (i <= B for the
  // prefixes, where entry B is the total); i is wave-uniform.
  auto ctx_at = [&](int i) { return per_wave ? __builtin_amdgcn_readlane(r_ctx, i) : ctx_s[i]; };
  auto pref_at = [&](int i) {
    return per_wave ? (i >= B ? tot_pref : __builtin_amdgcn_readlane(r_pref, i)) : stage_pref[i];
  };
  auto tail_at = [&](int i) {
    return per_wave ? (i >= B ? tot_tail : __builtin_amdgcn_readlane(r_tail, i)) : tail_pref[i];
  };

  // ---- Key stages.
  const int G = p.groups;
  const int group = gw % G;
  const int wi = gw / G;
  const int nw = nwaves / G;
  const int j0 = group * JPG;         // first decode row of this wave
  const int jn = min(JPG, p.N - j0);  // decode rows this wave owns
  // Share [floor(wi*S/nw), floor((wi+1)*S/nw)) in 32-bit arithmetic: with S = sq*nw + sr,
  // floor(wi*S/nw) = wi*sq + floor(wi*sr/nw), and wi*sr < nw^2 fits. sr waves of each
  // group take sq + 1 units, the others sq.
  const int S = SMALL ? 0 : pref_at(B);
  const int sq = S / nw, sr = S - sq * nw;
  const bool s_valid = SMALL && ss < (ctx_at(sb) + kStage - 1) / kStage;  // this wave's small-call stage exists
  const uint8_t* kv_g = p.kv + 16 * g;  // this lane's first key slice
  const uint8_t* kv_s = p.kv + kD;      // scales
  {
    // NT column tiles u0 .. u0+NT-1 of the stage starting at token tok0, whose table entries
    // (lane l: the entry of token tok0 + l) are in tab: their rows' keys into the B-operand
    // slots of s (row 0 when the stage is not live or an entry is outside the cache).
    auto gather_tiles = [&](int tok0, int u0, bool live, int tab, auto& s) {
      constexpr int NT = sizeof(s.scale) / sizeof(float);
      int ph[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) ph[u] = __shfl(tab, (u0 + u) * 16 + c);
      const uint32_t smask = (1u << p.bshift) - 1u;  // slot of a token in its block
      const uint32_t tok = (uint32_t)(tok0 + c);
      s.bad = 0;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const uint32_t slot = (tok + 16u * (u0 + u)) & smask;
        const bool inb = (uint32_t)ph[u] < p.nblk;
        const uint32_t row = (live && inb) ? ((uint32_t)ph[u] << p.bshift) | slot : 0u;
        s.bad |= (inb ? 0 : 1) << u;
        const uint8_t* kp = kv_g + (uint64_t)row * kRow;
        s.lo[u] = load16(kp);
        s.hi[u] = load16(kp + 64);
        s.scale[u] = *reinterpret_cast<const float*>(kv_s + (uint64_t)row * kRow);
      }
    };
    // Contraction and epilogue of those tiles of the stage at token tc for the owned decode
    // rows: lane group g keeps row jl's head sum of tile g in keep[jl] (positions from
    // t_need on are past ctx). wget(m) gives the lane's weights of row tile m.
    auto compute_tiles = [&](const Operand (&qa)[TILES], auto&& wget, const auto& s, int tc, int u0, int t_need,
                             float (&keep)[JPG]) {
      constexpr int NT = sizeof(s.scale) / sizeof(float);
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int ug = u0 + u;
        const int t = tc + ug * 16 + c;
        const bool in_ctx = t < t_need;
        const bool ok = in_ctx && !((s.bad >> u) & 1);
        // Past ctx the column is masked below; a bad table entry poisons it with NaN.
        const float sc = ok ? s.scale[u] : (in_ctx ? __builtin_nanf("") : 0.0f);
        i32x4 lo = s.lo[u], hi = s.hi[u];
        if (__ballot(__float_as_int(sc) < 0) != 0) {  // wave-uniform: rare
          const int flip = (__float_as_int(sc) < 0) ? (int)0x80808080 : 0;
          lo ^= flip;
          hi ^= flip;
        }
        const Operand kb = to_operand(lo, hi);
        const float sabs = __builtin_fabsf(sc);
#pragma unroll
        for (int jl = 0; jl < JPG; ++jl) {
          f32x4 acc[TPJ];
#pragma unroll
          for (int mm = 0; mm < TPJ; ++mm) {
            const int m = jl * TPJ + mm;
            acc[mm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[m].k[0], kb.k[0], f32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int k = 1; k < 4; ++k)
              acc[mm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[m].k[k], kb.k[k], acc[mm], 0, 0, 0);
          }
          float part = 0.0f;
#pragma unroll
          for (int mm = 0; mm < TPJ; ++mm) {
            const f32x4 wm = wget(jl * TPJ + mm);
#pragma unroll
            for (int v = 0; v < 4; ++v)
              part = __builtin_fmaf(wm[v], __builtin_elementwise_maximum(acc[mm][v], 0.0f), part);
          }
          part = sum_lane_groups(part);
          if (g == ug) keep[jl] = part * sabs;
        }
        // The half form keeps one tile's operands and accumulators live at a time: its
        // register budget is that of two waves per SIMD.
        if constexpr (HALF) __builtin_amdgcn_sched_barrier(0);
      }
    };
    // The stage's 64 logits of the jn owned decode rows (row jl of out0 + jl * L; positions
    // from nv[jl] on are past the row's causal limit, from t_end on past the output row).
    auto store_stage = [&](int tc, int t_end, const int (&nv)[JPG], float* out0, int jn, const float (&keep)[JPG]) {
      const int t = tc + lane;  // lane (g, c) stores token 16g + c of the stage
      if (t < t_end) {
#pragma unroll
        for (int jl = 0; jl < JPG; ++jl)
          if (jl < jn) out0[(int64_t)jl * L + t] = (t < nv[jl]) ? keep[jl] : -__builtin_inff();
      }
    };
    if constexpr (SMALL) {
      if (s_valid) {  // wave-uniform
        const int ctx = ctx_at(sb);
        const int tc = ss * kStage;
        const int t_end = min(tc + kStage, L);
        const int t_need = min(t_end, ctx);
        int nv[JPG];
#pragma unroll
        for (int jl = 0; jl < JPG; ++jl) nv[jl] = min(ctx - p.N + jl + 1, L);
        Keys<kTilesPerStage> sx;
        gather_tiles(tc, 0, true, tab_s, sx);
        Operand qs[TILES];
#pragma unroll
        for (int m = 0; m < TILES; ++m) qs[m] = to_operand(qraw_s[m][0], qraw_s[m][1]);
        float keep[JPG];
#pragma unroll
        for (int jl = 0; jl < JPG; ++jl) keep[jl] = 0.0f;
        compute_tiles(qs, [&](int m) { return wv_s[m]; }, sx, tc, 0, t_need, keep);
        store_stage(tc, t_end, nv, p.out + (int64_t)sb * p.N * L, min(JPG, p.N), keep);
      }
    } else if (wi < nw) {
    int lo = wi * sq + (wi * sr) / nw;
    const int hi = (wi + 1) * sq + ((wi + 1) * sr) / nw;
    int b = 0;
    if (lo < hi) {
      if (per_wave) {  // the prefix entries <= lo are a run from entry 0: count them
        const uint64_t le = __ballot(lane < B && r_pref <= lo);
        b = __popcll(le) - 1;
      } else {
        b = locate(stage_pref, B, lo);
      }
    }
    while (lo < hi) {
      // Segment: stages [s0, s0 + nstage) of request b, the stages whose units fall in
      // [lo, seg_hi); none when the share holds only the request's start units.
      const int pb = pref_at(b);
      const int seg_hi = min(hi, pref_at(b + 1));
      const int s0 = max(lo - pb - kStartUnits, 0);
      const int nstage = seg_hi - pb - kStartUnits - s0;
      if (nstage > 0) {
        const int ctx = ctx_at(b);
        const int t0 = s0 * kStage;
        const int t_end = min((s0 + nstage) * kStage, L);
        const int t_need = min(t_end, ctx);
        float* const out0 = p.out + (int64_t)(b * p.N + j0) * L;

        int nv[JPG];  // visible positions of each owned decode row
#pragma unroll
        for (int jl = 0; jl < JPG; ++jl) nv[jl] = min(ctx - p.N + (j0 + jl) + 1, L);

        const int32_t* btb = p.bt + (int64_t)b * p.W;
        const int wmax = p.W - 1;
        auto load_table = [&](int st) -> int {
          return btb[st < nstage ? min((t0 + st * kStage + lane) >> p.bshift, wmax) : 0];
        };
        // Table entries of the first two stages first: the gathers wait for them, and a
        // wait on a load also waits for every load issued before it.
        int tab0 = load_table(0);
        int tab1 = load_table(1);
        __builtin_amdgcn_sched_barrier(0);
        // Query rows of this segment: raw bytes now, f16 A operands once the first key
        // gathers are on their way (the conversion then overlaps their latency).
        i32x4 qraw[TILES][2];
        f32x4 wv[TILES];
        {
          const uint8_t* qb = p.q + ((int64_t)b * p.N + j0) * p.H * kD;
          const float* wb = p.w + ((int64_t)b * p.N + j0) * p.H;
          // Row tiles of decode rows past N repeat the last row (never stored).
          auto row_tile = [&](int m) { return min(m / TPJ, jn - 1) * TPJ + m % TPJ; };
#pragma unroll
          for (int m = 0; m < TILES; ++m) wv[m] = *reinterpret_cast<const f32x4*>(wb + row_tile(m) * 16 + 4 * g);
#pragma unroll
          for (int m = 0; m < TILES; ++m) {
            const uint8_t* qr = qb + (row_tile(m) * 16 + c) * kD;
            qraw[m][0] = load16(qr + 16 * g);
            qraw[m][1] = load16(qr + 64 + 16 * g);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        Operand qa[TILES];

        if constexpr (!HALF) {
          // Software pipeline: keys of two stages in flight, table entries two stages ahead
          // of their use; the compute of stage s waits only for stage s's loads, and its
          // registers are refilled with stage s+2 right after.
          // The prologue issues in the loop's order (keys of a stage, then the table entries
          // two stages on), so the wait counts computed for the loop's first pass hold for
          // every pass; stages past the segment issue harmless loads of row 0, so the loop
          // body is straight-line code. sched_barrier(0) keeps the scheduler from pulling a
          // use of a load up next to it, which would serialise the latencies.
          auto issue_keys = [&](int st, int tab, Keys<kTilesPerStage>& s) {
            gather_tiles(t0 + st * kStage, 0, st < nstage, tab, s);
          };
          auto compute_store = [&](int st, const Keys<kTilesPerStage>& s) {
            float keep[JPG];
#pragma unroll
            for (int jl = 0; jl < JPG; ++jl) keep[jl] = 0.0f;
            compute_tiles(qa, [&](int m) { return wv[m]; }, s, t0 + st * kStage, 0, t_need, keep);
            store_stage(t0 + st * kStage, t_end, nv, out0, jn, keep);
          };
          Keys<kTilesPerStage> sa, sb;
          issue_keys(0, tab0, sa);
          tab0 = load_table(2);
          issue_keys(1, tab1, sb);
          tab1 = load_table(3);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int m = 0; m < TILES; ++m) qa[m] = to_operand(qraw[m][0], qraw[m][1]);
          for (int st = 0; st < nstage; st += 2) {
            compute_store(st, sa);
            issue_keys(st + 2, tab0, sa);
            tab0 = load_table(st + 4);
            if (st + 1 < nstage) compute_store(st + 1, sb);
            issue_keys(st + 3, tab1, sb);
            tab1 = load_table(st + 5);
          }
        } else {
          // Half-stage pipeline: the two halves (32 tokens each) of the next stage are in
          // flight while a stage is computed, and table entries are loaded two stages
          // ahead of their use; the prologue issues in the loop's order here too. Half the
          // key registers of the form above, so two workgroups fit on a CU with the same
          // bytes in flight per CU. The weights wait in this wave's LDS slots (read back as
          // broadcasts) instead of 4 * TILES VGPRs.
          Keys<2> sa, sb;
          int tn = tab0;   // entries of the stage whose halves are issued next
          int tnn = tab1;  // and of the one after it
          gather_tiles(t0, 0, 0 < nstage, tn, sa);
          gather_tiles(t0, 2, 0 < nstage, tn, sb);
          tn = tnn;
          tnn = load_table(2);
          __builtin_amdgcn_sched_barrier(0);
          if (c == 0) {
#pragma unroll
            for (int m = 0; m < TILES; ++m) wsh[wave][m][g] = wv[m];
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int m = 0; m < TILES; ++m) qa[m] = to_operand(qraw[m][0], qraw[m][1]);
          auto wget = [&](int m) { return wsh[wave][m][g]; };
          for (int st = 0; st < nstage; ++st) {
            const int tc = t0 + st * kStage;
            float keep[JPG];
#pragma unroll
            for (int jl = 0; jl < JPG; ++jl) keep[jl] = 0.0f;
            compute_tiles(qa, wget, sa, tc, 0, t_need, keep);
            gather_tiles(tc + kStage, 0, st + 1 < nstage, tn, sa);
            compute_tiles(qa, wget, sb, tc, 2, t_need, keep);
            store_stage(tc, t_end, nv, out0, jn, keep);
            gather_tiles(tc + kStage, 2, st + 1 < nstage, tn, sb);
            tn = tnn;
            tnn = load_table(st + 3);
          }
        }
      }

      lo = seg_hi;
      ++b;
      while (b < B && pref_at(b + 1) <= lo) ++b;  // skip requests without stages
    }
    }
  }

  // ---- -inf tail: positions past each request's last key stage, every row. Each wave
  // takes a contiguous run of 1 KB chunks and walks it row by row (LDS is read only
  // where the run enters another request).
  {
    // The waves with a longer stage share (sq + 1 units; in a small call, the waves that
    // own a stage) take kStageChunks chunks fewer than the others (none if the tail is
    // short), so they are not the last to finish: heavy waves split the first C_H chunks
    // equally, the light ones the rest.
    const int C = tail_at(B);
    const int nH = SMALL ? (v_all < nwaves ? v_all : 0) : G * sr, nL = nwaves - nH;
    const bool heavy = SMALL ? (s_valid && nH > 0) : (wi < nw && ((wi + 1) * sr) / nw > (wi * sr) / nw);
    const int heavy_before = SMALL ? (nH > 0 ? v_below : 0) : G * min((wi * sr) / nw, sr) + (heavy ? group : 0);
    const int cH = max(0, (int)(((uint32_t)C + (uint32_t)nH * kStageChunks) / (uint32_t)nwaves) - kStageChunks);
    const int CH = nH * cH, CL = C - CH;
    int ci, ce;
    if (heavy) {
      ci = heavy_before * cH;
      ce = ci + cH;
    } else {
      const int li = gw - heavy_before;  // index among the light waves
      const int lq = CL / nL, lr = CL - lq * nL;
      ci = CH + li * lq + (li * lr) / nL;
      ce = CH + (li + 1) * lq + ((li + 1) * lr) / nL;
    }
    ci = __builtin_amdgcn_readfirstlane(ci);
    ce = __builtin_amdgcn_readfirstlane(ce);
    if (ci < ce) {
      const f32x4 ninf = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
      int b = per_wave ? __popcll(__ballot(lane < B && r_tail <= ci)) - 1 : locate(tail_pref, B, ci);
      b = __builtin_amdgcn_readfirstlane(b);
      int tail0 = 0, per_row = 1, j = 0, k = 0;
      auto enter = [&](int local) {  // request b, chunk `local` of its N rows
        tail0 = __builtin_amdgcn_readfirstlane(((ctx_at(b) + kStage - 1) / kStage) * kStage);
        per_row = (L - tail0 + kTailChunk - 1) / kTailChunk;
        j = local / per_row;
        k = local - j * per_row;
      };
      enter(ci - __builtin_amdgcn_readfirstlane(tail_at(b)));
      for (;;) {
        float* rp = p.out + (int64_t)(b * p.N + j) * L;
        const int start = tail0 + k * kTailChunk;
        const int end = min(start + kTailChunk, L);
        const int pos = start + 4 * lane;
        if (p.vec_store && pos + 4 <= end) {
          __builtin_nontemporal_store(ninf, reinterpret_cast<f32x4*>(rp + pos));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (pos + i < end) rp[pos + i] = -__builtin_inff();
        }
        if (++ci >= ce) break;
        if (++k == per_row) {
          k = 0;
          if (++j == p.N) {  // the next request that has a tail
            while (b + 1 < B && __builtin_amdgcn_readfirstlane(tail_at(b + 1)) <= ci) ++b;
            enter(ci - __builtin_amdgcn_readfirstlane(tail_at(b)));
          }
        }
      }
    }
  }
}

using KernelFn = void (*)(Params);

template <int TPJ, int JPG>
constexpr KernelFn kfn() { return paged_logits_kernel<TPJ, JPG, false, false>; }
template <int TPJ, int JPG>
constexpr KernelFn kfs() { return paged_logits_kernel<TPJ, JPG, true, false>; }
template <int TPJ, int JPG>
constexpr KernelFn kfh() { return paged_logits_kernel<TPJ, JPG, false, true>; }

// [TPJ-1][JPG-1]; TPJ = H/16 in 1..8, JPG = decode rows per wave: min(N, T/TPJ) with
// T = 8 row tiles (128 f16 query VGPRs) for pages under 64 tokens and T = 4 (64 VGPRs,
// two workgroups per CU) otherwise; 1 for H > 64 (up to 8 row tiles).
constexpr KernelFn kTable[8][4] = {
    {kfn<1, 1>(), kfn<1, 2>(), kfn<1, 3>(), kfn<1, 4>()},
    {kfn<2, 1>(), kfn<2, 2>(), kfn<2, 3>(), kfn<2, 4>()},
    {kfn<3, 1>(), kfn<3, 2>(), nullptr, nullptr},
    {kfn<4, 1>(), kfn<4, 2>(), nullptr, nullptr},
    {kfn<5, 1>(), nullptr, nullptr, nullptr},
    {kfn<6, 1>(), nullptr, nullptr, nullptr},
    {kfn<7, 1>(), nullptr, nullptr, nullptr},
    {kfn<8, 1>(), nullptr, nullptr, nullptr},
};

// Small-call forms, [TPJ-1][JPG-1] for up to 4 row tiles.
constexpr KernelFn kTableSmall[4][4] = {
    {kfs<1, 1>(), kfs<1, 2>(), kfs<1, 3>(), kfs<1, 4>()},
    {kfs<2, 1>(), kfs<2, 2>(), nullptr, nullptr},
    {kfs<3, 1>(), nullptr, nullptr, nullptr},
    {kfs<4, 1>(), nullptr, nullptr, nullptr},
};

// Half-stage forms, [TPJ-1][JPG-1]: several decode rows per wave, or more than 64 heads.
constexpr KernelFn kTableHalf[8][4] = {
    {nullptr, kfh<1, 2>(), kfh<1, 3>(), kfh<1, 4>()},
    {nullptr, kfh<2, 2>(), kfh<2, 3>(), kfh<2, 4>()},
    {nullptr, kfh<3, 2>(), nullptr, nullptr},
    {nullptr, kfh<4, 2>(), nullptr, nullptr},
    {kfh<5, 1>(), nullptr, nullptr, nullptr},
    {kfh<6, 1>(), nullptr, nullptr, nullptr},
    {kfh<7, 1>(), nullptr, nullptr, nullptr},
    {kfh<8, 1>(), nullptr, nullptr, nullptr},
};

// Compute units of the current device, read once per device.
int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}

// Up to 64 requests the schedule lives in registers and the kernel uses no LDS.
size_t logits_lds_bytes(int32_t batch) {
  return batch <= kWave ? 0 : (size_t)(3 * (int64_t)batch + 2 + 2 * kWavesPerGroup) * 4;
}

}  // namespace

hipError_t launch_logits(const LogitsLaunch& a, hipStream_t stream) {
  const int tpj = a.heads / 16;
  // Decode rows per wave: with pages under 64 tokens a wave holds up to 8 row tiles, so
  // the key rows of a stage are gathered once for all of a request's decode rows (in the
  // half-stage form below, two workgroups per CU); with 64-token pages up to 4, in whole
  // stages, two workgroups per CU when a request has several row groups (measured faster
  // there for N = 4).
  const int max_tiles = a.block_shift < 6 ? 8 : 4;
  const int per_wave = tpj <= max_tiles ? max_tiles / tpj : 1;
  const int jpg = a.next_n < per_wave ? a.next_n : per_wave;
  Params p;
  p.q = a.q;
  p.kv = a.kv;
  p.w = a.w;
  p.ctx_lens = a.ctx_lens;
  p.bt = a.bt;
  p.out = a.out;
  p.nblk = a.num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)a.num_blocks;
  p.B = a.batch;
  p.N = a.next_n;
  p.H = a.heads;
  p.W = a.bt_stride;
  p.L = a.max_model_len;
  p.bshift = a.block_shift;
  p.Wt = a.bt_stride << a.block_shift;
  p.groups = (a.next_n + jpg - 1) / jpg;
  p.vec_store = (a.max_model_len % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.out) & 15) == 0);
  KernelFn fn = kTable[tpj - 1][jpg - 1];
  const size_t lds = logits_lds_bytes(a.batch);
  // One round of persistent workgroups, one or two per CU, but no more waves than there
  // can be work for: the host knows an upper bound of the key stages (every request at its
  // largest context) and of the tail chunks, and small calls then launch a small grid.
  const int64_t ctx_cap = a.max_model_len < (int64_t)p.Wt ? a.max_model_len : (int64_t)p.Wt;
  const int64_t stage_bound = (int64_t)a.batch * ((ctx_cap + kStage - 1) / kStage + kStartUnits) * p.groups;
  const int64_t tail_bound = (int64_t)a.batch * a.next_n * ((a.max_model_len + kTailChunk - 1) / kTailChunk);
  const int64_t need = (std::max(stage_bound, tail_bound) + kWavesPerGroup - 1) / kWavesPerGroup;
  const int cus = compute_units();
  int64_t per_cu = 1;
  if (a.batch <= kWave && p.groups == 1 && tpj * jpg <= 4 && need <= 2 * (int64_t)cus) {
    // Small calls: when two workgroups per CU hold a wave for every stage of every request
    // at its largest context (one row group, at most 64 requests), each wave takes one
    // stage, fixed by its index, and issues its table and query loads beside the context
    // lengths: the schedule's round trips (context lengths, then table entries, then keys)
    // become one.
    fn = kTableSmall[tpj - 1][jpg - 1];
    per_cu = 2;
  } else if (a.block_shift < 6 && (jpg > 1 || tpj > 4)) {
    // A wave holding several decode rows, or more than 64 heads (pages under 64 tokens):
    // the half-stage form, whose registers fit two workgroups per CU (with whole stages
    // the 5..8-tile waves take the whole register file, one wave per SIMD). Measured
    // faster or equal on every shape tried: N = 2..4 at H = 32..80, H = 96 and 128 at N = 1.
    fn = kTableHalf[tpj - 1][jpg - 1];
    per_cu = 2;
  } else if (a.block_shift >= 6 && p.groups > 1 && tpj * jpg <= 4) {
    // With whole stages, four waves per CU measured faster than eight on single-token pages
    // and on single-group calls: each wave takes twice the stages and pays the start-up -
    // schedule, table and query loads queued behind the other waves' gathers - half as
    // often. With 64-token pages and several query groups per request (every key stage
    // read once per group, the later reads mostly from L2) eight waves per CU were faster
    // (4 to 10%): the key reads are whole lines and the wave is waiting on latency, not on
    // HBM. Two waves per CU, or a deeper prefetch (three or four stages in flight per
    // wave), were slower everywhere.
    per_cu = 2;
  }
  const int blocks = (int)std::max<int64_t>(1, std::min(per_cu * cus, need));
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace mqa
