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
// row is exactly the k largest e; no separate tie rule is needed.
//
// Cost model. A workgroup's waves share their CU's four SIMDs: with 16 waves on a CU
// every instruction a wave issues costs about 16 cycles of the workgroup's time. Per-element
// work is therefore kept to a few vector instructions (buffer loads clamped onto the last
// visible element, lane masks from one compare each, a NaN-propagating maximum for the
// finiteness test, emission from bit masks). Rows are spread over several workgroups only
// when one would take much longer than the synchronisation between them (~1-2 us per
// exchange through memory).
//
// Whole-row select (select_row): one workgroup holds the row in registers, 8 values per
// thread. A block min/max reduction sets 2048 first-level bins linear in the value
// (monotone, so bins are ordered like the logits; rows holding a non-finite value use the
// top 12 key bits instead, constant rows a single bin). An LDS histogram and a scan from
// the top find the bin holding the k-th element (every wave finishes the search itself
// after one barrier). Each lane marks its elements above that bin and in it in two bit
// masks; a lane scan of the mask populations and the wave totals (one barrier) give every
// lane its first slots: positions above the bin go straight to the output row, the bin's
// own elements to an LDS candidate list. A small list is finished by counting, for each
// candidate, the candidates above it (the count is the slot); a large one by further
// 11-bit radix digits of e, or over the whole row if the bin holds more than the list.
//
// Modes (nv is known only on the device):
//   max_model_len <= 8192: one launch, workgroup r (1024 threads) selects row r whole, or
//     writes it directly when nv <= k, or drops the row's smallest element when nv = k + 1.
//     No workspace.
//   8192 < max_model_len <= 32768: one launch, workgroup r selects row r whole with 32
//     values per thread. No workspace.
//   max_model_len > 32768: one launch of the chunked kernel (one workgroup per CU). Rows
//     of at most 32768 are selected whole; longer rows are cut into 8192-element chunks:
//     a row's chunks add their 12-bit key histograms into the row's histogram in the
//     workspace, then each chunk splits itself against the row's threshold bin and the
//     last one finishes the row's candidates (see the chunked section below).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "launch.h"

namespace mqa {
namespace {

constexpr int kPer = 8;                           // logits per thread of a row select
constexpr int kRowThreads = 1024;                 // workgroup size of every kernel here
constexpr int kRowLen = kRowThreads * kPer;       // 8192: rows selected with 8 values per thread
constexpr int kWidePer = 32;                      // logits per thread of a wide row select
constexpr int kWideLen = kRowThreads * kWidePer;  // 32768: rows one workgroup selects whole
constexpr int kChunkThreads = kRowThreads;        // chunked rows: workgroup size
constexpr int kChunkPer = 8;                      // logits per thread of a chunk
constexpr int kChunk = kChunkThreads * kChunkPer; // 8192-element chunks
constexpr int kLinBins = 2048;                    // first level of a whole-row select (linear)
constexpr int kKeyBits = 12;                      // first level of a chunked row (top key bits)
constexpr int kKeyBins = 1 << kKeyBits;           // 4096
constexpr int kCoarseBins = 64;                   // chunked rows: top 6 key bits, 64 key bins each
constexpr int kRowCap = 8192;                     // LDS candidates of a whole-row select (64 KB)
constexpr int kChunkCap = kRowCap;                // LDS (and workspace) candidates of a chunked row
constexpr int kRankMax = 256;                     // candidate lists up to this size are ranked
constexpr int kMaxK = 2048;                       // largest k the library accepts

struct Params {
  const float* logits;
  const int32_t* ctx_lens;
  int32_t* idx;
  // Workspace of the chunked mode (null otherwise), zero between calls: per row r,
  uint32_t* counters;     // [rows][4]: chunk histograms added, chunks split, emitted, candidates
  uint32_t* hist;         // [rows][kKeyBins] 12-bit key histogram
  uint32_t* coarse;       // [rows][kCoarseBins] the same counts over the top 6 key bits
  uint64_t* cand;         // [rows][kChunkCap] threshold-bin candidates
  int32_t rows, N, W, L, k;
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t compose(uint32_t key, int t) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
}

__device__ __forceinline__ int position(uint64_t e) { return (int)(0xFFFFFFFFu - (uint32_t)e); }

__device__ __forceinline__ int visible(const Params& p, int row) {
  const int b = row / p.N;
  const int j = row - b * p.N;
  const int ctx = max(0, min(p.ctx_lens[b], min(p.W, p.L)));
  return max(0, min(ctx - p.N + j + 1, p.L));
}

// Per-wave scratch slot groups (each group has one slot per wave), one group per use so
// that consecutive block operations need no barrier between them for the scratch itself.
enum { kRedLo = 0, kRedHi, kRedBad, kRedBin, kRedEmit, kRedCand, kRedLoc, kRedGroups };

template <int T>
struct Core {
  static constexpr int kWaves = T / 64;
  uint32_t hist[kKeyBins];
  uint32_t red[kRedGroups * kWaves];
  uint32_t n_out, bin, above, base_a, base_b, last, count;
  int32_t loc[4];  // the chunk located last: row, chunk, visible, chunks of the row
};

template <int T, int CAP>
struct Full : Core<T> {
  static constexpr int kCap = CAP;
  uint64_t cand[CAP];
};

// Wave-aggregated append to an LDS counter. Must be called by all 64 lanes of a wave.
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

// Running min / max over the lanes (lane 63 ends with the wave's value).
template <bool Max, int Ctrl, int Rows>
__device__ __forceinline__ float minmax_step(float v) {
  const int id = __float_as_int(Max ? -__builtin_inff() : __builtin_inff());
  const float o = __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(v), Ctrl, Rows, 0xf, false));
  return Max ? fmaxf(v, o) : fminf(v, o);
}

template <bool Max>
__device__ __forceinline__ float wave_scan_minmax(float v) {
  v = minmax_step<Max, 0x111, 0xf>(v);  // row_shr:1
  v = minmax_step<Max, 0x112, 0xf>(v);  // row_shr:2
  v = minmax_step<Max, 0x114, 0xf>(v);  // row_shr:4
  v = minmax_step<Max, 0x118, 0xf>(v);  // row_shr:8
  v = minmax_step<Max, 0x142, 0xa>(v);  // row_bcast:15
  v = minmax_step<Max, 0x143, 0xc>(v);  // row_bcast:31
  return v;
}

// Inclusive prefix sum within each 16-lane row of a wave (row-0 DPP shifts): lane l of
// row 0 ends with the sum of lanes 0..l.
__device__ __forceinline__ uint32_t row16_prefix(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  return v;
}

// Minimum (maximum) over lanes 0..15, returned to every lane.
template <bool Max>
__device__ __forceinline__ float row16_minmax(float v) {
  v = minmax_step<Max, 0x111, 0xf>(v);
  v = minmax_step<Max, 0x112, 0xf>(v);
  v = minmax_step<Max, 0x114, 0xf>(v);
  v = minmax_step<Max, 0x118, 0xf>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
}

// Exclusive prefix sum over the T threads in thread order, through the scratch slots of
// `group`. Also returns the block total. One barrier.
template <int T>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, Core<T>& sh, int group, uint32_t& total) {
  constexpr int W = T / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t* red = sh.red + group * W;
  const uint32_t incl = wave_scan_add(v);
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const uint32_t t = red[w];
    before += w < wave ? t : 0u;
    all += t;
  }
  total = all;
  return before + incl - v;
}

// Finds the bin B (scanning from the top of nbins) with above(B) < rem <= above(B) +
// hist[B]; leaves B in sh.bin and above(B) in sh.above. All threads must call it.
template <int T>
__device__ void find_bin(Core<T>& sh, int nbins, uint32_t rem) {
  const int per = nbins / T;
  const int top = nbins - 1 - per * (int)threadIdx.x;
  uint32_t cnt[kKeyBins / T] = {}, sum = 0;
  for (int i = 0; i < per; ++i) {
    cnt[i] = sh.hist[top - i];
    sum += cnt[i];
  }
  if (threadIdx.x == 0) {
    sh.bin = 0;
    sh.above = 0;
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan<T>(sum, sh, kRedBin, total);
  for (int i = 0; i < per; ++i) {
    if (run < rem && rem <= run + cnt[i]) {
      sh.bin = (uint32_t)(top - i);
      sh.above = run;
    }
    run += cnt[i];
  }
  __syncthreads();
}

template <int T>
__device__ __forceinline__ void clear_hist(Core<T>& sh, int nbins) {
  for (int i = threadIdx.x; i < nbins; i += T) sh.hist[i] = 0;
  __syncthreads();
}

// Selects the `rem` largest of the n candidates in sh.cand by counting, for each, the
// candidates above it; e is unique, so a selected candidate's rank is its slot after the
// sh.n_out positions already emitted. n <= kRankMax <= T: four lanes share a candidate
// (each counts over a quarter of the list, two DPP steps add the parts) when the list is
// short enough, else one lane counts over all of it.
template <int T, int CAP>
__device__ void rank_select(Full<T, CAP>& sh, int n, uint32_t rem, int32_t* out, int k) {
  static_assert(kRankMax <= T, "one lane per candidate at least");
  const uint32_t base = sh.n_out;
  if (4 * n <= T) {  // uniform
    const int i = threadIdx.x >> 2, part = threadIdx.x & 3;
    const uint64_t e = i < n ? sh.cand[i] : 0;
    uint32_t rank = 0;
    for (int j = part; j < n; j += 4) rank += sh.cand[j] > e ? 1u : 0u;
    rank += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)rank, 0xB1, 0xf, 0xf, false);  // quad_perm 1,0,3,2
    rank += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)rank, 0x4E, 0xf, 0xf, false);  // quad_perm 2,3,0,1
    if (i < n && part == 0 && rank < rem && base + rank < (uint32_t)k) out[base + rank] = position(e);
  } else {
    const int i = threadIdx.x;
    const uint64_t e = i < n ? sh.cand[i] : 0;
    uint32_t rank = 0;
#pragma unroll 8
    for (int j = 0; j < n; ++j) rank += sh.cand[j] > e ? 1u : 0u;
    if (i < n && rank < rem && base + rank < (uint32_t)k) out[base + rank] = position(e);
  }
  __syncthreads();
}

// Radix refinement over the candidate list (FromRow = false) or the whole visible row
// (FromRow = true), for elements matching `prefix` under `pmask`; bits [0, top) of e are
// still undecided. Emits through sh.n_out.
template <int T, int CAP, bool FromRow>
__device__ void refine(Full<T, CAP>& sh, const float* row, int n, uint64_t prefix, uint64_t pmask, int top,
                       uint32_t rem, int32_t* out, int k) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  auto fetch = [&](int i) -> uint64_t { return FromRow ? compose(order_key(row[i]), i) : sh.cand[i]; };
  while (top > 0) {
    const int shift = top > 11 ? top - 11 : 0;
    const uint64_t dmask = (1ull << (top - shift)) - 1;
    clear_hist<T>(sh, kLinBins);
    for (int i = threadIdx.x; i < n; i += T) {
      const uint64_t e = fetch(i);
      if ((e & pmask) == prefix) atomicAdd(&sh.hist[(e >> shift) & dmask], 1u);
    }
    __syncthreads();
    find_bin<T>(sh, kLinBins, rem);
    const uint64_t bin = sh.bin;
    const uint32_t above = sh.above;
    const uint32_t cnt = sh.hist[bin];
    for (int base = wave * 64; base < n; base += T) {  // emit the higher bins
      const int i = base + lane;
      const uint64_t e = i < n ? fetch(i) : 0;
      const bool take = i < n && (e & pmask) == prefix && ((e >> shift) & dmask) > bin;
      const int slot = wave_append(take, &sh.n_out);
      if (slot >= 0 && slot < k) out[slot] = position(e);
    }
    rem -= above;
    prefix |= bin << shift;
    pmask |= dmask << shift;
    top = shift;
    __syncthreads();
    if (cnt == rem) {  // the whole threshold bin is selected
      for (int base = wave * 64; base < n; base += T) {
        const int i = base + lane;
        const uint64_t e = i < n ? fetch(i) : 0;
        const int slot = wave_append(i < n && (e & pmask) == prefix, &sh.n_out);
        if (slot >= 0 && slot < k) out[slot] = position(e);
      }
      __syncthreads();
      return;
    }
  }
}

// Finishes the candidate list sh.cand[0, n) (all matching prefix/pmask, bits [0, top)
// undecided): `rem` of them are selected.
template <int T, int CAP>
__device__ void finish_candidates(Full<T, CAP>& sh, int n, uint64_t prefix, uint64_t pmask, int top, uint32_t rem,
                                  int32_t* out, int k) {
  if (n <= kRankMax)
    rank_select<T, CAP>(sh, n, rem, out, k);
  else
    refine<T, CAP, false>(sh, nullptr, n, prefix, pmask, top, rem, out, k);
}

// Rows with nv <= k.
template <int T>
__device__ void select_trivial_row(const Params& p, int r, int nv) {
  int32_t* out = p.idx + (int64_t)r * p.k;
  for (int i = threadIdx.x; i < p.k; i += T) out[i] = i < nv ? i : -1;
}

// The threshold bin of a block histogram of nbins = PER * T bins: the bin B with
// above(B) < rem <= above(B) + hist[B], counting from the top bin, for rem <= the total.
// Thread t owns bins [nbins - PER*(t+1), nbins - PER*t). Each wave scans its own bins and
// publishes its total; after one barrier every wave finds the owning wave from the
// totals, rescans that wave's bins from LDS and so knows B, above(B) and hist[B]
// without a second barrier. Uses the kRedBin scratch slots.
template <int T, int PER>
__device__ __forceinline__ void threshold_bin(Core<T>& sh, uint32_t rem, uint32_t& bin, uint32_t& above,
                                              uint32_t& count) {
  constexpr int W = T / 64;
  static_assert(W <= 16, "wave totals fit one 16-lane row");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int nbins = PER * T;
  uint32_t* red = sh.red + kRedBin * W;
  auto lane_bins = [&](int w, uint32_t (&c)[PER]) {
    const int lo = nbins - PER * (w * 64 + lane + 1);
#pragma unroll
    for (int j = 0; j < PER; ++j) c[j] = sh.hist[lo + j];
  };
  uint32_t c[PER];
  lane_bins(wave, c);
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) sum += c[j];
  const uint32_t incl = wave_scan_add(sum);
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  // Wave totals in lanes 0..W-1; the owner is the first wave whose inclusive prefix
  // reaches rem.
  const uint32_t wt = lane < W ? red[lane] : 0u;
  const uint32_t wi = row16_prefix(wt);
  const uint64_t reach = __ballot(lane < W && wi >= rem);
  const int ow = __builtin_ctzll(reach);  // rem <= total: some wave reaches it
  const uint32_t ow_before = (uint32_t)__builtin_amdgcn_readlane((int)(wi - wt), ow);
  // Rescan the owner's bins (the owner's own registers would do; every wave reads LDS).
  uint32_t oc[PER];
  lane_bins(ow, oc);
  uint32_t osum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) osum += oc[j];
  const uint32_t oincl = ow_before + wave_scan_add(osum);
  const uint64_t lreach = __ballot(oincl >= rem);
  const int ol = __builtin_ctzll(lreach);
  uint32_t run = (uint32_t)__builtin_amdgcn_readlane((int)(oincl - osum), ol);
  // Walk lane ol's bins from its top bin down.
  const int olo = nbins - PER * (ow * 64 + ol + 1);
  bin = 0;
  above = 0;
  count = 0;
  bool found = false;
#pragma unroll
  for (int j = PER - 1; j >= 0; --j) {
    const uint32_t cj = (uint32_t)__builtin_amdgcn_readlane((int)oc[j], ol);
    const bool hit = !found && rem <= run + cj;
    bin = hit ? (uint32_t)(olo + j) : bin;
    above = hit ? run : above;
    count = hit ? cj : count;
    found = found || hit;
    run += cj;
  }
}

// Rows with k < nv <= PER * T: the whole select by one workgroup of T threads. Element
// i*T + t of the row sits in thread t's register i. Loads past nv are clamped onto the last
// visible element, which leaves min, max and finiteness unchanged; histogram and emit
// count only the elements below nv. When the threshold bin holds more elements than the
// candidate list (CAP), the finish refines over the row itself.
template <int T, int CAP, int PER>
__device__ void select_row(const Params& p, int r, int nv, Full<T, CAP>& sh) {
  constexpr int W = T / 64;
  const int k = p.k;
  const float* row = p.logits + (int64_t)r * p.L;
  int32_t* out = p.idx + (int64_t)r * k;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, nv * 4, 0x00020000);
  const uint32_t last = (uint32_t)(nv - 1) * 4u;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t off = min((uint32_t)threadIdx.x * 4u + (uint32_t)(i * T * 4), last);
    v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  }
  for (int i = threadIdx.x; i < kKeyBins; i += T) sh.hist[i] = 0;
  // Min / max of the visible values; a non-finite value anywhere switches to key bins
  // (the wave reports it as an infinite maximum). The maximum propagates NaN, so one test
  // of the lane's extremes finds any NaN or infinity among its values.
  float lo = __builtin_inff(), hi = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    lo = fminf(lo, v[i]);
    hi = __builtin_elementwise_maximum(hi, v[i]);
  }
  const uint64_t bad = __ballot(!__builtin_isfinite(hi) || !__builtin_isfinite(lo));
  lo = wave_scan_minmax<false>(lo);
  hi = wave_scan_minmax<true>(bad ? -__builtin_inff() : hi);
  if (lane == 63) {
    sh.red[kRedLo * W + wave] = __float_as_uint(lo);
    sh.red[kRedHi * W + wave] = __float_as_uint(bad ? __builtin_inff() : hi);
  }
  __syncthreads();
  lo = row16_minmax<false>(__uint_as_float(lane < W ? sh.red[kRedLo * W + lane] : 0x7f800000u));
  hi = row16_minmax<true>(__uint_as_float(lane < W ? sh.red[kRedHi * W + lane] : 0xff800000u));
  const bool nonfinite = !__builtin_isfinite(hi);
  // Binning: linear in the value when the visible values are finite and spread; by the
  // top key bits when some value is not finite (or the spread is not representable);
  // a single bin when all values are equal (then the refinement starts at bit 64).
  // Every form is monotone in the value, so bins are ordered like the logits.
  const float spread = hi - lo;
  const float scale = kLinBins / spread;
  const bool linear = !nonfinite && hi > lo && __builtin_isfinite(spread) && __builtin_isfinite(scale) && scale > 0.0f;
  const bool keyed = !linear && (nonfinite || hi > lo);
  const int tid = (int)threadIdx.x;
  // Lanes whose element i is below nv (one compare; recomputed where needed, which costs
  // less than holding 2 * PER scalar registers).
  auto inm = [&](int i) { return __ballot(tid < nv - i * T); };
  uint32_t bin[PER];
  if (linear) {
#pragma unroll
    for (int i = 0; i < PER; ++i) bin[i] = min((uint32_t)(kLinBins - 1), (uint32_t)((v[i] - lo) * scale));
  } else if (keyed) {
#pragma unroll
    for (int i = 0; i < PER; ++i) bin[i] = order_key(v[i]) >> (32 - kKeyBits);
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) bin[i] = 0u;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (__builtin_amdgcn_inverse_ballot_w64(inm(i))) atomicAdd(&sh.hist[bin[i]], 1u);
  __syncthreads();
  uint32_t bin0, above, cnt0;
  if (keyed)
    threshold_bin<T, kKeyBins / T>(sh, (uint32_t)k, bin0, above, cnt0);
  else
    threshold_bin<T, kLinBins / T>(sh, (uint32_t)k, bin0, above, cnt0);
  const uint32_t rem = (uint32_t)k - above;
  const bool whole = cnt0 == rem;
  // Emit the elements above the threshold bin (the whole bin too when it is all taken)
  // straight to the output row and collect the bin's own elements into the candidate
  // list. Each lane marks its visible elements in two bit masks (above the bin / in it);
  // lane and wave prefix sums of the mask populations give every lane its first output
  // and candidate slots (wave totals through LDS, one barrier). above(bin0) < k, so every
  // output slot is in range; candidate slots past CAP are dropped (the finish then
  // refines over the row).
  const uint32_t thr = whole ? bin0 : bin0 + 1;
  const int vis = min(PER, (nv - tid + T - 1) / T);  // elements i < vis are visible
  uint32_t ma = 0, mb = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    ma |= (bin[i] >= thr ? 1u : 0u) << i;
    mb |= (bin[i] == bin0 ? 1u : 0u) << i;
  }
  static_assert(PER <= 32, "a lane's element masks fit 32 bits");
  const uint32_t vmask = vis >= 32 ? ~0u : (1u << max(vis, 0)) - 1u;
  ma &= vmask;
  mb = whole ? 0u : (mb & vmask);
  const uint32_t la = (uint32_t)__popc(ma), lb = (uint32_t)__popc(mb);
  const uint32_t ia = wave_scan_add(la), ib = wave_scan_add(lb);
  if (lane == 63) {
    sh.red[kRedEmit * W + wave] = ia;
    sh.red[kRedCand * W + wave] = ib;
  }
  if (threadIdx.x == 0) sh.n_out = above;  // the finish appends after the emitted elements
  __syncthreads();
  const uint32_t ca = lane < W ? sh.red[kRedEmit * W + lane] : 0u;
  const uint32_t cb = lane < W ? sh.red[kRedCand * W + lane] : 0u;
  uint32_t oa = (uint32_t)__builtin_amdgcn_readlane((int)(row16_prefix(ca) - ca), wave) + ia - la;
  uint32_t ob = (uint32_t)__builtin_amdgcn_readlane((int)(row16_prefix(cb) - cb), wave) + ib - lb;
  while (ma) {
    const int i = __builtin_ctz(ma);
    ma &= ma - 1u;
    out[oa++] = i * T + tid;
  }
  while (mb) {  // the threshold bin's elements (few): their keys are read again
    const int i = __builtin_ctz(mb);
    mb &= mb - 1u;
    const int t = i * T + tid;
    if (ob < (uint32_t)CAP) sh.cand[ob] = compose(order_key(row[t]), t);
    ++ob;
  }
  if (!whole) {
    __syncthreads();  // the candidate list is complete
    // Key bins fix the top 12 bits of e; linear or single bins fix none.
    const uint64_t prefix = keyed ? (uint64_t)bin0 << (64 - kKeyBits) : 0ull;
    const uint64_t pmask = keyed ? (uint64_t)(kKeyBins - 1) << (64 - kKeyBits) : 0ull;
    const int top = keyed ? 64 - kKeyBits : 64;
    if (PER * T <= CAP || cnt0 <= (uint32_t)CAP) {  // uniform
      finish_candidates<T, CAP>(sh, (int)cnt0, prefix, pmask, top, rem, out, k);
    } else if (keyed) {
      refine<T, CAP, true>(sh, row, nv, prefix, pmask, top, rem, out, k);
    } else {
      // Linear or single bins are not key-bit prefixes: select over the whole row again
      // by radix digits of e from the top, rewriting every output slot (the barrier
      // orders these stores after the ones above).
      if (threadIdx.x == 0) sh.n_out = 0;
      __syncthreads();
      refine<T, CAP, true>(sh, row, nv, 0ull, 0ull, 64, (uint32_t)k, out, k);
    }
  }
}

// Rows with nv = k + 1 (the reproducer's shape: ctx = 2049 with k = 2048): every visible
// position but the one with the smallest order key e is selected. One block minimum of e
// (a butterfly over each wave, one barrier) finds it, and the other positions are written
// in position order, position t to slot t or t - 1: no histogram, threshold or ranking.
// Used by the short-row kernel (max_model_len <= 8192: decode bs=1 at ctx 2049 goes
// 5.05 -> 4.1 us); the wide and chunked kernels keep their code as it is, which the extra
// branch made slower (their register budgets are tighter).
template <int T, int CAP>
__device__ void drop_min_row(const Params& p, int r, int nv, Full<T, CAP>& sh) {
  constexpr int W = T / 64;
  constexpr int PER = 4;
  static_assert(PER * T > kMaxK, "a row of k + 1 elements fits PER values per thread");
  const float* row = p.logits + (int64_t)r * p.L;
  int32_t* out = p.idx + (int64_t)r * p.k;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = (int)threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, nv * 4, 0x00020000);
  const uint32_t last = (uint32_t)(nv - 1) * 4u;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t off = min((uint32_t)tid * 4u + (uint32_t)(i * T * 4), last);
    v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  }
  uint64_t mn = ~0ull;  // larger than every composed key
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int t = i * T + tid;
    const uint64_t e = compose(order_key(v[i]), t);
    mn = (t < nv && e < mn) ? e : mn;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)mn, o);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(mn >> 32), o);
    const uint64_t x = ((uint64_t)hi << 32) | lo;
    mn = x < mn ? x : mn;
  }
  if (lane == 0) {
    sh.red[kRedLo * W + wave] = (uint32_t)(mn >> 32);
    sh.red[kRedHi * W + wave] = (uint32_t)mn;
  }
  __syncthreads();
  uint64_t bm = ~0ull;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const uint64_t x = ((uint64_t)sh.red[kRedLo * W + w] << 32) | sh.red[kRedHi * W + w];
    bm = x < bm ? x : bm;
  }
  const int px = position(bm);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int t = i * T + tid;
    if (t < nv && t != px) out[t - (t > px ? 1 : 0)] = t;
  }
}

// Whole-row select with the fewest values per thread that hold the row: a phase costs
// about one instruction per value a thread holds, and rows shorter than the kernel's
// longest (clamped loads past nv only repeat the last value) need not pay for it. MAXPER is
// the longest form a kernel needs.
template <int T, int CAP, int MAXPER, bool DROP_MIN = false>
__device__ void select_row_fit(const Params& p, int r, int nv, Full<T, CAP>& sh) {
  if (DROP_MIN && nv == p.k + 1) {  // uniform, like every branch here
    drop_min_row<T, CAP>(p, r, nv, sh);
  } else if (nv <= 4 * T) {
    select_row<T, CAP, 4>(p, r, nv, sh);
  } else if (MAXPER <= 8 || nv <= 8 * T) {
    select_row<T, CAP, 8>(p, r, nv, sh);
  } else if constexpr (MAXPER > 8) {
    if (nv <= 16 * T)
      select_row<T, CAP, 16>(p, r, nv, sh);
    else
      select_row<T, CAP, MAXPER>(p, r, nv, sh);
  }
}

// max_model_len <= kRowLen: one launch, workgroup r selects row r, no workspace.
__global__ __launch_bounds__(kRowThreads) void topk_rows_kernel(Params p) {
  __shared__ Full<kRowThreads, kRowCap> sh;
  const int r = blockIdx.x;
  const int nv = visible(p, r);
  if (nv <= p.k) select_trivial_row<kRowThreads>(p, r, nv);
  else select_row_fit<kRowThreads, kRowCap, kPer, true>(p, r, nv, sh);
}

// kRowLen < max_model_len <= kWideLen: one launch, workgroup r selects row r with 32
// values per thread, no workspace. (Splitting such rows over several workgroups measured
// slower: the synchronisation between them costs more than the row's instructions.)
__global__ __launch_bounds__(kRowThreads) void topk_rows_wide_kernel(Params p) {
  __shared__ Full<kRowThreads, kRowCap> sh;
  const int r = blockIdx.x;
  const int nv = visible(p, r);
  if (nv <= p.k) select_trivial_row<kRowThreads>(p, r, nv);
  else select_row_fit<kRowThreads, kRowCap, kWidePer>(p, r, nv, sh);
}

// ---- Chunked mode (max_model_len > kWideLen): one launch, no schedule pass.
// Rows with k < nv <= kWideLen are one work item each (a whole-row select); rows longer
// than that are cut into kChunk-element chunks, one item each. The items form one list,
// heaviest first (the chunk items row by row, then the whole rows by cost class), dealt to
// the workgroups in a snake; every workgroup derives the list from context_lens itself.
// The grid is as many workgroups as fit on the GPU at once (one per CU).
//   Phase 1, no waiting: for each of its chunks of a long row, a workgroup adds the
//   chunk's 12-bit key histogram into the row's histogram (global atomics) and then counts
//   the chunk.
//   Phase 2: for each of its chunks of a several-chunk row, it waits until the row's count
//   shows every chunk's histogram, takes the threshold bin from the row's histogram, emits
//   the chunk's elements above it and collects those in it into the row's candidate list;
//   the workgroup that counts a row's last chunk finishes the row's candidates and returns
//   the row's workspace to zero, so the next call needs no clearing pass or memset.
//   Phase 3, no waiting: it selects its whole rows and writes its trivial rows. Coming
//   after the splits, the row finishes (which the snake does not weigh) run while other
//   workgroups still select whole rows, instead of after the heaviest of them.
// A wait only ever waits for phase-1 work, and phase 1 never waits, so with every
// workgroup resident the waits end; the wait is bounded all the same, and a workgroup whose
// wait runs out builds the row's histogram from the row itself (the same counts, so the
// same threshold as every other chunk of the row: slower, not different).
// Data crosses workgroups on different XCDs, whose L2 caches are not coherent with each
// other within a kernel: histograms and counters only through atomics, candidates through
// agent-scope stores, and the readers use agent-scope loads (both bypass the non-coherent
// L2 state); a writer waits for its memory operations to complete before it counts. No
// device-scope fence is used (each costs microseconds on gfx950).

constexpr int kCT = kChunkThreads;

__device__ __forceinline__ uint64_t load_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Row counters in the workspace: chunk histograms added, chunks split, positions
// emitted, candidates collected.
enum { kCntHist = 0, kCntSplit = 1, kCntEmit = 2, kCntCand = 3 };

// Polls of a row's histogram count before a workgroup builds the histogram itself
// (~0.5 us each, with a short sleep between polls).
constexpr int kWaitPolls = 1 << 16;

// Chunk items of a row with nv visible positions: its chunk count (at least 5) when it is
// longer than a workgroup selects whole, else 0.
__device__ __forceinline__ uint32_t chunks_of(const Params& p, int nv) {
  return nv > kWideLen ? (uint32_t)((nv + kChunk - 1) / kChunk) : 0u;
}

// Rows selected whole (k < nv <= kWideLen) fall in four cost classes, heaviest first: the
// values per thread select_row_fit gives them (32, 16, 8, 4), each costing about twice the
// next. -1 for every other row.
constexpr int kWholeClasses = 4;
__device__ __forceinline__ int whole_class(const Params& p, int nv) {
  if (nv <= p.k || nv > kWideLen) return -1;
  return nv > 16 * kCT ? 0 : nv > 8 * kCT ? 1 : nv > 4 * kCT ? 2 : 3;
}

// Walks the chunk items of a call in increasing order, rows kCT at a time: thread t holds
// row base + t, its visible count, its chunk count and the exclusive prefix of the counts
// in the block. With every row in one block (rows <= kCT) the visible counts, once read,
// are kept (held): later passes and other numberings reuse them instead of reading
// context_lens again.
struct Cursor {
  int base = -kCT;
  uint32_t first = 0, total = 0;  // items before the block, items in it
  uint32_t excl = 0, nch = 0;
  int nv = 0;
  bool held = false;  // nv is row threadIdx.x's visible count (all rows in one block)
};

// A cursor at the start of another numbering, keeping the visible counts `from` holds.
__device__ __forceinline__ Cursor restart(const Cursor& from) {
  Cursor c;
  c.nv = from.nv;
  c.held = from.held;
  return c;
}

struct Item {
  int r, c, nv, nch;
};

// Back to the first item. With all rows in one block the block's scan is kept.
__device__ __forceinline__ void rewind(const Params& p, Cursor& cu) {
  if (p.rows <= kCT && cu.base >= 0) {
    cu.base = 0;
    cu.first = 0;
  } else {
    cu.base = -kCT;
    cu.first = cu.total = 0;
  }
}

// Finds item `item` of the numbering in which row r holds count(nv_r) consecutive items;
// returns false past the last one. Every thread calls it with the same item, and the
// items of successive calls (after a rewind) do not decrease.
template <typename Count>
__device__ bool locate(const Params& p, Cursor& cu, Core<kCT>& sh, uint32_t item, Item& it, Count count) {
  __syncthreads();  // the previous item's readers of sh.loc and of the scan scratch are done
  while (item >= cu.first + cu.total) {  // uniform
    cu.first += cu.total;
    cu.base += kCT;
    if (cu.base >= p.rows) return false;
    const int row = cu.base + (int)threadIdx.x;
    if (!cu.held) cu.nv = row < p.rows ? visible(p, row) : 0;  // uniform
    cu.held = p.rows <= kCT;
    cu.nch = count(cu.nv);
    cu.excl = block_exclusive_scan<kCT>(cu.nch, sh, kRedLoc, cu.total);
    __syncthreads();  // every thread has read the scan scratch
  }
  // No global load below: a wait for one would also wait for the caller's loads in flight.
  const uint32_t li = item - cu.first;
  if (li >= cu.excl && li < cu.excl + cu.nch) {  // exactly one thread
    sh.loc[0] = cu.base + (int)threadIdx.x;
    sh.loc[1] = (int)(li - cu.excl);
    sh.loc[2] = cu.nv;
    sh.loc[3] = (int)cu.nch;
  }
  __syncthreads();
  it.r = sh.loc[0];
  it.c = sh.loc[1];
  it.nv = sh.loc[2];
  it.nch = sh.loc[3];
  return true;
}

// Issues the loads of an item's chunk: element i*kCT + threadIdx.x of
// [c*kChunk, c*kChunk + kChunk) in v[i], loads past the row's visible end clamped onto its
// last visible element. Nothing waits for them here.
__device__ __forceinline__ void fetch_chunk(const Params& p, const Item& it, float (&v)[kChunkPer]) {
  const int base = it.c * kChunk;
  const int n = min(kChunk, it.nv - base);  // >= 1: chunks start below nv
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p.logits + (int64_t)it.r * p.L + base), 0, n * 4, 0x00020000);
  const uint32_t last = (uint32_t)(n - 1) * 4u;
#pragma unroll
  for (int i = 0; i < kChunkPer; ++i) {
    const uint32_t off = min((uint32_t)threadIdx.x * 4u + (uint32_t)(i * kCT * 4), last);
    v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  }
}

// Adds the 12-bit key histogram of the chunk in v (its visible elements) into sh.hist;
// the caller synchronises before reading it.
__device__ __forceinline__ void count_chunk(Core<kCT>& sh, const Item& it, const float (&v)[kChunkPer]) {
  const int n = it.nv - it.c * kChunk;
  const int tid = (int)threadIdx.x;
#pragma unroll
  for (int i = 0; i < kChunkPer; ++i)
    if (__builtin_amdgcn_inverse_ballot_w64(__ballot(tid < n - i * kCT)))
      atomicAdd(&sh.hist[order_key(v[i]) >> (32 - kKeyBits)], 1u);
}

// The row's whole histogram built by this workgroup alone, into sh.hist.
__device__ void build_row_hist(const Params& p, Core<kCT>& sh, const Item& it) {
  clear_hist<kCT>(sh, kKeyBins);
  for (int c = 0; c < it.nch; ++c) {
    const Item ci = {it.r, c, it.nv, it.nch};
    float v[kChunkPer];
    fetch_chunk(p, ci, v);
    count_chunk(sh, ci, v);
  }
  __syncthreads();
}

using ChunkFull = Full<kCT, kChunkCap>;

// Finishes row it.r after its last chunk: selects `k - above` of the threshold bin's
// candidates (or refines over the row when the bin held more than the list) and returns
// the row's workspace (histogram, counters, the candidate entries written) to zero.
__device__ void finish_row(const Params& p, ChunkFull& sh, const Item& it, uint32_t bin0, uint32_t above,
                           uint32_t cnt0) {
  const int k = p.k;
  const uint32_t rem = (uint32_t)k - above;
  int32_t* out = p.idx + (int64_t)it.r * k;
  if (cnt0 != rem) {  // uniform: the bin is not taken whole
    if (threadIdx.x == 0) sh.n_out = above;  // the chunks emitted exactly `above`
    const uint64_t prefix = (uint64_t)bin0 << (64 - kKeyBits);
    const uint64_t pmask = (uint64_t)(kKeyBins - 1) << (64 - kKeyBits);
    uint64_t* cand = p.cand + (int64_t)it.r * kChunkCap;
    if (cnt0 <= (uint32_t)kChunkCap) {
      for (int i = threadIdx.x; i < (int)cnt0; i += kCT) {
        sh.cand[i] = load_agent(cand + i);
        cand[i] = 0;  // the list is read once; the next call finds it zero
      }
      __syncthreads();
      finish_candidates<kCT, kChunkCap>(sh, (int)cnt0, prefix, pmask, 64 - kKeyBits, rem, out, k);
    } else {  // the chunks stored the first kChunkCap candidates
      for (int i = threadIdx.x; i < kChunkCap; i += kCT) cand[i] = 0;
      __syncthreads();
      refine<kCT, kChunkCap, true>(sh, p.logits + (int64_t)it.r * p.L, it.nv, prefix, pmask, 64 - kKeyBits, rem,
                                   out, k);
    }
  }
  uint4* gh = reinterpret_cast<uint4*>(p.hist + (int64_t)it.r * kKeyBins);
  for (int i = threadIdx.x; i < kKeyBins / 4; i += kCT) gh[i] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x < kCoarseBins) p.coarse[(int64_t)it.r * kCoarseBins + threadIdx.x] = 0u;
  if (threadIdx.x < 4) store_agent(p.counters + 4 * (int64_t)it.r + threadIdx.x, 0u);
}

// Phase 2 for one chunk whose values are in v: wait for the row's histogram, threshold
// bin, emission and candidates, count; the last chunk of the row finishes it.
__device__ void split_chunk(const Params& p, ChunkFull& sh, const Item& it, const float (&v)[kChunkPer]) {
  constexpr int W = kCT / 64;
  const int k = p.k;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t* cnt = p.counters + 4 * (int64_t)it.r;
  // Wait (thread 0) until every chunk of the row has added its histogram.
  if (tid == 0) {
    int polls = 0;
    while (load_agent(&cnt[kCntHist]) < (uint32_t)it.nch && ++polls < kWaitPolls) __builtin_amdgcn_s_sleep(2);
    sh.last = polls < kWaitPolls ? 1u : 0u;
  }
  __syncthreads();
  uint32_t bin0, above, cnt0;
  if (sh.last) {  // uniform
    // The threshold bin from the row's coarse counts, then from the 64 key bins of the
    // coarse bin holding it: wave 0, two loads of 256 bytes (lane l reads the l-th bin from
    // the top), no scan of the 4096 bins. The row holds more than k visible elements, so
    // both searches end inside their bins.
    if (wave == 0) {
      const uint32_t cc = load_agent(p.coarse + (int64_t)it.r * kCoarseBins + (kCoarseBins - 1 - lane));
      const uint32_t cincl = wave_scan_add(cc);
      const int ol = __builtin_ctzll(__ballot(cincl >= (uint32_t)k));
      const uint32_t above_c = (uint32_t)__builtin_amdgcn_readlane((int)(cincl - cc), ol);
      const int cb = kCoarseBins - 1 - ol;
      const uint32_t fc = load_agent(p.hist + (int64_t)it.r * kKeyBins + cb * 64 + (63 - lane));
      const uint32_t fincl = wave_scan_add(fc);
      const int fl = __builtin_ctzll(__ballot(above_c + fincl >= (uint32_t)k));
      const uint32_t above_f = (uint32_t)__builtin_amdgcn_readlane((int)(fincl - fc), fl);
      const uint32_t count_f = (uint32_t)__builtin_amdgcn_readlane((int)fc, fl);
      if (lane == 0) {
        sh.bin = (uint32_t)(cb * 64 + 63 - fl);
        sh.above = above_c + above_f;
        sh.count = count_f;
      }
    }
    __syncthreads();
    bin0 = sh.bin;
    above = sh.above;
    cnt0 = sh.count;
  } else {
    build_row_hist(p, sh, it);
    threshold_bin<kCT, kKeyBins / kCT>(sh, (uint32_t)k, bin0, above, cnt0);
  }
  const bool whole = cnt0 == (uint32_t)k - above;
  // Elements above the threshold bin (the whole bin too when all of it is taken) go to
  // the output, the bin's own elements to the row's candidate list; slots from one pair
  // of global atomics per workgroup, a prefix over the waves' counts and each lane's
  // prefix over the populations of its two element masks.
  const uint32_t thr = whole ? bin0 : bin0 + 1;
  const int base = it.c * kChunk;
  const int vis = min(kChunkPer, (it.nv - base - tid + kCT - 1) / kCT);  // visible elements
  uint32_t ma = 0, mb = 0;
#pragma unroll
  for (int i = 0; i < kChunkPer; ++i) {
    const uint32_t d = order_key(v[i]) >> (32 - kKeyBits);
    ma |= (d >= thr ? 1u : 0u) << i;
    mb |= (d == bin0 ? 1u : 0u) << i;
  }
  static_assert(kChunkPer < 32, "a lane's element masks fit 32 bits");
  const uint32_t vmask = (1u << max(vis, 0)) - 1u;
  ma &= vmask;
  mb = whole ? 0u : (mb & vmask);
  const uint32_t la = (uint32_t)__popc(ma), lb = (uint32_t)__popc(mb);
  const uint32_t la_incl = wave_scan_add(la), lb_incl = wave_scan_add(lb);
  if (lane == 63) {
    sh.red[kRedEmit * W + wave] = la_incl;
    sh.red[kRedCand * W + wave] = lb_incl;
  }
  __syncthreads();
  const uint32_t ca = lane < W ? sh.red[kRedEmit * W + lane] : 0u;
  const uint32_t cb = lane < W ? sh.red[kRedCand * W + lane] : 0u;
  const uint32_t ia = row16_prefix(ca), ib = row16_prefix(cb);
  if (tid == 0) {
    const uint32_t ta = (uint32_t)__builtin_amdgcn_readlane((int)ia, W - 1);
    const uint32_t tb = (uint32_t)__builtin_amdgcn_readlane((int)ib, W - 1);
    sh.base_a = ta ? atomicAdd(&cnt[kCntEmit], ta) : 0u;
    sh.base_b = tb ? atomicAdd(&cnt[kCntCand], tb) : 0u;
  }
  __syncthreads();
  uint32_t oa = sh.base_a + (uint32_t)__builtin_amdgcn_readlane((int)(ia - ca), wave) + la_incl - la;
  uint32_t ob = sh.base_b + (uint32_t)__builtin_amdgcn_readlane((int)(ib - cb), wave) + lb_incl - lb;
  int32_t* out = p.idx + (int64_t)it.r * k;
  uint64_t* cand = p.cand + (int64_t)it.r * kChunkCap;
  // Each element is taken from the registers (unrolled, predicated), none is read again.
#pragma unroll
  for (int i = 0; i < kChunkPer; ++i) {
    if ((mb >> i) & 1u) {
      if (ob < (uint32_t)kChunkCap) store_agent(cand + ob, compose(order_key(v[i]), base + i * kCT + tid));
      ++ob;
    }
  }
#pragma unroll
  for (int i = 0; i < kChunkPer; ++i) {
    if ((ma >> i) & 1u) {
      if (oa < (uint32_t)k) out[oa] = base + i * kCT + tid;
      ++oa;
    }
  }
  // Count the chunk once every store of it has completed; the workgroup that counts the
  // row's last chunk finishes the row.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) sh.last = atomicAdd(&cnt[kCntSplit], 1u) + 1u == (uint32_t)it.nch ? 1u : 0u;
  __syncthreads();
  if (sh.last) finish_row(p, sh, it, bin0, above, cnt0);  // uniform
}

// Items of the call: chunk items, then the whole rows of each cost class (one reduction
// pass over the rows, one barrier per block of rows; the per-class counts of one block
// fit 16 bits). When every row is in one block that the chunk cursor has scanned, the
// visible counts are the cursor's and nothing is loaded.
struct ItemTotals {
  uint32_t chunks;
  uint32_t whole[kWholeClasses];
};
__device__ ItemTotals item_totals(const Params& p, Core<kCT>& sh, const Cursor& cu) {
  constexpr int W = kCT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const bool cached = cu.held;  // uniform
  ItemTotals t = {0u, {0u, 0u, 0u, 0u}};
  for (int base = 0; base < p.rows; base += kCT) {
    const int row = base + (int)threadIdx.x;
    const int nv = cached ? cu.nv : (row < p.rows ? visible(p, row) : 0);
    const int cls = whole_class(p, nv);
    const uint32_t a = wave_scan_add(chunks_of(p, nv));
    const uint32_t b = wave_scan_add((cls == 0 ? 1u : 0u) | (cls == 1 ? 1u << 16 : 0u));
    const uint32_t c = wave_scan_add((cls == 2 ? 1u : 0u) | (cls == 3 ? 1u << 16 : 0u));
    if (base > 0) __syncthreads();  // the previous block's readers of these slots are done
    if (lane == 63) {
      sh.red[kRedLo * W + wave] = a;
      sh.red[kRedHi * W + wave] = b;
      sh.red[kRedBad * W + wave] = c;
    }
    __syncthreads();
    uint32_t ta = 0, tb = 0, tc = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      ta += sh.red[kRedLo * W + w];
      tb += sh.red[kRedHi * W + w];
      tc += sh.red[kRedBad * W + w];
    }
    t.chunks += ta;
    t.whole[0] += tb & 0xFFFFu;
    t.whole[1] += tb >> 16;
    t.whole[2] += tc & 0xFFFFu;
    t.whole[3] += tc >> 16;
  }
  // No barrier here: the next writers of these scratch slots (a row select) run after
  // locate()'s barrier.
  return t;
}

__global__ __launch_bounds__(kCT) void topk_chunked_kernel(Params p) {
  __shared__ ChunkFull sh;
  const int tid = (int)threadIdx.x;
  // Work is dealt out in one list, heaviest items first: chunk items (row by row), then
  // whole rows class by class; position j of the list goes to workgroup j mod G on even
  // rounds j / G and to G - 1 - j mod G on odd ones (a snake), so a workgroup that takes a
  // heavy item early takes a light one late. Dealing items row by row instead put up to
  // three long whole rows on one workgroup (mixed batch: 36 us of top-k on the slowest
  // workgroup against a median of 20).
  const uint32_t G = gridDim.x, g = blockIdx.x;
  auto position = [&](uint32_t m) -> uint64_t { return (uint64_t)m * G + ((m & 1u) ? G - 1u - g : g); };
  auto chunk_count = [&](int nv) { return chunks_of(p, nv); };
  Cursor cu;
  Item it;
  // Phase 1: histograms of this workgroup's chunks of several-chunk rows (the chunk items
  // come first in the list, so the numbering of chunk items alone finds them).
  for (uint32_t m = 0;; ++m) {
    if (!locate(p, cu, sh, (uint32_t)min<uint64_t>(position(m), 0xFFFFFFFFu), it, chunk_count)) break;
    float v[kChunkPer];
    fetch_chunk(p, it, v);
    for (int i = tid; i < kKeyBins; i += kCT) sh.hist[i] = 0;
    __syncthreads();
    count_chunk(sh, it, v);
    __syncthreads();
    uint32_t* gh = p.hist + (int64_t)it.r * kKeyBins;
    uint32_t* gc = p.coarse + (int64_t)it.r * kCoarseBins;
    static_assert(kKeyBins / kCoarseBins == 64 && kKeyBins % kCT == 0, "a wave's 64 lanes hold one coarse bin's key bins");
    for (int i = tid; i < kKeyBins; i += kCT) {
      const uint32_t c = sh.hist[i];
      if (c) atomicAdd(&gh[i], c);
      // The 64 lanes of a wave hold the 64 key bins of coarse bin i / 64.
      const uint32_t cs = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_add(c), 63);
      if ((tid & 63) == 0 && cs) atomicAdd(&gc[i >> 6], cs);
    }
    // Count the chunk once its histogram has reached the row's (atomics complete).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) atomicAdd(&p.counters[4 * (int64_t)it.r + kCntHist], 1u);
  }
  // The item totals, after the chunks are counted (before any wait on other workgroups).
  const ItemTotals tot = item_totals(p, sh, cu);
  // Phase 2: split this workgroup's chunks of several-chunk rows. Each chunk is loaded
  // again (mostly from cache) before the wait for its row's histogram, so the load and
  // the wait overlap.
  rewind(p, cu);
  for (uint32_t m = 0;; ++m) {
    const uint64_t j = position(m);
    if (j >= tot.chunks || !locate(p, cu, sh, (uint32_t)j, it, chunk_count)) break;
    float v[kChunkPer];
    fetch_chunk(p, it, v);
    split_chunk(p, sh, it, v);
  }
  // Phase 3: whole rows, class by class (their list positions follow the chunk items);
  // trivial rows.
  {
    const uint32_t nwhole = tot.whole[0] + tot.whole[1] + tot.whole[2] + tot.whole[3];
    Cursor cw;
    int cls_at = -1;  // class the cursor numbers
    for (uint32_t m = 0;; ++m) {
      const uint64_t j = position(m);
      if (j < tot.chunks) continue;
      uint32_t w = (uint32_t)(j - tot.chunks);
      if (w >= nwhole) break;
      // Class of list position w (w < nwhole), without indexing the totals (which would
      // put them in memory).
      int cls = 0;
      if (w >= tot.whole[0]) {
        w -= tot.whole[0];
        cls = 1;
        if (w >= tot.whole[1]) {
          w -= tot.whole[1];
          cls = 2;
          if (w >= tot.whole[2]) {
            w -= tot.whole[2];
            cls = 3;
          }
        }
      }
      if (cls != cls_at) {  // a new numbering: start over
        cw = restart(cu);
        cls_at = cls;
      }
      if (!locate(p, cw, sh, w, it, [&](int nv) { return whole_class(p, nv) == cls ? 1u : 0u; })) break;
      select_row_fit<kCT, kChunkCap, kWidePer>(p, it.r, it.nv, sh);
    }
  }
  for (int r = blockIdx.x; r < p.rows; r += gridDim.x) {
    const int nv = visible(p, r);
    if (nv <= p.k) select_trivial_row<kCT>(p, r, nv);
  }
}

// Workspace layout (chunked mode): counters [rows][4] u32 | hist [rows][kKeyBins] u32 |
// coarse [rows][kCoarseBins] u32 | cand [rows][kChunkCap] u64; every region 16-byte aligned
// (the histograms are cleared as uint4; the workspace base is 16-byte aligned).
struct Layout {
  size_t counters, hist, coarse, cand, total;
};

Layout layout(int64_t rows) {
  static_assert((8 * kChunkCap) % 16 == 0, "candidate lists keep 16-byte alignment");
  Layout l;
  l.counters = 0;
  l.hist = (size_t)16 * rows;
  l.coarse = l.hist + (size_t)4 * kKeyBins * rows;
  l.cand = l.coarse + (size_t)4 * kCoarseBins * rows;
  l.total = l.cand + (size_t)8 * kChunkCap * rows;
  return l;
}

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

// Chunked-kernel workgroups one CU holds at once (read once per device).
int chunked_per_cu() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, topk_chunked_kernel, kCT, 0) != hipSuccess || n <= 0) n = 1;
    __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}

// Scratch of the no-allocation entry point: one copy per device, held until the process
// ends. Host code never uses this name as an address (on the host it is a stand-in, not
// device memory): topk_static_scratch() looks the device address up once per device.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

}  // namespace

size_t topk_static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t topk_static_scratch(void** ptr) {
  static std::atomic<void*> per_device[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = per_device[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    per_device[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

size_t topk_workspace_bytes(int64_t rows, int32_t max_model_len) {
  if (max_model_len <= kWideLen) return 0;
  return layout(rows).total;
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.batch * a.next_n;
  if (rows > 0x7fffffff) return hipErrorInvalidConfiguration;
  Params p = {};
  p.logits = a.logits;
  p.ctx_lens = a.ctx_lens;
  p.idx = a.idx;
  p.rows = (int32_t)rows;
  p.N = a.next_n;
  p.W = a.token_capacity;
  p.L = a.max_model_len;
  p.k = a.k;
  if (a.max_model_len <= kRowLen) {  // every row fits one workgroup, 8 values per thread
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, stream, p);
    return hipGetLastError();
  }
  if (a.max_model_len <= kWideLen) {  // every row fits one workgroup, 32 values per thread
    hipLaunchKernelGGL(topk_rows_wide_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, stream, p);
    return hipGetLastError();
  }
  const Layout l = layout(rows);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  p.counters = reinterpret_cast<uint32_t*>(ws + l.counters);
  p.hist = reinterpret_cast<uint32_t*>(ws + l.hist);
  p.coarse = reinterpret_cast<uint32_t*>(ws + l.coarse);
  p.cand = reinterpret_cast<uint64_t*>(ws + l.cand);
  // Every workgroup resident at once (the waits assume it; see above), and no more than
  // the chunks can need (every row at its longest).
  const int64_t cap = a.max_model_len < a.token_capacity ? a.max_model_len : a.token_capacity;
  const int64_t items = rows * ((cap + kChunk - 1) / kChunk);
  const int64_t resident = (int64_t)chunked_per_cu() * compute_units();
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(resident, std::max(items, rows)));
  hipLaunchKernelGGL(topk_chunked_kernel, dim3(grid), dim3(kCT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mqa
