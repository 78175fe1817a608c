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
// Row classes (nv known only on the device):
//   trivial  nv <= k: every visible position, no logits read.
//   whole    k < nv <= 8192 (8 logits per thread) or <= 32768 (32 per thread): one
//            workgroup of 1024 threads owns the row, its logits in registers. A block
//            min/max reduction sets 2048 first-level bins linear in the value (monotone,
//            so bins are ordered like the logits; rows holding a non-finite value use the
//            top 12 key bits instead, constant rows a single bin). An LDS histogram and a
//            scan from the top find the bin holding the k-th element (every wave finishes
//            the search itself after one barrier). Each lane marks its elements above
//            that bin and in it in two bit masks; a lane scan of the mask populations and
//            the 16 wave totals (one barrier) give every lane its first slots, and each
//            lane walks its set bits: positions above the bin go straight to the output
//            row, the bin's own elements to an LDS candidate list. A small list is finished by
//            counting, for each candidate, the candidates above it (the count is the
//            slot); a large one by further 11-bit radix digits of e, or over the whole
//            row if the bin holds more than the list (kCap). One CU serves a row, so the
//            time is set by the instructions each wave issues: per-element work is kept
//            to a few vector instructions (buffer loads clamped onto the last visible
//            element, lane masks from one compare each, a NaN-propagating maximum for the
//            finiteness test, emission by walking set bits).
//   long     nv > 8192 when max_model_len > 32768: 8192-element chunks. A
//            schedule kernel lists the rows of each class and the long rows' chunks and
//            clears their histograms; persistent kernels then add each chunk's 12-bit key
//            histogram into the row's global histogram (the next chunk's loads in flight
//            meanwhile), emit each chunk's elements above the threshold bin (slots from
//            one pair of global atomics per workgroup, a prefix over the waves' counts
//            and the lanes' mask populations) and collect its threshold-bin elements, and
//            finish each row's candidates in LDS. If the threshold bin holds more than
//            kCap elements (extreme ties, e.g. a constant row) the finish refines over
//            the whole row from global memory: slower, same result. The finishing pass's
//            spare workgroups select the call's rows of at most 8192 and the trivial rows
//            (selecting rows up to 32768 whole there was slower: the wide select in the
//            same kernel costs its other paths, and the rows queue behind other items).
// When max_model_len <= 8192 (8 per thread) or <= 32768 (32 per thread) no row is long:
// one launch, one workgroup per row, no workspace.
#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.h"

namespace mqa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 8;                   // logits per thread per chunk
constexpr int kChunk = kThreads * kPer;   // 8192
constexpr int kWidePer = 32;              // logits per thread of a whole-row select
constexpr int kWide = kThreads * kWidePer;  // 32768: rows one workgroup selects alone
constexpr int kLinBins = 2048;            // first level of a short row (linear bins)
constexpr int kKeyBits = 12;              // first level of a long row (top key bits)
constexpr int kKeyBins = 1 << kKeyBits;   // 4096
constexpr int kCap = 8192;                // LDS candidate slots (64 KB)
constexpr int kRankMax = 256;             // candidate lists up to this size are ranked

enum { kMetaLong = 0, kMetaChunks = 1, kMetaShort = 2, kMetaTrivial = 3 };

struct Params {
  const float* logits;
  const int32_t* ctx_lens;
  int32_t* idx;
  // Workspace (long-row mode only; null otherwise).
  uint32_t* meta;         // [8]: long rows, long chunks, short rows, trivial rows
  uint32_t* long_rows;    // [rows] row id of each long-row slot
  uint32_t* short_rows;   // [rows]
  uint32_t* triv_rows;    // [rows]
  uint32_t* chunk_items;  // [rows * nchunk_max][2]: long-row slot, chunk
  uint32_t* counters;     // [rows][2] per slot: emitted, candidates
  uint32_t* hist;         // [rows][kKeyBins] per slot
  uint64_t* cand;         // [rows][kCap] per slot
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

// Per-wave scratch slots, one region per use so that consecutive block operations need
// no barrier between them for the scratch itself.
enum { kRedLo = 0, kRedHi = kWaves, kRedBad = 2 * kWaves, kRedBin = 3 * kWaves, kRedEmit = 4 * kWaves,
       kRedCand = 5 * kWaves, kRedSize = 6 * kWaves };

struct Core {
  uint32_t hist[kKeyBins];
  uint32_t red[kRedSize];
  uint32_t n_out, bin, above, base_a, base_b;
};

struct Full : Core {
  uint64_t cand[kCap];
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

// Exclusive prefix sum over the 1024 threads in thread order, through the kWaves scratch
// slots at `slot`. Also returns the block total. One barrier.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, Core& sh, int slot, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_scan_add(v);
  if (lane == 63) sh.red[slot + wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = sh.red[slot + w];
    before += w < wave ? t : 0u;
    all += t;
  }
  total = all;
  return before + incl - v;
}

// Finds the bin B (scanning from the top of nbins) with above(B) < rem <= above(B) +
// hist[B]; leaves B in sh.bin and above(B) in sh.above. All threads must call it.
__device__ void find_bin(Core& sh, int nbins, uint32_t rem) {
  const int per = nbins / kThreads;  // 2 or 4
  const int top = nbins - 1 - per * (int)threadIdx.x;
  uint32_t cnt[kKeyBins / kThreads] = {}, sum = 0;
  for (int i = 0; i < per; ++i) {
    cnt[i] = sh.hist[top - i];
    sum += cnt[i];
  }
  if (threadIdx.x == 0) {
    sh.bin = 0;
    sh.above = 0;
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan(sum, sh, kRedBin, total);
  for (int i = 0; i < per; ++i) {
    if (run < rem && rem <= run + cnt[i]) {
      sh.bin = (uint32_t)(top - i);
      sh.above = run;
    }
    run += cnt[i];
  }
  __syncthreads();
}

__device__ __forceinline__ void clear_hist(Core& sh, int nbins) {
  for (int i = threadIdx.x; i < nbins; i += kThreads) sh.hist[i] = 0;
  __syncthreads();
}

// Selects the `rem` largest of the n candidates in sh.cand by counting, for each, the
// candidates above it; e is unique, so a selected candidate's rank is its slot after the
// sh.n_out positions already emitted. n <= kRankMax.
__device__ void rank_select(Full& sh, int n, uint32_t rem, int32_t* out, int k) {
  const uint32_t base = sh.n_out;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const uint64_t e = sh.cand[i];
    uint32_t rank = 0;
#pragma unroll 8
    for (int j = 0; j < n; ++j) rank += sh.cand[j] > e ? 1u : 0u;
    if (rank < rem && base + rank < (uint32_t)k) out[base + rank] = position(e);
  }
  __syncthreads();
}

// Radix refinement over the candidate list (FromRow = false) or the whole visible row
// (FromRow = true), for elements matching `prefix` under `pmask`; bits [0, top) of e are
// still undecided. Emits through sh.n_out.
template <bool FromRow>
__device__ void refine(Full& sh, const float* row, int n, uint64_t prefix, uint64_t pmask, int top,
                       uint32_t rem, int32_t* out, int k) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  auto fetch = [&](int i) -> uint64_t { return FromRow ? compose(order_key(row[i]), i) : sh.cand[i]; };
  while (top > 0) {
    const int shift = top > 11 ? top - 11 : 0;
    const uint64_t dmask = (1ull << (top - shift)) - 1;
    clear_hist(sh, kLinBins);
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint64_t e = fetch(i);
      if ((e & pmask) == prefix) atomicAdd(&sh.hist[(e >> shift) & dmask], 1u);
    }
    __syncthreads();
    find_bin(sh, kLinBins, rem);
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
    top = shift;
    __syncthreads();
    if (cnt == rem) {  // the whole threshold bin is selected
      for (int base = wave * 64; base < n; base += kThreads) {
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
__device__ void finish_candidates(Full& sh, int n, uint64_t prefix, uint64_t pmask, int top, uint32_t rem,
                                  int32_t* out, int k) {
  if (n <= kRankMax)
    rank_select(sh, n, rem, out, k);
  else
    refine<false>(sh, nullptr, n, prefix, pmask, top, rem, out, k);
}

// Rows with nv <= k.
__device__ void select_trivial_row(const Params& p, int r, int nv) {
  int32_t* out = p.idx + (int64_t)r * p.k;
  for (int i = threadIdx.x; i < p.k; i += kThreads) out[i] = i < nv ? i : -1;
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

// The threshold bin of a block histogram of nbins = PER * kThreads bins: the bin B with
// above(B) < rem <= above(B) + hist[B], counting from the top bin, for rem <= the total.
// Thread t owns bins [nbins - PER*(t+1), nbins - PER*t). Each wave scans its own bins and
// publishes its total; after one barrier every wave finds the owning wave from the
// totals, rescans that wave's bins from LDS and so knows B, above(B) and hist[B]
// without a second barrier. Uses the kRedBin scratch slots.
template <int PER>
__device__ __forceinline__ void threshold_bin(Core& sh, uint32_t rem, uint32_t& bin, uint32_t& above,
                                              uint32_t& count) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int nbins = PER * kThreads;
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
  if (lane == 63) sh.red[kRedBin + wave] = incl;
  __syncthreads();
  // Wave totals in lanes 0..15; the owner is the first wave whose inclusive prefix
  // reaches rem.
  const uint32_t wt = lane < kWaves ? sh.red[kRedBin + lane] : 0u;
  const uint32_t wi = row16_prefix(wt);
  const uint64_t reach = __ballot(lane < kWaves && wi >= rem);
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

// Rows with k < nv <= PER * kThreads: the whole select by one workgroup. Element
// i*kThreads + t of the row sits in thread t's register i. Loads past nv are clamped onto
// the last visible element, which leaves min, max and finiteness unchanged; histogram and
// emit count only the elements below nv. PER = 8 serves rows up to 8192 (every tie set
// fits the candidate list); PER = 32 rows up to 32768, whose threshold bin can exceed the
// list, in which case the finish refines over the row itself.
template <int PER>
__device__ void select_row(const Params& p, int r, int nv, Full& sh) {
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
    const uint32_t off = min((uint32_t)threadIdx.x * 4u + (uint32_t)(i * kThreads * 4), last);
    v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  }
  for (int i = threadIdx.x; i < kKeyBins; i += kThreads) sh.hist[i] = 0;
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
    sh.red[kRedLo + wave] = __float_as_uint(lo);
    sh.red[kRedHi + wave] = __float_as_uint(bad ? __builtin_inff() : hi);
  }
  __syncthreads();
  lo = row16_minmax<false>(__uint_as_float(lane < kWaves ? sh.red[kRedLo + lane] : 0x7f800000u));
  hi = row16_minmax<true>(__uint_as_float(lane < kWaves ? sh.red[kRedHi + lane] : 0xff800000u));
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
  auto inm = [&](int i) { return __ballot(tid < nv - i * kThreads); };
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
    threshold_bin<kKeyBins / kThreads>(sh, (uint32_t)k, bin0, above, cnt0);
  else
    threshold_bin<kLinBins / kThreads>(sh, (uint32_t)k, bin0, above, cnt0);
  const uint32_t rem = (uint32_t)k - above;
  const bool whole = cnt0 == rem;
  // Emit the elements above the threshold bin (the whole bin too when it is all taken)
  // straight to the output row and collect the bin's own elements into the candidate
  // list. Each lane marks its visible elements in two bit masks (above the bin / in it);
  // lane and wave prefix sums of the mask populations give every lane its first output
  // and candidate slots (wave totals through LDS, one barrier), and each lane then walks
  // only its set bits. above(bin0) < k, so every output slot is in range; candidate
  // slots past kCap are dropped (the finish then refines over the row).
  const uint32_t thr = whole ? bin0 : bin0 + 1;
  const int vis = min(PER, (nv - tid + kThreads - 1) / kThreads);  // elements i < vis are visible
  uint32_t ma = 0, mb = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    ma |= (bin[i] >= thr ? 1u : 0u) << i;
    mb |= (bin[i] == bin0 ? 1u : 0u) << i;
  }
  const uint32_t vmask = vis >= 32 ? ~0u : (1u << max(vis, 0)) - 1u;
  ma &= vmask;
  mb = whole ? 0u : (mb & vmask);
  const uint32_t la = (uint32_t)__popc(ma), lb = (uint32_t)__popc(mb);
  const uint32_t ia = wave_scan_add(la), ib = wave_scan_add(lb);
  if (lane == 63) {
    sh.red[kRedEmit + wave] = ia;
    sh.red[kRedCand + wave] = ib;
  }
  if (threadIdx.x == 0) sh.n_out = above;  // the finish appends after the emitted elements
  __syncthreads();
  const uint32_t ca = lane < kWaves ? sh.red[kRedEmit + lane] : 0u;
  const uint32_t cb = lane < kWaves ? sh.red[kRedCand + lane] : 0u;
  uint32_t oa = (uint32_t)__builtin_amdgcn_readlane((int)(row16_prefix(ca) - ca), wave) + ia - la;
  uint32_t ob = (uint32_t)__builtin_amdgcn_readlane((int)(row16_prefix(cb) - cb), wave) + ib - lb;
  while (ma) {
    const int i = __builtin_ctz(ma);
    ma &= ma - 1u;
    out[oa++] = i * kThreads + tid;
  }
  while (mb) {  // the threshold bin's elements (few): their keys are read again
    const int i = __builtin_ctz(mb);
    mb &= mb - 1u;
    const int t = i * kThreads + tid;
    if (ob < (uint32_t)kCap) sh.cand[ob] = compose(order_key(row[t]), t);
    ++ob;
  }
  if (!whole) {
    __syncthreads();  // the candidate list is complete
    // Key bins fix the top 12 bits of e; linear or single bins fix none.
    const uint64_t prefix = keyed ? (uint64_t)bin0 << (64 - kKeyBits) : 0ull;
    const uint64_t pmask = keyed ? (uint64_t)(kKeyBins - 1) << (64 - kKeyBits) : 0ull;
    const int top = keyed ? 64 - kKeyBits : 64;
    if (PER * kThreads <= kCap || cnt0 <= (uint32_t)kCap) {  // uniform
      finish_candidates(sh, (int)cnt0, prefix, pmask, top, rem, out, k);
    } else if (keyed) {
      refine<true>(sh, row, nv, prefix, pmask, top, rem, out, k);
    } else {
      // Linear or single bins are not key-bit prefixes: select over the whole row again
      // by radix digits of e from the top, rewriting every output slot (the barrier
      // orders these stores after the ones above).
      if (threadIdx.x == 0) sh.n_out = 0;
      __syncthreads();
      refine<true>(sh, row, nv, 0ull, 0ull, 64, (uint32_t)k, out, k);
    }
  }
}

// When no row can exceed kWide: one launch, workgroup r selects row r with 32 values per
// thread (no workspace, none of the long-row passes).
__global__ __launch_bounds__(kThreads) void topk_rows_wide_kernel(Params p) {
  __shared__ Full sh;
  const int r = blockIdx.x;
  const int nv = visible(p, r);
  if (nv <= p.k) select_trivial_row(p, r, nv);
  else select_row<kWidePer>(p, r, nv, sh);
}

// One 8192-element chunk of a long row: element i*kThreads + threadIdx.x of
// [base, base + kChunk) in register i (loads past the row's visible end are clamped onto
// its last visible element), and where the chunk belongs.
struct Chunk {
  int slot, r, nv, base;
  float v[kPer];
};

// Issues the loads of chunk item `item`; nothing waits for them here, so the caller can
// prefetch the next item while it works on the current one.
__device__ __forceinline__ void fetch_chunk(const Params& p, int item, Chunk& c) {
  c.slot = (int)p.chunk_items[2 * item];
  c.base = (int)p.chunk_items[2 * item + 1] * kChunk;
  c.r = (int)p.long_rows[c.slot];
  c.nv = visible(p, c.r);
  const int n = min(kChunk, c.nv - c.base);  // >= 1: chunks start below nv
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p.logits + (int64_t)c.r * p.L + c.base), 0, n * 4, 0x00020000);
  const uint32_t last = (uint32_t)(n - 1) * 4u;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t off = min((uint32_t)threadIdx.x * 4u + (uint32_t)(i * kThreads * 4), last);
    c.v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  }
}

// Pass 1. Implicit mode (no workspace): workgroup r handles row r. Scheduled mode:
// persistent workgroups walk the long rows' chunks (histograms); the short and trivial
// rows wait for the last pass, whose workgroups are mostly idle otherwise, so that they
// do not lengthen this one.
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(Params p) {
  __shared__ Full sh;
  if (p.meta == nullptr) {
    const int r = blockIdx.x;
    const int nv = visible(p, r);
    if (nv <= p.k) select_trivial_row(p, r, nv);
    else select_row<kPer>(p, r, nv, sh);
    return;
  }
  const int nc = (int)p.meta[kMetaChunks];
  if ((int)blockIdx.x >= nc) return;
  const int tid = (int)threadIdx.x;
  Chunk cur, nxt;
  fetch_chunk(p, blockIdx.x, cur);
  clear_hist(sh, kKeyBins);
  for (int item = blockIdx.x; item < nc; item += gridDim.x) {
    if (item + (int)gridDim.x < nc) fetch_chunk(p, item + gridDim.x, nxt);  // uniform
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (__builtin_amdgcn_inverse_ballot_w64(__ballot(tid < cur.nv - cur.base - i * kThreads)))
        atomicAdd(&sh.hist[order_key(cur.v[i]) >> (32 - kKeyBits)], 1u);
    __syncthreads();
    // Add the chunk's bins into the row's histogram, clearing them for the next chunk.
    uint32_t* gh = p.hist + (int64_t)cur.slot * kKeyBins;
    for (int i = tid; i < kKeyBins; i += kThreads) {
      const uint32_t c = sh.hist[i];
      sh.hist[i] = 0;
      if (c) atomicAdd(&gh[i], c);
    }
    __syncthreads();
    cur = nxt;
  }
}

// This workgroup's share of the histograms of `nlong` long-row slots (8-byte stores:
// the workspace is 8-byte aligned).
__device__ void clear_long_hist(const Params& p, uint32_t nlong) {
  uint2* gh = reinterpret_cast<uint2*>(p.hist);
  const int64_t words = (int64_t)nlong * (kKeyBins / 2);
  const int64_t per = (words + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < words ? lo + per : words;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) gh[i] = make_uint2(0u, 0u);
}

// Schedule for long-row mode. Workgroup 0 classifies every row, lists the rows of each
// class and the long rows' chunks (offsets from block scans) and clears the long rows'
// counters; every workgroup counts the long rows and clears its share of their
// histograms (16 KB each: one workgroup alone spent tens of microseconds on it).
__global__ __launch_bounds__(kThreads) void topk_schedule_kernel(Params p) {
  __shared__ Core sh;
  if (blockIdx.x != 0) {
    uint32_t nlong = 0;
    for (int base = 0; base < p.rows; base += kThreads) {
      const int r = base + (int)threadIdx.x;
      const int nv = r < p.rows ? visible(p, r) : 0;
      uint32_t tl;
      block_exclusive_scan((r < p.rows && nv > p.k && nv > kChunk) ? 1u : 0u, sh, kRedLo, tl);
      nlong += tl;
      __syncthreads();  // the scratch slots are reused by the next block of rows
    }
    clear_long_hist(p, nlong);
    return;
  }
  uint32_t off_l = 0, off_s = 0, off_t = 0, off_c = 0;
  for (int base = 0; base < p.rows; base += kThreads) {
    const int r = base + (int)threadIdx.x;
    const bool in = r < p.rows;
    const int nv = in ? visible(p, r) : 0;
    const uint32_t is_long = in && nv > p.k && nv > kChunk;
    const uint32_t is_short = in && nv > p.k && nv <= kChunk;
    const uint32_t is_triv = in && nv <= p.k;
    const uint32_t nch = is_long ? (uint32_t)((nv + kChunk - 1) / kChunk) : 0u;
    uint32_t tl, tt, tc;
    const uint32_t el = block_exclusive_scan(is_long | (is_short << 16), sh, kRedLo, tl);  // < 2^16 each
    const uint32_t et = block_exclusive_scan(is_triv, sh, kRedHi, tt);
    const uint32_t ec = block_exclusive_scan(nch, sh, kRedBad, tc);
    if (is_long) {
      const uint32_t slot = off_l + (el & 0xFFFFu);
      p.long_rows[slot] = (uint32_t)r;
      p.counters[2 * slot] = 0u;
      p.counters[2 * slot + 1] = 0u;
      const uint32_t first = off_c + ec;
      for (uint32_t c = 0; c < nch; ++c) {
        p.chunk_items[2 * (first + c)] = slot;
        p.chunk_items[2 * (first + c) + 1] = c;
      }
    }
    if (is_short) p.short_rows[off_s + (el >> 16)] = (uint32_t)r;
    if (is_triv) p.triv_rows[off_t + et] = (uint32_t)r;
    off_l += tl & 0xFFFFu;
    off_s += tl >> 16;
    off_t += tt;
    off_c += tc;
    __syncthreads();  // the scratch slots are reused by the next block of rows
  }
  clear_long_hist(p, off_l);
  if (threadIdx.x == 0) {
    p.meta[kMetaLong] = off_l;
    p.meta[kMetaChunks] = off_c;
    p.meta[kMetaShort] = off_s;
    p.meta[kMetaTrivial] = off_t;
  }
}

// Pass 2 (long rows): threshold bin from the row's histogram; emit the chunk's elements
// above it, collect those in it.
__global__ __launch_bounds__(kThreads) void topk_split_kernel(Params p) {
  __shared__ Core sh;
  const int nc = (int)p.meta[kMetaChunks];
  if ((int)blockIdx.x >= nc) return;
  const int k = p.k;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The row histogram arrives 16 bytes per thread (kKeyBins = 4 * kThreads).
  static_assert(kKeyBins == 4 * kThreads, "one uint4 of the histogram per thread");
  auto fetch_hist = [&](int slot) {
    return reinterpret_cast<const uint4*>(p.hist + (int64_t)slot * kKeyBins)[tid];
  };
  Chunk cur, nxt;
  fetch_chunk(p, blockIdx.x, cur);
  uint4 hcur = fetch_hist(cur.slot), hnxt;
  for (int item = blockIdx.x; item < nc; item += gridDim.x) {
    if (item + (int)gridDim.x < nc) {  // uniform: prefetch the next item
      fetch_chunk(p, item + gridDim.x, nxt);
      hnxt = fetch_hist(nxt.slot);
    }
    reinterpret_cast<uint4*>(sh.hist)[tid] = hcur;
    __syncthreads();
    uint32_t bin0, above, cnt0;
    threshold_bin<kKeyBins / kThreads>(sh, (uint32_t)k, bin0, above, cnt0);
    const bool whole = cnt0 == (uint32_t)k - above;
    // Elements above the threshold bin (the whole bin too when all of it is taken) go to
    // the output, the bin's own elements to the row's candidate list; slots from one
    // pair of global atomics per workgroup, a prefix over the waves' counts and each
    // lane's prefix over the populations of its two element masks; each lane then walks
    // its set bits.
    const uint32_t thr = whole ? bin0 : bin0 + 1;
    const int vis = min(kPer, (cur.nv - cur.base - tid + kThreads - 1) / kThreads);  // visible elements
    uint32_t ma = 0, mb = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t d = order_key(cur.v[i]) >> (32 - kKeyBits);
      ma |= (d >= thr ? 1u : 0u) << i;
      mb |= (d == bin0 ? 1u : 0u) << i;
    }
    static_assert(kPer < 32, "a lane's element masks fit 32 bits");
    const uint32_t vmask = (1u << max(vis, 0)) - 1u;
    ma &= vmask;
    mb = whole ? 0u : (mb & vmask);
    const uint32_t la = (uint32_t)__popc(ma), lb = (uint32_t)__popc(mb);
    const uint32_t la_incl = wave_scan_add(la), lb_incl = wave_scan_add(lb);
    if (lane == 63) {
      sh.red[kRedEmit + wave] = la_incl;
      sh.red[kRedCand + wave] = lb_incl;
    }
    __syncthreads();
    const uint32_t ca = lane < kWaves ? sh.red[kRedEmit + lane] : 0u;
    const uint32_t cb = lane < kWaves ? sh.red[kRedCand + lane] : 0u;
    const uint32_t ia = row16_prefix(ca), ib = row16_prefix(cb);
    if (tid == 0) {
      const uint32_t ta = (uint32_t)__builtin_amdgcn_readlane((int)ia, kWaves - 1);
      const uint32_t tb = (uint32_t)__builtin_amdgcn_readlane((int)ib, kWaves - 1);
      sh.base_a = ta ? atomicAdd(&p.counters[2 * cur.slot], ta) : 0u;
      sh.base_b = tb ? atomicAdd(&p.counters[2 * cur.slot + 1], tb) : 0u;
    }
    __syncthreads();
    uint32_t oa = sh.base_a + (uint32_t)__builtin_amdgcn_readlane((int)(ia - ca), wave) + la_incl - la;
    uint32_t ob = sh.base_b + (uint32_t)__builtin_amdgcn_readlane((int)(ib - cb), wave) + lb_incl - lb;
    int32_t* out = p.idx + (int64_t)cur.r * k;
    uint64_t* cand = p.cand + (int64_t)cur.slot * kCap;
    while (ma) {
      const int i = __builtin_ctz(ma);
      ma &= ma - 1u;
      const uint32_t ra = oa++;
      if (ra < (uint32_t)k) out[ra] = cur.base + i * kThreads + tid;
    }
    while (mb) {  // the threshold bin's elements (few): their keys are read again
      const int i = __builtin_ctz(mb);
      mb &= mb - 1u;
      const int t = cur.base + i * kThreads + tid;
      const uint32_t rb = ob++;
      if (rb < (uint32_t)kCap) cand[rb] = compose(order_key(p.logits[(int64_t)cur.r * p.L + t]), t);
    }
    // The next item's first LDS writes (histogram, then the slots above) come after
    // barriers every wave passes only once it has read this item's.
    cur = nxt;
    hcur = hnxt;
  }
}

// Pass 3: refine each long row's candidates; then the short rows (whole selection) and
// the trivial rows.
__global__ __launch_bounds__(kThreads) void topk_finish_kernel(Params p) {
  __shared__ Full sh;
  const int nl = (int)p.meta[kMetaLong];
  const int ns = (int)p.meta[kMetaShort];
  const int nt = (int)p.meta[kMetaTrivial];
  for (int item = blockIdx.x; item < nl + ns + nt; item += gridDim.x) {
    if (item >= nl) {  // uniform
      if (item < nl + ns) {
        const int r = (int)p.short_rows[item - nl];
        select_row<kPer>(p, r, visible(p, r), sh);
        __syncthreads();
      } else {
        const int r = (int)p.triv_rows[item - nl - ns];
        select_trivial_row(p, r, visible(p, r));
      }
      continue;
    }
    const int slot = item;
    const int r = (int)p.long_rows[slot];
    const int nv = visible(p, r);
    const int k = p.k;
    const uint32_t* gh = p.hist + (int64_t)slot * kKeyBins;
    reinterpret_cast<uint4*>(sh.hist)[threadIdx.x] = reinterpret_cast<const uint4*>(gh)[threadIdx.x];
    __syncthreads();
    uint32_t bin0, above, cnt0;
    threshold_bin<kKeyBins / kThreads>(sh, (uint32_t)k, bin0, above, cnt0);
    const uint32_t rem = (uint32_t)k - above;
    __syncthreads();  // every wave is done with the histogram before the next item's copy
    if (cnt0 == rem) continue;  // the split pass took the whole bin (uniform)
    const float* row = p.logits + (int64_t)r * p.L;
    int32_t* out = p.idx + (int64_t)r * k;
    if (threadIdx.x == 0) sh.n_out = above;  // the split pass emitted exactly `above`
    const uint64_t prefix = (uint64_t)bin0 << (64 - kKeyBits);
    const uint64_t pmask = (uint64_t)(kKeyBins - 1) << (64 - kKeyBits);
    if (cnt0 <= (uint32_t)kCap) {
      const uint64_t* cand = p.cand + (int64_t)slot * kCap;
      for (int i = threadIdx.x; i < (int)cnt0; i += kThreads) sh.cand[i] = cand[i];
      __syncthreads();
      finish_candidates(sh, (int)cnt0, prefix, pmask, 64 - kKeyBits, rem, out, k);
    } else {
      __syncthreads();
      refine<true>(sh, row, nv, prefix, pmask, 64 - kKeyBits, rem, out, k);
    }
    __syncthreads();
  }
}

// Workspace layout (long-row mode): meta[8] | long_rows | short_rows | triv_rows |
// chunk_items | counters | hist | cand, each region 16-byte aligned (the histograms are
// read as uint4; the workspace base is 16-byte aligned).
struct Layout {
  size_t meta, long_rows, short_rows, triv_rows, chunk_items, counters, hist, cand, total;
};

Layout layout(int64_t rows, int32_t L) {
  auto up16 = [](size_t x) { return (x + 15) & ~(size_t)15; };
  const int64_t nchunk = (L + kChunk - 1) / kChunk;
  Layout l;
  l.meta = 0;
  l.long_rows = 32;
  l.short_rows = up16(l.long_rows + 4 * rows);
  l.triv_rows = up16(l.short_rows + 4 * rows);
  l.chunk_items = up16(l.triv_rows + 4 * rows);
  l.counters = up16(l.chunk_items + 8 * rows * nchunk);
  l.hist = up16(l.counters + 8 * rows);
  l.cand = up16(l.hist + (size_t)4 * kKeyBins * rows);
  l.total = l.cand + (size_t)8 * kCap * rows;
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
  if (max_model_len <= kWide) return 0;
  return layout(rows, max_model_len).total;
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
  if (a.max_model_len <= kChunk) {  // every row fits one workgroup, 8 values per thread
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
  }
  if (a.max_model_len <= kWide) {  // every row fits one workgroup, 32 values per thread
    hipLaunchKernelGGL(topk_rows_wide_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
  }
  const Layout l = layout(rows, a.max_model_len);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  p.meta = reinterpret_cast<uint32_t*>(ws + l.meta);
  p.long_rows = reinterpret_cast<uint32_t*>(ws + l.long_rows);
  p.short_rows = reinterpret_cast<uint32_t*>(ws + l.short_rows);
  p.triv_rows = reinterpret_cast<uint32_t*>(ws + l.triv_rows);
  p.chunk_items = reinterpret_cast<uint32_t*>(ws + l.chunk_items);
  p.counters = reinterpret_cast<uint32_t*>(ws + l.counters);
  p.hist = reinterpret_cast<uint32_t*>(ws + l.hist);
  p.cand = reinterpret_cast<uint64_t*>(ws + l.cand);
  const unsigned persistent = (unsigned)compute_units();
  hipLaunchKernelGGL(topk_schedule_kernel, dim3(persistent), dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(topk_rows_kernel, dim3(persistent), dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(topk_split_kernel, dim3(persistent), dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(persistent), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mqa
