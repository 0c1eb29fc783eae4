// topselect.hip -- gfx950 kernels and the C ABI of the batched per-row sampler.
//
// Every call enqueues two kernels on the caller's stream:
//
//   ts_stream_kernel  rows x chunks workgroups of 256 threads (4 waves). Each workgroup streams
//                     one contiguous chunk (<= 8192 logits) of one row from HBM exactly once and
//                     keeps it in registers. A histogram of a quarter of the chunk (the first
//                     two load slots of every wave), 256 bins reaching down from the sample
//                     maximum, gives a threshold L_c: the lower edge of the bin holding the
//                     sample's j-th largest key, j a safety multiple of the chunk's share of k.
//                     Every wave then works alone (no further
//                     barriers): it stages the float4 quads whose maximum reaches L_c, extracts
//                     their elements >= L_c in id order and stores them as candidates in its own
//                     slice of the workspace, with a 32-byte summary (count, L_c, maximum, NaN
//                     and overflow flags).
//   ts_row_kernel     one 512-thread workgroup per row. It gathers the row's candidates into
//                     LDS, selects their exact top-k, and certifies it: when the smallest
//                     selected key is >= every L_c, every row element that could rank above it
//                     is a candidate, so the candidate top-k IS the row top-k. Otherwise
//                     (adversarial or tie-heavy rows) it falls back to the exact row-streaming
//                     path. Then the top-p mass cut and the Gumbel argmax run on the top-k set.
//
// The stream kernel is bound by vector-ALU issue as much as by HBM: a wave64 VALU instruction
// occupies its SIMD for four cycles, so the per-element work between the loads and the
// candidate stores is a handful of instructions per float4 (one three-input max chain, two
// unordered compares, one threshold compare, a ballot).
//
// Row paths (chosen per row on the device from that row's k, p, T):
//   CAND    k_eff <= 2048: candidates + certified selection as above.
//   GREEDY  T == 0: the first token of the row ordering (max key, lowest id).
//   FULL    top-k and top-p both off (sampling): each wave computes its Gumbel argmax relative
//           to its own maximum; the row kernel folds the wave winners.
//   STREAM  everything else (k > 2048, top-p with top-k off, failed certification): the row
//           kernel re-reads the row from global memory once per radix pass.
//   NONE    invalid row: outputs poisoned.
//
// Page citations (title, then section):
//   [DETK]   vLLM PR #55122 "[Kernel] Make persistent_topk deterministic": "Changes" (exact
//            radix select, pass skipping, index-ordered ties, per-CTA counts merged in CTA
//            order).
//   [TOPP]   "Split top-p numerical reference and conservative gate": "Source basis",
//            "Independent binary64 numerical reference".
//   [GUMBEL] prhub summary of vLLM PR #45996: "implementation breakdown", "key source
//            excerpts".
//   [LOGP]   RL-Kernel issue #332: "Contract constants", "Integration".
#include <float.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "topselect.h"
#include "topselect_testing.h"
#include "ts_device.hpp"
#include "ts_host.hpp"

using namespace tsd;

namespace {

enum Mode : int { kModeTopk = 0, kModeTopp = 1, kModeSample = 2 };
enum Path : int { kPathNone = 0, kPathCand = 1, kPathGreedy = 2, kPathFull = 3, kPathStream = 4, kPathNucleus = 5 };

// stream kernel
constexpr int kT1 = 256;                            // threads per chunk workgroup
constexpr int kW1 = kT1 / 64;                       // waves per chunk workgroup
constexpr int kS1 = 8;                              // float4 loads per thread
constexpr int kChunkMax = kT1 * 4 * kS1;            // 8192 logits per chunk
constexpr int kHBits = 11;                          // sample histogram digit (top key bits)
constexpr int kHBins = 1 << kHBits;
constexpr int kHWords = kHBins + kHBins / 8;        // padded: 4 spare words after every 32 bins
constexpr int kH2Bits = 8;                          // second-level digit inside the chosen bin
constexpr int kH2Bins = 1 << kH2Bits;
constexpr int kSampleSlots = 2;                     // slots whose keys form the sample
constexpr int kQStage = 128;                        // staged quads per wave (a power of two)
static_assert((kQStage & (kQStage - 1)) == 0, "stage ranks wrap with a mask");
constexpr int kRefine = 16;                         // sampled keys in a chosen bin that call for a finer level
constexpr int kCapW = kChunkMax / kW1 / 2;          // candidate slots per wave, at most: half of its
                                                     // share (less 32), so that the workspace takes no
                                                     // more bytes than the logits it covers
constexpr int kCapSmall = 256;                      // waves of at most this many elements keep a slot
                                                     // for each; larger ones get half their share
// A wave that finds more candidates than its slice holds flags it overflowed and its row takes
// the exact path, unless every one of its elements is the same key (a uniform slice, which
// stores nothing).
// row kernel
constexpr int kRT = 512;                            // threads per row workgroup
constexpr int kRW = kRT / 64;
constexpr int kFastK = 2048;                        // largest k taking the candidate path
constexpr int kDBits = 11;                          // radix digit of the row selects
constexpr int kDBins = 1 << kDBits;                 // = 4 bins per row-kernel thread
constexpr int kLdsCand = 12288;                     // candidates the row kernel holds in LDS
constexpr int kSlab = 8192;                         // row elements per row-streaming Gumbel slab
constexpr int kValueOrderMax = 8192;                // value-ordered top-k: k_max limit (sort size)
constexpr int kVisU = 6;                            // LDS items per thread per visitor round
constexpr int kGatherB = 10;                        // wave slices per gather batch
constexpr uint32_t kSmallBin = 64;                  // boundary bins up to this size are resolved by one wave
constexpr int kMaxSeg = 1024;                       // wave slices per row the gather indexes
constexpr int kSegPT = kMaxSeg / kRT;               // slice counts scanned per thread
constexpr int kBPT = kDBins / kRT;                  // histogram bins owned per thread
static_assert((kBPT == 2 || kBPT % 4 == 0) && kSegPT >= 1, "row-kernel geometry");

// Summary of one wave's share of a chunk (32 bytes).
struct WaveInfo {
  uint32_t count;     // candidates stored (CAND), capped at the slice capacity
  uint32_t thr;       // L_c as a key: every key >= thr of the wave's elements is a candidate
  uint32_t kmax;      // largest key among the wave's elements
  uint32_t flags;     // bit 0: NaN seen; bit 1: candidates overflowed the slice
  uint32_t kmax_idx;  // lowest id holding kmax (GREEDY)
  float best_s;       // FULL sampling: best score relative to kmax's value
  int32_t best_idx;
  uint32_t first;     // UNIFORM slices: the id of the wave's first element
};
static_assert(sizeof(WaveInfo) == 32, "WaveInfo layout");
// kFlagUniform: every one of the wave's `count` elements holds the key kmax, so the slice
// stores no entries: entry j is (kmax, first + j). Only such slices may count past the
// slice capacity.
constexpr uint32_t kFlagNan = 1u, kFlagOverflow = 2u, kFlagUniform = 4u;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Per-row state of the nucleus passes. The exact fixed-point mass of every nucleus bin
// (value-linear bins in a window below the row maximum, and one bin for everything below
// it), then the counts of the tokens above the cut bin (and those min-p keeps), the best Gumbel score of the
// kept tokens above the cut bin, as (ordered score << 32 | ~id) so that the maximum prefers
// the lowest id on equal scores, and the number of cut-bin tokens listed (the list itself
// lives in the row's candidate slices, which nucleus rows leave unused).
constexpr int kSplitCUs = 256;   // row-kernel workgroups that fill the chip (one per CU: its LDS)
constexpr int kNucBins = 1024;   // nucleus bins (value-linear window below the maximum, and bin 0)
constexpr int64_t kSplitNokV = 100000;         // calls without a top-k array: the split nucleus
constexpr int64_t kSplitNokLogits = 6400000;   // for rows up to this long, calls up to this size
constexpr int kCodeCap = 4096;   // split nucleus: tokens sharing the cut bin's code, listed at most
constexpr int kCodePer = kCodeCap / kRT;
struct NucRow {
  uint64_t mass[kNucBins];     // exact fixed-point mass per bin
  uint64_t best;               // best (ordered score << 32 | ~id) of the kept tokens above the cut bin
  uint32_t nlist;              // tokens of the cut bin, listed by the cut pass
  uint32_t nabove;             // tokens in bins above the cut bin
  uint32_t kabove;             // of those, the ones min-p keeps (all of them without min-p)
  uint32_t ticket;             // split nucleus: workgroups of the row that finished their part
  uint32_t pad[2];
};
static_assert(sizeof(NucRow) % 16 == 0, "NucRow is zeroed in 16-byte words");

struct Params {
  const float* x;
  int64_t stride;
  int32_t V;
  int32_t rows;
  const int32_t* k;
  const float* p;
  const float* t;
  const float* minp;           // min-p per row, or NULL (off)
  const int32_t* lengths;      // top-k select: valid keys per row (clamped to V), or NULL
  const int32_t* offsets;      // top-k select: added to every emitted id, or NULL
  int32_t order;               // top-k select: TS_ORDER_INDEX or TS_ORDER_VALUE
  const uint64_t* seed;
  int32_t k_max;
  int32_t chunks;
  int32_t chunk_len;
  int32_t cap_w;
  int32_t xcd_map;
  int32_t force_exact;
  int32_t direct;              // rows of <= kLdsCand logits: the row kernel alone, row in LDS
  int32_t nucleus;             // top-k off for every row: the nucleus pass spreads top-p work
  int32_t split;               // workgroups per row of the row kernel's split nucleus (0: none)
  int32_t codes;               // split nucleus, sampling: the parts store per-token bin codes
  struct NucRow* nuc;          // per row: the nucleus pass's histograms
  int32_t* out_idx;
  int32_t* out_kept;
  uint8_t* out_mask;
  int32_t* out_token;
  int32_t* status;
  float* out_logp;             // sampling with logprobs: selected-token logprob, lse (or NULL)
  float* out_lse;
  double* wsum;                // per wave slice: sum of exp((x - wave max) / T), or NULL
  WaveInfo* info;
  uint2* cand;
};

struct RowPlan {
  int32_t n;                   // the row's valid length (V unless top-k select lengths are given)
  int32_t k_eff;
  float p;
  float t;
  float minp;                  // 0 = off
  int32_t path;
  int32_t bad;
};

// LDS of the row kernel (about 141 KB; one workgroup per CU)
struct Smem {
  uint32_t ckey[kLdsCand];     // candidates (id order), keys and ids in separate arrays
  uint32_t cidx[kLdsCand];
  alignas(16) uint32_t hist[kDBins];   // count histogram; each thread reads and re-zeroes its own bins
  alignas(16) uint64_t mhi[kDBins];    // mass histogram (fixed-point sums)
  uint32_t kkey[kFastK];       // the kept set P, compacted for the Gumbel draws
  uint32_t kidx[kFastK];
  uint32_t segoff[kMaxSeg + 1];
  uint32_t red[5 * kRW];
  uint64_t red64[2 * kRW];
  float reds[kRW];
  int32_t redi[kRW];
  uint32_t res[4];
  uint64_t res64[4];
  uint32_t kcount[2];
  uint32_t bkey[kSmallBin];    // a small boundary bin, collected for one wave to rank
  uint32_t bidx[kSmallBin];
  uint64_t bmass[kSmallBin];
  uint32_t bres[4];
  uint32_t bcount;             // zero outside collect_bin .. its resolution
};

// LDS of the stream kernel (about 20 KB)
struct Smem1 {
  uint32_t hist[kHWords];      // sample keys by their top 11 bits
  uint32_t hist2[kH2Bins];     // sample keys inside the chosen bin, by their next 8 bits
  alignas(16) uint32_t hwin[kH2Bins];   // sample keys in the 256 top-16-bit bins below the maximum
  uint32_t wmax[kW1];          // per wave: the sample's largest key
  uint4 stage_v[kW1][kQStage];
  uint32_t stage_q[kW1][kQStage];
  uint32_t res[4];
};

// ------------------------------------------------------------------ per-row plan
__device__ __forceinline__ RowPlan plan_row(const Params& P, int mode, int r) {
  RowPlan rp;
  rp.n = (mode == kModeTopk && P.lengths) ? max(0, min(P.lengths[r], P.V)) : P.V;
  const int32_t kr = P.k ? P.k[r] : P.V;
  rp.k_eff = kr < 1 ? 0 : min(kr, rp.n);
  rp.p = (mode != kModeTopk && P.p) ? P.p[r] : 1.0f;
  rp.t = (mode != kModeTopk && P.t) ? P.t[r] : 1.0f;
  rp.minp = (mode != kModeTopk && P.minp) ? P.minp[r] : 0.0f;
  int bad = TS_ROW_OK;
  if (kr < 1) bad = TS_ROW_BAD_K;
  else if (mode == kModeTopk && rp.k_eff > P.k_max) bad = TS_ROW_BAD_K;
  else if (mode != kModeTopk && !(rp.p > 0.0f && rp.p <= 1.0f)) bad = TS_ROW_BAD_P;
  else if (mode != kModeTopk && !(rp.t >= 0.0f && rp.t <= FLT_MAX)) bad = TS_ROW_BAD_T;
  else if (mode != kModeTopk && !(rp.minp >= 0.0f && rp.minp <= 1.0f)) bad = TS_ROW_BAD_MINP;
  rp.bad = bad;
  if (bad) rp.path = kPathNone;
  else if (mode == kModeTopk) rp.path = rp.k_eff <= kFastK ? kPathCand : kPathStream;
  else if (rp.t == 0.0f) rp.path = kPathGreedy;
  else if (rp.k_eff <= kFastK) rp.path = kPathCand;
  else if (rp.k_eff == P.V && rp.p == 1.0f && rp.minp == 0.0f) rp.path = kPathFull;
  else if (P.nucleus && rp.k_eff == P.V) rp.path = kPathNucleus;
  else rp.path = kPathStream;
  return rp;
}

// Rows of the row kernel's split nucleus: rows with top-p or min-p on and top-k off, in calls
// with a top-k array (whose value for the row reaches the row length, visible on the device
// only) and in small sampling calls without one that the host sends here.
__device__ __forceinline__ bool split_row(const Params& P, const RowPlan& rp) {
  return P.split && rp.path == kPathStream && rp.k_eff >= rp.n && (rp.p != 1.0f || rp.minp > 0.0f);
}

// ------------------------------------------------------------------ selection descriptor
// Elements are selected when the top (32 - lo) bits of their radix key exceed `prefix`, or
// equal it and their id is <= cutoff (lowest ids first among equal keys, [DETK] "Changes").
struct Sel {
  uint32_t prefix;
  int lo;
  uint32_t cutoff;
};
__device__ __forceinline__ bool sel_member(const Sel& s, uint32_t rk, uint32_t idx) {
  const uint32_t h = shr(rk, s.lo);
  return h > s.prefix || (h == s.prefix && idx <= s.cutoff);
}
__device__ __forceinline__ Sel sel_all() { return Sel{0u, 32, 0xFFFFFFFFu}; }

// ------------------------------------------------------------------ threshold-bin searches
// Workgroup-wide searches over the kDBins-bin histograms; thread t owns bins kBPT*t ..
// kBPT*t + kBPT - 1 (16-byte LDS reads), reads them and zeroes them for the next pass (no
// other thread touches them before the next pass's atomics, which follow two barriers).
//
// Reads thread t's kBPT count bins into c and zeroes them (16- or 8-byte LDS accesses).
__device__ __forceinline__ void take_bins(uint32_t* hist, int t, uint32_t* c) {
  if (kBPT == 2) {
    uint2* h2 = reinterpret_cast<uint2*>(hist) + t;
    const uint2 v = *h2;
    c[0] = v.x;
    c[1] = v.y;
    *h2 = make_uint2(0, 0);
  } else {
    uint4* h4 = reinterpret_cast<uint4*>(hist) + t * (kBPT / 4);
#pragma unroll
    for (int q = 0; q < kBPT / 4; ++q) {
      const uint4 v = h4[q];
      c[4 * q] = v.x;
      c[4 * q + 1] = v.y;
      c[4 * q + 2] = v.z;
      c[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int q = 0; q < kBPT / 4; ++q) h4[q] = make_uint4(0, 0, 0, 0);
  }
}

// Count: the highest bin b with (count in bins >= b) >= need. Writes res[0] = b,
// res[1] = count in bins > b, res[2] = count in b. Requires 1 <= need <= total.
__device__ __forceinline__ void search_count(Smem& sm, uint32_t need) {
  uint32_t c[kBPT];
  take_bins(sm.hist, threadIdx.x, c);
  uint32_t lsum = 0;
#pragma unroll
  for (int j = 0; j < kBPT; ++j) lsum += c[j];
  const uint32_t sfx = wave_incl_suffix(lsum);     // lanes >= this one, within the wave
  if (lane() == 0) sm.red[wave()] = sfx;
  bar();
  uint32_t above = 0;
#pragma unroll
  for (int w = 0; w < kRW; ++w) above += (w > wave()) ? sm.red[w] : 0u;
  const uint32_t excl = above + sfx - lsum;        // count in bins above this thread's bins
  if (excl < need && excl + lsum >= need) {
    uint32_t acc = excl;
    int j = kBPT - 1;
    for (; j > 0; --j) {
      if (acc + c[j] >= need) break;
      acc += c[j];
    }
    sm.res[0] = kBPT * threadIdx.x + j;
    sm.res[1] = acc;
    sm.res[2] = c[j];
  }
  bar();
}

// Mass: the highest bin b with ma + (mass in bins >= b) >= target_fx, masses being exact
// fixed-point sums (one 64-bit word floor(w * 2^S) per weight). Writes res[0] = b,
// res[1] = count above b, res[2] = count in b, res64[0] = ma + mass above b, res64[1] = mass
// of b. The caller guarantees that ma plus the whole histogram reaches the target.
// With zp > 0 the target is ceil(zp * Z), Z being the whole histogram's mass (the caller's
// first pass weighed every item into it): it is computed here from the waves' totals, after the
// exchange this search needs anyway, and left in res64[2].
__device__ __forceinline__ void search_mass(Smem& sm, uint64_t target_fx, uint64_t ma, float zp = 0.0f) {
  const int t = threadIdx.x;
  uint32_t c[kBPT];
  uint64_t mh[kBPT];
  take_bins(sm.hist, t, c);
#pragma unroll
  for (int j = 0; j < kBPT; ++j) mh[j] = sm.mhi[kBPT * t + j];
#pragma unroll
  for (int j = 0; j < kBPT; ++j) sm.mhi[kBPT * t + j] = 0;
  uint32_t lc = 0;
  uint64_t lh = 0;
#pragma unroll
  for (int j = 0; j < kBPT; ++j) {
    lc += c[j];
    lh += mh[j];
  }
  const uint32_t sc = wave_incl_suffix(lc);
  const uint64_t sh = wave_incl_suffix64(lh);
  if (lane() == 0) {
    sm.red[wave()] = sc;
    sm.red64[wave()] = sh;
  }
  bar();
  uint32_t ac = 0;
  uint64_t ah = 0, z = 0;
#pragma unroll
  for (int w = 0; w < kRW; ++w) {
    const bool up = w > wave();
    ac += up ? sm.red[w] : 0u;
    ah += up ? sm.red64[w] : 0ull;
    z += sm.red64[w];
  }
  if (zp > 0.0f) {
    target_fx = topp_target(zp, z);
    if (threadIdx.x == 0) sm.res64[2] = target_fx;
  }
  uint32_t xc = ac + sc - lc;
  uint64_t xh = ma + ah + sh - lh;
  if (xh < target_fx && xh + lh >= target_fx) {
    int j = kBPT - 1;
    for (; j > 0; --j) {
      if (xh + mh[j] >= target_fx) break;
      xh += mh[j];
      xc += c[j];
    }
    sm.res[0] = kBPT * t + j;
    sm.res[1] = xc;
    sm.res[2] = c[j];
    sm.res64[0] = xh;
    sm.res64[1] = mh[j];
  }
  bar();
}

// ------------------------------------------------------------------ radix digits
// The first radix pass over keys in [lo_rk, hi_rk]: the bits above the highest bit where the
// bounds differ are common (prefix); the digit is the next min(kDBits, lo) bits.
struct Digit {
  int lo;
  int sh;
  uint32_t dm;
  uint32_t prefix;
};
__device__ __forceinline__ Digit first_digit(uint32_t hi_rk, uint32_t lo_rk) {
  Digit g;
  g.lo = (hi_rk == lo_rk) ? 0 : 32 - __clz((int)(hi_rk ^ lo_rk));
  g.prefix = shr(hi_rk, g.lo);
  const int d = min(kDBits, g.lo);
  g.sh = g.lo - d;
  g.dm = (1u << d) - 1u;
  return g;
}

// ------------------------------------------------------------------ histogram adds
// Count-histogram increment by the calling (active) lanes. When every active lane hits the
// same bin (runs of equal keys), one lane adds their number: same-address LDS atomics from
// a whole wave would otherwise serialize.
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t b) {
  const uint64_t act = __ballot(1);
  const uint32_t b0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)b);
  if (__ballot(b == b0) == act) {
    if ((uint32_t)lane() == (uint32_t)__builtin_ctzll(act)) atomicAdd(&h[b0], (uint32_t)__popcll(act));
  } else {
    atomicAdd(&h[b], 1u);
  }
}

// ------------------------------------------------------------------ small boundary bins
// When a radix pass leaves c <= kSmallBin items in the boundary bin, one visit collects
// them and wave 0 ranks them directly (key descending, then id ascending: the row order),
// in place of further passes over the whole set.
template <class Vis>
__device__ __forceinline__ void collect_bin(const Vis& vis, uint32_t prefix, int lo, Smem& sm) {
  vis([&](uint32_t rk, uint32_t idx) {
    if (shr(rk, lo) == prefix) {
      const uint32_t p = atomicAdd(&sm.bcount, 1u);
      if (p < kSmallBin) {
        sm.bkey[p] = rk;
        sm.bidx[p] = idx;
      }
    }
  });
  bar();
}

// Wave 0: lane l < c loads collected item l into (k, x) and returns its rank, the number of
// collected items before it in the row order (a permutation of 0 .. c-1 since ids differ).
__device__ __forceinline__ uint32_t bin_rank(uint32_t c, uint32_t& k, uint32_t& x, const Smem& sm) {
  const uint32_t l = (uint32_t)lane();
  k = 0u;
  x = 0xFFFFFFFFu;
  if (l < c) {
    k = sm.bkey[l];
    x = sm.bidx[l];
  }
  uint32_t rank = 0;
  const uint32_t cu = (uint32_t)__builtin_amdgcn_readfirstlane((int)c);   // uniform trip count
  for (uint32_t j = 0; j < cu; ++j) {
    const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)k, (int)j);
    const uint32_t xj = (uint32_t)__builtin_amdgcn_readlane((int)x, (int)j);
    rank += (kj > k || (kj == k && xj < x)) ? 1u : 0u;
  }
  return rank;
}

// The `need` first (row order) of the c collected items of the bin (prefix, lo): the
// selection is every key above the need-th item, and that item's equal keys up to its id.
template <class Vis>
__device__ __forceinline__ Sel small_topk(const Vis& vis, uint32_t prefix, int lo, uint32_t c, uint32_t need,
                                          Smem& sm) {
  collect_bin(vis, prefix, lo, sm);
  if (wave() == 0) {
    uint32_t k, x;
    const uint32_t rank = bin_rank(c, k, x, sm);
    if ((uint32_t)lane() < c && rank == need - 1u) {
      sm.bres[0] = k;
      sm.bres[1] = x;
    }
    if (lane() == 0) sm.bcount = 0;
  }
  bar();
  return Sel{sm.bres[0], 0, sm.bres[1]};
}

// ------------------------------------------------------------------ exact count select
// MSB-first radix select of the `need` largest radix keys among the items the visitor
// yields (vis(f) calls f(rk, idx) for this thread's items; the union over threads must be
// n_in_play items with hi_rk >= rk >= lo_rk). Bits above the highest bit where hi_rk and
// lo_rk differ are common and skipped. A pass stops early when the threshold bin holds
// exactly the slots still unfilled ([DETK] "Changes": pass skipping). The count histogram
// is zero on entry and on return.
// With `prebuilt`, the caller has already counted the first pass (digit first_digit(hi_rk,
// lo_rk)) into the histogram and passed a barrier; it may do so only when that pass runs
// (need >= 1 and hi_rk != lo_rk).
// On return: items with shr(rk, lo) > prefix are selected; eq_take of the tie_cnt items with
// shr(rk, lo) == prefix must still be taken (lowest ids first).
template <class Vis>
__device__ __forceinline__ void count_select(const Vis& vis, uint32_t need, uint32_t n_in_play, uint32_t hi_rk,
                                             uint32_t lo_rk, Smem& sm, uint32_t& prefix, int& lo,
                                             uint32_t& eq_take, uint32_t& tie_cnt, bool prebuilt = false) {
  lo = (hi_rk == lo_rk) ? 0 : 32 - __clz((int)(hi_rk ^ lo_rk));
  prefix = shr(hi_rk, lo);
  tie_cnt = n_in_play;
  bool counted = prebuilt;
  while (lo > 0 && need > 0) {
    const int d = min(kDBits, lo);
    const int sh = lo - d;
    const uint32_t dm = (1u << d) - 1u;
    const uint32_t pre = prefix;
    const int lo_now = lo;
    uint32_t* hist = sm.hist;
    if (!counted) {
      vis([&](uint32_t rk, uint32_t) {
        if (shr(rk, lo_now) == pre) hist_add(hist, (rk >> sh) & dm);
      });
      bar();
    }
    counted = false;
    search_count(sm, need);
    const uint32_t bin = sm.res[0], above = sm.res[1], cnt = sm.res[2];
    need -= above;
    prefix = (prefix << d) | bin;
    lo = sh;
    tie_cnt = cnt;
    if (cnt == need) break;
  }
  eq_take = need;
}

// Full selection (with the lowest-id tie cutoff) of the `need` largest keys.
// idx_lo / idx_hi bound the ids of the items.
template <class Vis>
__device__ __forceinline__ Sel select_topk(const Vis& vis, uint32_t need, uint32_t n_in_play, uint32_t hi_key,
                                           uint32_t lo_key, uint32_t idx_lo, uint32_t idx_hi, Smem& sm,
                                           bool prebuilt = false) {
  Sel s;
  uint32_t eq_take, tie_cnt;
  {
    // count_select's passes, leaving early for a small boundary bin
    int lo = (hi_key == lo_key) ? 0 : 32 - __clz((int)(hi_key ^ lo_key));
    uint32_t prefix = shr(hi_key, lo);
    tie_cnt = n_in_play;
    bool counted = prebuilt;
    while (lo > 0 && need > 0) {
      const int d = min(kDBits, lo);
      const int sh = lo - d;
      const uint32_t dm = (1u << d) - 1u;
      const uint32_t pre = prefix;
      const int lo_now = lo;
      if (!counted) {
        vis([&](uint32_t rk, uint32_t) {
          if (shr(rk, lo_now) == pre) hist_add(sm.hist, (rk >> sh) & dm);
        });
        bar();
      }
      counted = false;
      search_count(sm, need);
      const uint32_t bin = sm.res[0], above = sm.res[1], cnt = sm.res[2];
      need -= above;
      prefix = (prefix << d) | bin;
      lo = sh;
      tie_cnt = cnt;
      if (cnt == need) break;
      if (cnt <= kSmallBin) return small_topk(vis, prefix, lo, cnt, need, sm);
    }
    s.prefix = prefix;
    s.lo = lo;
    eq_take = need;
  }
  s.cutoff = 0xFFFFFFFFu;
  if (eq_take < tie_cnt) {
    // the eq_take lowest ids among the tied items: select on ~id
    const uint32_t pre = s.prefix;
    const int lo = s.lo;
    auto tvis = [&](auto f) {
      vis([&](uint32_t rk, uint32_t idx) {
        if (shr(rk, lo) == pre) f(~idx, idx);
      });
    };
    uint32_t p2, e2, t2;
    int lo2;
    count_select(tvis, eq_take, tie_cnt, ~idx_lo, ~idx_hi, sm, p2, lo2, e2, t2);
    s.cutoff = ~shl(p2, lo2);
  }
  return s;
}

// ------------------------------------------------------------------ mass select (top-p)
// Visit the items [0, n) of an LDS (key, id) array pair: kVisU per thread per round, all LDS
// reads of a round issued before any item is used. f(rk, idx) is called for each item.
template <class F>
__device__ __forceinline__ void lds_for(const uint32_t* ka, const uint32_t* ia, uint32_t n, F f) {
  for (uint32_t base = threadIdx.x; base < n; base += kRT * kVisU) {
    uint32_t k[kVisU], x[kVisU];
#pragma unroll
    for (int u = 0; u < kVisU; ++u) {
      const uint32_t i = min(base + u * kRT, n - 1);   // clamped: in bounds, result unused past n
      k[u] = ka[i];
      x[u] = ia[i];
    }
#pragma unroll
    for (int u = 0; u < kVisU; ++u) {
      if (base + u * kRT < n) f(k[u], x[u]);
    }
  }
}

// Visitor over LDS arrays (a fixed type, so that a select can continue on a list it built).
struct LdsVis {
  const uint32_t* ka;
  const uint32_t* ia;
  uint32_t n;
  template <class F>
  __device__ __forceinline__ void operator()(F f) const { lds_for(ka, ia, n, f); }
};

// Smallest prefix of the row ordering whose exact fixed-point mass reaches `target_fx`
// ([TOPP] "Independent binary64 numerical reference", steps 4-5, with the predicate kept in
// probability space, [TOPP] "Source basis"). kvis(f) calls f(rk, idx) for this thread's items
// of K; wmass(rk) returns the fixed-point weight of a key (computed only for items still in
// play). Result: Sel of the kept set P (a canonical prefix) and |P| in `kept`. Both histograms
// are zero on entry and on return. With `prebuilt`, the caller has already accumulated the
// first pass (digit first_digit(hi_key, lo_key), counts and masses) and passed a barrier; it
// may do so only when hi_key != lo_key. ma0 and n_above0 are the mass and the count of items
// above the ones in play. COLLECT (the row-streaming path, whose LDS candidate arrays are
// free): a boundary bin that fits in LDS is copied there and the select continues on it.
template <bool COLLECT = false, class KVis, class WMass>
__device__ __forceinline__ Sel select_mass(const KVis& kvis, const WMass& wmass, uint64_t target_fx,
                                           uint32_t n_in_play, uint32_t hi_key, uint32_t lo_key,
                                           uint32_t idx_lo, uint32_t idx_hi, Smem& sm, uint32_t& kept,
                                           bool prebuilt = false, uint64_t ma0 = 0, uint32_t n_above0 = 0,
                                           float zp = 0.0f) {
  int lo = (hi_key == lo_key) ? 0 : 32 - __clz((int)(hi_key ^ lo_key));
  uint32_t prefix = shr(hi_key, lo);
  uint32_t n_above = n_above0, tie_cnt = n_in_play;
  uint64_t ma = ma0, bin_m = 0;
  bool single = false, ran = false, counted = prebuilt;
  while (lo > 0) {
    const int d = min(kDBits, lo);
    const int sh = lo - d;
    const uint32_t dm = (1u << d) - 1u;
    const uint32_t pre = prefix;
    const int lo_now = lo;
    ran = true;
    if (!counted) {
      kvis([&](uint32_t rk, uint32_t) {
        if (shr(rk, lo_now) == pre) {
          const uint32_t b = (rk >> sh) & dm;
          hist_add(sm.hist, b);
          atomicAdd((unsigned long long*)&sm.mhi[b], (unsigned long long)wmass(rk));
        }
      });
      bar();
    }
    counted = false;
    search_mass(sm, target_fx, ma, zp);
    if (zp > 0.0f) {   // the first search took the target from the prebuilt histogram
      target_fx = sm.res64[2];
      zp = 0.0f;
    }
    const uint32_t bin = sm.res[0];
    n_above += sm.res[1];
    tie_cnt = sm.res[2];
    ma = sm.res64[0];
    bin_m = sm.res64[1];
    prefix = (prefix << d) | bin;
    lo = sh;
    if (tie_cnt == 1) { single = true; break; }
    if (tie_cnt <= kSmallBin) {
      // Rank the bin's items, lay their masses out in row order, and cut at the first
      // prefix whose mass (above the bin plus the prefix) reaches the target.
      collect_bin(kvis, prefix, lo, sm);
      if (wave() == 0) {
        uint32_t k, x;
        const uint32_t c = tie_cnt;
        const uint32_t rank = bin_rank(c, k, x, sm);
        const bool in = (uint32_t)lane() < c;
        if (in) sm.bmass[rank] = wmass(k);
        wave_lds_sync();
        const uint64_t cum = wave_incl_scan64(in ? sm.bmass[lane()] : 0ull);
        const uint64_t hit = __ballot(in && ma + cum >= target_fx);
        const uint32_t j = hit ? (uint32_t)__builtin_ctzll(hit) : c - 1u;   // the bin reaches it
        if (in && rank == j) {
          sm.bres[0] = k;
          sm.bres[1] = x;
        }
        if (lane() == 0) {
          sm.bres[2] = j + 1u;
          sm.bcount = 0;
        }
      }
      bar();
      kept = n_above + sm.bres[2];
      return Sel{sm.bres[0], 0, sm.bres[1]};
    }
    if constexpr (COLLECT) {
      if (lo > 0 && tie_cnt <= (uint32_t)kLdsCand) {
        const uint32_t pre2 = prefix;
        const int lo2 = lo;
        kvis([&](uint32_t rk, uint32_t idx) {
          if (shr(rk, lo2) == pre2) {
            const uint32_t p = atomicAdd(&sm.bcount, 1u);
            if (p < (uint32_t)kLdsCand) {
              sm.ckey[p] = rk;
              sm.cidx[p] = idx;
            }
          }
        });
        bar();
        if (threadIdx.x == 0) sm.bcount = 0;   // read by no one before the next barrier
        const uint32_t base_key = shl(prefix, lo);
        return select_mass<false>(LdsVis{sm.ckey, sm.cidx, tie_cnt}, wmass, target_fx, tie_cnt,
                                  base_key | ((1u << lo) - 1u), base_key, idx_lo, idx_hi, sm, kept, false,
                                  ma, n_above);
      }
    }
  }
  uint32_t take = 1;
  if (!single && tie_cnt > 1) {
    // The boundary key is shared by tie_cnt items of identical weight q (same key, same
    // fp32 logit, same weight): take the fewest of them, lowest ids first, that bring the
    // mass to the target.
    const uint64_t q = ran ? bin_m / tie_cnt : wmass(prefix);
    const uint64_t rest = target_fx > ma ? target_fx - ma : 0ull;
    const uint64_t j = q > 0 ? (rest + q - 1) / q : (uint64_t)tie_cnt;
    take = (uint32_t)min(max(j, (uint64_t)1), (uint64_t)tie_cnt);
  }
  Sel s{prefix, lo, 0xFFFFFFFFu};
  if (take < tie_cnt) {
    const uint32_t pre = prefix;
    const int lo_ = lo;
    auto tvis = [&](auto f) {
      kvis([&](uint32_t rk, uint32_t idx) {
        if (shr(rk, lo_) == pre) f(~idx, idx);
      });
    };
    uint32_t p2, e2, t2;
    int lo2;
    count_select(tvis, take, tie_cnt, ~idx_lo, ~idx_hi, sm, p2, lo2, e2, t2);
    s.cutoff = ~shl(p2, lo2);
  }
  kept = n_above + take;
  return s;
}

// ------------------------------------------------------------------ misc helpers

// The perturbed score (x - m) / T + g of token idx, with 1 / T rounded once per row (the
// same reciprocal on every path, so every path forms the same score; a correctly rounded
// division per token costs ten vector instructions). The compiler hoists 1.0f / t out of the
// callers' loops.
__device__ __forceinline__ float gumbel_score(uint32_t key, uint32_t idx, float m, float t,
                                              uint32_t r, uint32_t k0, uint32_t k1) {
  const uint4 w = philox4x32_10(idx >> 2, r, k0, k1);
  const float g = gumbel_from_uniform(uniform_from_word(pick_word(w, idx & 3u)));
  return (key2f(key) - m) * (1.0f / t) + g;
}


// Ordered emission over an id-ordered source, E consecutive items per thread per tile (all
// loads of a tile are issued before any is used); out(pos, idx) writes selected item `idx`
// at `pos`, positions following the source order.
template <int E, class Get, class Mem, class Out>
__device__ __forceinline__ void emit_ordered(uint32_t n, const Get& get, const Mem& mem, const Out& out,
                                             uint32_t& run, Smem& sm) {
  for (uint32_t base = 0; base < n; base += kRT * E) {
    uint32_t rk[E], idx[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t i = base + threadIdx.x * E + e;
      rk[e] = 0;
      idx[e] = 0;
      if (i < n) get(i, rk[e], idx[e]);
    }
    bool sel[E];
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t i = base + threadIdx.x * E + e;
      sel[e] = (i < n) && mem(rk[e], idx[e]);
      cnt += sel[e] ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t pos = block_excl_scan<kRW>(cnt, sm.red, tot);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (sel[e]) out(run + pos++, idx[e]);
    }
    run += tot;
  }
}


// lds_for over K = (kkey, kidx)[0, n) that also passes each item's position: f(i, key, id).
template <class F>
__device__ __forceinline__ void kvis_i(uint32_t n, F f, Smem& sm) {
  for (uint32_t base = threadIdx.x; base < n; base += kRT * kVisU) {
    uint32_t k[kVisU], x[kVisU];
#pragma unroll
    for (int u = 0; u < kVisU; ++u) {
      const uint32_t i = min(base + u * kRT, n - 1);   // clamped: in bounds, result unused past n
      k[u] = sm.kkey[i];
      x[u] = sm.kidx[i];
    }
#pragma unroll
    for (int u = 0; u < kVisU; ++u) {
      if (base + u * kRT < n) f(base + u * kRT, k[u], x[u]);
    }
  }
}

// Append the items of [0, n) of (ka, ia) that satisfy `mem` to (dkey, didx), in any order:
// per round, a wave scan of the per-lane counts and one LDS atomic per wave reserve room.
// Returns the count (entries past `cap` are dropped). Ends with a barrier. The slot's counter
// must be zero on entry: the row kernel clears it at its start, and a workgroup compacts once.
template <class Mem>
__device__ __forceinline__ uint32_t append_members(const uint32_t* ka, const uint32_t* ia, uint32_t n,
                                                   const Mem& mem, uint32_t* dkey, uint32_t* didx,
                                                   uint32_t cap, int slot, Smem& sm) {
  uint32_t* counter = &sm.kcount[slot];
  for (uint32_t base = threadIdx.x - (uint32_t)lane(); base < n; base += kRT * kVisU) {
    // wave-uniform loop: base is the wave's first item of the round
    uint32_t k[kVisU], x[kVisU];
    bool m[kVisU];
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < kVisU; ++u) {
      const uint32_t i = min(base + (uint32_t)lane() + u * kRT, n - 1);
      k[u] = ka[i];
      x[u] = ia[i];
    }
#pragma unroll
    for (int u = 0; u < kVisU; ++u) {
      const uint32_t i = base + (uint32_t)lane() + u * kRT;
      m[u] = i < n && mem(k[u], x[u]);
      c += m[u] ? 1u : 0u;
    }
    const uint32_t incl = wave_incl_scan(c);
    const uint32_t tot = wave_total(incl);
    uint32_t wbase = 0;
    if (tot) {
      if (lane() == 63) wbase = atomicAdd(counter, tot);
      wbase = (uint32_t)__builtin_amdgcn_readlane((int)wbase, 63);
    }
    uint32_t pos = wbase + incl - c;
#pragma unroll
    for (int u = 0; u < kVisU; ++u) {
      if (m[u]) {
        if (pos < cap) {
          dkey[pos] = k[u];
          didx[pos] = x[u];
        }
        ++pos;
      }
    }
  }
  bar();
  return *counter;
}

// ------------------------------------------------------------------ stream kernel
// Sample histogram word of bin b: four spare words after every 32 bins, so that lane l's 32
// bins (wave 0's search reads them as eight 16-byte loads) start 4*l banks apart.
__device__ __forceinline__ int hword(uint32_t b) { return (int)(b + 4u * (b >> 5)); }

// Wave 0 only: the highest bin b of a sample histogram with (count in bins >= b) >= thr.
// Writes res[0] = b, res[1] = count in bins > b.
__device__ __forceinline__ void search_hist(const uint32_t* hist, uint32_t thr, Smem1& sm) {
  constexpr int kG = 8;   // 8 groups of 4 bins per lane
  const int l = lane();
  const uint4* h4 = reinterpret_cast<const uint4*>(hist) + 9 * l;
  // only the lane sums stay live (the chunk's data occupies most registers); the one lane
  // that holds the bin reads its 32 bins again
  uint32_t lsum = 0;
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    const uint4 v = h4[i];
    lsum += v.x + v.y + v.z + v.w;
  }
  const uint32_t excl = wave_incl_suffix(lsum) - lsum;
  const uint64_t bal = __ballot(excl + lsum >= thr);
  const int L = bal ? 63 - __clzll((long long)bal) : -1;
  if (l == L) {
    uint32_t acc = excl;
    int bin = 0;
    bool done = false;
#pragma unroll
    for (int i = kG - 1; i >= 0; --i) {
      const uint4 v = h4[i];
      const uint32_t c[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (!done && acc + c[j] >= thr) { bin = 4 * i + j; done = true; }
        if (!done) acc += c[j];
      }
    }
    sm.res[0] = (uint32_t)(32 * L + bin);
    sm.res[1] = acc;
  }
}

// Wave 0 only: the same search over the 256-bin second level (four bins per lane); also
// writes res[1] = count in bins above b and res[2] = count in b.
__device__ __forceinline__ void search_hist2(const uint32_t* hist, uint32_t thr, Smem1& sm) {
  const int l = lane();
  const uint4 v = reinterpret_cast<const uint4*>(hist)[l];
  const uint32_t lsum = v.x + v.y + v.z + v.w;
  const uint32_t excl = wave_incl_suffix(lsum) - lsum;
  const uint64_t bal = __ballot(excl + lsum >= thr);
  const int L = bal ? 63 - __clzll((long long)bal) : -1;
  if (l == L) {
    const uint32_t c[4] = {v.x, v.y, v.z, v.w};
    uint32_t acc = excl;
    int j = 3;
    for (; j > 0; --j) {
      if (acc + c[j] >= thr) break;
      acc += c[j];
    }
    sm.res[0] = (uint32_t)(4 * L + j);
    sm.res[1] = acc;
    sm.res[2] = c[j];
  }
}

template <int NT>
__device__ __forceinline__ void fill_bytes_nt(uint8_t* dst, int64_t n, uint8_t v) {
  const uintptr_t a = (uintptr_t)dst;
  int64_t head = (int64_t)((4u - (a & 3u)) & 3u);
  if (head > n) head = n;
  for (int64_t i = threadIdx.x; i < head; i += NT) dst[i] = v;
  uint32_t* d32 = reinterpret_cast<uint32_t*>(dst + head);
  const int64_t n32 = (n - head) >> 2;
  const uint32_t wv = (uint32_t)v * 0x01010101u;
  for (int64_t i = threadIdx.x; i < n32; i += NT) d32[i] = wv;
  for (int64_t i = head + n32 * 4 + threadIdx.x; i < n; i += NT) dst[i] = v;
}

template <int MODE>
__global__ __launch_bounds__(kT1) __attribute__((amdgpu_waves_per_eu(7))) void ts_stream_kernel(Params P) {
  __shared__ Smem1 sm;
  const int b = (int)blockIdx.x;
  int L = b;
  if (P.xcd_map) {   // keep the chunks of a row on one XCD (workgroups go round-robin over 8)
    const int per = (P.rows * P.chunks) >> 3;
    L = (b & 7) * per + (b >> 3);
  }
  const int r = L / P.chunks;
  const int c = L - r * P.chunks;
  const int c0 = c * P.chunk_len;
  // the row's valid length: V, or its clamped length for top-k select rows of varying length
  const int vrow = (MODE == kModeTopk && P.lengths) ? max(0, min(P.lengths[r], P.V)) : P.V;
  const int n = max(0, min(P.chunk_len, vrow - c0));   // 0: the chunk lies past the row's end
  const float* base = P.x + (int64_t)r * P.stride + c0;
  const bool aligned = ((uintptr_t)base & 15u) == 0;
  const int nq = (n + 3) >> 2;
  const int qw = (nq + kW1 - 1) / kW1;
  // the wave index lives in a scalar register and the thread index is rebuilt from it and the
  // lane, so that no vector register holds the thread index through the whole kernel
  const int w = __builtin_amdgcn_readfirstlane(wave()), l = lane();
  const int tid = (w << 6) | l;
  const int q_lo = w * qw;
  const int q_hi = min(q_lo + qw, nq);
  const int nfull = n >> 2;

  // Issue every load of the chunk before consuming any. Addresses are clamped into the
  // chunk, so all loads are in bounds and every loaded value is an element of the chunk (a
  // lane past its wave's range reads a duplicate); duplicates cannot change a maximum or the
  // NaN flag, and candidate extraction masks them by position.
  uint4 raw[kS1];
  if (aligned && nfull > 0) {
#pragma unroll
    for (int s = 0; s < kS1; ++s) {
      const int q = min(q_lo + s * 64 + l, nfull - 1);
      // streamed once: a non-temporal load keeps the chunk from displacing cached data
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + q);
      raw[s] = make_uint4(v.x, v.y, v.z, v.w);
    }
    if (nfull * 4 < n) {   // one partial quad at the end of the chunk
#pragma unroll
      for (int s = 0; s < kS1; ++s) {
        const int q = q_lo + s * 64 + l;
        if (q == nfull && q < q_hi) {
          const uint32_t* s32 = reinterpret_cast<const uint32_t*>(base);
          raw[s].x = s32[4 * q];
          raw[s].y = s32[min(4 * q + 1, n - 1)];
          raw[s].z = s32[min(4 * q + 2, n - 1)];
          raw[s].w = s32[min(4 * q + 3, n - 1)];
        }
      }
    }
  } else if (n > 0) {
    const uint32_t* s32 = reinterpret_cast<const uint32_t*>(base);
#pragma unroll
    for (int s = 0; s < kS1; ++s) {
      const int e0 = 4 * (q_lo + s * 64 + l);
      raw[s].x = s32[min(e0, n - 1)];
      raw[s].y = s32[min(e0 + 1, n - 1)];
      raw[s].z = s32[min(e0 + 2, n - 1)];
      raw[s].w = s32[min(e0 + 3, n - 1)];
    }
  } else {   // empty chunk: nothing is loaded; -inf cannot raise a maximum or set a flag
#pragma unroll
    for (int s = 0; s < kS1; ++s) raw[s] = make_uint4(0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u);
  }
  // The row's parameters are read only now, so the chunk's loads above are already in
  // flight while these small loads resolve.
  const RowPlan rp = plan_row(P, MODE, r);
  const int path = rp.path;
  const bool cand = path == kPathCand;

  auto xval = [&](int s, int e) -> float {
    return __uint_as_float(e == 0 ? raw[s].x : (e == 1 ? raw[s].y : (e == 2 ? raw[s].z : raw[s].w)));
  };
  auto nvalid = [&](int s) -> int {   // valid elements in this lane's quad of slot s (0..4)
    const int q = q_lo + s * 64 + l;
    return (q < q_hi) ? min(max(n - 4 * q, 0), 4) : 0;
  };

  // The candidate threshold comes from a sample, the first kSampleSlots slots of every wave
  // (a quarter of the chunk spread over four segments), so it is known while the rest of
  // the chunk is still arriving. Any threshold is correct (the row kernel certifies); the
  // margin only makes a failed certification rare: the sample's count above the row's k-th
  // key has mean mu = k * ns / V, and the threshold sits mu + 5 sqrt(mu) + 5 keys down (a
  // Poisson tail below 1e-7 per workgroup for every k up to the fast path's limit).
  // Work happens on the fp32 values: a key >= threshold-key test is a float >= test against
  // the threshold's float (ordered keys are a monotone map of fp32, with -0 == +0 in both).
  // The threshold is located in a window of 256 bins of 2^16 keys below the sample maximum
  // (a relative 2^-7 of the value or finer), else in two levels over the whole key range: a
  // 2048-bin histogram of the top 11 key bits, then a 256-bin one of the next 8 bits of the
  // sample keys inside the chosen bin.
  // A sample element's key, recomputed at each use: the empty asm hides the value from
  // common-subexpression elimination, which would otherwise keep eight keys live across the
  // barriers (the chunk's 32 data registers leave no room for them).
  auto skey = [&](int s, int e) -> uint32_t {
    float xv = xval(s, e);
    asm volatile("" : "+v"(xv));
    return f2key(xv);
  };
  uint32_t thr = kKeyNegInf;   // reported: every valid non-NaN element with key >= thr is emitted
  float thr_f = -INFINITY;
  if (cand) {
    for (int i = tid; i < kHWords / 4; i += kT1) reinterpret_cast<uint4*>(sm.hist)[i] = make_uint4(0, 0, 0, 0);
    if (tid < kH2Bins) {
      sm.hist2[tid] = 0u;
      sm.hwin[tid] = 0u;
    }
    bar();   // LDS only: the loads above stay in flight
    {
      // the sample's largest value (fmaxf passes over NaN), one word per wave
      float smx = -INFINITY;
#pragma unroll
      for (int s = 0; s < kSampleSlots; ++s) {
        const int nv = nvalid(s);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float xv = xval(s, e);
          asm volatile("" : "+v"(xv));
          if (e < nv) smx = fmaxf(smx, xv);
        }
      }
      const uint32_t wmx = wave_max(f2key(smx));
      if (l == 0) sm.wmax[w] = wmx;
    }
    uint32_t ns = 0;   // valid sample elements of the workgroup
#pragma unroll
    for (int ww = 0; ww < kW1; ++ww) {
      const int lo_q = ww * qw, hi_q = min(lo_q + qw, nq);
      const int e_hi = min(min(4 * (lo_q + 64 * kSampleSlots), 4 * hi_q), n);
      ns += (uint32_t)max(e_hi - 4 * lo_q, 0);
    }
    const float mu = (float)rp.k_eff * (float)ns / (float)P.V;
    const uint32_t jt = (uint32_t)ceilf(mu + 5.0f * sqrtf(mu) + 5.0f);
    if (jt < ns) {
      // Window histogram: 256 bins of 2^16 keys (aligned to the key's top 16 bits) reaching
      // down from the sample maximum's bin, about two binades. When the sample's jt-th
      // largest key lies inside, one pass and one search locate it, and only the sample keys
      // near the top touch LDS. Otherwise the two-level search over the whole key range
      // below runs instead.
      bar();
      const uint32_t kmw = max(max(sm.wmax[0], sm.wmax[1]), max(sm.wmax[2], sm.wmax[3])) >> 16;
#pragma unroll
      for (int s = 0; s < kSampleSlots; ++s) {
        const int nv = nvalid(s);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t d = kmw - (skey(s, e) >> 16);   // NaN keys above the maximum wrap high
          if (e < nv && d < (uint32_t)kH2Bins) atomicAdd(&sm.hwin[d], 1u);
        }
      }
      bar();
      // every wave searches the 256 bins itself (four per lane, bin 0 = the top), so no
      // barrier follows: the first bin where the running count from the top reaches jt
      const uint4 hv = reinterpret_cast<const uint4*>(sm.hwin)[l];
      const uint32_t c4[4] = {hv.x, hv.y, hv.z, hv.w};
      const uint32_t lsum = hv.x + hv.y + hv.z + hv.w;
      const uint32_t incl = wave_incl_scan(lsum);
      const uint64_t hit = __ballot(incl >= jt);
      uint32_t tk = 0, in_bin = 0, need = 0;
      int rem = 0;
      if (hit) {
        const int L = (int)__builtin_ctzll(hit);
        uint32_t acc = incl - lsum, jb = 3;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          if (jb == 3u && acc + c4[j] >= jt) jb = (uint32_t)j;
          if (jb == 3u) acc += c4[j];
        }
        const uint32_t b = 4u * (uint32_t)L + (uint32_t)__builtin_amdgcn_readlane((int)jb, L);
        const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)acc, L);
        tk = (kmw - b) << 16;
        in_bin = (uint32_t)__builtin_amdgcn_readlane((int)(jb == 0 ? c4[0] : jb == 1 ? c4[1] : jb == 2 ? c4[2] : c4[3]), L);
        need = jt - above;   // >= 1
        rem = 16;
      } else {
        // the jt-th largest lies below the window: 2048 bins of the top 11 key bits, then
        // 256 of the next 8 inside the chosen bin
#pragma unroll
        for (int s = 0; s < kSampleSlots; ++s) {
          const int nv = nvalid(s);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e < nv) atomicAdd(&sm.hist[hword(skey(s, e) >> (32 - kHBits))], 1u);
        }
        bar();   // sample histogram complete
        if (w == 0) search_hist(sm.hist, jt, sm);
        bar();
        const uint32_t b1 = sm.res[0];
        const uint32_t need2 = jt - sm.res[1];   // >= 1
#pragma unroll
        for (int s = 0; s < kSampleSlots; ++s) {
          const int nv = nvalid(s);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = skey(s, e);
            if (e < nv && (key >> (32 - kHBits)) == b1)
              atomicAdd(&sm.hist2[(key >> (32 - kHBits - kH2Bits)) & (kH2Bins - 1)], 1u);
          }
        }
        bar();
        if (w == 0) search_hist2(sm.hist2, need2, sm);
        bar();
        tk = (b1 << (32 - kHBits)) | (sm.res[0] << (32 - kHBits - kH2Bits));
        in_bin = sm.res[2];
        need = need2 - sm.res[1];
        rem = 32 - kHBits - kH2Bits;
      }
      // Narrow value ranges (a near-uniform row puts every sampled key in one bin): refine
      // through the remaining key bits, at most 8 at a time, while the chosen bin still holds
      // more than kRefine sampled keys. Never taken on spread-out rows.
#pragma unroll 1
      for (int lvl = 0; lvl < 2 && in_bin > (uint32_t)kRefine && rem > 0; ++lvl) {
        const int bits = min(kH2Bits, rem);
        const int sh = rem - bits;
        const uint32_t pre = tk >> (sh + bits);
        if (tid < kH2Bins) sm.hist2[tid] = 0u;
        bar();
#pragma unroll
        for (int s = 0; s < kSampleSlots; ++s) {
          const int nv = nvalid(s);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = skey(s, e);
            // narrow rows put whole waves in one bin: one atomic per wave then
            if (e < nv && (key >> (sh + bits)) == pre) hist_add(sm.hist2, (key >> sh) & ((1u << bits) - 1u));
          }
        }
        bar();
        if (w == 0) search_hist2(sm.hist2, need, sm);
        bar();
        tk |= sm.res[0] << sh;
        in_bin = sm.res[2];
        need -= sm.res[1];
        rem = sh;
      }
      if (tk > kKeyNegInf) {
        thr = tk;
        thr_f = key2f(tk);
      }
    }
  }

  // From here on every wave works alone. Each slot as it arrives: the quad maximum feeds the
  // wave maximum and the candidate test. It is the IEEE 754-2019 maximum (two v_maximum3),
  // which propagates NaN, so a lane's running maximum is NaN exactly when one of its elements
  // was: the NaN flag needs no compares of its own (a row holding a NaN is rejected whatever
  // its maximum). A quad whose maximum reaches the threshold is staged (values and quad
  // index) at its ballot rank, which keeps the staged quads in id order; ranks past the
  // stage's end wrap around it (distinct addresses, no write conflicts), and the stage's
  // contents are then unused: more hits than it holds take the register path below. One loop serves every path (off the
  // candidate path the test compares against NaN and never hits), so that each slot is
  // processed as it arrives, with no branch besides the stage write's: every instruction
  // after the last data arrive is on the critical path.
  const float stage_thr = cand ? thr_f : __builtin_nanf("");
  float fmx = -INFINITY;
  uint32_t run = 0;
#pragma unroll
  for (int s = 0; s < kS1; ++s) {
    const float mq = __builtin_elementwise_maximum(__builtin_elementwise_maximum(xval(s, 0), xval(s, 1)),
                                                   __builtin_elementwise_maximum(xval(s, 2), xval(s, 3)));
    fmx = __builtin_elementwise_maximum(fmx, mq);
    const bool hit = mq >= stage_thr;
    const uint64_t mk = __ballot(hit);
    const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, run)) &
                         ((uint32_t)kQStage - 1u);
    if (hit) {
      sm.stage_v[w][pos] = raw[s];
      sm.stage_q[w][pos] = (uint32_t)(q_lo + s * 64 + l);
    }
    run += (uint32_t)__popcll(mk);
  }
  const bool nan_lane = __builtin_isnan(fmx);
  const uint32_t kmax = wave_max(f2key(nan_lane ? -INFINITY : fmx));
  uint32_t flags = (__ballot(nan_lane) != 0ull) ? kFlagNan : 0u;
  const int64_t seg = ((int64_t)r * P.chunks + c) * kW1 + w;
  if (MODE == kModeSample && P.wsum) {
    // [LOGP] "Design: the numeric contract": the wave's share of S = sum exp((x - m) / T),
    // here relative to the wave maximum (the row kernel rescales each share to the row
    // maximum). exp(y) = 2^(y log2 e) in fp32 by the hardware exp2 (results below 2^-126
    // flush to 0: the share holds the maximum's 1, so they are below its resolution), four
    // elements per fp32 partial, binary64 accumulation, a fixed lane tree: the same bits for
    // every launch of this vocabulary.
    double acc = 0.0;
    if (rp.bad == TS_ROW_OK && rp.t > 0.0f && kmax > kKeyNegInf && kmax < kKeyPosInf) {
      const float m_w = key2f(kmax);
      const float c2f = (float)(1.4426950408889634 / (double)rp.t);
#pragma unroll
      for (int s = 0; s < kS1; ++s) {
        const int nv = nvalid(s);
        float ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < nv) ps += __builtin_amdgcn_exp2f((xval(s, e) - m_w) * c2f);
        acc += (double)ps;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (l == 0) P.wsum[seg] = acc;
  }

  uint32_t count = 0, kmax_idx = 0xFFFFFFFFu;
  float best_s = -INFINITY;
  int32_t best_idx = 0x7FFFFFFF;

  if (cand) {
    uint2* out = P.cand + seg * P.cap_w;
    const uint32_t cap = (uint32_t)P.cap_w;
    if (run <= (uint32_t)kQStage) {
      wave_lds_sync();
      // Extract the staged quads' elements >= thr in id order: a wave scan of the per-lane
      // counts gives each lane its first position, and a lane's elements follow in order.
      // When the wave's slice has room for the whole batch (always, unless the caller capped
      // the slices) the stores need no bound check.
      for (uint32_t i0 = 0; i0 < run; i0 += 64) {
        const uint32_t i = i0 + (uint32_t)l;   // < kQStage: entries at or past run are stale, masked below
        const uint4 v = sm.stage_v[w][i];
        const uint32_t q = sm.stage_q[w][i];
        const float y[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
        const int e_lim = (i < run && (int)q < q_hi) ? min(n - 4 * (int)q, 4) : 0;   // valid elements of the quad
        uint32_t at[4];   // position among the lane's selected elements
        bool sel[4];
        uint32_t cc = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sel[e] = e < e_lim && y[e] >= thr_f;
          at[e] = cc;
          cc += sel[e] ? 1u : 0u;
        }
        const uint32_t incl = wave_incl_scan(cc);
        const uint32_t pos = count + incl - cc;
        const uint32_t total = wave_total(incl);
        const uint32_t id0 = (uint32_t)(c0 + 4 * (int)q);
        if (count + total <= cap) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (sel[e]) out[pos + at[e]] = make_uint2(f2key(y[e]), id0 + (uint32_t)e);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (sel[e] && pos + at[e] < cap) out[pos + at[e]] = make_uint2(f2key(y[e]), id0 + (uint32_t)e);
        }
        count += total;
      }
    } else {
      // More hits than the stage holds. When every valid element of the wave is one key
      // (a constant stretch of the row, e.g. an all-equal row) the slice is uniform and
      // stores nothing; otherwise the same ordered list, straight from registers.
      // Every value this wave loaded is an element of the chunk (lanes past the wave's range
      // hold duplicates), so comparing all of them with the maximum's bits is a test that can
      // only be stricter than needed (and needs no validity masks).
      const uint32_t mbits = __float_as_uint(key2f(kmax));
      uint32_t other = 0u;
#pragma unroll
      for (int s = 0; s < kS1; ++s)
        other |= (raw[s].x ^ mbits) | (raw[s].y ^ mbits) | (raw[s].z ^ mbits) | (raw[s].w ^ mbits);
      if (__ballot(other != 0u) == 0ull) {
        // m_w >= thr_f: the wave has hits, every one of them equal to m_w
        flags |= kFlagUniform;
        count = (uint32_t)max(0, min(4 * q_hi, n) - 4 * q_lo);
      } else {
#pragma unroll
      for (int s = 0; s < kS1; ++s) {
        const int nv = nvalid(s);
        uint64_t mk[4];
        uint32_t slot_cnt = 0, lane_off = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mk[e] = __ballot(e < nv && xval(s, e) >= thr_f);
          slot_cnt += (uint32_t)__popcll(mk[e]);
          lane_off += mbcnt(mk[e]);
        }
        uint32_t pos = count + lane_off;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((mk[e] >> l) & 1ull) {
            if (pos < cap) out[pos] = make_uint2(f2key(xval(s, e)), (uint32_t)(c0 + 4 * (q_lo + s * 64 + l) + e));
            ++pos;
          }
        }
        count += slot_cnt;
      }
      }
    }
    if (count > cap && !(flags & kFlagUniform)) {
      flags |= kFlagOverflow;
      count = cap;
    }
  } else if (path == kPathGreedy) {
    const float m_w = key2f(kmax);
    uint32_t mi = 0xFFFFFFFFu;
#pragma unroll
    for (int s = 0; s < kS1; ++s) {
      const int nv = nvalid(s);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (e < nv && xval(s, e) == m_w) mi = min(mi, (uint32_t)(c0 + 4 * (q_lo + s * 64 + l) + e));
      }
    }
    kmax_idx = wave_min(mi);
  } else if (path == kPathFull && MODE == kModeSample) {
    // Gumbel argmax of the wave's elements relative to the wave maximum (one Philox block
    // per quad).
    const float m_w = key2f(kmax);
    const uint64_t sd = P.seed[r];
    // the key is uniform: scalar registers keep the ten round keys out of the vector file
    const uint32_t k0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sd);
    const uint32_t k1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sd >> 32));
    const float inv_t = 1.0f / rp.t;   // one rounding per row instead of a division per token
    // Branch-free over the slots, so that the eight Philox chains can interleave: every
    // lane draws for every slot (a lane past its range draws for ids it then ignores), and
    // the argmax keeps (score, lowest id) through selects, a tree within each quad. The
    // winner does not depend on the order of the comparisons (ties compare ids).
    auto better = [](float sa, int32_t ia, float sb, int32_t ib) {
      return sb > sa || (sb == sa && ib < ia);
    };
    float bs = -INFINITY;
    int32_t bi = 0x7FFFFFFF;
#pragma unroll
    for (int s = 0; s < kS1; ++s) {
      const int q = q_lo + s * 64 + l;
      const int nv = nvalid(s);
      const uint32_t tok0 = (uint32_t)(c0 + 4 * q);
      const uint4 wd = philox4x32_10(tok0 >> 2, (uint32_t)r, k0, k1);
      const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
      float sc[4];
      int32_t id[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float g = gumbel_from_uniform(uniform_from_word(words[e]));
        sc[e] = e < nv ? (xval(s, e) - m_w) * inv_t + g : -INFINITY;
        id[e] = e < nv ? (int32_t)(tok0 + e) : 0x7FFFFFFF;
      }
      const bool b01 = better(sc[0], id[0], sc[1], id[1]);
      const float s01 = b01 ? sc[1] : sc[0];
      const int32_t i01 = b01 ? id[1] : id[0];
      const bool b23 = better(sc[2], id[2], sc[3], id[3]);
      const float s23 = b23 ? sc[3] : sc[2];
      const int32_t i23 = b23 ? id[3] : id[2];
      const bool bq = better(s01, i01, s23, i23);
      const float sq = bq ? s23 : s01;
      const int32_t iq = bq ? i23 : i01;
      const bool bb = better(bs, bi, sq, iq);
      bs = bb ? sq : bs;
      bi = bb ? iq : bi;
    }
    wave_argmax(bs, bi);
    best_s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bs), 63));
    best_idx = __builtin_amdgcn_readlane(bi, 63);
  }

  if (MODE == kModeTopp && P.out_mask) {
    fill_bytes_nt<kT1>(P.out_mask + (int64_t)r * P.V + c0, n, (path == kPathFull) ? (uint8_t)1 : (uint8_t)0);
  }
  if (c == 0 && tid == 0 && split_row(P, rp)) P.nuc[r].ticket = 0u;   // the split nucleus's counter
  if (path == kPathNucleus) {
    // this workgroup's share of zeroing the row's nucleus histograms
    uint4* z = reinterpret_cast<uint4*>(P.nuc + r);
    const int nz = (int)(sizeof(NucRow) / sizeof(uint4));
    const int per = (nz + P.chunks - 1) / P.chunks;
    for (int i = c * per + tid; i < min(nz, (c + 1) * per); i += kT1) z[i] = make_uint4(0, 0, 0, 0);
  }
  if (l == 0) {
    WaveInfo wi;
    wi.count = count;
    wi.thr = thr;
    wi.kmax = kmax;
    wi.flags = flags;
    wi.kmax_idx = kmax_idx;
    wi.best_s = best_s;
    wi.best_idx = best_idx;
    wi.first = (flags & kFlagUniform) ? (uint32_t)(c0 + 4 * q_lo) : 0u;
    P.info[seg] = wi;
  }
}

// ------------------------------------------------------------------ row kernel
// Top-k select output in the canonical order (value descending, id ascending): the cnt
// selected items sit unordered in a[0, cnt) as (key << 32 | ~id); a bitonic network sorts
// them descending in LDS (padding 0 sorts last: every real key is above 0), then row slot j
// gets off + id_j. cnt <= cap, cap a power of two.
__device__ __forceinline__ void emit_value_order(uint64_t* a, uint32_t cnt, uint32_t cap, int32_t* orow,
                                                 uint32_t kmx, int32_t off) {
  uint32_t nn = 1;
  while (nn < cnt) nn <<= 1;
  for (uint32_t i = cnt + threadIdx.x; i < nn; i += kRT) a[i] = 0ull;
  bar();
  for (uint32_t kk = 2; kk <= nn; kk <<= 1) {
    for (uint32_t jj = kk >> 1; jj > 0; jj >>= 1) {
      for (uint32_t i = threadIdx.x; i < nn; i += kRT) {
        const uint32_t l = i ^ jj;
        if (l > i) {
          const uint64_t x = a[i], y = a[l];
          const bool desc = (i & kk) == 0;   // this pair's block sorts descending
          if (desc ? x < y : x > y) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      bar();
    }
  }
  (void)cap;
  for (uint32_t j = threadIdx.x; j < cnt && j < kmx; j += kRT) orow[j] = off + (int32_t)(~(uint32_t)a[j]);
}

// Thread 0, sampling with logprobs: [LOGP] "Design: the numeric contract" with temperature in
// the epilogue: logp = min(x_t / T - lse, 0) for the sampled token t. A rejected row
// (tok < 0) gets NaN for both; greedy rows (T == 0) get lse = +inf and logp = 0.
__device__ __forceinline__ void put_logp(const Params& P, int r, int32_t tok, float t, double lse) {
  if (!P.out_logp && !P.out_lse) return;
  float lp = __builtin_nanf(""), ls = __builtin_nanf("");
  if (tok >= 0 && t == 0.0f) {
    lp = 0.0f;
    ls = INFINITY;
  } else if (tok >= 0) {
    const double xt = (double)P.x[(int64_t)r * P.stride + tok];
    lp = (float)fmin(xt / (double)t - lse, 0.0);
    ls = (float)lse;
  }
  if (P.out_logp) P.out_logp[r] = lp;
  if (P.out_lse) P.out_lse[r] = ls;
}

template <int MODE>
__device__ __forceinline__ void finish_cand(const Params& P, const RowPlan& rp, int r, uint32_t kmax, uint32_t klo,
                                            uint64_t seed, uint32_t total, const Sel& sk, Smem& sm, double lse) {
  // K = the candidates selected by sk, compacted into (kkey, kidx) in any order: every step
  // below is order-independent.
  const uint32_t nk = min(append_members(sm.ckey, sm.cidx, total,
                                         [&](uint32_t rk, uint32_t idx) { return sel_member(sk, rk, idx); },
                                         sm.kkey, sm.kidx, (uint32_t)kFastK, 0, sm),
                          (uint32_t)kFastK);
  const float m = key2f(kmax);
  const float t = rp.t;
  auto kvis = [&](auto f) { lds_for(sm.kkey, sm.kidx, nk, f); };
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  float* const gsc = reinterpret_cast<float*>(sm.ckey);   // Gumbel scores, gsc[i] for item i of K
  Sel sp = sel_all();
  uint32_t kept = nk;
  if (rp.p != 1.0f) {
    // One visit of K computes every weight once: Z, and the counts and masses of the mass
    // select's first pass. One 64-bit word floor(w * 2^S) per weight sums exactly
    // (S = 63 - bitlen(|K|); truncation costs < |K| * 2^-S of Z >= 1).
    const int S = 63 - bitlen(nk);
    const double c2 = kLog2e / (double)t;
    auto wmass = [&](uint32_t rk) { return mass32_of(weight32(rk, m, c2), S); };
    const Digit g = first_digit(kmax, klo);
    const bool pre = g.lo > 0;
    // When sampling, the same visit draws every item's Gumbel score into gsc[i] (the
    // candidate keys are dead once K is compacted), so the draw overlaps the mass select
    // and no kept-set compaction is needed.
    uint64_t zh = 0, zl = 0;
    for (uint32_t base = threadIdx.x; base < nk; base += kRT * kVisU) {
      uint32_t kr[kVisU], kx[kVisU];
#pragma unroll
      for (int u = 0; u < kVisU; ++u) {
        const uint32_t i = min(base + u * kRT, nk - 1);   // clamped: in bounds, unused past nk
        kr[u] = sm.kkey[i];
        kx[u] = sm.kidx[i];
      }
#pragma unroll
      for (int u = 0; u < kVisU; ++u) {
        const uint32_t i = base + u * kRT;
        if (i < nk) {
          const uint64_t q = wmass(kr[u]);
          zh += q;
          if (pre) {
            const uint32_t b = (kr[u] >> g.sh) & g.dm;
            atomicAdd(&sm.hist[b], 1u);
            atomicAdd((unsigned long long*)&sm.mhi[b], (unsigned long long)q);
          }
          if (MODE == kModeSample) gsc[i] = gumbel_score(kr[u], kx[u], m, t, (uint32_t)r, k0, k1);
        }
      }
    }
    // [TOPP] reference steps 4-5 in exact fixed point: keep the shortest prefix whose mass is
    // >= p * Z, i.e. >= ceil(p * Z) since masses are integers. With the first pass prebuilt,
    // Z is the histogram's total and the first search computes the target from it; else a
    // block sum of the items' masses gives it.
    if (pre) {
      bar();   // completes the atomics and the scores' stores
      sp = select_mass(kvis, wmass, 0ull, nk, kmax, klo, 0u, (uint32_t)(P.V - 1), sm, kept, true, 0ull, 0u, rp.p);
    } else {
      block_sum2_u64<kRW>(zh, zl, sm.red64);   // its barriers also complete the stores
      const uint64_t target_fx = topp_target(rp.p, zh);
      sp = select_mass(kvis, wmass, target_fx, nk, kmax, klo, 0u, (uint32_t)(P.V - 1), sm, kept, false);
    }
  }
  // min-p after top-p: the members of P whose weight is >= min_p (the maximum has weight 1),
  // again a canonical prefix ([LOGP] relay order temperature -> top-k -> top-p -> min-p).
  const double c2m = kLog2e / (double)t;
  const bool minp_on = rp.minp > 0.0f;   // uniform: the weight is computed only when min-p is on
  auto keep = [&](uint32_t rk, uint32_t idx) {
    bool in = sel_member(sp, rk, idx);
    if (minp_on) in = in && weight32(rk, m, c2m) >= rp.minp;
    return in;
  };
  if (MODE == kModeTopp) {
    if (rp.minp > 0.0f) {
      uint64_t c = 0, z = 0;
      kvis([&](uint32_t rk, uint32_t idx) { c += keep(rk, idx) ? 1u : 0u; });
      block_sum2_u64<kRW>(c, z, sm.red64);
      kept = (uint32_t)c;
    }
    if (threadIdx.x == 0) P.out_kept[r] = (int32_t)kept;
    if (P.out_mask) {
      uint8_t* mrow = P.out_mask + (int64_t)r * P.V;
      kvis([&](uint32_t rk, uint32_t idx) {
        if (keep(rk, idx) && idx < (uint32_t)P.V) mrow[idx] = 1;
      });
    }
  } else {
    // Gumbel-max over the kept set: the scores drawn above, masked by membership; without
    // top-p P = K and the scores are drawn here.
    float bs = -INFINITY;
    int32_t bi = 0x7FFFFFFF;
    if (rp.p != 1.0f) {
      kvis_i(nk, [&](uint32_t i, uint32_t rk, uint32_t idx) {
        if (keep(rk, idx)) {
          const float sc = gsc[i];
          if (sc > bs || (sc == bs && (int32_t)idx < bi)) { bs = sc; bi = (int32_t)idx; }
        }
      }, sm);
    } else {
      for (uint32_t i = threadIdx.x; i < nk; i += kRT) {
        const uint32_t idx = sm.kidx[i];
        if (!keep(sm.kkey[i], idx)) continue;
        const float sc = gumbel_score(sm.kkey[i], idx, m, t, (uint32_t)r, k0, k1);
        if (sc > bs || (sc == bs && (int32_t)idx < bi)) { bs = sc; bi = (int32_t)idx; }
      }
    }
    const int32_t tok = block_argmax<kRW>(bs, bi, sm.reds, sm.redi, nullptr, true);
    if (threadIdx.x == 0) {
      P.out_token[r] = tok;
      put_logp(P, r, tok, t, lse);
    }
  }
}

// Visits a row in global memory, f(key, id) for each of its first V elements (ids rising
// along a thread's calls): 8 float4 loads per thread per round with the next round in flight
// when the row is 16-byte aligned, else 16 scalar loads per thread per round.
template <class F>
__device__ __forceinline__ void visit_row(const float* row, uint32_t V, F f) {
  const bool al4 = ((uintptr_t)row & 15u) == 0;
  if (al4) {   // 8 float4 loads per thread per round; the next round loads during this one
    const uint32_t nq = V >> 2;
    const uint4* rq = reinterpret_cast<const uint4*>(row);
    uint4 v[8], nx[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t q = u * kRT + threadIdx.x;
      v[u] = q < nq ? rq[q] : make_uint4(0, 0, 0, 0);
    }
    for (uint32_t base = 0; base < nq; base += kRT * 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t q = base + kRT * 8 + u * kRT + threadIdx.x;
        nx[u] = q < nq ? rq[q] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t q = base + u * kRT + threadIdx.x;
        if (q < nq) {
          f(f2key(__uint_as_float(v[u].x)), 4 * q);
          f(f2key(__uint_as_float(v[u].y)), 4 * q + 1);
          f(f2key(__uint_as_float(v[u].z)), 4 * q + 2);
          f(f2key(__uint_as_float(v[u].w)), 4 * q + 3);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = nx[u];
    }
    for (uint32_t i = 4 * nq + threadIdx.x; i < V; i += kRT) f(f2key(row[i]), i);
  } else {
    for (uint32_t base = 0; base < V; base += kRT * 16) {
      uint32_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint32_t j = base + u * kRT + threadIdx.x;
        v[u] = 0;
        if (j < V) v[u] = f2key(row[j]);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint32_t j = base + u * kRT + threadIdx.x;
        if (j < V) f(v[u], j);
      }
    }
  }
}

template <int MODE>
__device__ __forceinline__ void row_stream(const Params& P, const RowPlan& rp, int r, uint32_t kmax,
                                           uint32_t kmin, uint64_t seed, Smem& sm, double lse) {
  // The exact path over the raw row in global memory, one read of the row per pass.
  const float* row = P.x + (int64_t)r * P.stride;
  const uint32_t V = (uint32_t)rp.n;   // the row's valid length
  auto rvis = [&](auto f) { visit_row(row, V, f); };
  const uint32_t ke = (uint32_t)rp.k_eff;
  Sel sk = sel_all();
  if (ke < V) sk = select_topk(rvis, ke, V, kmax, kmin, 0u, V - 1, sm);
  if (MODE == kModeTopk) {
    int32_t* orow = P.out_idx + (int64_t)r * P.k_max;
    const uint32_t kmx = (uint32_t)P.k_max;
    const int32_t off = P.offsets ? P.offsets[r] : 0;
    if (P.order == TS_ORDER_VALUE) {
      // K (<= 8192 items, checked by the host) gathered from the row into the free candidate
      // arrays, then sorted there
      uint64_t* a = reinterpret_cast<uint64_t*>(sm.ckey);
      rvis([&](uint32_t rk, uint32_t idx) {
        if (sel_member(sk, rk, idx)) {
          const uint32_t at = atomicAdd(&sm.bcount, 1u);
          if (at < (uint32_t)kValueOrderMax) a[at] = ((uint64_t)rk << 32) | (uint32_t)~idx;
        }
      });
      bar();
      const uint32_t nk = min(sm.bcount, (uint32_t)kValueOrderMax);
      bar();
      if (threadIdx.x == 0) sm.bcount = 0;
      emit_value_order(a, nk, (uint32_t)kValueOrderMax, orow, kmx, off);
    } else {
      uint32_t run = 0;
      emit_ordered<4>(V, [&](uint32_t i, uint32_t& rk, uint32_t& idx) { rk = f2key(row[i]); idx = i; },
                      [&](uint32_t rk, uint32_t idx) { return sel_member(sk, rk, idx); },
                      [&](uint32_t pos, uint32_t idx) { if (pos < kmx) orow[pos] = off + (int32_t)idx; }, run, sm);
    }
    for (int i = rp.k_eff + threadIdx.x; i < P.k_max; i += kRT) orow[i] = -1;
    return;
  }
  const float m = key2f(kmax);
  const float t = rp.t;
  auto kvis = [&](auto f) {
    rvis([&](uint32_t rk, uint32_t idx) {
      if (sel_member(sk, rk, idx)) f(rk, idx);
    });
  };
  Sel sp = sel_all();
  uint32_t kept = ke;
  if (rp.p != 1.0f) {
    // One visit of K: Z and the mass select's first pass (counts and masses of the first
    // digit over [klo, kmax], where every key of K lies).
    const int S = 63 - bitlen(ke);
    const double c2 = kLog2e / (double)t;
    auto wmass = [&](uint32_t rk) { return mass32_of(weight32(rk, m, c2), S); };
    const uint32_t klo = (sk.lo >= 32) ? kmin : max(kmin, shl(sk.prefix, sk.lo));
    const Digit g = first_digit(kmax, klo);
    const bool pre = g.lo > 0;
    uint64_t zh = 0, zl = 0;
    kvis([&](uint32_t rk, uint32_t) {
      const uint64_t q = wmass(rk);
      zh += q;
      if (pre) {
        const uint32_t b = (rk >> g.sh) & g.dm;
        hist_add(sm.hist, b);
        atomicAdd((unsigned long long*)&sm.mhi[b], (unsigned long long)q);
      }
    });
    block_sum2_u64<kRW>(zh, zl, sm.red64);   // its barriers also complete the atomics
    sp = select_mass<true>(kvis, wmass, topp_target(rp.p, zh), ke, kmax, klo, 0u, V - 1, sm, kept, pre);
  }
  // min-p after top-p (as on the candidate path)
  const double c2m = kLog2e / (double)t;
  const bool minp_on = rp.minp > 0.0f;   // uniform: the weight is computed only when min-p is on
  auto keep = [&](uint32_t rk, uint32_t idx) {
    bool in = sel_member(sp, rk, idx);
    if (minp_on) in = in && weight32(rk, m, c2m) >= rp.minp;
    return in;
  };
  if (MODE == kModeTopp) {
    if (rp.minp > 0.0f) {
      uint64_t c = 0, z = 0;
      kvis([&](uint32_t rk, uint32_t idx) { c += keep(rk, idx) ? 1u : 0u; });
      block_sum2_u64<kRW>(c, z, sm.red64);
      kept = (uint32_t)c;
    }
    if (threadIdx.x == 0) P.out_kept[r] = (int32_t)kept;
    if (P.out_mask) {
      uint8_t* mrow = P.out_mask + (int64_t)r * P.V;
      kvis([&](uint32_t rk, uint32_t idx) {
        if (keep(rk, idx)) mrow[idx] = 1;
      });
    }
  } else {
    // Gumbel-max over P. Per slab of kSlab row elements the members of P are compacted
    // into LDS first, so that noise is drawn only for them (members are scattered: drawing
    // in place would run the generator in nearly every wave for every element).
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    constexpr int kPer = kSlab / kRT;
    float bs = -INFINITY;
    int32_t bi = 0x7FFFFFFF;
    auto load = [&](uint32_t s0, uint32_t (&key)[kPer]) {
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const uint32_t i = s0 + (uint32_t)(u * kRT) + threadIdx.x;
        key[u] = i < V ? __float_as_uint(row[i]) : 0u;
      }
    };
    uint32_t cur[kPer], nxt[kPer];
    load(0, cur);
    for (uint32_t s0 = 0; s0 < V; s0 += (uint32_t)kSlab) {
      load(s0 + (uint32_t)kSlab, nxt);   // the next slab loads while this one is processed
      uint64_t bal[kPer];
      uint32_t tot = 0;
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const uint32_t i = s0 + (uint32_t)(u * kRT) + threadIdx.x;
        cur[u] = f2key(__uint_as_float(cur[u]));
        bool mem = i < V && sel_member(sk, cur[u], i) && sel_member(sp, cur[u], i);
        if (minp_on) mem = mem && weight32(cur[u], m, c2m) >= rp.minp;
        bal[u] = __ballot(mem);
        tot += (uint32_t)__popcll(bal[u]);
      }
      if (tot) {   // wave-uniform: one reservation per wave and slab
        uint32_t wbase = 0;
        if (lane() == 0) wbase = atomicAdd(&sm.bcount, tot);
        wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)wbase);
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          if ((bal[u] >> lane()) & 1ull) {
            const uint32_t at = wbase + mbcnt(bal[u]);   // < kSlab: one slab's members
            sm.ckey[at] = cur[u];
            sm.cidx[at] = s0 + (uint32_t)(u * kRT) + threadIdx.x;
          }
          wbase += (uint32_t)__popcll(bal[u]);
        }
      }
      bar();
      const uint32_t nq = sm.bcount;
      // four independent draws per thread per step
      for (uint32_t q0 = threadIdx.x; q0 < nq; q0 += 4 * kRT) {
        float sc[4];
        uint32_t id[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t q = min(q0 + (uint32_t)(e * kRT), nq - 1u);
          id[e] = sm.cidx[q];
          sc[e] = gumbel_score(sm.ckey[q], id[e], m, t, (uint32_t)r, k0, k1);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (q0 + (uint32_t)(e * kRT) < nq && (sc[e] > bs || (sc[e] == bs && (int32_t)id[e] < bi))) {
            bs = sc[e];
            bi = (int32_t)id[e];
          }
        }
      }
      bar();
      if (threadIdx.x == 0) sm.bcount = 0;
#pragma unroll
      for (int u = 0; u < kPer; ++u) cur[u] = nxt[u];
      bar();
    }
    const int32_t tok = block_argmax<kRW>(bs, bi, sm.reds, sm.redi, nullptr, true);
    if (threadIdx.x == 0) {
      P.out_token[r] = tok;
      put_logp(P, r, tok, t, lse);
    }
  }
}

// The row's candidates when there are more than LDS holds: they stay in their slices in
// global memory (sm.segoff holds the slices' exclusive offsets and the total). One pass
// counts their first digit over [cmin, kmax] and finds the bin holding the ke-th largest;
// the candidates with keys at or above that bin's low edge (a superset of the candidates'
// top ke) are then counted per slice and gathered into LDS in id order. When every
// candidate key is equal, the first ke in id order are gathered directly. Returns the
// number gathered, 0 when they would not fit; *lo_key is a lower bound of their keys.
__device__ __forceinline__ uint32_t gather_filtered(const Params& P, int r, int nseg, uint32_t ke, uint32_t kmax,
                                                    uint32_t cmin, Smem& sm, uint32_t* lo_key) {
  const uint2* base = P.cand + (int64_t)r * nseg * P.cap_w;
  const uint32_t j = (uint32_t)lane();
  // per_batch(sb, cnt, first, gs): kGatherB slices sb, sb + kRW, ... of this wave, with
  // entry `lane` of each already loaded into first[u]
  auto batches = [&](auto per_batch) {
    for (int sb = wave(); sb < nseg; sb += kRW * kGatherB) {
      uint32_t cnt[kGatherB];
#pragma unroll
      for (int u = 0; u < kGatherB; ++u) {
        const int sl = min(sb + u * kRW, nseg);   // slice nseg has no candidates
        cnt[u] = sm.segoff[min(sl + 1, nseg)] - sm.segoff[sl];
      }
      const uint2* gs = base + (int64_t)sb * P.cap_w;
      uint2 first[kGatherB];
#pragma unroll
      for (int u = 0; u < kGatherB; ++u) {
        first[u] = make_uint2(0, 0);
        if (j < cnt[u]) first[u] = gs[(int64_t)u * kRW * P.cap_w + j];
      }
      per_batch(sb, cnt, first, gs);
    }
  };
  // f(jj, w, ok) over a slice's entries in id order, 64 per (wave-uniform) call; entries
  // past the first 64 load 8 rounds at a time
  auto slice_chunks = [&](const uint2* gsl, uint32_t cnt, uint2 first, auto f) {
    f(j, first, j < cnt);
    for (uint32_t j0 = 64; j0 < cnt; j0 += 64 * 8) {
      uint2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t jj = j0 + 64 * u + j;
        v[u] = jj < cnt ? gsl[jj] : make_uint2(0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + 64 * u < cnt) f(j0 + 64 * u + j, v[u], j0 + 64 * u + j < cnt);
      }
    }
  };
  const Digit g = first_digit(kmax, cmin);
  if (g.lo == 0) {
    // every candidate key is equal: the first ke candidates in id order are the top ke
    *lo_key = kmax;
    const uint32_t nk = min(sm.segoff[nseg], ke);
    for (int sl = wave(); sl < nseg; sl += kRW) {
      const uint32_t o = sm.segoff[sl];
      if (o >= nk) break;   // slices are in id order
      const uint32_t c = min(sm.segoff[sl + 1], nk) - o;
      const uint2* gsl = base + (int64_t)sl * P.cap_w;
      slice_chunks(gsl, c, j < c ? gsl[j] : make_uint2(0, 0), [&](uint32_t jj, uint2 w, bool ok) {
        if (ok) {
          sm.ckey[o + jj] = w.x;
          sm.cidx[o + jj] = w.y;
        }
      });
    }
    bar();
    return nk;
  }
  // pass 1: first-digit histogram of every candidate
  batches([&](int, const uint32_t (&cnt)[kGatherB], const uint2 (&first)[kGatherB], const uint2* gs) {
#pragma unroll
    for (int u = 0; u < kGatherB; ++u) {
      slice_chunks(gs + (int64_t)u * kRW * P.cap_w, cnt[u], first[u], [&](uint32_t, uint2 w, bool ok) {
        if (ok) hist_add(sm.hist, (w.x >> g.sh) & g.dm);
      });
    }
  });
  bar();
  search_count(sm, ke);
  if (sm.res[1] + sm.res[2] > (uint32_t)kLdsCand) return 0u;
  const uint32_t thr_key = shl((g.prefix << (g.lo - g.sh)) | sm.res[0], g.sh);
  *lo_key = thr_key;
  // pass 2: per-slice counts of the kept candidates, in sm.kkey (not yet in use)
  batches([&](int sb, const uint32_t (&cnt)[kGatherB], const uint2 (&first)[kGatherB], const uint2* gs) {
#pragma unroll
    for (int u = 0; u < kGatherB; ++u) {
      uint32_t c = 0;
      slice_chunks(gs + (int64_t)u * kRW * P.cap_w, cnt[u], first[u], [&](uint32_t, uint2 w, bool ok) {
        c += (uint32_t)__popcll(__ballot(ok && w.x >= thr_key));
      });
      const int sl = sb + u * kRW;
      if (j == 0 && sl < nseg) sm.kkey[sl] = c;
    }
  });
  bar();
  uint32_t nf;
  {
    const int s0 = kSegPT * (int)threadIdx.x;
    uint32_t cs[kSegPT], csum = 0;
#pragma unroll
    for (int q = 0; q < kSegPT; ++q) {
      cs[q] = s0 + q < nseg ? sm.kkey[s0 + q] : 0u;
      csum += cs[q];
    }
    uint32_t off = block_excl_scan<kRW>(csum, sm.red, nf);   // barrier before the writes
#pragma unroll
    for (int q = 0; q < kSegPT; ++q) {
      if (s0 + q < nseg) sm.kkey[s0 + q] = off;
      off += cs[q];
    }
  }
  if (nf > (uint32_t)kLdsCand) return 0u;   // uniform: every thread holds the scan total
  bar();
  // pass 3: the kept candidates into LDS at their id-ordered positions
  batches([&](int sb, const uint32_t (&cnt)[kGatherB], const uint2 (&first)[kGatherB], const uint2* gs) {
#pragma unroll
    for (int u = 0; u < kGatherB; ++u) {
      uint32_t pos = sm.kkey[min(sb + u * kRW, nseg - 1)];
      slice_chunks(gs + (int64_t)u * kRW * P.cap_w, cnt[u], first[u], [&](uint32_t, uint2 w, bool ok) {
        const bool keep = ok && w.x >= thr_key;
        const uint64_t bal = __ballot(keep);
        const uint32_t at = pos + mbcnt(bal);
        if (keep && at < nf) {
          sm.ckey[at] = w.x;
          sm.cidx[at] = w.y;
        }
        pos += (uint32_t)__popcll(bal);
      });
    }
  });
  bar();
  return nf;
}

// The top ke candidates of a row whose candidates all hold one key (kmax == every slice's
// threshold) when some of its slices are uniform (they store nothing): the first ke
// candidates in id order, read from the stored slices or made up from the uniform ones (whose
// key and first id are in their wave summaries). Returns the number gathered.
__device__ __forceinline__ uint32_t gather_equal(const Params& P, int r, int nseg, uint32_t ke, Smem& sm) {
  const uint2* base = P.cand + (int64_t)r * nseg * P.cap_w;
  const WaveInfo* inf = P.info + (int64_t)r * nseg;
  const uint32_t nk = min(sm.segoff[nseg], ke);
  for (int sl = wave(); sl < nseg; sl += kRW) {
    const uint32_t o = sm.segoff[sl];
    if (o >= nk) break;   // slices are in id order
    const uint32_t c = min(sm.segoff[sl + 1], nk) - o;
    const WaveInfo wi = inf[sl];
    const bool uni = (wi.flags & kFlagUniform) != 0;
    const uint2* gsl = base + (int64_t)sl * P.cap_w;
    for (uint32_t jj = (uint32_t)lane(); jj < c; jj += 64) {
      const uint2 w = uni ? make_uint2(wi.kmax, wi.first + jj) : gsl[jj];
      sm.ckey[o + jj] = w.x;
      sm.cidx[o + jj] = w.y;
    }
  }
  bar();
  return nk;
}

// ------------------------------------------------------------------ nucleus pass
// Rows with top-k off and top-p or min-p on (NUCLEUS): rows x chunks workgroups, run after
// the stream kernel. Each weighs its chunk against the row maximum (the same fixed-point
// masses as the exact top-p select: S = 63 - bitlen(V)), bins the tokens by value in the
// window below the row maximum (nuc_bin), and adds each bin's mass into the row's NucRow.
// The cut pass then finds the bin where the nucleus ends and counts, draws and lists the
// tokens; the row kernel finishes the cut bin.
// f(x, i) for the n elements of a chunk starting at `row` (NT threads; float4 loads, four
// per thread in flight, when the chunk is 16-byte aligned).
template <int NT, class F>
__device__ __forceinline__ void chunk_visit(const float* row, int n, F f) {
  if (((uintptr_t)row & 15u) == 0) {
    const int nq = n >> 2;
    const float4* rq = reinterpret_cast<const float4*>(row);
    for (int q0 = threadIdx.x; q0 < nq; q0 += 4 * NT) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + u * NT;
        v[u] = q < nq ? rq[q] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + u * NT;
        if (q < nq) {
          f(v[u].x, (uint32_t)(4 * q));
          f(v[u].y, (uint32_t)(4 * q + 1));
          f(v[u].z, (uint32_t)(4 * q + 2));
          f(v[u].w, (uint32_t)(4 * q + 3));
        }
      }
    }
    for (int i = 4 * nq + (int)threadIdx.x; i < n; i += NT) f(row[i], (uint32_t)i);
  } else {
    for (int i = threadIdx.x; i < n; i += NT) f(row[i], (uint32_t)i);
  }
}

// Bins of the nucleus passes: value-linear over the window [lo, m] below the row maximum m,
// bins 1 .. kNucBins - 1, and bin 0 for every token below lo (and -inf). (Each workgroup adds
// its non-empty bins to the row's histograms with global atomics, so the bin count is kept
// moderate.) lo = m + T (ln((1 - p)
// / V) - 1): a token below it has weight exp((x - m) / T) < (1 - p) / (e V), so the tokens of
// bin 0 together hold less than (1 - p) / e of the total mass (the maximum's weight is 1) and
// the nucleus's last token lies in the window; its bin then holds few tokens. Only the size
// of that bin depends on this bound, not the result (any bin is cut exactly). The bin is a
// monotone function of x, so every bin is a contiguous key range. p == 1 (no cut): one bin.
static_assert(kNucBins % kT1 == 0 && kNucBins % kRT == 0 && kNucBins <= kDBins, "nucleus bins");
struct NucBin {
  float lo;
  float scale;
};
__device__ __forceinline__ NucBin nuc_bin_params(float m, float p, float t, int V) {
  if (!(p < 1.0f)) return NucBin{-INFINITY, 0.0f};
  const double span = (double)t * (1.0 - log((1.0 - (double)p) / (double)V));   // > 0
  return NucBin{(float)((double)m - span), (float)((double)(kNucBins - 1) / span)};
}
__device__ __forceinline__ uint32_t nuc_bin(float x, const NucBin& nb) {
  if (!(x >= nb.lo)) return 0u;
  const float f = (x - nb.lo) * nb.scale;   // >= 0; a monotone function of x
  return min(1u + (uint32_t)f, (uint32_t)(kNucBins - 1));
}

constexpr int kNT = 256;   // threads of the histogram pass: 8 workgroups per CU, so a decode grid
                           // (1216) is resident at once (with 512, 1024 are and 192 wait)
struct SmemN {
  uint64_t mass[kNucBins];
  uint32_t red[4 * (kNT / 64)];
};

// The row plan and maximum key of a NUCLEUS row from its wave summaries (common to the nucleus
// kernels). Returns false for rows that are not NUCLEUS or that the row kernel rejects.
struct NucPlan {
  RowPlan rp;
  uint32_t kmax;
};
template <int MODE, int NT, int NW>
__device__ __forceinline__ bool nucleus_plan(const Params& P, int r, uint32_t* red, NucPlan& np) {
  np.rp = plan_row(P, MODE, r);
  if (np.rp.path != kPathNucleus) return false;        // uniform
  const int nseg = P.chunks * kW1;
  const WaveInfo* inf = P.info + (int64_t)r * nseg;
  uint32_t kmax = 0, dummy = 0u, dummy2 = 0xFFFFFFFFu, flags = 0;
  for (int i = threadIdx.x; i < nseg; i += NT) {
    const WaveInfo wi = inf[i];
    kmax = max(kmax, wi.kmax);
    flags |= wi.flags;
  }
  block_reduce4<NW>(kmax, dummy, dummy2, flags, red);
  np.kmax = kmax;
  return !((flags & kFlagNan) || kmax >= kKeyPosInf || kmax <= kKeyNegInf);
}

template <int MODE>
__global__ __launch_bounds__(kNT) void ts_nucleus_kernel(Params P) {
  __shared__ SmemN sm;
  const int b = (int)blockIdx.x;
  int L = b;
  if (P.xcd_map) {
    const int per = (P.rows * P.chunks) >> 3;
    L = (b & 7) * per + (b >> 3);
  }
  const int r = L / P.chunks;
  const int c = L - r * P.chunks;
  NucPlan np;
  if (!nucleus_plan<MODE, kNT, kNT / 64>(P, r, sm.red, np)) return;   // uniform
  const RowPlan& rp = np.rp;
  const uint32_t kmax = np.kmax;
  for (int i = threadIdx.x; i < kNucBins; i += kNT) sm.mass[i] = 0ull;
  const float m = key2f(kmax);
  const double c2 = kLog2e / (double)rp.t;
  const int S = 63 - bitlen((uint32_t)P.V);
  const NucBin nb = nuc_bin_params(m, rp.p, rp.t, P.V);
  const int c0 = c * P.chunk_len;
  const int n = max(0, min(P.chunk_len, P.V - c0));
  const float* row = P.x + (int64_t)r * P.stride + c0;
  bar();
  // Bin 0 (below the window) holds most of a spread row's tokens: its mass is summed in
  // registers and added once per wave instead of by LDS atomics on one address.
  uint64_t z0m = 0;
  chunk_visit<kNT>(row, n, [&](float x, uint32_t) {
    const uint32_t bin = nuc_bin(x, nb);
    const uint64_t q = massf(x, m, c2, S);
    if (bin == 0u) z0m += q;
    else if (q) atomicAdd((unsigned long long*)&sm.mass[bin], (unsigned long long)q);
  });
  {
    const uint64_t wm = readlane64(wave_incl_scan64(z0m), 63);
    if (lane() == 0 && wm) atomicAdd((unsigned long long*)&sm.mass[0], (unsigned long long)wm);
  }
  bar();
  NucRow* nr = P.nuc + r;
  for (int i = threadIdx.x; i < kNucBins; i += kNT) {
    const uint64_t q = sm.mass[i];
    if (q) atomicAdd((unsigned long long*)&nr->mass[i], (unsigned long long)q);
  }
}

// Second nucleus pass (rows x chunks, after the histograms are complete): every workgroup of a
// row finds the same cut bin - the bin holding the nucleus's last token - from the row's
// masses. Its chunk's tokens in bins above the cut are all in the nucleus: sampling draws
// their Gumbel scores (min-p kept ones) into the row's best; top-p with a mask writes their
// bytes. Tokens of the cut bin are appended, in any order, to the row's list for the row
// kernel's exact cut.
struct SmemC {
  uint32_t red[4 * kW1];
  uint64_t red64[2 * kW1];
  uint32_t res[2];
  uint32_t mkey[kW1][256];     // a wave's kept tokens, compacted across load slots for the noise
  uint32_t mid[kW1][256];
};

template <int MODE>
__global__ __launch_bounds__(kT1) void ts_nucleus_cut_kernel(Params P) {
  __shared__ SmemC sm;
  const int b = (int)blockIdx.x;
  int L = b;
  if (P.xcd_map) {
    const int per = (P.rows * P.chunks) >> 3;
    L = (b & 7) * per + (b >> 3);
  }
  const int r = L / P.chunks;
  const int c = L - r * P.chunks;
  NucPlan np;
  if (!nucleus_plan<MODE, kT1, kW1>(P, r, sm.red, np)) return;
  const RowPlan& rp = np.rp;
  NucRow* nr = P.nuc + r;
  const NucBin nb = nuc_bin_params(key2f(np.kmax), rp.p, rp.t, P.V);
  int cut = -1;
  if (rp.p != 1.0f) {
    constexpr int kB = kNucBins / kT1;                 // 4 bins per thread, thread t: 4t .. 4t+3
    uint64_t ms[kB], tsum = 0;
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      ms[j] = nr->mass[kB * threadIdx.x + j];
      tsum += ms[j];
    }
    const uint64_t suf = wave_incl_suffix64(tsum);    // this and higher lanes of the wave
    if (lane() == 0) sm.red64[wave()] = suf;
    if (threadIdx.x == 0) sm.res[0] = 0xFFFFFFFFu;
    bar();
    uint64_t above = suf - tsum, z = 0;
#pragma unroll
    for (int w = 0; w < kW1; ++w) {
      z += sm.red64[w];
      if (w > wave()) above += sm.red64[w];
    }
    const uint64_t target = topp_target(rp.p, z);
    if (above < target && above + tsum >= target) {
      uint64_t acc = above;
      int j = kB - 1;
      for (; j > 0; --j) {
        if (acc + ms[j] >= target) break;
        acc += ms[j];
      }
      sm.res[0] = (uint32_t)(kB * threadIdx.x + j);
    }
    bar();
    cut = (int)sm.res[0];
  }
  const float m = key2f(np.kmax);
  const double c2 = kLog2e / (double)rp.t;
  const bool minp_on = rp.minp > 0.0f;
  const uint64_t seed = (MODE == kModeSample) ? P.seed[r] : 0ull;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int c0 = c * P.chunk_len;
  const int n = max(0, min(P.chunk_len, P.V - c0));
  const float* row = P.x + (int64_t)r * P.stride + c0;
  uint8_t* mrow = (MODE == kModeTopp && P.out_mask) ? P.out_mask + (int64_t)r * P.V + c0 : nullptr;
  // the chunk in registers: thread t holds quads t, t + kT1, ... (ids rise along them)
  constexpr int kQ = kChunkMax / 4 / kT1;
  float4 v[kQ];
  const int nq = (n + 3) >> 2;
  const bool al = ((uintptr_t)row & 15u) == 0;
#pragma unroll
  for (int s = 0; s < kQ; ++s) {
    const int q = (int)threadIdx.x + s * kT1;
    v[s] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    if (q < nq) {
      if (al && 4 * q + 3 < n) {
        v[s] = reinterpret_cast<const float4*>(row)[q];
      } else {
        v[s].x = row[4 * q];
        v[s].y = 4 * q + 1 < n ? row[4 * q + 1] : -INFINITY;
        v[s].z = 4 * q + 2 < n ? row[4 * q + 2] : -INFINITY;
        v[s].w = 4 * q + 3 < n ? row[4 * q + 3] : -INFINITY;
      }
    }
  }
  auto elem = [&](int s, int e) { return e == 0 ? v[s].x : (e == 1 ? v[s].y : (e == 2 ? v[s].z : v[s].w)); };
  auto valid = [&](int s, int e) { return 4 * ((int)threadIdx.x + s * kT1) + e < n; };
  // cut-bin members: count (one LDS add per wave, one global reservation per workgroup)
  uint32_t mine = 0;
  if (cut >= 0) {
#pragma unroll
    for (int s = 0; s < kQ; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (valid(s, e) && (int)nuc_bin(elem(s, e), nb) == cut) ++mine;
  }
  const uint32_t wincl = wave_incl_scan(mine);
  const uint32_t wtot = wave_total(wincl);
  if (threadIdx.x == 0) sm.res[1] = 0u;
  bar();
  uint32_t wbase = 0;
  if (lane() == 0 && wtot) wbase = atomicAdd(&sm.res[1], wtot);
  bar();
  if (threadIdx.x == 0 && sm.res[1]) sm.res[0] = atomicAdd(&nr->nlist, sm.res[1]);
  bar();
  const int nseg = P.chunks * kW1;
  uint2* list = P.cand + (int64_t)r * nseg * P.cap_w;
  const uint32_t cap_list = (uint32_t)min((int64_t)kLdsCand, (int64_t)nseg * P.cap_w);
  uint32_t at = sm.res[0] + (uint32_t)__builtin_amdgcn_readfirstlane((int)wbase) + wincl - mine;
  uint64_t best = 0;
  uint64_t n_up = 0, k_up = 0;   // this thread's tokens above the cut bin, and those min-p keeps
  const int w = wave(), l = lane();
  // Sampling: the kept tokens are scattered over the wave's lanes and slots. They are
  // compacted into the wave's LDS buffer across slots (flushed when the next slot would
  // overflow it, and at the end), so the generator and the noise run on full lanes, once per
  // member: not once per quad of every lane whenever any lane has one, nor once per slot.
  constexpr uint32_t kMemCap = sizeof(sm.mkey[0]) / sizeof(sm.mkey[0][0]);
  uint32_t nmem = 0;   // wave-uniform
  auto flush = [&]() {
    if (nmem) {
      wave_lds_sync();
      for (uint32_t j = (uint32_t)l; j < nmem; j += 64) {
        const uint32_t key = sm.mkey[w][j], id = sm.mid[w][j];
        const float sc = gumbel_score(key, id, m, rp.t, (uint32_t)r, k0, k1);
        best = max(best, ((uint64_t)f2key(sc) << 32) | (uint32_t)~id);
      }
      wave_lds_sync();
      nmem = 0;
    }
  };
#pragma unroll
  for (int s = 0; s < kQ; ++s) {
    const uint32_t id0 = (uint32_t)(c0 + 4 * ((int)threadIdx.x + s * kT1));
    bool mem[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = f2key(elem(s, e));
      const int bin = (int)nuc_bin(elem(s, e), nb);
      mem[e] = false;
      if (!valid(s, e)) continue;
      if (bin == cut) {
        if (at < cap_list) list[at] = make_uint2(key, id0 + e);
        ++at;
      } else if (bin > cut) {
        mem[e] = !minp_on || weight32(key, m, c2) >= rp.minp;
        ++n_up;
        k_up += mem[e] ? 1u : 0u;
      }
    }
    if (MODE == kModeSample) {
      uint64_t bal[4];
      uint32_t cnt = 0;   // this slot's members over the wave: at most 256 = kMemCap
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bal[e] = __ballot(mem[e]);
        cnt += (uint32_t)__popcll(bal[e]);
      }
      if (nmem + cnt > kMemCap) flush();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (mem[e]) {
          const uint32_t pos = nmem + mbcnt(bal[e]);
          sm.mkey[w][pos] = f2key(elem(s, e));
          sm.mid[w][pos] = id0 + (uint32_t)e;
        }
        nmem += (uint32_t)__popcll(bal[e]);
      }
    }
    if (MODE == kModeTopp && mrow) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (mem[e]) mrow[id0 - c0 + e] = 1;
    }
  }
  if (MODE == kModeSample) flush();
  // the workgroup's tokens above the cut bin (and those min-p keeps): one atomic each
  block_sum2_u64<kW1>(n_up, k_up, sm.red64);
  if (threadIdx.x == 0 && n_up) {
    atomicAdd(&nr->nabove, (uint32_t)n_up);
    atomicAdd(&nr->kabove, (uint32_t)k_up);
  }
  if (MODE == kModeSample) {
    uint32_t hi = (uint32_t)(best >> 32);
    hi = block_max_u32<kW1>(hi, sm.red);
    uint32_t lo = ((uint32_t)(best >> 32) == hi) ? (uint32_t)best : 0u;
    lo = block_max_u32<kW1>(lo, sm.red);
    if (threadIdx.x == 0 && (hi | lo)) atomicMax((unsigned long long*)&nr->best, ((unsigned long long)hi << 32) | lo);
  }
}

// f(v, q, live) for the quads q in [qa, qb) of a row of V elements (elements past V read as
// -inf), in rounds of U quads per thread: quads base + u * kRT + tid, u < U, with the round
// index uniform over the workgroup so that f may use wave-wide operations (every lane calls it
// each round; `live` tells whether its quad exists). An aligned row takes 16-byte loads of its
// whole quads, the next round's issued before this round is visited (indexes clamped into the
// row, so every load is in bounds; quads past the range are replaced by -inf with selects, so
// that no other load stands between a round's loads and their use), then a partial last quad
// in a round of its own by element loads; an unaligned row takes element loads.
template <int U = 8, class F>
__device__ __forceinline__ void visit_quads(const float* row, uint32_t V, uint32_t qa, uint32_t qb, F f) {
  constexpr uint32_t kStep = kRT * U;
  const uint32_t nfull = V >> 2;
  auto slow = [&](uint32_t a, uint32_t b) {
    for (uint32_t base = a; base < b; base += kStep) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = base + u * kRT + threadIdx.x;
        v[u] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (q < b) {
          v[u].x = row[4 * q];
          if (4 * q + 1 < V) v[u].y = row[4 * q + 1];
          if (4 * q + 2 < V) v[u].z = row[4 * q + 2];
          if (4 * q + 3 < V) v[u].w = row[4 * q + 3];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = base + u * kRT + threadIdx.x;
        f(v[u], q, q < b);
      }
    }
  };
  if (((uintptr_t)row & 15u) != 0 || nfull == 0) {
    slow(qa, qb);
    return;
  }
  const float4* row4 = reinterpret_cast<const float4*>(row);
  const uint32_t qe = min(qb, nfull);       // the range's whole quads end here
  auto load = [&](float4 (&v)[U], uint32_t base) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = row4[min(base + u * kRT + threadIdx.x, nfull - 1u)];
  };
  float4 v[U];
  if (qa < qe) load(v, qa);
  for (uint32_t base = qa; base < qe; base += kStep) {
    float4 nx[U];
    load(nx, base + kStep);          // unconditional (clamped), so the waits below count it
    asm volatile("" ::: "memory");   // keep the next round's loads issued ahead of this round's work
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t q = base + u * kRT + threadIdx.x;
      const bool in = q < qe;
      const float4 w = make_float4(in ? v[u].x : -INFINITY, in ? v[u].y : -INFINITY, in ? v[u].z : -INFINITY,
                                   in ? v[u].w : -INFINITY);
      f(w, q, in);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = nx[u];
  }
  if (qb > qe && qb > qa) slow(max(qa, qe), qb);   // the partial last quad
}

// The largest of each of two 64-bit values over the row workgroup (red: 2 * kRW words).
__device__ __forceinline__ void block_max2_u64(uint64_t& a, uint64_t& b, uint64_t* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a = max(a, (uint64_t)__shfl_xor((unsigned long long)a, o));
    b = max(b, (uint64_t)__shfl_xor((unsigned long long)b, o));
  }
  if (lane() == 0) {
    red[wave()] = a;
    red[kRW + wave()] = b;
  }
  bar();
  a = 0;
  b = 0;
#pragma unroll
  for (int w = 0; w < kRW; ++w) {
    a = max(a, red[w]);
    b = max(b, red[kRW + w]);
  }
  bar();
}

// Top-p (and min-p after it) over whole rows whose k reaches the row length, in calls with a
// top-k array (the host cannot see the array's values, so the nucleus passes over the chunk
// workgroups do not run for them) and in small sampling calls without one (fewer launches than
// the nucleus passes). The row kernel runs P.split workgroups per row; each takes
// a contiguous part of the row and, with the row maximum m known from the wave summaries:
//  - bins every token's exact fixed-point mass by value in the window below m (nuc_bin; bin 0
//    below the window, summed in registers);
//  - sampling: draws the Gumbel score of every token of the window that min-p keeps (one
//    Philox block per quad) and keeps the best per bin (p == 1: one best for the row), since
//    the kept set is every bin above the cut plus a prefix of the cut bin, whichever bin that
//    turns out to be;
//  - stores its bins into its own slot in the row's candidate area (unused by rows of this
//    kind) and counts itself done on the row's counter.
// The workgroup that counts last (no workgroup ever waits for another) sums the slots, finds
// the cut bin where the mass from the top reaches ceil(p * Z), lists that bin's tokens in LDS
// from one compare-only read of the row (top-p masks: also marks the tokens above the cut),
// and takes the exact cut inside it with the same fixed-point select as the exact path. The
// sampled token is the best of the bins above the cut and of the selected members of the cut
// bin. Returns false only in the finishing workgroup, when the cut bin holds more tokens than
// the LDS list (the caller then takes the row-streaming path, which writes the same mask
// bytes).
template <int MODE>
__device__ __forceinline__ bool row_nucleus(const Params& P, const RowPlan& rp, int r, uint32_t kmax,
                                            uint64_t seed, Smem& sm, double lse, int part) {
  const float* row = P.x + (int64_t)r * P.stride;
  const uint32_t V = (uint32_t)rp.n;
  const float m = key2f(kmax);
  const float t = rp.t;
  const double c2 = kLog2e / (double)t;
  const int S = 63 - bitlen(V);
  const bool minp_on = rp.minp > 0.0f;
  const bool binned = rp.p != 1.0f;          // p == 1: min-p alone keeps every token it passes
  auto wmass = [&](uint32_t rk) { return mass32_of(weight32(rk, m, c2), S); };
  auto ok = [&](uint32_t rk) { return !minp_on || weight32(rk, m, c2) >= rp.minp; };
  const NucBin nb = nuc_bin_params(m, rp.p, t, (int)V);
  NucRow* nr = P.nuc + r;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int G = P.split;
  // the parts' slots: 2 * kNucBins words each, masses then best scores
  uint64_t* slots = reinterpret_cast<uint64_t*>(P.cand + (int64_t)r * P.chunks * kW1 * P.cap_w);
  const uint32_t nq = (V + 3) >> 2;
  const uint32_t per = (nq + (uint32_t)G - 1) / (uint32_t)G;
  const uint32_t qa = min(nq, (uint32_t)part * per), qb = min(nq, qa + per);
  uint64_t* bbest = sm.mhi + kNucBins;      // the upper half of the mass histogram (zero)
  // Sampling: every part also stores one byte per token, its bin / 4 (0 for bins 0-3 and past the
  // row), in one word per quad after the parts' slots, so that the finishing workgroup can find
  // the cut bin's tokens without reading the row's values (a quarter of the bytes).
  uint32_t* const codes = reinterpret_cast<uint32_t*>(slots + (int64_t)G * 2 * kNucBins);
  const bool scored = MODE == kModeSample && binned;   // the parts keep the best score per bin
  const bool coded = scored && P.codes != 0;           // and store the codes (when they fit)

  // ---- this workgroup's part: masses by bin, and the best score per bin
  uint64_t z0 = 0, best = 0;
  visit_quads(row, V, qa, qb, [&](const float4& v, uint32_t q, bool live) {
    const float xs[4] = {v.x, v.y, v.z, v.w};
    uint32_t bin[4];
    bool cand[4];
    bool any = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bin[e] = binned ? nuc_bin(xs[e], nb) : 1u;
      if (binned && live) {
        const uint64_t q64 = massf(xs[e], m, c2, S);   // 0 for the -inf past the row end
        if (bin[e] == 0u) z0 += q64;
        else if (q64) atomicAdd((unsigned long long*)&sm.mhi[bin[e]], (unsigned long long)q64);
      }
      cand[e] = MODE == kModeSample && live && 4 * q + e < V && bin[e] != 0u && ok(f2key(xs[e]));
      any |= cand[e];
    }
    if (coded && live)   // written through like the slots (elements past the row are -inf: bin 0)
      __hip_atomic_store(codes + q, (bin[0] >> 2) | ((bin[1] >> 2) << 8) | ((bin[2] >> 2) << 16) | ((bin[3] >> 2) << 24),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (MODE == kModeSample && any) {
      const uint4 w = philox4x32_10(q, (uint32_t)r, k0, k1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (cand[e]) {
          const float g = gumbel_from_uniform(uniform_from_word(pick_word(w, (uint32_t)e)));
          const float sc = (xs[e] - m) * (1.0f / t) + g;   // as gumbel_score
          const uint64_t pk = ((uint64_t)f2key(sc) << 32) | (uint32_t)~(4 * q + e);
          if (binned) atomicMax((unsigned long long*)&bbest[bin[e]], (unsigned long long)pk);
          else best = max(best, pk);
        }
      }
    }
  });
  {
    uint64_t zl = 0;
    block_sum2_u64<kRW>(z0, zl, sm.red64);   // its barriers also complete the LDS atomics
  }
  uint64_t* mine = slots + (int64_t)part * 2 * kNucBins;
  static_assert(kNucBins % (2 * kRT) == 0, "bins in pairs per thread");
  // The slots are written with device-scope atomic stores, which write through to the point
  // of coherence of all XCDs, and read with device-scope atomic loads. Every thread waits for
  // its stores to complete before the barrier; the counter's fetch-add then releases the part
  // and, in the last workgroup, acquires the others (one agent-scope fence pair per
  // workgroup: a fence in every thread costs tens of microseconds in L2 write-backs).
  auto put = [&](uint64_t* a, uint64_t v) { __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  if (binned) {
    for (int i = 2 * (int)threadIdx.x; i < kNucBins; i += 2 * kRT) {
      put(mine + i, sm.mhi[i] + (i == 0 ? z0 : 0ull));
      put(mine + i + 1, sm.mhi[i + 1]);
      sm.mhi[i] = 0;
      sm.mhi[i + 1] = 0;
      if (MODE == kModeSample) {
        put(mine + kNucBins + i, bbest[i]);
        put(mine + kNucBins + i + 1, bbest[i + 1]);
        bbest[i] = 0;
        bbest[i + 1] = 0;
      }
    }
  } else if (MODE == kModeSample) {
    uint32_t hi = (uint32_t)(best >> 32);
    hi = block_max_u32<kRW>(hi, sm.red);
    uint32_t lo = ((uint32_t)(best >> 32) == hi) ? (uint32_t)best : 0u;
    lo = block_max_u32<kRW>(lo, sm.red);
    if (threadIdx.x == 0) put(mine + kNucBins, ((unsigned long long)hi << 32) | lo);
  }
  // publish the part (every store complete), then count it; the workgroup that counts last
  // finishes the row
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  bar();
  if (threadIdx.x == 0) sm.res[3] = __hip_atomic_fetch_add(&nr->ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  bar();
  const bool last = sm.res[3] == (uint32_t)(G - 1);
  bar();
  if (!last) return true;

  // ---- the row's finish: the cut bin from the whole histogram
  int cut = -1;                 // bins above it are kept whole; p == 1: every token
  uint64_t target = 0, ma = 0;
  if (binned) {
    uint64_t zh = 0, zl = 0;
    for (int i = 2 * (int)threadIdx.x; i < kNucBins; i += 2 * kRT) {
      uint64_t m0 = 0, m1 = 0;
      for (int g = 0; g < G; ++g) {
        m0 += __hip_atomic_load(slots + (int64_t)g * 2 * kNucBins + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        m1 += __hip_atomic_load(slots + (int64_t)g * 2 * kNucBins + i + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      sm.mhi[i] = m0;
      sm.mhi[i + 1] = m1;
      zh += m0 + m1;
    }
    block_sum2_u64<kRW>(zh, zl, sm.red64);
    target = topp_target(rp.p, zh);
    search_mass(sm, target, 0ull);           // also clears the histograms for the exact cut
    cut = (int)sm.res[0];
    ma = sm.res64[0];
  }
  auto best_of = [&](int g, int b) {        // part g's best packed score in bin b
    return (uint64_t)__hip_atomic_load(slots + (int64_t)g * 2 * kNucBins + kNucBins + b, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  };
  uint32_t nlist = 0;                       // the cut bin's tokens, listed in (ckey, cidx)
  bool listed = false;
  uint64_t bst = 0;                         // sampling: the best packed score above the cut bin
  if (scored) {
    // The best score above the cut bin against the cut bin's best: when the former is larger
    // it is the sample, whichever prefix of the cut bin the cut keeps (the kept tokens of the
    // cut bin score at most its best), and the cut bin's tokens are not needed.
    uint64_t bc = 0;
    for (int i = cut + 1 + (int)threadIdx.x; i < kNucBins; i += kRT)
      for (int g = 0; g < G; ++g) bst = max(bst, best_of(g, i));
    if ((int)threadIdx.x < G) bc = best_of((int)threadIdx.x, cut);
    block_max2_u64(bst, bc, sm.red64);
    if (bst > bc) {
      if (threadIdx.x == 0) {
        const int32_t tok = (int32_t)~(uint32_t)bst;
        P.out_token[r] = tok;
        put_logp(P, r, tok, t, lse);
      }
      return true;
    }
    if (coded && cut >= 4) {
      // The tokens whose code is the cut bin's (bins 4 * (cut / 4) .. + 3): their ids into the
      // LDS list (one reservation per wave and word), then their values, kept when their bin is
      // the cut bin. More than kCodeCap of them: the value scan below instead.
      const uint32_t want = (uint32_t)cut >> 2;
      const uint64_t* cw = reinterpret_cast<const uint64_t*>(codes);
      const uint32_t nw = (nq + 1u) >> 1;   // words of two quads (tokens 8j .. 8j + 7)
      auto load = [&](uint64_t (&v)[8], uint32_t base) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = __hip_atomic_load(cw + min(base + u * kRT + threadIdx.x, nw - 1u), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
      };
      uint64_t v[8];
      load(v, 0u);
      for (uint32_t base = 0; base < nw; base += kRT * 8) {
        uint64_t nx[8];
        load(nx, base + kRT * 8);        // clamped: in bounds; the next round in flight
        asm volatile("" ::: "memory");
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t jw = base + u * kRT + threadIdx.x;
          uint32_t hits = 0;
          if (jw < nw) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (2 * jw + (uint32_t)(e >> 2) < nq && (uint32_t)((v[u] >> (8 * e)) & 0xFFu) == want) hits |= 1u << e;
          }
          if (__ballot(hits != 0u)) {
            const uint32_t nh = (uint32_t)__popc(hits);
            const uint32_t incl = wave_incl_scan(nh);
            const uint32_t tot = wave_total(incl);
            uint32_t wb = 0;
            if (lane() == 0) wb = atomicAdd(&sm.bcount, tot);
            uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane((int)wb) + incl - nh;
            while (hits) {
              const uint32_t e = (uint32_t)__builtin_ctz(hits);
              hits &= hits - 1u;
              if (pos < (uint32_t)kCodeCap) sm.cidx[pos] = 8 * jw + e;
              ++pos;
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = nx[u];
      }
      bar();
      const uint32_t nc = sm.bcount;
      bar();
      if (nc <= (uint32_t)kCodeCap) {
        uint32_t id[kCodePer];
        float xv[kCodePer];
#pragma unroll
        for (int u = 0; u < kCodePer; ++u) {
          const uint32_t i = u * kRT + threadIdx.x;
          id[u] = i < nc ? sm.cidx[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kCodePer; ++u) xv[u] = (u * kRT + threadIdx.x < nc && id[u] < V) ? row[id[u]] : -INFINITY;
        if (threadIdx.x == 0) sm.bcount = 0;
        bar();                             // every listed id read before the list is rewritten
#pragma unroll
        for (int u = 0; u < kCodePer; ++u) {
          if (u * kRT + threadIdx.x < nc && nuc_bin(xv[u], nb) == (uint32_t)cut) {
            const uint32_t pos = atomicAdd(&sm.bcount, 1u);
            sm.ckey[pos] = f2key(xv[u]);
            sm.cidx[pos] = id[u];
          }
        }
        listed = true;
      } else if (threadIdx.x == 0) {
        sm.bcount = 0;
      }
      bar();
      if (listed) {
        nlist = sm.bcount;
        bar();
        if (threadIdx.x == 0) sm.bcount = 0;   // zero again outside the small-bin collections
        bar();
      }
    }
  }
  uint32_t un = 0;                          // tokens above the cut bin (top-p masks: min-p's share)
  uint64_t uk = 0;
  if (!listed) {
    // the cut bin as a key range [ka, kb): nuc_bin is monotone in the value up to m
    auto first_key = [&](uint32_t b) {        // smallest key <= kmax whose bin is >= b, else kmax + 1
      uint32_t lo = kKeyNegInf, hi = kmax + 1u;
      while (lo < hi) {
        const uint32_t mid = lo + ((hi - lo) >> 1);
        if (nuc_bin(key2f(mid), nb) >= b) hi = mid;
        else lo = mid + 1u;
      }
      return lo;
    };
    const uint32_t ka = binned ? first_key((uint32_t)cut) : kKeyNegInf;
    const uint32_t kb = binned ? first_key((uint32_t)cut + 1u) : kKeyNegInf;
    // one read of the row: the cut bin's tokens into the LDS list; top-p masks also mark the
    // tokens above the cut that min-p keeps
    uint8_t* mrow = (MODE == kModeTopp && P.out_mask) ? P.out_mask + (int64_t)r * P.V : nullptr;
    uint32_t n_up = 0, k_up = 0;
    // as values: x >= xb is key >= kb, and x >= xa is key >= ka (keys order the values, -0 as +0)
    const float xa = key2f(ka), xb = key2f(kb);
    if (binned || MODE == kModeTopp) visit_quads(row, V, 0u, nq, [&](const float4& v, uint32_t q, bool live) {
      const float xs[4] = {v.x, v.y, v.z, v.w};
      const float qmax = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v.x, v.y), __builtin_elementwise_maximum(v.z, v.w));
      const float qmin = __builtin_elementwise_minimum(__builtin_elementwise_minimum(v.x, v.y), __builtin_elementwise_minimum(v.z, v.w));
      bool inl[4] = {false, false, false, false};
      uint32_t nin = 0;
      if (binned) {
        // xb > -inf here, so the -inf that pads a quad is never above the cut
#pragma unroll
        for (int e = 0; e < 4; ++e) n_up += xs[e] >= xb ? 1u : 0u;
        if (qmax >= xa && qmin < xb) {   // some token of the quad may lie in the cut bin
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            inl[e] = live && 4 * q + e < V && xs[e] >= xa && xs[e] < xb;
            nin += inl[e] ? 1u : 0u;
          }
        }
      }
      if (MODE == kModeTopp && qmax >= xb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool keep = live && 4 * q + e < V && xs[e] >= xb && ok(f2key(xs[e]));
          k_up += keep ? 1u : 0u;
          if (keep && mrow) mrow[4 * q + e] = 1;
        }
      }
      const uint64_t any = __ballot(nin != 0u);
      if (any) {   // cut-bin tokens: one LDS reservation per wave and round
        const uint32_t incl = wave_incl_scan(nin);
        const uint32_t tot = wave_total(incl);
        uint32_t wb = 0;
        if (lane() == 0) wb = atomicAdd(&sm.bcount, tot);
        uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane((int)wb) + incl - nin;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (inl[e]) {
            if (pos < (uint32_t)kLdsCand) {
              sm.ckey[pos] = f2key(xs[e]);
              sm.cidx[pos] = 4 * q + e;
            }
            ++pos;
          }
        }
      }
    });
    bar();
    nlist = sm.bcount;
    bar();
    if (threadIdx.x == 0) sm.bcount = 0;   // zero again outside the small-bin collections
    bar();
    if (nlist > (uint32_t)kLdsCand) return false;
    if (MODE == kModeTopp) {
      uint64_t a = n_up, b = k_up;
      block_sum2_u64<kRW>(a, b, sm.red64);
      un = (uint32_t)a;
      uk = b;
    }
  }
  Sel sp = sel_all();
  if (binned) {
    // the exact cut inside the cut bin (a bin is a contiguous key range)
    uint32_t top_key = 0u, base_key = 0xFFFFFFFFu;
    for (uint32_t i = threadIdx.x; i < nlist; i += kRT) {
      top_key = max(top_key, sm.ckey[i]);
      base_key = min(base_key, sm.ckey[i]);
    }
    top_key = block_max_u32<kRW>(top_key, sm.red);
    base_key = block_min_u32<kRW>(base_key, sm.red);
    uint32_t kept_unused;
    sp = select_mass<false>(LdsVis{sm.ckey, sm.cidx, nlist}, wmass, target, nlist, top_key, base_key, 0u, V - 1,
                            sm, kept_unused, false, ma, un);
  }
  if (MODE == kModeTopp) {
    uint8_t* mrow = P.out_mask ? P.out_mask + (int64_t)r * P.V : nullptr;
    uint64_t c = threadIdx.x == 0 ? uk : 0ull, z = 0;
    for (uint32_t i = threadIdx.x; i < nlist; i += kRT) {
      if (sel_member(sp, sm.ckey[i], sm.cidx[i]) && ok(sm.ckey[i])) {
        c += 1;
        if (mrow) mrow[sm.cidx[i]] = 1;
      }
    }
    block_sum2_u64<kRW>(c, z, sm.red64);
    if (threadIdx.x == 0) P.out_kept[r] = (int32_t)c;
  } else if (MODE == kModeSample) {
    if (binned) {
      for (uint32_t i = threadIdx.x; i < nlist; i += kRT) {
        const uint32_t key = sm.ckey[i], id = sm.cidx[i];
        if (sel_member(sp, key, id) && ok(key)) {
          const float sc = gumbel_score(key, id, m, t, (uint32_t)r, k0, k1);
          bst = max(bst, ((uint64_t)f2key(sc) << 32) | (uint32_t)~id);
        }
      }
    } else {
      for (int g = threadIdx.x; g < G; g += kRT) bst = max(bst, best_of(g, 0));
    }
    uint32_t hi = (uint32_t)(bst >> 32);
    hi = block_max_u32<kRW>(hi, sm.red);
    uint32_t lo = ((uint32_t)(bst >> 32) == hi) ? (uint32_t)bst : 0u;
    lo = block_max_u32<kRW>(lo, sm.red);
    const int32_t tok = (int32_t)~lo;
    if (threadIdx.x == 0) {
      P.out_token[r] = tok;
      put_logp(P, r, tok, t, lse);
    }
  }
  return true;
}

// The row kernel's side of a NUCLEUS row (both nucleus passes done): Z and the cut bin come
// from the row's histograms exactly as the second pass found them; the cut bin's tokens come
// from the row's list into LDS for the exact cut, the same fixed-point select as the exact
// path. Tokens above the cut bin were handled by the second pass (their best score, their
// mask bytes). Returns false (nothing written) when the cut bin holds more tokens than LDS:
// the caller then runs the row-streaming path.
template <int MODE>
__device__ __forceinline__ bool nucleus_finish(const Params& P, const RowPlan& rp, int r, uint32_t kmax,
                                               uint64_t seed, Smem& sm, double lse) {
  const int nseg = P.chunks * kW1;
  const NucRow* nr = P.nuc + r;
  const uint32_t V = (uint32_t)P.V;
  const float m = key2f(kmax);
  const float t = rp.t;
  const double c2 = kLog2e / (double)t;
  const int S = 63 - bitlen(V);
  const bool minp_on = rp.minp > 0.0f;
  auto wmass = [&](uint32_t rk) { return mass32_of(weight32(rk, m, c2), S); };
  auto ok = [&](uint32_t rk) { return !minp_on || weight32(rk, m, c2) >= rp.minp; };
  // the masses into LDS for the search (the bins past kNucBins and the count histogram stay
  // zero: the cut pass counted the tokens itself)
  constexpr int kPerT = kNucBins / kRT;
  uint64_t zh = 0, zl = 0;
#pragma unroll
  for (int j = 0; j < kPerT; ++j) {
    const int i = (int)threadIdx.x + j * kRT;
    const uint64_t q = nr->mass[i];
    sm.mhi[i] = q;
    zh += q;
  }
  const uint32_t n_list = nr->nlist, n_up = nr->nabove, k_up = nr->kabove;
  block_sum2_u64<kRW>(zh, zl, sm.red64);
  uint32_t ncut = 0;            // tokens in the cut bin (the bin holding the nucleus's last token)
  Sel sp = sel_all();
  if (rp.p != 1.0f) {
    const uint64_t target = topp_target(rp.p, zh);
    // the mass above the cut bin (the cut pass found the same bin); the search also clears
    // the LDS histograms for the select below
    search_mass(sm, target, 0ull);
    const uint32_t n_above = n_up;   // counted by the cut pass for the same cut bin
    ncut = n_list;
    const uint64_t ma = sm.res64[0];
    // the cut pass listed at most this many (the LDS, and the row's candidate slices); a
    // longer cut bin was not stored whole and the row takes the row-streaming path
    const uint32_t cap_list = (uint32_t)min((int64_t)kLdsCand, (int64_t)nseg * P.cap_w);
    if (ncut > cap_list) return false;
    const uint2* list = P.cand + (int64_t)r * nseg * P.cap_w;   // ncut entries, any order
    for (uint32_t i0 = threadIdx.x; i0 < ncut; i0 += 8 * kRT) {
      uint2 e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = i0 + u * kRT;
        e[u] = i < ncut ? list[i] : make_uint2(0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = i0 + u * kRT;
        if (i < ncut) {
          sm.ckey[i] = e[u].x;
          sm.cidx[i] = e[u].y;
        }
      }
    }
    bar();
    // the cut bin's key range, from its tokens (a bin is a contiguous key range)
    uint32_t top_key = 0u, base_key = 0xFFFFFFFFu;
    for (uint32_t i = threadIdx.x; i < ncut; i += kRT) {
      top_key = max(top_key, sm.ckey[i]);
      base_key = min(base_key, sm.ckey[i]);
    }
    top_key = block_max_u32<kRW>(top_key, sm.red);
    base_key = block_min_u32<kRW>(base_key, sm.red);
    uint32_t kept_unused;
    sp = select_mass<false>(LdsVis{sm.ckey, sm.cidx, ncut}, wmass, target, ncut, top_key, base_key, 0u, V - 1,
                            sm, kept_unused, false, ma, n_above);
  }
  if (MODE == kModeTopp) {
    // kept: tokens of bins above the cut that min-p keeps, plus the cut bin's kept members
    uint64_t c = threadIdx.x == 0 ? (uint64_t)k_up : 0ull, z = 0;
    uint8_t* mrow = P.out_mask ? P.out_mask + (int64_t)r * P.V : nullptr;
    for (uint32_t i = threadIdx.x; i < ncut; i += kRT) {
      if (sel_member(sp, sm.ckey[i], sm.cidx[i]) && ok(sm.ckey[i])) {
        c += 1;
        if (mrow) mrow[sm.cidx[i]] = 1;
      }
    }
    block_sum2_u64<kRW>(c, z, sm.red64);
    if (threadIdx.x == 0) P.out_kept[r] = (int32_t)c;
  } else if (MODE == kModeSample) {
    uint64_t best = threadIdx.x == 0 ? nr->best : 0ull;
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    for (uint32_t i = threadIdx.x; i < ncut; i += kRT) {
      const uint32_t key = sm.ckey[i], id = sm.cidx[i];
      if (sel_member(sp, key, id) && ok(key)) {
        const float sc = gumbel_score(key, id, m, t, (uint32_t)r, k0, k1);
        best = max(best, ((uint64_t)f2key(sc) << 32) | (uint32_t)~id);
      }
    }
    uint32_t hi = (uint32_t)(best >> 32);
    hi = block_max_u32<kRW>(hi, sm.red);
    uint32_t lo = ((uint32_t)(best >> 32) == hi) ? (uint32_t)best : 0u;
    lo = block_max_u32<kRW>(lo, sm.red);
    const int32_t tok = (int32_t)~lo;
    if (threadIdx.x == 0) {
      P.out_token[r] = tok;
      put_logp(P, r, tok, t, lse);
    }
  }
  return true;
}

// Top-k select output of a certified candidate selection: the selected ids ascending (or in
// the row ordering for TS_ORDER_VALUE), shifted by the row's offset, then -1 padding.
__device__ __forceinline__ void emit_topk_cand(const Params& P, const RowPlan& rp, int r, uint32_t ntot,
                                               const Sel& sk, Smem& sm) {
  int32_t* orow = P.out_idx + (int64_t)r * P.k_max;
  const uint32_t kmx = (uint32_t)P.k_max;
  const int32_t off = P.offsets ? P.offsets[r] : 0;
  if (P.order == TS_ORDER_VALUE) {
    // K (<= kFastK items) compacted, then sorted in the free mass histogram
    const uint32_t nk = min(append_members(sm.ckey, sm.cidx, ntot,
                                           [&](uint32_t rk, uint32_t idx) { return sel_member(sk, rk, idx); },
                                           sm.kkey, sm.kidx, (uint32_t)kFastK, 0, sm),
                            (uint32_t)kFastK);
    uint64_t* a = reinterpret_cast<uint64_t*>(sm.mhi);
    for (uint32_t i = threadIdx.x; i < nk; i += kRT) a[i] = ((uint64_t)sm.kkey[i] << 32) | (uint32_t)~sm.kidx[i];
    emit_value_order(a, nk, (uint32_t)kDBins, orow, kmx, off);
  } else {
    uint32_t run = 0;
    // 12 items per thread: up to 6144 candidates per block scan
    emit_ordered<12>(ntot, [&](uint32_t i, uint32_t& rk, uint32_t& idx) { rk = sm.ckey[i]; idx = sm.cidx[i]; },
                    [&](uint32_t rk, uint32_t idx) { return sel_member(sk, rk, idx); },
                    [&](uint32_t pos, uint32_t idx) { if (pos < kmx) orow[pos] = off + (int32_t)idx; },
                    run, sm);
  }
  for (int i = rp.k_eff + threadIdx.x; i < P.k_max; i += kRT) orow[i] = -1;
}

// LONG: rows of more wave slices than one gather batch per wave covers (long rows) take the
// flat gather; it is compiled into a kernel of its own so that the common kernel's code and
// register allocation stay as they are without it.
template <int MODE, bool LONG>
__global__ __launch_bounds__(kRT) void ts_row_kernel(Params P) {
  __shared__ Smem sm;
  // With the stream kernel's XCD mapping (rows 8x .. 8x + rows/8 - 1 on XCD x, workgroups
  // being dealt round-robin over the 8 XCDs), workgroup b takes a row whose summaries and
  // candidates were written on its own XCD.
  const int b = (int)blockIdx.x;
  // workgroups past the rows are the other parts of split-nucleus rows (part 1 of every row,
  // then part 2, ...); for the other rows they end here
  const int part = b < P.rows ? 0 : 1 + (b - P.rows) / P.rows;
  const int bb = part ? (b - P.rows) % P.rows : b;
  const int r = P.xcd_map ? (bb & 7) * (P.rows >> 3) + (bb >> 3) : bb;
  if (part && !split_row(P, plan_row(P, MODE, r))) return;
  const int nseg = P.chunks * kW1;
  const WaveInfo* inf = P.info + (int64_t)r * nseg;
  uint32_t flags = 0, kmax = 0, thr_max = 0, cmin = 0xFFFFFFFFu;
  uint32_t kw0 = kKeyNegInf;   // the maximum key of this thread's first slice
  double ws0 = 0.0;            // and its exponential sum (sampling with logprobs)
  uint32_t cnt0 = 0;           // and its candidate count
  // At most one slice per thread: the slice offsets come with the summaries' reduction.
  const bool one_slice = !P.direct && nseg <= kRT;
  RowPlan rp;
  if (P.direct) {
    // The whole row is the candidate set: its keys and ids go straight to LDS (no stream
    // kernel ran). Every element is a candidate, so the certification below always holds
    // (thr_max = 0); cmin is the row's smallest key.
    rp = plan_row(P, MODE, r);
    const float* row = P.x + (int64_t)r * P.stride;
#pragma unroll 4
    for (int i = threadIdx.x; i < rp.n; i += kRT) {
      const float v = row[i];
      const uint32_t key = f2key(v);
      flags |= (v != v) ? kFlagNan : 0u;
      kmax = max(kmax, key);
      cmin = min(cmin, key);
      sm.ckey[i] = key;
      sm.cidx[i] = (uint32_t)i;
    }
  } else {
    // Aggregate the wave summaries. Their loads are issued first; the row parameters and
    // the seed load while they are in flight. Counts go to LDS for the slice offsets. With
    // logprobs, this thread's first slice's exponential sum loads alongside.
    if (MODE == kModeSample && P.wsum && (int)threadIdx.x < nseg) ws0 = P.wsum[(int64_t)r * nseg + threadIdx.x];
    for (int i = threadIdx.x; i < nseg; i += kRT) {
      const WaveInfo wi = inf[i];
      if (i == (int)threadIdx.x) {
        kw0 = wi.kmax;
        cnt0 = wi.count;
      }
      flags |= wi.flags;
      kmax = max(kmax, wi.kmax);
      thr_max = max(thr_max, wi.thr);
      cmin = min(cmin, wi.thr);
      if (!one_slice && i < kMaxSeg) sm.segoff[i] = wi.count;
    }
    rp = plan_row(P, MODE, r);
  }
  const uint64_t seed = (MODE == kModeSample) ? P.seed[r] : 0ull;
  // zero the histograms (each select leaves them zero again), the small-bin counter and the
  // compaction counter (one compaction per workgroup)
  if (threadIdx.x == 0) {
    sm.bcount = 0;
    sm.kcount[0] = 0;
  }
  for (int i = threadIdx.x; i < kDBins / 4; i += kRT) reinterpret_cast<uint4*>(sm.hist)[i] = make_uint4(0, 0, 0, 0);
  for (int i = threadIdx.x; i < kDBins / 2; i += kRT) {
    reinterpret_cast<uint4*>(sm.mhi)[i] = make_uint4(0, 0, 0, 0);
  }
  // kmax, thr_max: maxima; cmin: every candidate key is >= the smallest threshold
  uint32_t seg_total = 0;
  if (one_slice) {
    uint32_t excl;
    block_reduce4_scan<kRW>(kmax, thr_max, cmin, flags, cnt0, excl, seg_total, sm.red);
    if ((int)threadIdx.x < nseg) sm.segoff[threadIdx.x] = excl;
    if (threadIdx.x == 0) sm.segoff[nseg] = seg_total;
    bar();   // the offsets are visible to the gathers, and `red` is free again
  } else {
    block_reduce4<kRW>(kmax, thr_max, cmin, flags, sm.red);
  }
  const bool nan = (flags & kFlagNan) != 0;
  int st = TS_ROW_OK;
  if (MODE == kModeTopk) {
    if (nan) st = TS_ROW_NONFINITE;
  } else if (nan || kmax >= kKeyPosInf || kmax <= kKeyNegInf) {
    st = TS_ROW_NONFINITE;
  }
  if (st == TS_ROW_OK) st = rp.bad;
  if (part == 0 && threadIdx.x == 0 && P.status) P.status[r] = st;
  // Sampling with logprobs: lse = m/T + log S over the whole row, S combined from the wave
  // shares in wave order, each rescaled from its wave maximum to the row maximum m.
  double lse = 0.0;
  if (MODE == kModeSample && P.wsum) {
    double zpart = 0.0;
    if (st == TS_ROW_OK && rp.t > 0.0f && P.direct) {
      // the row is in LDS: S directly, exp(y) = 2^(y log2 e) in fp32 (hardware exp2, as in
      // the stream kernel), binary64 accumulation
      const float m_f = key2f(kmax);
      const float c2f = (float)(1.4426950408889634 / (double)rp.t);
      for (int i = threadIdx.x; i < rp.n; i += kRT)
        zpart += (double)__builtin_amdgcn_exp2f((key2f(sm.ckey[i]) - m_f) * c2f);
    } else if (st == TS_ROW_OK && rp.t > 0.0f) {
      // each wave's share rescaled by exp((m_w - m) / T), fp32-accurate (the weights' form)
      const float m_f = key2f(kmax);
      const double c2 = kLog2e / (double)rp.t;
      if ((int)threadIdx.x < nseg && kw0 > kKeyNegInf) zpart += ws0 * (double)weight32(kw0, m_f, c2);
      for (int i = kRT + (int)threadIdx.x; i < nseg; i += kRT) {
        const uint32_t kw = inf[i].kmax;
        if (kw > kKeyNegInf) zpart += P.wsum[(int64_t)r * nseg + i] * (double)weight32(kw, m_f, c2);
      }
    }
    const double z = block_sum_f64<kRW>(zpart, reinterpret_cast<double*>(sm.red64));
    lse = (double)key2f(kmax) / (double)rp.t + log_fast(z);
  }

  if (MODE == kModeTopp && P.direct && P.out_mask) {
    // no stream kernel wrote the mask row: all ones for a full row, else zeros (the kept
    // tokens are marked below, after every zero has landed)
    fill_bytes_nt<kRT>(P.out_mask + (int64_t)r * P.V, P.V,
                       (st == TS_ROW_OK && rp.path == kPathFull) ? (uint8_t)1 : (uint8_t)0);
    bar_all();
  }
  if (st != TS_ROW_OK) {
    if (part) return;
    if (MODE == kModeTopp && rp.path == kPathFull && P.out_mask && !P.direct) {
      fill_bytes_nt<kRT>(P.out_mask + (int64_t)r * P.V, P.V, 0);   // chunks had written ones
    }
    if (MODE == kModeTopk) {
      for (int i = threadIdx.x; i < P.k_max; i += kRT) P.out_idx[(int64_t)r * P.k_max + i] = -1;
    } else if (MODE == kModeTopp) {
      if (threadIdx.x == 0) P.out_kept[r] = 0;
    } else {
      if (threadIdx.x == 0) {
        P.out_token[r] = -1;
        put_logp(P, r, -1, rp.t, lse);
      }
    }
    return;
  }

  const int path = rp.path;
  if (path == kPathGreedy) {
    // slices are in id order: the lowest id holding the row maximum
    uint32_t idx = 0xFFFFFFFFu;
    if (P.direct) {
      for (int i = threadIdx.x; i < rp.n; i += kRT)
        if (sm.ckey[i] == kmax) idx = min(idx, (uint32_t)i);
    } else {
      for (int i = threadIdx.x; i < nseg; i += kRT) {
        const WaveInfo wi = inf[i];
        if (wi.kmax == kmax) idx = min(idx, wi.kmax_idx);
      }
    }
    idx = block_min_u32<kRW>(idx, sm.red);
    if (MODE == kModeTopp) {
      if (threadIdx.x == 0) {
        P.out_kept[r] = 1;
        if (P.out_mask && idx < (uint32_t)P.V) P.out_mask[(int64_t)r * P.V + idx] = 1;
      }
    } else if (MODE == kModeSample) {
      if (threadIdx.x == 0) {
        P.out_token[r] = (int32_t)idx;
        put_logp(P, r, (int32_t)idx, rp.t, lse);
      }
    }
    return;
  }
  if (path == kPathFull) {
    if (MODE == kModeTopp) {
      if (threadIdx.x == 0) P.out_kept[r] = P.V;
    } else if (MODE == kModeSample) {
      const float m = key2f(kmax);
      float bs = -INFINITY;
      int32_t bi = 0x7FFFFFFF;
      if (P.direct) {
        const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
        for (int i = threadIdx.x; i < rp.n; i += kRT) {
          const float sc = gumbel_score(sm.ckey[i], (uint32_t)i, m, rp.t, (uint32_t)r, k0, k1);
          if (sc > bs) { bs = sc; bi = i; }   // ids rise along a thread's elements
        }
      } else {
        for (int i = threadIdx.x; i < nseg; i += kRT) {
          const WaveInfo wi = inf[i];
          const float adj = wi.best_s + (key2f(wi.kmax) - m) * (1.0f / rp.t);
          if (adj > bs || (adj == bs && wi.best_idx < bi)) { bs = adj; bi = wi.best_idx; }
        }
      }
      bi = block_argmax<kRW>(bs, bi, sm.reds, sm.redi, nullptr, true);
      if (threadIdx.x == 0) {
        P.out_token[r] = bi;
        put_logp(P, r, bi, rp.t, lse);
      }
    }
    return;
  }

  if (path == kPathNucleus && nucleus_finish<MODE>(P, rp, r, kmax, seed, sm, lse)) return;

  // the smallest key the exact path must consider (a lower bound of the row's k-th key)
  uint32_t kfloor = kKeyNegInf;
  if (path == kPathCand && P.direct) {
    const uint32_t ntot = (uint32_t)rp.n;
    if (ntot && !P.force_exact) {
      const uint32_t ke = (uint32_t)rp.k_eff;
      auto vis = [&](auto f) { lds_for(sm.ckey, sm.cidx, ntot, f); };
      Sel sk = sel_all();
      uint32_t min_sel = cmin;
      if (ntot > ke) {
        sk = select_topk(vis, ke, ntot, kmax, cmin, 0u, (uint32_t)(P.V - 1), sm, false);
        min_sel = shl(sk.prefix, sk.lo);
      }
      if (MODE == kModeTopk) {
        emit_topk_cand(P, rp, r, ntot, sk, sm);
        return;
      }
      finish_cand<MODE>(P, rp, r, kmax, max(cmin, min_sel), seed, ntot, sk, sm, lse);
      return;
    }
  } else if (path == kPathCand && nseg <= kMaxSeg) {
    const uint32_t ke = (uint32_t)rp.k_eff;
    // exclusive prefix of the slice counts: the candidates' flat, id-ordered index space
    // (with one slice per thread it came with the summaries' reduction)
    uint32_t total = seg_total;
    if (!one_slice) {
      const int s0 = kSegPT * (int)threadIdx.x;   // kSegPT consecutive slices per thread
      uint32_t cs[kSegPT], csum = 0;
#pragma unroll
      for (int q = 0; q < kSegPT; ++q) {
        cs[q] = s0 + q < nseg ? sm.segoff[s0 + q] : 0u;
        csum += cs[q];
      }
      uint32_t off = block_excl_scan<kRW>(csum, sm.red, total);   // barrier before the writes
#pragma unroll
      for (int q = 0; q < kSegPT; ++q) {
        if (s0 + q < nseg) sm.segoff[s0 + q] = off;
        off += cs[q];
      }
      if (threadIdx.x == 0) sm.segoff[nseg] = total;
    }
    // Wave w published the elements >= its threshold (at most the cap of them when it
    // overflowed): at least `total` elements are >= cmin, so the k-th key is >= cmin (used
    // only when a top-k select runs, k < V).
    if (total >= ke && ke < (uint32_t)rp.n) kfloor = cmin;
    const bool fast = !P.force_exact && (flags & kFlagOverflow) == 0 && total >= ke;
    uint32_t ntot = 0, lo_key = cmin;
    bool pre = false;
    if (fast && (flags & kFlagUniform)) {
      // Some slice is uniform (it stores nothing). When every candidate is one key its first
      // ke in id order are the top ke; otherwise (a constant stretch among other candidates)
      // the row takes the exact path.
      if (cmin == kmax) {
        bar();
        ntot = gather_equal(P, r, nseg, ke, sm);
        lo_key = kmax;
      }
    } else if (fast && total <= (uint32_t)kLdsCand) {
      if (!one_slice) bar();   // the offsets just written (with one slice per thread, already)
      // The top-k select's first pass is counted while the candidates are written to LDS:
      // every candidate key lies in [cmin, kmax], so its digit needs no prefix test.
      const Digit g0 = first_digit(kmax, cmin);
      pre = total > ke && g0.lo > 0;
      auto put = [&](uint32_t f, uint2 v) {
        sm.ckey[f] = v.x;
        sm.cidx[f] = v.y;
        if (pre) atomicAdd(&sm.hist[(v.x >> g0.sh) & g0.dm], 1u);
      };
      {
        // Wave w copies slices w, w + kRW, ...: lane l takes slots l, l + 64, ... of each
        // (coalesced). Per batch of kGatherB slices the offsets are read first, then every load
        // is issued (two per slice and lane when a slice of the batch holds more than 64, so
        // that such slices cost no second round trip), then the candidates are written; slices
        // holding more than 64 * NL finish afterwards.
        const uint32_t j = (uint32_t)lane();
        auto batch = [&](const uint2* gs, const uint32_t* o, const uint32_t* cnt, auto nl) {
          constexpr uint32_t NL = decltype(nl)::value;
          uint2 v[kGatherB][NL];
#pragma unroll
          for (int u = 0; u < kGatherB; ++u) {
#pragma unroll
            for (uint32_t e = 0; e < NL; ++e) {
              const uint32_t jj = 64u * e + j;
              v[u][e] = jj < cnt[u] ? gs[(int64_t)u * kRW * P.cap_w + jj] : make_uint2(0, 0);
            }
          }
          bool more = false;
#pragma unroll
          for (int u = 0; u < kGatherB; ++u) {
#pragma unroll
            for (uint32_t e = 0; e < NL; ++e) {
              const uint32_t jj = 64u * e + j;
              if (jj < cnt[u]) put(o[u] + jj, v[u][e]);
            }
            more |= cnt[u] > 64u * NL;
          }
          if (more) {   // wave-uniform: some slice of the batch holds more than 64 * NL candidates
#pragma unroll
            for (int u = 0; u < kGatherB; ++u) {
              for (uint32_t j0 = 64u * NL; j0 < cnt[u]; j0 += 256u) {   // 4 loads in flight per lane
                uint2 w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const uint32_t jj = j0 + 64u * e + j;
                  w[e] = jj < cnt[u] ? gs[(int64_t)u * kRW * P.cap_w + jj] : make_uint2(0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const uint32_t jj = j0 + 64u * e + j;
                  if (jj < cnt[u]) put(o[u] + jj, w[e]);
                }
              }
            }
          }
        };
        // Rows of more slices than one batch per wave covers (long rows): each thread takes
        // the flat candidate positions tid, tid + kRT, ... instead, finds each one's slice by a
        // branch-free binary search of the slice offsets in LDS (the E searches interleave),
        // and issues all its loads at once, so that the gather is one round trip.
        auto flat = [&](auto ne) {
          constexpr int E = decltype(ne)::value;
          const uint2* gr = P.cand + (int64_t)r * nseg * P.cap_w;
          const uint32_t ns = (uint32_t)nseg;
          uint32_t sl[E], so[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            sl[e] = 0;
            so[e] = 0;   // segoff[0]
          }
          // the largest slice whose offset is <= f (segoff[nseg] = total exceeds every f)
          for (uint32_t bb = 1u << (31 - __builtin_clz(ns - 1)); bb > 0; bb >>= 1) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const uint32_t f = min((uint32_t)(e * kRT) + threadIdx.x, total - 1);
              const uint32_t t = sl[e] + bb;
              const uint32_t sv = sm.segoff[min(t, ns)];
              if (sv <= f) {
                sl[e] = t;
                so[e] = sv;
              }
            }
          }
          uint2 v[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const uint32_t f = (uint32_t)(e * kRT) + threadIdx.x;
            v[e] = f < total ? gr[(int64_t)sl[e] * P.cap_w + (f - so[e])] : make_uint2(0, 0);
          }
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const uint32_t f = (uint32_t)(e * kRT) + threadIdx.x;
            if (f < total) put(f, v[e]);
          }
        };
        static_assert(kLdsCand <= 24 * kRT, "flat gather covers the LDS candidate capacity");
        if constexpr (LONG) {
          if (total <= 8u * kRT) flat(std::integral_constant<int, 8>{});
          else if (total <= 16u * kRT) flat(std::integral_constant<int, 16>{});
          else flat(std::integral_constant<int, 24>{});
        } else for (int sb = wave(); sb < nseg; sb += kRW * kGatherB) {
          uint32_t o[kGatherB], cnt[kGatherB], mx = 0;
#pragma unroll
          for (int u = 0; u < kGatherB; ++u) {
            const int sl = min(sb + u * kRW, nseg);   // slice nseg has no candidates
            o[u] = sm.segoff[sl];
            cnt[u] = sm.segoff[min(sl + 1, nseg)] - o[u];
            mx = max(mx, cnt[u]);
          }
          const uint2* gs = P.cand + ((int64_t)r * nseg + sb) * P.cap_w;
          // two loads per slice and lane only in top-k select (its k = 2048 rows publish
          // slices of 65-128 candidates); the sampling kernels run faster without that code
          if constexpr (MODE == kModeTopk) {
            if (mx > 64u) batch(gs, o, cnt, std::integral_constant<uint32_t, 2>{});
            else batch(gs, o, cnt, std::integral_constant<uint32_t, 1>{});
          } else {
            const uint32_t j = (uint32_t)lane();
            uint2 v[kGatherB];
#pragma unroll
            for (int u = 0; u < kGatherB; ++u) {
              v[u] = make_uint2(0, 0);
              if (j < cnt[u]) v[u] = gs[(int64_t)u * kRW * P.cap_w + j];
            }
            bool more = false;
#pragma unroll
            for (int u = 0; u < kGatherB; ++u) {
              if (j < cnt[u]) put(o[u] + j, v[u]);
              more |= cnt[u] > 64u;
            }
            if (more) {   // wave-uniform: some slice of the batch holds more than 64 candidates
#pragma unroll
              for (int u = 0; u < kGatherB; ++u) {
                for (uint32_t j0 = 64u; j0 < cnt[u]; j0 += 256u) {   // 4 loads in flight per lane
                  uint2 w[4];
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    const uint32_t jj = j0 + 64u * e + j;
                    w[e] = jj < cnt[u] ? gs[(int64_t)u * kRW * P.cap_w + jj] : make_uint2(0, 0);
                  }
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    const uint32_t jj = j0 + 64u * e + j;
                    if (jj < cnt[u]) put(o[u] + jj, w[e]);
                  }
                }
              }
            }
          }
        }
      }
      bar();
      ntot = total;
    } else if (fast) {
      bar();
      ntot = gather_filtered(P, r, nseg, ke, kmax, cmin, sm, &lo_key);
    }
    if (ntot) {
      auto vis = [&](auto f) { lds_for(sm.ckey, sm.cidx, ntot, f); };
      Sel sk = sel_all();
      uint32_t min_sel = lo_key;
      if (ntot > ke) {
        sk = select_topk(vis, ke, ntot, kmax, lo_key, 0u, (uint32_t)(P.V - 1), sm, pre);
        min_sel = shl(sk.prefix, sk.lo);
      }
      // Certification: every element of the row with a key >= the smallest selected key
      // was published by its wave, so the candidates' top-k is the row's top-k.
      if (min_sel >= thr_max) {
        if (MODE == kModeTopk) {
          emit_topk_cand(P, rp, r, ntot, sk, sm);
          return;
        }
        finish_cand<MODE>(P, rp, r, kmax, max(lo_key, min_sel), seed, ntot, sk, sm, lse);
        return;
      }
    }
  }
  // top-k off (k >= the row length) with top-p or min-p on, in a call with a top-k array: the
  // split nucleus over this row's workgroups (the exact path when its cut bin is too long)
  if (split_row(P, rp) && row_nucleus<MODE>(P, rp, r, kmax, seed, sm, lse, part)) return;
  row_stream<MODE>(P, rp, r, kmax, kfloor, seed, sm, lse);
}

__global__ void ts_fill_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ void ts_noise_kernel(uint64_t seed, int32_t row, const int32_t* tokens, int64_t n,
                                uint32_t* out_word, float* out_u, float* out_g) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const uint32_t tok = (uint32_t)tokens[j];
  const uint4 w = philox4x32_10(tok >> 2, (uint32_t)row, (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint32_t wd = pick_word(w, tok & 3u);
  const float u = uniform_from_word(wd);
  if (out_word) out_word[j] = wd;
  if (out_u) out_u[j] = u;
  if (out_g) out_g[j] = gumbel_from_uniform(u);
}

__global__ void ts_noise_words_kernel(const uint32_t* words, int64_t n, float* out_u, float* out_g) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const float u = uniform_from_word(words[j]);
  if (out_u) out_u[j] = u;
  if (out_g) out_g[j] = gumbel_from_uniform(u);
}

}  // namespace

// ================================================================== host side
// Error reporting and the device check, shared with the other sources of the library.
namespace tsh {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

struct DevProps {
  bool probed = false;
  bool ok = false;
  std::string arch;
};
std::mutex g_dev_mu;
std::vector<DevProps> g_dev;

int check_device(int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TS_ERR_UNSUPPORTED, "no HIP device available");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
  DevProps& d = g_dev[dev];
  if (!d.probed) {
    hipDeviceProp_t prop;
    d.probed = true;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      d.arch = prop.gcnArchName;
      d.ok = d.arch.compare(0, 6, "gfx950") == 0;
    }
  }
  if (!d.ok) return fail(TS_ERR_UNSUPPORTED, "device %d is '%s', this library is built for gfx950", dev, d.arch.c_str());
  *dev_out = dev;
  return TS_OK;
}

const char* last_error() { return g_last_error.c_str(); }

}  // namespace tsh

namespace {

using tsh::check_device;
using tsh::fail;

// Test hooks (topselect_testing.h): per calling thread, so that a setting made by one thread
// never reaches another thread's calls or workspace sizes.
thread_local int64_t g_knob_chunk = 0;
thread_local int64_t g_knob_exact = 0;
thread_local int64_t g_knob_direct = 1;
thread_local int64_t g_knob_nucleus = 0;

struct Plan {
  int64_t chunks = 0, chunk_len = 0, cap_w = 0;
  size_t off_info = 0, off_cand = 0, off_wsum = 0, off_nuc = 0, total = 0;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Chunking of a row and the workspace layout: per (row, chunk, wave) a WaveInfo, then per
// (row, chunk, wave) a slice of cap_w candidate slots, then per (row, chunk, wave) one double
// (the wave's exponential sum, used by sampling with logprobs).
bool make_plan(int64_t rows, int64_t V, Plan& pl, int64_t cap_limit = kCapW) {
  if (rows < 0 || V < 1 || V > TS_MAX_VOCAB) return false;
  int64_t ce = g_knob_chunk;
  if (ce <= 0) ce = kChunkMax;
  const int64_t chunks0 = (V + ce - 1) / ce;
  int64_t len = (V + chunks0 - 1) / chunks0;
  len = (len + 3) & ~int64_t(3);
  pl.chunk_len = len;
  pl.chunks = (V + len - 1) / len;
  const int64_t qw = ((len + 3) / 4 + kW1 - 1) / kW1;   // quads per wave
  const int64_t share = 4 * qw;                          // elements per wave, at most
  // half the share, less 32 entries: the summaries, partial sums and per-row histograms
  // then fit too, so that a default-chunked workspace is no larger than the logits
  const int64_t cap = share <= kCapSmall ? share : std::max<int64_t>(share / 2 - 32, kCapSmall);
  pl.cap_w = std::min<int64_t>(cap, cap_limit);
  const int64_t rr = rows > 0 ? rows : 1;
  if (rr * pl.chunks * kW1 > (int64_t)0x7FFFFFFF) return false;
  const size_t nseg = (size_t)(rr * pl.chunks * kW1);
  size_t b = 0;
  pl.off_info = b;
  b += align256(nseg * sizeof(WaveInfo));
  pl.off_cand = b;
  b += align256(nseg * (size_t)pl.cap_w * sizeof(uint2));
  pl.off_wsum = b;
  b += align256(nseg * sizeof(double));
  pl.off_nuc = b;
  b += align256((size_t)rr * sizeof(NucRow));
  pl.total = b;
  return true;
}

template <int MODE>
int launch(const float* x, int64_t rows, int64_t V, int64_t stride, const int32_t* k, int32_t k_max,
           const float* p, const float* t, const uint64_t* seed, int32_t* out_idx, int32_t* out_kept,
           uint8_t* out_mask, int32_t* out_token, int32_t* status, void* ws, size_t ws_bytes,
           void* stream, float* out_logp = nullptr, float* out_lse = nullptr,
           const float* minp = nullptr, const int32_t* lengths = nullptr, const int32_t* offsets = nullptr,
           int order = TS_ORDER_INDEX, int64_t cap_limit = kCapW) {
  if (rows < 0) return fail(TS_ERR_INVALID_ARG, "rows = %lld < 0", (long long)rows);
  if (V < 1 || V > TS_MAX_VOCAB) return fail(TS_ERR_INVALID_ARG, "vocab = %lld outside [1, 2^30]", (long long)V);
  if (stride < V) return fail(TS_ERR_INVALID_ARG, "row_stride %lld < vocab %lld", (long long)stride, (long long)V);
  if (rows == 0) return TS_OK;   // an empty batch: nothing to read or write
  if (!x) return fail(TS_ERR_INVALID_ARG, "logits pointer is NULL");
  if (rows > 0x7FFFFFFF) return fail(TS_ERR_INVALID_ARG, "rows too large");
  Plan pl;
  if (!make_plan(rows, V, pl, cap_limit)) return fail(TS_ERR_INVALID_ARG, "rows x chunks too large");
  if (!ws) return fail(TS_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)ws & 255u) != 0) return fail(TS_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < pl.total)
    return fail(TS_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, pl.total);
  int dev;
  int rc = check_device(&dev);
  if (rc != TS_OK) return rc;
  Params P;
  memset(&P, 0, sizeof(P));
  P.x = x;
  P.stride = stride;
  P.V = (int32_t)V;
  P.rows = (int32_t)rows;
  P.k = k;
  P.p = p;
  P.t = t;
  P.seed = seed;
  P.minp = minp;
  P.lengths = lengths;
  P.offsets = offsets;
  P.order = order;
  P.k_max = k_max;
  P.chunks = (int32_t)pl.chunks;
  P.chunk_len = (int32_t)pl.chunk_len;
  P.cap_w = (int32_t)pl.cap_w;
  P.xcd_map = (pl.chunks > 1 && rows % 8 == 0) ? 1 : 0;
  P.force_exact = (int32_t)g_knob_exact;
  // Rows that fit the row kernel's LDS skip the stream kernel (unless a chunk size is forced).
  P.direct = (V <= kLdsCand && g_knob_chunk == 0 && g_knob_direct != 0) ? 1 : 0;
  // With a top-k array, rows whose k reaches the row length are seen on the device only: the
  // row kernel then runs up to 8 workgroups per row (one per CU across the batch) that share
  // such rows' nucleus work (the split nucleus); for the other rows the extra workgroups end
  // at once. Each part keeps its bins in a slot of 2 * kNucBins words inside the row's
  // candidate area; when sampling, the slots are followed by one byte per token (in 8-byte
  // words of two quads) if the area holds them beside at least one slot (the
  // allocation-free entry point's smaller slices do not: its parts then store no codes, and a
  // cut bin's tokens come from the row's values).
  const int64_t area = pl.chunks * kW1 * pl.cap_w * (int64_t)sizeof(uint2);
  const int64_t slot_bytes = 2 * kNucBins * (int64_t)sizeof(uint64_t);
  const int64_t code_bytes = ((V + 3) / 4 + 1) / 2 * (int64_t)sizeof(uint64_t);
  P.codes = (MODE == kModeSample && area - code_bytes >= slot_bytes) ? 1 : 0;
  const int64_t slots = (area - (P.codes ? code_bytes : 0)) / slot_bytes;
  const int64_t split = std::min<int64_t>({8, std::max<int64_t>(1, kSplitCUs / rows), slots});
  const bool nucleus_on = MODE != kModeTopk && !P.direct && !P.force_exact && (p != nullptr || minp != nullptr);
  // No top-k array: every row has top-k off, so rows with top-p or min-p on take the nucleus
  // passes (spread over the chunk workgroups, two launches more) or, when sampling in a call of
  // at most kSplitNokLogits logits over rows of at most kSplitNokV, the split nucleus, which is
  // faster there (fewer launches; the passes' wider grid wins on larger calls).
  const bool nok_split = MODE == kModeSample && k == nullptr && V <= kSplitNokV &&
                         (int64_t)rows * V <= kSplitNokLogits && split > 0 && g_knob_nucleus == 0;
  P.nucleus = (nucleus_on && k == nullptr && !nok_split) ? 1 : 0;
  P.split = (nucleus_on && (k != nullptr || nok_split) && split > 0) ? (int32_t)split : 0;
  const unsigned row_grid = (unsigned)(rows * (P.split ? P.split : 1));
  P.out_idx = out_idx;
  P.out_kept = out_kept;
  P.out_mask = out_mask;
  P.out_token = out_token;
  P.status = status;
  P.out_logp = out_logp;
  P.out_lse = out_lse;
  char* w = static_cast<char*>(ws);
  P.info = reinterpret_cast<WaveInfo*>(w + pl.off_info);
  P.cand = reinterpret_cast<uint2*>(w + pl.off_cand);
  P.wsum = (out_logp || out_lse) ? reinterpret_cast<double*>(w + pl.off_wsum) : nullptr;
  P.nuc = reinterpret_cast<NucRow*>(w + pl.off_nuc);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (!P.direct) {
    hipLaunchKernelGGL(ts_stream_kernel<MODE>, dim3((unsigned)(rows * pl.chunks)), dim3(kT1), 0, s, P);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "stream kernel launch failed: %s", hipGetErrorString(e));
  }
  if (P.nucleus) {
    hipLaunchKernelGGL(ts_nucleus_kernel<MODE>, dim3((unsigned)(rows * pl.chunks)), dim3(kNT), 0, s, P);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "nucleus kernel launch failed: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(ts_nucleus_cut_kernel<MODE>, dim3((unsigned)(rows * pl.chunks)), dim3(kT1), 0, s, P);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "nucleus cut kernel launch failed: %s", hipGetErrorString(e));
  }
  if (!P.direct && P.chunks * kW1 > kRW * kGatherB)
    hipLaunchKernelGGL((ts_row_kernel<MODE, true>), dim3(row_grid), dim3(kRT), 0, s, P);
  else
    hipLaunchKernelGGL((ts_row_kernel<MODE, false>), dim3(row_grid), dim3(kRT), 0, s, P);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "row kernel launch failed: %s", hipGetErrorString(e));
  return TS_OK;
}

// ------------------------------------------------------------------ allocation-free variant
// ts_sample_rows_noalloc keeps its workspace in this array: one copy per GPU, held until the
// process ends. Its candidate slices hold at most kCapNoAlloc candidates per wave (a wave with
// more flags an overflow and its row takes the exact path, which gives the same bytes), so the
// decode batch (64 x 151936) needs about 11 MB of it.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int64_t kCapNoAlloc = 256;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on each GPU (the host-side name is only a stand-in):
// looked up once per device, with that device current.
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;

int scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(TS_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TS_OK;
}

}  // namespace

// ================================================================== C ABI
extern "C" {

size_t ts_workspace_bytes(int op, int64_t rows, int64_t vocab, int32_t k_max) {
  (void)k_max;
  if (op < TS_OP_TOPK_SELECT || op > TS_OP_SAMPLE_ROWS) return 0;
  Plan pl;
  if (!make_plan(rows, vocab, pl)) return 0;
  return pl.total;
}

int ts_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(TS_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(TS_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  int dev;
  int rc = check_device(&dev);
  if (rc != TS_OK) return rc;
  const size_t words = workspace_bytes / 4;
  if (words == 0) return TS_OK;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(ts_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<uint32_t*>(workspace), words);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "fill launch failed: %s", hipGetErrorString(e));
  return TS_OK;
}

int ts_topk_select_rows(const float* keys, int64_t rows, int64_t row_len, int64_t row_stride,
                        const int32_t* lengths, const int32_t* k, int32_t k_max, int order,
                        const int32_t* offsets, int32_t* out_idx, int32_t* row_status, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (rows > 0 && (!k || !out_idx)) return fail(TS_ERR_INVALID_ARG, "k and out_idx are required");
  if (k_max < 1) return fail(TS_ERR_INVALID_ARG, "k_max = %d < 1", (int)k_max);
  if (order != TS_ORDER_INDEX && order != TS_ORDER_VALUE)
    return fail(TS_ERR_INVALID_ARG, "order = %d is neither TS_ORDER_INDEX nor TS_ORDER_VALUE", order);
  if (order == TS_ORDER_VALUE && k_max > kValueOrderMax)
    return fail(TS_ERR_INVALID_ARG, "value order supports k_max <= %d (got %d)", kValueOrderMax, (int)k_max);
  return launch<kModeTopk>(keys, rows, row_len, row_stride, k, k_max, nullptr, nullptr, nullptr,
                           out_idx, nullptr, nullptr, nullptr, row_status, workspace,
                           workspace_bytes, stream, nullptr, nullptr, nullptr, lengths, offsets, order);
}

int ts_topk_select(const float* keys, int64_t rows, int64_t row_len, int64_t row_stride,
                   const int32_t* k, int32_t k_max, int32_t* out_idx, int32_t* row_status,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return ts_topk_select_rows(keys, rows, row_len, row_stride, nullptr, k, k_max, TS_ORDER_INDEX, nullptr,
                             out_idx, row_status, workspace, workspace_bytes, stream);
}

int ts_topp_mask(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                 const int32_t* top_k, const float* top_p, const float* temperature,
                 int32_t* out_kept, uint8_t* out_mask, int32_t* row_status, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (rows > 0 && !out_kept) return fail(TS_ERR_INVALID_ARG, "out_kept is required");
  return launch<kModeTopp>(logits, rows, vocab, row_stride, top_k, 0, top_p, temperature, nullptr,
                           nullptr, out_kept, out_mask, nullptr, row_status, workspace,
                           workspace_bytes, stream);
}

int ts_sample_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                   const int32_t* top_k, const float* top_p, const float* temperature,
                   const uint64_t* seed, int32_t* out_token, int32_t* row_status, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (rows > 0 && (!seed || !out_token)) return fail(TS_ERR_INVALID_ARG, "seed and out_token are required");
  return launch<kModeSample>(logits, rows, vocab, row_stride, top_k, 0, top_p, temperature, seed,
                             nullptr, nullptr, nullptr, out_token, row_status, workspace,
                             workspace_bytes, stream);
}

int ts_sample_rows_noalloc(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                           const int32_t* top_k, const float* top_p, const float* temperature,
                           const uint64_t* seed, int32_t* out_token, int32_t* row_status, void* stream) {
  if (rows > 0 && (!seed || !out_token)) return fail(TS_ERR_INVALID_ARG, "seed and out_token are required");
  if (rows < 0) return fail(TS_ERR_INVALID_ARG, "rows = %lld < 0", (long long)rows);
  if (rows == 0) return TS_OK;
  Plan pl;
  if (!make_plan(rows, vocab, pl, kCapNoAlloc))
    return fail(TS_ERR_INVALID_ARG, "vocab = %lld or rows x chunks outside the supported range", (long long)vocab);
  if (pl.total > kScratchBytes)
    return fail(TS_ERR_INVALID_ARG,
                "%lld rows of %lld logits need %zu bytes of scratch; ts_sample_rows_noalloc holds %zu "
                "(use ts_sample_rows with a workspace)",
                (long long)rows, (long long)vocab, pl.total, kScratchBytes);
  int dev;
  int rc = check_device(&dev);
  if (rc != TS_OK) return rc;
  void* ws = nullptr;
  rc = scratch_address(dev, &ws);
  if (rc != TS_OK) return rc;
  return launch<kModeSample>(logits, rows, vocab, row_stride, top_k, 0, top_p, temperature, seed,
                             nullptr, nullptr, nullptr, out_token, row_status, ws, kScratchBytes, stream,
                             nullptr, nullptr, nullptr, nullptr, nullptr, TS_ORDER_INDEX, kCapNoAlloc);
}

int ts_sample_rows_logp(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                        const int32_t* top_k, const float* top_p, const float* temperature,
                        const uint64_t* seed, int32_t* out_token, float* out_logp, float* out_lse,
                        int32_t* row_status, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows > 0 && (!seed || !out_token || !out_logp))
    return fail(TS_ERR_INVALID_ARG, "seed, out_token and out_logp are required");
  return launch<kModeSample>(logits, rows, vocab, row_stride, top_k, 0, top_p, temperature, seed,
                             nullptr, nullptr, nullptr, out_token, row_status, workspace,
                             workspace_bytes, stream, out_logp, out_lse);
}

int ts_topp_mask_minp(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                      const int32_t* top_k, const float* top_p, const float* temperature,
                      const float* min_p, int32_t* out_kept, uint8_t* out_mask, int32_t* row_status,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (rows > 0 && (!out_kept || !min_p)) return fail(TS_ERR_INVALID_ARG, "min_p and out_kept are required");
  return launch<kModeTopp>(logits, rows, vocab, row_stride, top_k, 0, top_p, temperature, nullptr,
                           nullptr, out_kept, out_mask, nullptr, row_status, workspace,
                           workspace_bytes, stream, nullptr, nullptr, min_p);
}

int ts_sample_rows_minp(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                        const int32_t* top_k, const float* top_p, const float* temperature,
                        const float* min_p, const uint64_t* seed, int32_t* out_token,
                        int32_t* row_status, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows > 0 && (!seed || !out_token || !min_p))
    return fail(TS_ERR_INVALID_ARG, "min_p, seed and out_token are required");
  return launch<kModeSample>(logits, rows, vocab, row_stride, top_k, 0, top_p, temperature, seed,
                             nullptr, nullptr, nullptr, out_token, row_status, workspace,
                             workspace_bytes, stream, nullptr, nullptr, min_p);
}

int ts_gumbel_noise(uint64_t seed, int32_t row, const int32_t* tokens, int64_t n,
                    uint32_t* out_word, float* out_u, float* out_g, void* stream) {
  if (n < 0) return fail(TS_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return TS_OK;
  if (!tokens) return fail(TS_ERR_INVALID_ARG, "tokens is NULL");
  int dev;
  int rc = check_device(&dev);
  if (rc != TS_OK) return rc;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(ts_noise_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, seed, row,
                     tokens, n, out_word, out_u, out_g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "noise launch failed: %s", hipGetErrorString(e));
  return TS_OK;
}

int ts_noise_transform(const uint32_t* words, int64_t n, float* out_u, float* out_g, void* stream) {
  if (n < 0) return fail(TS_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return TS_OK;
  if (!words) return fail(TS_ERR_INVALID_ARG, "words is NULL");
  if (n > ((int64_t)1 << 40)) return fail(TS_ERR_INVALID_ARG, "n too large");
  int dev;
  int rc = check_device(&dev);
  if (rc != TS_OK) return rc;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(ts_noise_words_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, words, n, out_u, out_g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "noise launch failed: %s", hipGetErrorString(e));
  return TS_OK;
}

int64_t ts_debug_set(int knob, int64_t value) {
  switch (knob) {
    case TS_KNOB_CHUNK_ELEMS: {
      if (value != 0 && (value < 64 || value > kChunkMax || value % 64 != 0)) return -1;
      const int64_t old = g_knob_chunk;
      g_knob_chunk = value;
      return old;
    }
    case TS_KNOB_FORCE_EXACT: {
      const int64_t old = g_knob_exact;
      g_knob_exact = value ? 1 : 0;
      return old;
    }
    case TS_KNOB_DIRECT: {
      const int64_t old = g_knob_direct;
      g_knob_direct = value ? 1 : 0;
      return old;
    }
    case TS_KNOB_NUCLEUS_PASSES: {
      const int64_t old = g_knob_nucleus;
      g_knob_nucleus = value ? 1 : 0;
      return old;
    }
    default: return -1;
  }
}

const char* ts_status_string(int status) {
  switch (status) {
    case TS_OK: return "ok";
    case TS_ERR_INVALID_ARG: return "invalid argument";
    case TS_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TS_ERR_UNSUPPORTED: return "no supported (gfx950) device";
    case TS_ERR_LAUNCH: return "kernel launch failed";
    case TS_ROW_NONFINITE: return "row has NaN/+inf logits or only -inf";
    case TS_ROW_BAD_K: return "row k invalid";
    case TS_ROW_BAD_P: return "row top_p outside (0, 1]";
    case TS_ROW_BAD_T: return "row temperature negative or non-finite";
    case TS_ROW_BAD_MINP: return "row min_p outside [0, 1]";
    default: return "unknown status";
  }
}

const char* ts_last_error(void) { return tsh::last_error(); }

}  // extern "C"
