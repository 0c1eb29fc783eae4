// topselect.hip -- gfx950 kernels and the C ABI of the batched per-row sampler.
//
// Every call enqueues two kernels on the caller's stream:
//
//   ts_stream_kernel  rows x chunks workgroups of 256 threads. Each workgroup streams one
//                     contiguous chunk (<= 8192 logits) of one row from HBM exactly once,
//                     keeping the chunk's ordered keys in registers, and publishes a small
//                     summary of it. While the chunk arrives it builds a 12-bit histogram of
//                     the keys; from it the chunk picks a threshold L_c, the lower edge of
//                     the bin holding its m_c-th largest key, with m_c a safety multiple of
//                     the chunk's share of k, and writes every key >= L_c (id order) as a
//                     candidate.
//   ts_row_kernel     one 1024-thread workgroup per row. From the candidates it selects the
//                     row's exact top-k and certifies it: if the smallest selected key is
//                     >= every chunk's L_c, every row element that could rank above it is a
//                     candidate, so the candidate top-k IS the row top-k. Otherwise (adversarial
//                     or tie-heavy rows) it falls back to the exact row-streaming path. Then
//                     the top-p mass cut and the Gumbel argmax run on the top-k set.
//
// Row paths (chosen per row on the device from that row's k, p, T):
//   CAND    k_eff <= 2048: candidates + certified selection as above.
//   GREEDY  T == 0: the first token of the row ordering (max key, lowest id).
//   FULL    top-k and top-p both off (sampling): each chunk computes its Gumbel argmax
//           relative to its own maximum; the row kernel folds the chunk winners.
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
#include <vector>

#include "topselect.h"
#include "ts_device.hpp"

using namespace tsd;

namespace {

enum Mode : int { kModeTopk = 0, kModeTopp = 1, kModeSample = 2 };
enum Path : int { kPathNone = 0, kPathCand = 1, kPathGreedy = 2, kPathFull = 3, kPathStream = 4 };

// stream kernel
constexpr int kT1 = 256;                            // threads per chunk workgroup
constexpr int kW1 = kT1 / 64;                       // waves per chunk workgroup
constexpr int kS1 = 8;                              // float4 loads per thread
constexpr int kChunkMax = kT1 * 4 * kS1;            // 8192 logits per chunk
constexpr int kHBits = 11;                          // sample histogram digit (top key bits)
constexpr int kHBins = 1 << kHBits;
constexpr int kSampleSlots = 2;                     // slots whose keys form the sample
constexpr int kCapMax = 4096;                       // candidate slots per chunk
constexpr int kWStage = 512;                        // candidates staged per wave in LDS
// row kernel
constexpr int kFastK = 2048;                        // largest k taking the candidate path
constexpr int kBins = 256;                          // radix digit of 8 bits
constexpr int kCC = 8;                              // replicated count histograms
constexpr int kMC = 4;                              // replicated mass histograms
constexpr int kLdsCand = 8192;                      // candidates the row kernel keeps in LDS

struct ChunkInfo {
  uint32_t count;     // candidates written (CAND), capped at the chunk capacity
  uint32_t thr;       // L_c: every key >= thr of the chunk is a candidate (0: all)
  uint32_t kmax;      // largest key of the chunk's elements (0 if none)
  uint32_t kmin;      // smallest key of the chunk's elements (0xFFFFFFFF if none)
  uint32_t kmax_idx;  // lowest id holding kmax (GREEDY)
  uint32_t flags;     // bit 0: NaN seen; bit 1: candidates overflowed the capacity
  float best_s;       // FULL sampling: best score relative to the chunk maximum
  int32_t best_idx;
  uint32_t cmin;      // smallest candidate key written (0xFFFFFFFF if none)
};
static_assert(sizeof(ChunkInfo) == 36, "ChunkInfo layout");
constexpr uint32_t kFlagNan = 1u, kFlagOverflow = 2u;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Params {
  const float* x;
  int64_t stride;
  int32_t V;
  int32_t rows;
  const int32_t* k;
  const float* p;
  const float* t;
  const uint64_t* seed;
  int32_t k_max;
  int32_t chunks;
  int32_t chunk_len;
  int32_t cap_c;
  int32_t xcd_map;
  int32_t force_exact;
  int32_t leader_global;
  int32_t pad_;
  int32_t* out_idx;
  int32_t* out_kept;
  uint8_t* out_mask;
  int32_t* out_token;
  int32_t* status;
  ChunkInfo* info;
  uint2* cand;
};

struct RowPlan {
  int32_t k_eff;
  float p;
  float t;
  int32_t path;
  int32_t bad;
};

// LDS of the row kernel
struct Smem {
  // two histogram buffers: a pass fills one while the previous pass's one is cleared
  uint32_t hist[2][kBins * kCC];
  uint64_t mhist[2][kBins * kMC * 2];
  uint2 cand[kLdsCand];
  uint2 kset[kFastK];
  uint32_t red[kWaves];
  uint32_t red3[3 * kWaves];
  uint64_t red64[2 * kWaves];
  float reds[kWaves];
  int32_t redi[kWaves];
  uint32_t wave_tot[kWaves];
  uint32_t res[4];
  uint64_t res64[4];
  uint32_t segoff[1025];
  uint32_t kcount;
};

// LDS of the stream kernel
struct Smem1 {
  uint32_t hist[kHBins];
  uint2 stage[kW1][kWStage];
  uint32_t red3[3 * kW1];
  uint32_t red[kW1];
  float reds[kW1];
  int32_t redi[kW1];
  uint32_t wave_tot[kW1];
  uint32_t res[4];
};

// ------------------------------------------------------------------ per-row plan
__device__ __forceinline__ RowPlan plan_row(const Params& P, int mode, int r) {
  RowPlan rp;
  const int32_t kr = P.k ? P.k[r] : P.V;
  rp.k_eff = kr < 1 ? 0 : min(kr, P.V);
  rp.p = (mode != kModeTopk && P.p) ? P.p[r] : 1.0f;
  rp.t = (mode != kModeTopk && P.t) ? P.t[r] : 1.0f;
  int bad = TS_ROW_OK;
  if (kr < 1) bad = TS_ROW_BAD_K;
  else if (mode == kModeTopk && rp.k_eff > P.k_max) bad = TS_ROW_BAD_K;
  else if (mode != kModeTopk && !(rp.p > 0.0f && rp.p <= 1.0f)) bad = TS_ROW_BAD_P;
  else if (mode != kModeTopk && !(rp.t >= 0.0f && rp.t <= FLT_MAX)) bad = TS_ROW_BAD_T;
  rp.bad = bad;
  if (bad) rp.path = kPathNone;
  else if (mode == kModeTopk) rp.path = rp.k_eff <= kFastK ? kPathCand : kPathStream;
  else if (rp.t == 0.0f) rp.path = kPathGreedy;
  else if (rp.k_eff <= kFastK) rp.path = kPathCand;
  else if (rp.k_eff == P.V && rp.p == 1.0f) rp.path = kPathFull;
  else rp.path = kPathStream;
  return rp;
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
// Wave 0 only. Finds the highest bin b with (sum of counts in bins >= b) >= thr and writes
// res[0] = b, res[1] = count in bins > b, res[2] = count in b.
__device__ __forceinline__ void search_count(Smem& sm, int hb, uint32_t thr) {
  const int l = lane();
  uint32_t c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t s = 0;
#pragma unroll
    for (int cp = 0; cp < kCC; ++cp) s += sm.hist[hb][(4 * l + j) * kCC + cp];
    c[j] = s;
  }
  const uint32_t lsum = c[0] + c[1] + c[2] + c[3];
  const uint32_t excl = wave_incl_suffix(lsum) - lsum;
  const uint64_t bal = __ballot(excl + lsum >= thr);
  const int L = bal ? 63 - __clzll((long long)bal) : -1;
  if (l == L) {
    uint32_t acc = excl;
    int j = 3;
    for (; j > 0; --j) {
      if (acc + c[j] >= thr) break;
      acc += c[j];
    }
    sm.res[0] = 4 * L + j;
    sm.res[1] = acc;
    sm.res[2] = c[j];
  }
}

// Mass version: masses are exact (hi, lo) sums, compared with `target` after conversion to
// binary64. ma = mass already known to lie above the current prefix. Writes res[0] = bin,
// res[1] = count above, res[2] = count in bin, res64[0..1] = ma + mass above the bin,
// res64[2..3] = mass of the bin.
__device__ __forceinline__ void search_mass(Smem& sm, int hb, double target, uint64_t ma_hi, uint64_t ma_lo, int S) {
  const int l = lane();
  uint32_t c[4];
  uint64_t mh[4], ml[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t s = 0;
#pragma unroll
    for (int cp = 0; cp < kCC; ++cp) s += sm.hist[hb][(4 * l + j) * kCC + cp];
    c[j] = s;
    uint64_t h = 0, o = 0;
#pragma unroll
    for (int cp = 0; cp < kMC; ++cp) {
      h += sm.mhist[hb][((4 * l + j) * kMC + cp) * 2];
      o += sm.mhist[hb][((4 * l + j) * kMC + cp) * 2 + 1];
    }
    mh[j] = h;
    ml[j] = o;
  }
  const uint32_t lc = c[0] + c[1] + c[2] + c[3];
  const uint64_t lh = mh[0] + mh[1] + mh[2] + mh[3];
  const uint64_t lo_ = ml[0] + ml[1] + ml[2] + ml[3];
  const uint32_t xc = wave_incl_suffix(lc) - lc;
  const uint64_t xh = wave_incl_suffix64(lh) - lh;
  const uint64_t xl = wave_incl_suffix64(lo_) - lo_;
  const bool has = mass_to_double(ma_hi + xh + lh, ma_lo + xl + lo_, S) >= target;
  const uint64_t bal = __ballot(has);
  const int L = bal ? 63 - __clzll((long long)bal) : -1;
  if (l == L) {
    uint64_t ah = ma_hi + xh, al = ma_lo + xl;
    uint32_t ac = xc;
    int j = 3;
    for (; j > 0; --j) {
      if (mass_to_double(ah + mh[j], al + ml[j], S) >= target) break;
      ah += mh[j];
      al += ml[j];
      ac += c[j];
    }
    sm.res[0] = 4 * L + j;
    sm.res[1] = ac;
    sm.res[2] = c[j];
    sm.res64[0] = ah;
    sm.res64[1] = al;
    sm.res64[2] = mh[j];
    sm.res64[3] = ml[j];
  }
}

// Zero histogram buffer hb (count and mass); called by waves 1..15 while wave 0 searches
// the other buffer, or by the whole workgroup (first = 0, step = kThreads).
__device__ __forceinline__ void clear_hist(Smem& sm, int hb, int first, int step) {
  uint4* h = reinterpret_cast<uint4*>(sm.hist[hb]);
  for (int i = first; i < kBins * kCC / 4; i += step) h[i] = make_uint4(0, 0, 0, 0);
  uint4* m = reinterpret_cast<uint4*>(sm.mhist[hb]);
  for (int i = first; i < kBins * kMC; i += step) m[i] = make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void search_or_clear_count(Smem& sm, int hb, uint32_t thr) {
  if (wave() == 0) search_count(sm, hb, thr);
  else clear_hist(sm, hb ^ 1, (int)threadIdx.x - 64, kThreads - 64);
}

// ------------------------------------------------------------------ exact count select
// MSB-first radix select of the `need` largest radix keys among the items the visitor
// yields (vis(f) calls f(rk, idx) for this thread's items; the union over threads must be
// n_in_play items with hi_rk >= rk >= lo_rk). Bits above the highest bit where hi_rk and
// lo_rk differ are common and skipped. A pass stops early when the threshold bin holds
// exactly the slots still unfilled ([DETK] "Changes": pass skipping).
// On return: items with shr(rk, lo) > prefix are selected; eq_take of the tie_cnt items with
// shr(rk, lo) == prefix must still be taken (lowest ids first).
template <class Vis>
__device__ __forceinline__ void count_select(const Vis& vis, uint32_t need, uint32_t n_in_play, uint32_t hi_rk,
                             uint32_t lo_rk, Smem& sm, int& hb, uint32_t& prefix, int& lo,
                             uint32_t& eq_take, uint32_t& tie_cnt) {
  lo = (hi_rk == lo_rk) ? 0 : 32 - __clz((int)(hi_rk ^ lo_rk));
  prefix = shr(hi_rk, lo);
  tie_cnt = n_in_play;
  while (lo > 0 && need > 0) {
    const int d = min(8, lo);
    const int sh = lo - d;
    const uint32_t dm = (1u << d) - 1u;
    const uint32_t pre = prefix;
    const int lo_now = lo;
    const uint32_t copy = (uint32_t)lane() & (kCC - 1);
    uint32_t* hist = sm.hist[hb];   // zero on entry
    vis([&](uint32_t rk, uint32_t idx) {
      if (shr(rk, lo_now) == pre) atomicAdd(&hist[((rk >> sh) & dm) * kCC + copy], 1u);
    });
    bar();
    search_or_clear_count(sm, hb, need);
    bar();
    hb ^= 1;
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
                           uint32_t lo_key, uint32_t idx_lo, uint32_t idx_hi, Smem& sm, int& hb) {
  Sel s;
  uint32_t eq_take, tie_cnt;
  count_select(vis, need, n_in_play, hi_key, lo_key, sm, hb, s.prefix, s.lo, eq_take, tie_cnt);
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
    count_select(tvis, eq_take, tie_cnt, ~idx_lo, ~idx_hi, sm, hb, p2, lo2, e2, t2);
    s.cutoff = ~shl(p2, lo2);
  }
  return s;
}

// ------------------------------------------------------------------ mass select (top-p)
// Smallest prefix of the row ordering whose exact fixed-point mass reaches `target`
// ([TOPP] "Independent binary64 numerical reference", steps 4-5, with the predicate kept in
// probability space, [TOPP] "Source basis"). vis(f) calls f(rk, idx) for items of K; wfn(rk)
// returns the item's weight. Result: Sel of the kept set P (a canonical prefix) and |P|.
template <class Vis, class WFn>
__device__ __forceinline__ Sel select_mass(const Vis& vis, const WFn& wfn, double target, int S, uint32_t n_in_play,
                           uint32_t hi_key, uint32_t lo_key, uint32_t idx_lo, uint32_t idx_hi,
                           Smem& sm, int& hb, uint32_t& kept) {
  int lo = (hi_key == lo_key) ? 0 : 32 - __clz((int)(hi_key ^ lo_key));
  uint32_t prefix = shr(hi_key, lo);
  uint32_t n_above = 0, tie_cnt = n_in_play;
  uint64_t ma_hi = 0, ma_lo = 0, bin_hi = 0, bin_lo = 0;
  bool single = false, ran = false;
  while (lo > 0) {
    const int d = min(8, lo);
    const int sh = lo - d;
    const uint32_t dm = (1u << d) - 1u;
    const uint32_t pre = prefix;
    const int lo_now = lo;
    ran = true;
    const uint32_t cc = (uint32_t)lane() & (kCC - 1);
    const uint32_t mc = (uint32_t)lane() & (kMC - 1);
    uint32_t* hist = sm.hist[hb];      // both zero on entry
    uint64_t* mhist = sm.mhist[hb];
    vis([&](uint32_t rk, uint32_t idx) {
      if (shr(rk, lo_now) == pre) {
        const uint32_t b = (rk >> sh) & dm;
        const Mass m = mass_of(wfn(rk), S);
        atomicAdd(&hist[b * kCC + cc], 1u);
        atomicAdd((unsigned long long*)&mhist[(b * kMC + mc) * 2], (unsigned long long)m.hi);
        atomicAdd((unsigned long long*)&mhist[(b * kMC + mc) * 2 + 1], (unsigned long long)m.lo);
      }
    });
    bar();
    if (wave() == 0) search_mass(sm, hb, target, ma_hi, ma_lo, S);
    else clear_hist(sm, hb ^ 1, (int)threadIdx.x - 64, kThreads - 64);
    bar();
    hb ^= 1;
    const uint32_t bin = sm.res[0];
    n_above += sm.res[1];
    tie_cnt = sm.res[2];
    ma_hi = sm.res64[0];
    ma_lo = sm.res64[1];
    bin_hi = sm.res64[2];
    bin_lo = sm.res64[3];
    prefix = (prefix << d) | bin;
    lo = sh;
    if (tie_cnt == 1) { single = true; break; }
  }
  uint32_t take = 1;
  if (!single && tie_cnt > 1) {
    // The boundary key is shared by tie_cnt items of identical weight q (same key, same
    // fp32 logit, same binary64 weight): take the fewest of them, lowest ids first, that
    // bring the mass above to the target.
    uint64_t qh, ql;
    if (ran) {
      qh = bin_hi / tie_cnt;
      ql = bin_lo / tie_cnt;
    } else {  // every in-play key is equal and no pass ran
      const Mass q1 = mass_of(wfn(prefix), S);
      qh = q1.hi;
      ql = q1.lo;
    }
    const double q = mass_to_double(qh, ql, S);
    const double ma = mass_to_double(ma_hi, ma_lo, S);
    const double j = q > 0.0 ? ceil((target - ma) / q) : (double)tie_cnt;
    uint32_t t = (uint32_t)fmin(fmax(j, 1.0), (double)tie_cnt);
    while (t > 1 && mass_to_double(ma_hi + qh * (t - 1), ma_lo + ql * (t - 1), S) >= target) --t;
    while (t < tie_cnt && mass_to_double(ma_hi + qh * t, ma_lo + ql * t, S) < target) ++t;
    take = t;
  }
  Sel s{prefix, lo, 0xFFFFFFFFu};
  if (take < tie_cnt) {
    const uint32_t pre = prefix;
    const int lo_ = lo;
    auto tvis = [&](auto f) {
      vis([&](uint32_t rk, uint32_t idx) {
        if (shr(rk, lo_) == pre) f(~idx, idx);
      });
    };
    uint32_t p2, e2, t2;
    int lo2;
    count_select(tvis, take, tie_cnt, ~idx_lo, ~idx_hi, sm, hb, p2, lo2, e2, t2);
    s.cutoff = ~shl(p2, lo2);
  }
  kept = n_above + take;
  return s;
}

// ------------------------------------------------------------------ misc helpers

__device__ __forceinline__ double weight_of(uint32_t key, float m, float t) {
  return exp(((double)key2f(key) - (double)m) / (double)t);
}

__device__ __forceinline__ float gumbel_score(uint32_t key, uint32_t idx, float m, float t,
                                              uint32_t r, uint32_t k0, uint32_t k1) {
  const uint4 w = philox4x32_10(idx >> 2, r, k0, k1);
  const float g = gumbel_from_uniform(uniform_from_word(pick_word(w, idx & 3u)));
  return (key2f(key) - m) / t + g;
}

__device__ __forceinline__ int bitlen(uint32_t n) { return n ? 32 - __clz((int)n) : 0; }

// Ordered emission over an id-ordered source, E consecutive items per thread per tile (all
// loads of a tile are issued before any is used); out(pos, idx) writes selected item `idx`
// at `pos`, positions following the source order.
template <int E, class Get, class Mem, class Out>
__device__ __forceinline__ void emit_ordered(uint32_t n, const Get& get, const Mem& mem, const Out& out,
                                             uint32_t& run, Smem& sm) {
  for (uint32_t base = 0; base < n; base += kThreads * E) {
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
    uint32_t pos = block_excl_scan(cnt, sm.red, tot);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (sel[e]) out(run + pos++, idx[e]);
    }
    run += tot;
  }
}

// Visit items [0, n) of an indexable source, U per thread per round with all loads of a
// round issued first, so global-memory latency is paid once per round, not once per item.
template <int U, class Get, class F>
__device__ __forceinline__ void batched_for(uint32_t n, const Get& get, F f) {
  for (uint32_t base = 0; base < n; base += kThreads * U) {
    uint2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t j = base + u * kThreads + threadIdx.x;
      v[u] = make_uint2(0, 0);
      if (j < n) v[u] = get(j);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t j = base + u * kThreads + threadIdx.x;
      if (j < n) f(v[u].x, v[u].y);
    }
  }
}

// ------------------------------------------------------------------ stream kernel
// Wave 0 only: the highest bin b of the sample histogram with (count in bins >= b) >= thr.
// Writes res[0] = b, res[1] = count in bins > b, res[2] = count in b.
__device__ __forceinline__ void search_hist(Smem1& sm, uint32_t thr) {
  constexpr int kG = kHBins / 64 / 4;   // groups of 4 bins per lane
  const int l = lane();
  const uint4* h4 = reinterpret_cast<const uint4*>(sm.hist) + kG * l;
  uint32_t g[kG];
  uint32_t lsum = 0;
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    const uint4 v = h4[i];
    g[i] = v.x + v.y + v.z + v.w;
    lsum += g[i];
  }
  const uint32_t excl = wave_incl_suffix(lsum) - lsum;
  const uint64_t bal = __ballot(excl + lsum >= thr);
  const int L = bal ? 63 - __clzll((long long)bal) : -1;
  if (l == L) {
    uint32_t acc = excl;
    int gs = 0;
    bool done = false;
#pragma unroll
    for (int i = kG - 1; i >= 0; --i) {
      const bool hit = !done && (i == 0 || acc + g[i] >= thr);
      if (hit) { gs = i; done = true; }
      if (!done) acc += g[i];
    }
    const uint4 v = h4[gs];
    const uint32_t c[4] = {v.x, v.y, v.z, v.w};
    int j = 0;
    done = false;
    uint32_t cj = c[0];
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      const bool hit = !done && (i == 0 || acc + c[i] >= thr);
      if (hit) { j = i; cj = c[i]; done = true; }
      if (!done) acc += c[i];
    }
    sm.res[0] = (uint32_t)(kG * 4 * L + 4 * gs + j);
    sm.res[1] = acc;
    sm.res[2] = cj;
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
__global__ __launch_bounds__(kT1) void ts_stream_kernel(Params P) {
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
  const int n = min(P.chunk_len, P.V - c0);
  const float* base = P.x + (int64_t)r * P.stride + c0;
  const bool aligned = ((uintptr_t)base & 15u) == 0;
  const int nq = (n + 3) >> 2;
  const int qw = (nq + kW1 - 1) / kW1;
  const int w = wave(), l = lane();
  const int q_lo = w * qw;
  const int q_hi = min(q_lo + qw, nq);
  const int nfull = n >> 2;

  // Issue every load of the chunk before consuming any. Addresses are clamped into the
  // chunk so all loads are in bounds; elements past the end are masked afterwards.
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
  } else {
    const uint32_t* s32 = reinterpret_cast<const uint32_t*>(base);
#pragma unroll
    for (int s = 0; s < kS1; ++s) {
      const int e0 = 4 * (q_lo + s * 64 + l);
      raw[s].x = s32[min(e0, n - 1)];
      raw[s].y = s32[min(e0 + 1, n - 1)];
      raw[s].z = s32[min(e0 + 2, n - 1)];
      raw[s].w = s32[min(e0 + 3, n - 1)];
    }
  }
  // The row's parameters are read only now, so the chunk's loads above are already in
  // flight while these small loads resolve.
  const RowPlan rp = plan_row(P, MODE, r);
  const int path = rp.path;
  const bool cand = path == kPathCand;
  if (cand) {
    uint4* h = reinterpret_cast<uint4*>(sm.hist);
    for (int i = threadIdx.x; i < kHBins / 4; i += kT1) h[i] = make_uint4(0, 0, 0, 0);
  }
  bar();   // LDS only: the loads above stay in flight

  // Work on the fp32 values directly: a key >= threshold-key test is a float >= test against
  // the threshold's float (ordered keys are a monotone map of fp32, with -0 == +0 in both), so
  // only the sample and the selected candidates ever need their ordered key.
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
  // key has mean mu = k * ns / V, and the threshold sits mu + 6 sqrt(mu) + 10 keys down.
  uint32_t thr = kKeyNegInf;   // reported: every valid non-NaN element with key >= thr is emitted
  float thr_f = -INFINITY;
  if (cand) {
#pragma unroll
    for (int s = 0; s < kSampleSlots; ++s) {
      const int nv = nvalid(s);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < nv) atomicAdd(&sm.hist[f2key(xval(s, e)) >> (32 - kHBits)], 1u);
    }
    uint32_t ns = 0;   // valid sample elements of the workgroup
#pragma unroll
    for (int ww = 0; ww < kW1; ++ww) {
      const int lo_q = ww * qw, hi_q = min(lo_q + qw, nq);
      const int e_hi = min(min(4 * (lo_q + 64 * kSampleSlots), 4 * hi_q), n);
      ns += (uint32_t)max(e_hi - 4 * lo_q, 0);
    }
    const float mu = (float)rp.k_eff * (float)ns / (float)P.V;
    const uint32_t jt = (uint32_t)ceilf(mu + 6.0f * sqrtf(mu) + 10.0f);
    if (jt < ns) {
      bar();   // sample histogram complete
      if (w == 0) search_hist(sm, jt);
      bar();
      const uint32_t tk = sm.res[0] << (32 - kHBits);
      if (tk > kKeyNegInf) {
        thr = tk;
        thr_f = key2f(tk);
      }
    }
  }

  // Every slot, as it arrives: chunk statistics (float max, NaN flag) and, on the candidate
  // path, the ordered append of every value >= thr_f into this wave's LDS region. Ballots
  // give each selected element its position within the wave's segment ((slot, lane,
  // element) = id order); the waves' regions concatenate in wave order.
  float fmx = -INFINITY;
  uint32_t nan = 0;
  uint32_t run = 0;
#pragma unroll
  for (int s = 0; s < kS1; ++s) {
    const int nv = nvalid(s);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = xval(s, e);
      const bool valid = e < nv;
      fmx = valid ? fmaxf(fmx, x) : fmx;
      nan |= (valid && x != x) ? 1u : 0u;
    }
    if (cand) {
      uint64_t mk[4];
      uint32_t slot_cnt = 0, lane_off = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mk[e] = __ballot(e < nv && xval(s, e) >= thr_f);
        slot_cnt += (uint32_t)__popcll(mk[e]);
        lane_off += mbcnt(mk[e]);
      }
      uint32_t pos = run + lane_off;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((mk[e] >> l) & 1ull) {
          if (pos < (uint32_t)kWStage)
            sm.stage[w][pos] = make_uint2(f2key(xval(s, e)), (uint32_t)(c0 + 4 * (q_lo + s * 64 + l) + e));
          ++pos;
        }
      }
      run += slot_cnt;
    }
  }
  if (cand && l == 0) sm.wave_tot[w] = run;
  uint32_t kmax = f2key(fmx), kmin_unused = 0u;
  block_reduce3<kW1>(kmax, kmin_unused, nan, sm.red3);   // its barriers also publish wave_tot
  const float m_c = key2f(kmax);                          // the chunk maximum

  uint32_t count = 0, flags = nan ? kFlagNan : 0u, kmax_idx = 0xFFFFFFFFu;
  uint32_t cmin = 0xFFFFFFFFu;
  float best_s = -INFINITY;
  int32_t best_idx = 0x7FFFFFFF;

  if (cand) {
    uint32_t base = 0, total = 0;
    bool wave_ovf = false;
#pragma unroll
    for (int ww = 0; ww < kW1; ++ww) {
      const uint32_t t = sm.wave_tot[ww];
      base += (ww < w) ? t : 0u;
      total += t;
      wave_ovf |= t > (uint32_t)kWStage;
    }
    const uint32_t cap = (uint32_t)P.cap_c;
    uint2* out = P.cand + ((int64_t)r * P.chunks + c) * P.cap_c;
    if (!wave_ovf) {
      for (uint32_t i = (uint32_t)l; i < run; i += 64)
        if (base + i < cap) out[base + i] = sm.stage[w][i];
    } else {
      // a wave's region overflowed: store straight from registers (same positions)
      uint32_t rr = base;
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
        uint32_t pos = rr + lane_off;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((mk[e] >> l) & 1ull) {
            if (pos < cap) out[pos] = make_uint2(f2key(xval(s, e)), (uint32_t)(c0 + 4 * (q_lo + s * 64 + l) + e));
            ++pos;
          }
        }
        rr += slot_cnt;
      }
    }
    count = min(total, cap);
    if (total > cap) flags |= kFlagOverflow;
    cmin = thr;   // every candidate is >= thr: a valid lower bound for the row kernel
  } else if (path == kPathGreedy) {
    uint32_t mi = 0xFFFFFFFFu;
#pragma unroll
    for (int s = 0; s < kS1; ++s) {
      const int nv = nvalid(s);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (e < nv && xval(s, e) == m_c) mi = min(mi, (uint32_t)(c0 + 4 * (q_lo + s * 64 + l) + e));
      }
    }
    kmax_idx = block_min_u32<kW1>(mi, sm.red);
  } else if (path == kPathFull && MODE == kModeSample) {
    // Gumbel argmax of the chunk relative to the chunk maximum (one Philox block per quad).
    const uint64_t sd = P.seed[r];
    const uint32_t k0 = (uint32_t)sd, k1 = (uint32_t)(sd >> 32);
    float bs = -INFINITY;
    int32_t bi = 0x7FFFFFFF;
#pragma unroll
    for (int s = 0; s < kS1; ++s) {
      const int q = q_lo + s * 64 + l;
      const int nv = nvalid(s);
      if (nv > 0) {
        const uint32_t tok0 = (uint32_t)(c0 + 4 * q);
        const uint4 wd = philox4x32_10(tok0 >> 2, (uint32_t)r, k0, k1);
        const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e < nv) {
            const float g = gumbel_from_uniform(uniform_from_word(words[e]));
            const float sc = (xval(s, e) - m_c) / rp.t + g;
            const int32_t id = (int32_t)(tok0 + e);
            if (sc > bs || (sc == bs && id < bi)) { bs = sc; bi = id; }
          }
        }
      }
    }
    best_idx = block_argmax<kW1>(bs, bi, sm.reds, sm.redi, &best_s);
  }

  if (MODE == kModeTopp && P.out_mask) {
    fill_bytes_nt<kT1>(P.out_mask + (int64_t)r * P.V + c0, n, (path == kPathFull) ? (uint8_t)1 : (uint8_t)0);
  }
  if (threadIdx.x == 0) {
    ChunkInfo ci;
    ci.count = count;
    ci.thr = thr;
    ci.kmax = kmax;
    ci.kmin = kKeyNegInf;   // lower bound of every non-NaN key
    ci.kmax_idx = kmax_idx;
    ci.flags = flags;
    ci.best_s = best_s;
    ci.cmin = cmin;
    ci.best_idx = best_idx;
    P.info[(int64_t)r * P.chunks + c] = ci;
  }
}

// ------------------------------------------------------------------ row-kernel helpers
constexpr int kMaxSeg = 1024;   // chunks per row the row kernel indexes through LDS offsets

struct SegSrc {
  // The candidates of a row in id order: one LDS array, or the `chunks` global segments
  // (chunk c's list at glob + c * cap) addressed through the LDS prefix offsets segoff[].
  const uint2* lds;
  const uint2* glob;
  const uint32_t* segoff;   // chunks + 1 entries: exclusive prefix of the chunk counts
  uint32_t n;
  int chunks;
  int cap;
  bool in_lds;
  __device__ __forceinline__ uint2 item(uint32_t j) const {
    if (in_lds) return lds[j];
    int lo = 0, hi = chunks;   // largest c with segoff[c] <= j
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (segoff[mid] <= j) lo = mid; else hi = mid;
    }
    return glob[(int64_t)lo * cap + (j - segoff[lo])];
  }
};

template <class F>
__device__ __forceinline__ void seg_for_each(const SegSrc& src, F f) {
  batched_for<8>(src.n, [&](uint32_t j) { return src.item(j); }, f);
}

template <class Mem, class Out>
__device__ __forceinline__ void seg_emit_ordered(const SegSrc& src, const Mem& mem, const Out& out, Smem& sm) {
  uint32_t run = 0;
  emit_ordered<4>(src.n, [&](uint32_t i, uint32_t& rk, uint32_t& idx) {
    const uint2 v = src.item(i); rk = v.x; idx = v.y; }, mem, out, run, sm);
}

template <int MODE>
__device__ __forceinline__ void finish_kset(const Params& P, const RowPlan& rp, int r, uint32_t kmax, uint32_t klo,
                            uint64_t seed, Smem& sm, int& hb) {
  // K is in sm.kset (any order; every later step is order-independent).
  const uint32_t nk = min(sm.kcount, (uint32_t)kFastK);
  const float m = key2f(kmax);
  const float t = rp.t;
  auto kvis = [&](auto f) {
    for (uint32_t i = threadIdx.x; i < nk; i += kThreads) {
      const uint2 v = sm.kset[i];
      f(v.x, v.y);
    }
  };
  Sel sp = sel_all();
  uint32_t kept = nk;
  if (rp.p != 1.0f) {
    const int S = 63 - bitlen(nk);
    uint64_t zh = 0, zl = 0;
    kvis([&](uint32_t rk, uint32_t) {
      const Mass q = mass_of(weight_of(rk, m, t), S);
      zh += q.hi;
      zl += q.lo;
    });
    block_sum2_u64(zh, zl, sm.red64);
    const double target = (double)rp.p * mass_to_double(zh, zl, S);
    sp = select_mass(kvis, [&](uint32_t rk) { return weight_of(rk, m, t); }, target, S, nk, kmax,
                     klo, 0u, (uint32_t)(P.V - 1), sm, hb, kept);
  }
  if (MODE == kModeTopp) {
    if (threadIdx.x == 0) P.out_kept[r] = (int32_t)kept;
    if (P.out_mask) {
      uint8_t* mrow = P.out_mask + (int64_t)r * P.V;
      kvis([&](uint32_t rk, uint32_t idx) {
        if (sel_member(sp, rk, idx) && idx < (uint32_t)P.V) mrow[idx] = 1;
      });
    }
  } else {
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    float bs = -INFINITY;
    int32_t bi = 0x7FFFFFFF;
    kvis([&](uint32_t rk, uint32_t idx) {
      if (sel_member(sp, rk, idx)) {
        const float sc = gumbel_score(rk, idx, m, t, (uint32_t)r, k0, k1);
        if (sc > bs || (sc == bs && (int32_t)idx < bi)) { bs = sc; bi = (int32_t)idx; }
      }
    });
    const int32_t tok = block_argmax(bs, bi, sm.reds, sm.redi);
    if (threadIdx.x == 0) P.out_token[r] = tok;
  }
}

// ------------------------------------------------------------------ row kernel
template <int MODE>
__device__ __forceinline__ void row_stream(const Params& P, const RowPlan& rp, int r, uint32_t kmax,
                                           uint32_t kmin, uint64_t seed, Smem& sm, int& hb) {
  // The exact path over the raw row in global memory, one read of the row per pass.
  const float* row = P.x + (int64_t)r * P.stride;
  const uint32_t V = (uint32_t)P.V;
  const bool al4 = ((uintptr_t)row & 15u) == 0;
  auto rvis = [&](auto f) {
    if (al4) {   // 8 float4 loads in flight per thread per round
      const uint32_t nq = V >> 2;
      for (uint32_t base = 0; base < nq; base += kThreads * 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t q = base + u * kThreads + threadIdx.x;
          v[u] = make_uint4(0, 0, 0, 0);
          if (q < nq) v[u] = reinterpret_cast<const uint4*>(row)[q];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t q = base + u * kThreads + threadIdx.x;
          if (q < nq) {
            f(f2key(__uint_as_float(v[u].x)), 4 * q);
            f(f2key(__uint_as_float(v[u].y)), 4 * q + 1);
            f(f2key(__uint_as_float(v[u].z)), 4 * q + 2);
            f(f2key(__uint_as_float(v[u].w)), 4 * q + 3);
          }
        }
      }
      for (uint32_t i = 4 * nq + threadIdx.x; i < V; i += kThreads) f(f2key(row[i]), i);
    } else {
      batched_for<16>(V, [&](uint32_t j) { return make_uint2(f2key(row[j]), j); }, f);
    }
  };
  const uint32_t ke = (uint32_t)rp.k_eff;
  Sel sk = sel_all();
  if (ke < V) sk = select_topk(rvis, ke, V, kmax, kmin, 0u, V - 1, sm, hb);
  if (MODE == kModeTopk) {
    int32_t* orow = P.out_idx + (int64_t)r * P.k_max;
    const uint32_t kmx = (uint32_t)P.k_max;
    uint32_t run = 0;
    emit_ordered<4>(V, [&](uint32_t i, uint32_t& rk, uint32_t& idx) { rk = f2key(row[i]); idx = i; },
                 [&](uint32_t rk, uint32_t idx) { return sel_member(sk, rk, idx); },
                 [&](uint32_t pos, uint32_t idx) { if (pos < kmx) orow[pos] = (int32_t)idx; }, run, sm);
    for (int i = rp.k_eff + threadIdx.x; i < P.k_max; i += kThreads) orow[i] = -1;
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
    const int S = 63 - bitlen(ke);
    uint64_t zh = 0, zl = 0;
    kvis([&](uint32_t rk, uint32_t) {
      const Mass q = mass_of(weight_of(rk, m, t), S);
      zh += q.hi;
      zl += q.lo;
    });
    block_sum2_u64(zh, zl, sm.red64);
    const double target = (double)rp.p * mass_to_double(zh, zl, S);
    const uint32_t klo = (sk.lo >= 32) ? kmin : max(kmin, shl(sk.prefix, sk.lo));
    sp = select_mass(kvis, [&](uint32_t rk) { return weight_of(rk, m, t); }, target, S, ke, kmax,
                     klo, 0u, V - 1, sm, hb, kept);
  }
  if (MODE == kModeTopp) {
    if (threadIdx.x == 0) P.out_kept[r] = (int32_t)kept;
    if (P.out_mask) {
      uint8_t* mrow = P.out_mask + (int64_t)r * P.V;
      kvis([&](uint32_t rk, uint32_t idx) {
        if (sel_member(sp, rk, idx)) mrow[idx] = 1;
      });
    }
  } else {
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    float bs = -INFINITY;
    int32_t bi = 0x7FFFFFFF;
    kvis([&](uint32_t rk, uint32_t idx) {
      if (sel_member(sp, rk, idx)) {
        const float sc = gumbel_score(rk, idx, m, t, (uint32_t)r, k0, k1);
        if (sc > bs || (sc == bs && (int32_t)idx < bi)) { bs = sc; bi = (int32_t)idx; }
      }
    });
    const int32_t tok = block_argmax(bs, bi, sm.reds, sm.redi);
    if (threadIdx.x == 0) P.out_token[r] = tok;
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void ts_row_kernel(Params P) {
  __shared__ Smem sm;
  const int r = (int)blockIdx.x;
  const ChunkInfo* inf = P.info + (int64_t)r * P.chunks;
  // Aggregate the chunk summaries (one chunk per thread, then workgroup reductions). Their
  // loads are issued first; the row parameters and the seed load while they are in flight.
  uint32_t flags = 0, kmax = 0, kmin = 0xFFFFFFFFu, cmin = 0xFFFFFFFFu, total = 0, thr_max = 0;
  uint32_t my_count = 0;
  for (int c = threadIdx.x; c < P.chunks; c += kThreads) {
    const ChunkInfo ci = inf[c];
    flags |= ci.flags;
    kmax = max(kmax, ci.kmax);
    kmin = min(kmin, ci.kmin);
    cmin = min(cmin, ci.cmin);
    thr_max = max(thr_max, ci.thr);
    total += ci.count;
    my_count = ci.count;   // used only when chunks <= kThreads
  }
  const RowPlan rp = plan_row(P, MODE, r);
  const uint64_t seed = (MODE == kModeSample) ? P.seed[r] : 0ull;
  int hb = 0;   // histogram buffer of the next radix pass; both start zeroed
  clear_hist(sm, 0, (int)threadIdx.x, kThreads);
  clear_hist(sm, 1, (int)threadIdx.x, kThreads);
  block_reduce3(kmax, kmin, flags, sm.red3);
  {
    uint32_t none = 0;
    block_reduce3(thr_max, cmin, none, sm.red3);
  }
  total = (uint32_t)block_sum_u64(total, sm.red64);
  const bool nan = (flags & kFlagNan) != 0;
  int st = TS_ROW_OK;
  if (MODE == kModeTopk) {
    if (nan) st = TS_ROW_NONFINITE;
  } else if (nan || kmax >= kKeyPosInf || kmax <= kKeyNegInf) {
    st = TS_ROW_NONFINITE;
  }
  if (st == TS_ROW_OK) st = rp.bad;
  if (threadIdx.x == 0 && P.status) P.status[r] = st;

  if (st != TS_ROW_OK) {
    if (MODE == kModeTopp && rp.path == kPathFull && P.out_mask) {
      fill_bytes_nt<kThreads>(P.out_mask + (int64_t)r * P.V, P.V, 0);   // chunks had written ones
    }
    if (MODE == kModeTopk) {
      for (int i = threadIdx.x; i < P.k_max; i += kThreads) P.out_idx[(int64_t)r * P.k_max + i] = -1;
    } else if (MODE == kModeTopp) {
      if (threadIdx.x == 0) P.out_kept[r] = 0;
    } else {
      if (threadIdx.x == 0) P.out_token[r] = -1;
    }
    return;
  }

  const int path = rp.path;
  if (path == kPathGreedy) {
    // chunks are in id order: the lowest id holding the row maximum
    uint32_t idx = 0xFFFFFFFFu;
    for (int c = threadIdx.x; c < P.chunks; c += kThreads) {
      const ChunkInfo ci = inf[c];
      if (ci.kmax == kmax) idx = min(idx, ci.kmax_idx);
    }
    idx = block_min_u32(idx, sm.red);
    if (MODE == kModeTopp) {
      if (threadIdx.x == 0) {
        P.out_kept[r] = 1;
        if (P.out_mask && idx < (uint32_t)P.V) P.out_mask[(int64_t)r * P.V + idx] = 1;
      }
    } else if (MODE == kModeSample) {
      if (threadIdx.x == 0) P.out_token[r] = (int32_t)idx;
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
      for (int c = threadIdx.x; c < P.chunks; c += kThreads) {
        const ChunkInfo ci = inf[c];
        const float adj = ci.best_s + (key2f(ci.kmax) - m) / rp.t;
        if (adj > bs || (adj == bs && ci.best_idx < bi)) { bs = adj; bi = ci.best_idx; }
      }
      bi = block_argmax(bs, bi, sm.reds, sm.redi);
      if (threadIdx.x == 0) P.out_token[r] = bi;
    }
    return;
  }

  if (path == kPathCand) {
    const uint32_t ke = (uint32_t)rp.k_eff;
    bool ok = ((flags & kFlagOverflow) == 0) && total >= ke && !P.force_exact && P.chunks <= kMaxSeg;
    if (ok) {
      // exclusive prefix of the chunk counts: the candidates' flat, id-ordered index space
      uint32_t tot;
      const uint32_t off = block_excl_scan(threadIdx.x < (uint32_t)P.chunks ? my_count : 0u, sm.red, tot);
      if (threadIdx.x < (uint32_t)P.chunks) sm.segoff[threadIdx.x] = off;
      if (threadIdx.x == 0) sm.segoff[P.chunks] = tot;
      bar();
      SegSrc src;
      src.glob = P.cand + (int64_t)r * P.chunks * P.cap_c;
      src.segoff = sm.segoff;
      src.chunks = P.chunks;
      src.cap = P.cap_c;
      src.lds = sm.cand;
      src.n = total;
      src.in_lds = false;
      if (total <= (uint32_t)kLdsCand && !P.leader_global) {
        // gather the candidates into LDS: each chunk's list is copied by its own group of
        // threads, up to 8 loads in flight per thread
        const int G = kThreads / P.chunks;   // >= 1 because chunks <= kMaxSeg
        const int cg = (int)threadIdx.x / G;
        const int g = (int)threadIdx.x - cg * G;
        if (cg < P.chunks) {
          const uint32_t dst = sm.segoff[cg];
          const uint32_t nc = sm.segoff[cg + 1] - dst;
          const uint2* src_c = src.glob + (int64_t)cg * P.cap_c;
          for (uint32_t j0 = (uint32_t)g; j0 < nc; j0 += (uint32_t)G * 8u) {
            uint2 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const uint32_t j = j0 + (uint32_t)(u * G);
              v[u] = make_uint2(0, 0);
              if (j < nc) v[u] = src_c[j];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const uint32_t j = j0 + (uint32_t)(u * G);
              if (j < nc) sm.cand[dst + j] = v[u];
            }
          }
        }
        bar();
        src.in_lds = true;
      }
      auto vis = [&](auto f) { seg_for_each(src, f); };
      Sel sk = sel_all();
      uint32_t min_sel = cmin;
      if (total > ke) {
        sk = select_topk(vis, ke, total, kmax, cmin, 0u, (uint32_t)(P.V - 1), sm, hb);
        min_sel = shl(sk.prefix, sk.lo);
      }
      // Certification: every element of the row with a key >= the smallest selected key
      // was published by its chunk, so the candidates' top-k is the row's top-k.
      if (min_sel >= thr_max) {
        if (MODE == kModeTopk) {
          int32_t* orow = P.out_idx + (int64_t)r * P.k_max;
          const uint32_t kmx = (uint32_t)P.k_max;
          seg_emit_ordered(src, [&](uint32_t rk, uint32_t idx) { return sel_member(sk, rk, idx); },
                           [&](uint32_t pos, uint32_t idx) { if (pos < kmx) orow[pos] = (int32_t)idx; }, sm);
          for (int i = rp.k_eff + threadIdx.x; i < P.k_max; i += kThreads) orow[i] = -1;
          return;
        }
        if (threadIdx.x == 0) sm.kcount = 0;
        bar();
        vis([&](uint32_t rk, uint32_t idx) {
          // one LDS atomic per wave: the lowest active lane reserves room for the wave
          const bool mem = sel_member(sk, rk, idx);
          const uint64_t bal = __ballot(mem);
          if (bal) {
            const int leader = __ffsll((unsigned long long)bal) - 1;
            uint32_t base = 0;
            if (lane() == leader) base = atomicAdd(&sm.kcount, (uint32_t)__popcll(bal));
            base = (uint32_t)__shfl((int)base, leader, 64);
            const uint32_t pos = base + mbcnt(bal);
            if (mem && pos < (uint32_t)kFastK) sm.kset[pos] = make_uint2(rk, idx);
          }
        });
        bar();
        finish_kset<MODE>(P, rp, r, kmax, max(cmin, min_sel), seed, sm, hb);
        return;
      }
    }
  }
  row_stream<MODE>(P, rp, r, kmax, kmin, seed, sm, hb);
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

// ================================================================== host side
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

std::atomic<int64_t> g_knob_chunk{0};
std::atomic<int64_t> g_knob_exact{0};
std::atomic<int64_t> g_knob_leader_global{0};

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

struct Plan {
  int64_t chunks = 0, chunk_len = 0, cap_c = 0;
  size_t off_info = 0, off_cand = 0, total = 0;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool make_plan(int64_t rows, int64_t V, Plan& pl) {
  if (rows < 0 || V < 1 || V > TS_MAX_VOCAB) return false;
  int64_t ce = g_knob_chunk.load();
  if (ce <= 0) ce = kChunkMax;
  const int64_t chunks0 = (V + ce - 1) / ce;
  int64_t len = (V + chunks0 - 1) / chunks0;
  len = (len + 3) & ~int64_t(3);
  pl.chunk_len = len;
  pl.chunks = (V + len - 1) / len;
  pl.cap_c = len < kCapMax ? len : kCapMax;
  const int64_t rr = rows > 0 ? rows : 1;
  if (rr * pl.chunks > (int64_t)0x7FFFFFFF) return false;
  size_t b = 0;
  pl.off_info = b;
  b += align256((size_t)rr * pl.chunks * sizeof(ChunkInfo));
  pl.off_cand = b;
  b += align256((size_t)rr * pl.chunks * pl.cap_c * sizeof(uint2));
  pl.total = b;
  return true;
}

template <int MODE>
int launch(const float* x, int64_t rows, int64_t V, int64_t stride, const int32_t* k, int32_t k_max,
           const float* p, const float* t, const uint64_t* seed, int32_t* out_idx, int32_t* out_kept,
           uint8_t* out_mask, int32_t* out_token, int32_t* status, void* ws, size_t ws_bytes,
           void* stream) {
  if (!x) return fail(TS_ERR_INVALID_ARG, "logits pointer is NULL");
  if (rows < 0) return fail(TS_ERR_INVALID_ARG, "rows = %lld < 0", (long long)rows);
  if (V < 1 || V > TS_MAX_VOCAB) return fail(TS_ERR_INVALID_ARG, "vocab = %lld outside [1, 2^30]", (long long)V);
  if (stride < V) return fail(TS_ERR_INVALID_ARG, "row_stride %lld < vocab %lld", (long long)stride, (long long)V);
  if (rows > 0x7FFFFFFF) return fail(TS_ERR_INVALID_ARG, "rows too large");
  Plan pl;
  if (!make_plan(rows, V, pl)) return fail(TS_ERR_INVALID_ARG, "rows x chunks too large");
  if (rows == 0) return TS_OK;
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
  P.k_max = k_max;
  P.chunks = (int32_t)pl.chunks;
  P.chunk_len = (int32_t)pl.chunk_len;
  P.cap_c = (int32_t)pl.cap_c;
  P.xcd_map = (pl.chunks > 1 && rows % 8 == 0) ? 1 : 0;
  P.force_exact = (int32_t)g_knob_exact.load();
  P.leader_global = (int32_t)g_knob_leader_global.load();
  P.out_idx = out_idx;
  P.out_kept = out_kept;
  P.out_mask = out_mask;
  P.out_token = out_token;
  P.status = status;
  char* w = static_cast<char*>(ws);
  P.info = reinterpret_cast<ChunkInfo*>(w + pl.off_info);
  P.cand = reinterpret_cast<uint2*>(w + pl.off_cand);
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(ts_stream_kernel<MODE>, dim3((unsigned)(rows * pl.chunks)), dim3(kT1), 0, s, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "stream kernel launch failed: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(ts_row_kernel<MODE>, dim3((unsigned)rows), dim3(kThreads), 0, s, P);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "row kernel launch failed: %s", hipGetErrorString(e));
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

int ts_topk_select(const float* keys, int64_t rows, int64_t row_len, int64_t row_stride,
                   const int32_t* k, int32_t k_max, int32_t* out_idx, int32_t* row_status,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (rows > 0 && (!k || !out_idx)) return fail(TS_ERR_INVALID_ARG, "k and out_idx are required");
  if (k_max < 1) return fail(TS_ERR_INVALID_ARG, "k_max = %d < 1", (int)k_max);
  return launch<kModeTopk>(keys, rows, row_len, row_stride, k, k_max, nullptr, nullptr, nullptr,
                           out_idx, nullptr, nullptr, nullptr, row_status, workspace,
                           workspace_bytes, stream);
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

int64_t ts_debug_set(int knob, int64_t value) {
  switch (knob) {
    case TS_KNOB_CHUNK_ELEMS: {
      if (value != 0 && (value < 64 || value > kChunkMax || value % 64 != 0)) return -1;
      return g_knob_chunk.exchange(value);
    }
    case TS_KNOB_FORCE_EXACT: return g_knob_exact.exchange(value ? 1 : 0);
    case TS_KNOB_LEADER_GLOBAL: return g_knob_leader_global.exchange(value ? 1 : 0);
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
    default: return "unknown status";
  }
}

const char* ts_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
