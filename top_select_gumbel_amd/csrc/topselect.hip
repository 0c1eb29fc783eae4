// topselect.hip -- gfx950 kernels and the C ABI of the batched per-row sampler.
//
// One kernel launch per call. The grid is rows x chunks workgroups of 1024 threads; each
// workgroup streams one contiguous chunk (<= 40960 logits) of one row from HBM exactly
// once, keeping the chunk's ordered keys in registers. The last workgroup of a row to
// finish (elected with an atomic counter, so no workgroup ever waits on another) becomes
// the row's leader and finishes the row from the chunks' published results.
//
// Row paths (chosen per row on the device from that row's k, p, T):
//   CAND    k_eff <= 2048: every chunk publishes its exact local top-k (index order); the
//           leader selects the row's top-k from those candidates, then (top-p / sampling)
//           runs the mass-carrying radix cut and the Gumbel argmax on that small set.
//           Correct because the row's top-k restricted to a chunk is contained in that
//           chunk's own top-k (vLLM PR #55122, "Changes": per-CTA counts, CTA-order merge).
//   GREEDY  T == 0: the first token of the row ordering (max key, lowest id).
//   FULL    top-k and top-p both off (sampling): each chunk computes its Gumbel argmax
//           relative to its own maximum; the leader folds the chunk winners.
//   STREAM  everything else (k > 2048, or top-p with top-k off): the leader re-reads the
//           row from global memory once per radix pass.
//   NONE    invalid row: outputs poisoned.
//
// Page citations (title, then section):
//   [DETK]   vLLM PR #55122 "[Kernel] Make persistent_topk deterministic": "Changes".
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

constexpr int kSlots = 10;                          // float4 loads per thread per chunk
constexpr int kChunkMax = kThreads * 4 * kSlots;    // 40960 logits per workgroup
constexpr int kFastK = 2048;                        // largest k taking the candidate path
constexpr int kCapChunk = 4096;                     // candidate slots per chunk in workspace
constexpr int kBins = 256;                          // radix digit of 8 bits
constexpr int kCC = 16;                             // replicated count histograms
constexpr int kMC = 4;                              // replicated mass histograms
constexpr int kLdsCand = 8192;                      // candidates the leader keeps in LDS

struct ChunkInfo {
  uint32_t count;     // candidates published (CAND)
  uint32_t cmin;      // smallest key among them (0xFFFFFFFF if none)
  uint32_t kmax;      // largest key of the chunk's elements (0 if none)
  uint32_t kmin;      // smallest key of the chunk's elements (0xFFFFFFFF if none)
  uint32_t kmax_idx;  // lowest id holding kmax (GREEDY)
  uint32_t nan;       // 1 if the chunk holds a NaN
  float best_s;       // FULL sampling: best score relative to the chunk maximum
  int32_t best_idx;
};
static_assert(sizeof(ChunkInfo) == 32, "ChunkInfo layout");

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
  uint32_t* counters;
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

struct Smem {
  uint32_t hist[kBins * kCC];
  uint64_t mhist[kBins * kMC * 2];
  uint2 cand[kLdsCand];
  uint2 kset[kFastK];
  uint32_t red[kWaves];
  uint32_t red3[3 * kWaves];
  uint64_t red64[kWaves];
  float reds[kWaves];
  int32_t redi[kWaves];
  uint32_t wave_tot[kWaves];
  uint32_t res[4];
  uint64_t res64[4];
  uint32_t kcount;
  uint32_t is_last;
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
__device__ __forceinline__ void search_count(Smem& sm, uint32_t thr) {
  const int l = lane();
  uint32_t c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t s = 0;
#pragma unroll
    for (int cp = 0; cp < kCC; ++cp) s += sm.hist[(4 * l + j) * kCC + cp];
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
__device__ __forceinline__ void search_mass(Smem& sm, double target, uint64_t ma_hi, uint64_t ma_lo, int S) {
  const int l = lane();
  uint32_t c[4];
  uint64_t mh[4], ml[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t s = 0;
#pragma unroll
    for (int cp = 0; cp < kCC; ++cp) s += sm.hist[(4 * l + j) * kCC + cp];
    c[j] = s;
    uint64_t h = 0, o = 0;
#pragma unroll
    for (int cp = 0; cp < kMC; ++cp) {
      h += sm.mhist[((4 * l + j) * kMC + cp) * 2];
      o += sm.mhist[((4 * l + j) * kMC + cp) * 2 + 1];
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

__device__ __forceinline__ void clear_hist(Smem& sm, bool with_mass) {
  uint4* h = reinterpret_cast<uint4*>(sm.hist);
  for (int i = threadIdx.x; i < kBins * kCC / 4; i += kThreads) h[i] = make_uint4(0, 0, 0, 0);
  if (with_mass) {
    uint4* m = reinterpret_cast<uint4*>(sm.mhist);
    for (int i = threadIdx.x; i < kBins * kMC; i += kThreads) m[i] = make_uint4(0, 0, 0, 0);
  }
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
                             uint32_t lo_rk, Smem& sm, uint32_t& prefix, int& lo,
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
    clear_hist(sm, false);
    bar();
    const uint32_t copy = (uint32_t)lane() & (kCC - 1);
    vis([&](uint32_t rk, uint32_t idx) {
      if (shr(rk, lo_now) == pre) atomicAdd(&sm.hist[((rk >> sh) & dm) * kCC + copy], 1u);
    });
    bar();
    if (wave() == 0) search_count(sm, need);
    bar();
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
                           uint32_t lo_key, uint32_t idx_lo, uint32_t idx_hi, Smem& sm) {
  Sel s;
  uint32_t eq_take, tie_cnt;
  count_select(vis, need, n_in_play, hi_key, lo_key, sm, s.prefix, s.lo, eq_take, tie_cnt);
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
// Smallest prefix of the row ordering whose exact fixed-point mass reaches `target`
// ([TOPP] "Independent binary64 numerical reference", steps 4-5, with the predicate kept in
// probability space, [TOPP] "Source basis"). vis(f) calls f(rk, idx) for items of K; wfn(rk)
// returns the item's weight. Result: Sel of the kept set P (a canonical prefix) and |P|.
template <class Vis, class WFn>
__device__ __forceinline__ Sel select_mass(const Vis& vis, const WFn& wfn, double target, int S, uint32_t n_in_play,
                           uint32_t hi_key, uint32_t lo_key, uint32_t idx_lo, uint32_t idx_hi,
                           Smem& sm, uint32_t& kept) {
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
    clear_hist(sm, true);
    bar();
    const uint32_t cc = (uint32_t)lane() & (kCC - 1);
    const uint32_t mc = (uint32_t)lane() & (kMC - 1);
    vis([&](uint32_t rk, uint32_t idx) {
      if (shr(rk, lo_now) == pre) {
        const uint32_t b = (rk >> sh) & dm;
        const Mass m = mass_of(wfn(rk), S);
        atomicAdd(&sm.hist[b * kCC + cc], 1u);
        atomicAdd((unsigned long long*)&sm.mhist[(b * kMC + mc) * 2], (unsigned long long)m.hi);
        atomicAdd((unsigned long long*)&sm.mhist[(b * kMC + mc) * 2 + 1], (unsigned long long)m.lo);
      }
    });
    bar();
    if (wave() == 0) search_mass(sm, target, ma_hi, ma_lo, S);
    bar();
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
    count_select(tvis, take, tie_cnt, ~idx_lo, ~idx_hi, sm, p2, lo2, e2, t2);
    s.cutoff = ~shl(p2, lo2);
  }
  kept = n_above + take;
  return s;
}

// ------------------------------------------------------------------ misc helpers
__device__ __forceinline__ void fill_bytes(uint8_t* dst, int64_t n, uint8_t v) {
  const uintptr_t a = (uintptr_t)dst;
  int64_t head = (int64_t)((4u - (a & 3u)) & 3u);
  if (head > n) head = n;
  for (int64_t i = threadIdx.x; i < head; i += kThreads) dst[i] = v;
  uint32_t* d32 = reinterpret_cast<uint32_t*>(dst + head);
  const int64_t n32 = (n - head) >> 2;
  const uint32_t w = (uint32_t)v * 0x01010101u;
  for (int64_t i = threadIdx.x; i < n32; i += kThreads) d32[i] = w;
  for (int64_t i = head + n32 * 4 + threadIdx.x; i < n; i += kThreads) dst[i] = v;
}

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

// Ordered emission over a tile-structured source: one item per thread per tile, in id
// order across the workgroup; out(pos, idx) writes selected item `idx` at `pos`.
template <class Get, class Mem, class Out>
__device__ __forceinline__ void emit_ordered(uint32_t n, const Get& get, const Mem& mem, const Out& out,
                             uint32_t& run, Smem& sm) {
  for (uint32_t base = 0; base < n; base += kThreads) {
    const uint32_t i = base + threadIdx.x;
    uint32_t rk = 0, idx = 0;
    bool s = false;
    if (i < n) {
      get(i, rk, idx);
      s = mem(rk, idx);
    }
    uint32_t tot;
    const uint32_t pos = block_excl_scan(s ? 1u : 0u, sm.red, tot);
    if (s) out(run + pos, idx);
    run += tot;
  }
}

// ------------------------------------------------------------------ chunk phase
template <int MODE>
__device__ __forceinline__ void chunk_phase(const Params& P, const RowPlan& rp, int r, int c, Smem& sm) {
  const int c0 = c * P.chunk_len;
  const int n = min(P.chunk_len, P.V - c0);
  const float* base = P.x + (int64_t)r * P.stride + c0;
  const bool aligned = ((uintptr_t)base & 15u) == 0;
  const int nq = (n + 3) >> 2;
  const int qw = (nq + kWaves - 1) / kWaves;
  const int w = wave(), l = lane();
  const int q_lo = w * qw;
  const int q_hi = min(q_lo + qw, nq);

  // Stream the chunk: all loads are issued before any is consumed. Addresses are clamped
  // into the chunk so every load is in bounds; elements past the end are masked afterwards.
  const int nfull = n >> 2;                 // quads with four valid elements
  uint4 raw[kSlots];
  if (aligned && nfull > 0) {
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const int q = min(q_lo + s * 64 + l, nfull - 1);
      raw[s] = *reinterpret_cast<const uint4*>(base + 4 * q);
    }
    if (nfull * 4 < n) {                    // one partial quad at the end of the chunk
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
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
    for (int s = 0; s < kSlots; ++s) {
      const int e0 = 4 * (q_lo + s * 64 + l);
      raw[s].x = s32[min(e0, n - 1)];
      raw[s].y = s32[min(e0 + 1, n - 1)];
      raw[s].z = s32[min(e0 + 2, n - 1)];
      raw[s].w = s32[min(e0 + 3, n - 1)];
    }
  }
  // Ordered keys; 0 marks an element past the end of the chunk. The one NaN pattern whose
  // key would be 0 (all bits set) is moved to key 1, which is still a NaN key.
  uint32_t kk[kSlots][4];
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int q = q_lo + s * 64 + l;
    const int nv = (q < q_hi) ? min(max(n - 4 * q, 0), 4) : 0;   // valid elements in the quad
    const uint32_t bits[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = max(f2key(__uint_as_float(bits[e])), 1u);
      kk[s][e] = (e < nv) ? key : 0u;
      // keep the key opaque so the conversion temporaries are not kept alive
      __asm__ volatile("" : "+v"(kk[s][e]));
    }
  }
  // max key, min key and the NaN flag of the chunk (NaN keys lie above +inf's key or below
  // -inf's key).
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu, nan = 0;
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = kk[s][e];
      kmax = max(kmax, key);
      kmin = min(kmin, key ? key : 0xFFFFFFFFu);
      nan |= (key > kKeyPosInf || (key != 0u && key < kKeyNegInf)) ? 1u : 0u;
    }
  }
  block_reduce3(kmax, kmin, nan, sm.red3);

  const int path = rp.path;
  auto vis = [&](auto f) {
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = kk[s][e];
        if (key) f(key, (uint32_t)(c0 + 4 * (q_lo + s * 64 + l) + e));
      }
    }
  };

  uint32_t count = 0, cmin = 0xFFFFFFFFu, kmax_idx = 0xFFFFFFFFu;
  float best_s = -INFINITY;
  int32_t best_idx = 0x7FFFFFFF;

  if (path == kPathCand) {
    // Exact local top-k of the chunk (or the whole chunk when it is not longer than k).
    Sel s = sel_all();
    if (n > rp.k_eff) {
      s = select_topk(vis, (uint32_t)rp.k_eff, (uint32_t)n, kmax, kmin == 0xFFFFFFFFu ? kmax : kmin,
                      (uint32_t)c0, (uint32_t)(c0 + n - 1), sm);
    }
    // Ordered emission straight from registers: ballots give each element its position
    // (wave-contiguous segments, each in (slot, lane, element) = id order).
    uint64_t selbits = 0;
    uint32_t wtot = 0;
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = kk[sl][e];
        const uint32_t idx = (uint32_t)(c0 + 4 * (q_lo + sl * 64 + l) + e);
        const bool m = key != 0u && sel_member(s, key, idx);
        selbits |= m ? (1ull << (sl * 4 + e)) : 0ull;
        wtot += (uint32_t)__popcll(__ballot(m));
      }
    }
    if (l == 0) sm.wave_tot[w] = wtot;
    bar();
    uint32_t run = 0, tot = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const uint32_t t = sm.wave_tot[ww];
      run += (ww < w) ? t : 0u;
      tot += t;
    }
    bar();
    uint2* out = P.cand + ((int64_t)r * P.chunks + c) * P.cap_c;
    const uint32_t cap = (uint32_t)P.cap_c;
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      uint64_t m[4];
      uint32_t slot_cnt = 0, lane_off = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[e] = __ballot((selbits >> (sl * 4 + e)) & 1ull);
        slot_cnt += (uint32_t)__popcll(m[e]);
        lane_off += mbcnt(m[e]);
      }
      uint32_t pos = run + lane_off;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((selbits >> (sl * 4 + e)) & 1ull) {
          const uint32_t idx = (uint32_t)(c0 + 4 * (q_lo + sl * 64 + l) + e);
          if (pos < cap) out[pos] = make_uint2(kk[sl][e], idx);
          cmin = min(cmin, kk[sl][e]);
          ++pos;
        }
      }
      run += slot_cnt;
    }
    count = min(tot, cap);
    cmin = block_min_u32(cmin, sm.red);
  } else if (path == kPathGreedy) {
    uint32_t mi = 0xFFFFFFFFu;
    vis([&](uint32_t key, uint32_t idx) {
      if (key == kmax) mi = min(mi, idx);
    });
    kmax_idx = block_min_u32(mi, sm.red);
  } else if (path == kPathFull && MODE == kModeSample) {
    const float m_c = key2f(kmax);
    const uint64_t sd = P.seed[r];
    const uint32_t k0 = (uint32_t)sd, k1 = (uint32_t)(sd >> 32);
    float bs = -INFINITY;
    int32_t bi = 0x7FFFFFFF;
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int q = q_lo + sl * 64 + l;
      if (q < q_hi) {
        const uint32_t tok0 = (uint32_t)(c0 + 4 * q);
        const uint4 wd = philox4x32_10(tok0 >> 2, (uint32_t)r, k0, k1);
        const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (kk[sl][e]) {
            const float g = gumbel_from_uniform(uniform_from_word(words[e]));
            const float sc = (key2f(kk[sl][e]) - m_c) / rp.t + g;
            const int32_t id = (int32_t)(tok0 + e);
            if (sc > bs || (sc == bs && id < bi)) { bs = sc; bi = id; }
          }
        }
      }
    }
    best_idx = block_argmax(bs, bi, sm.reds, sm.redi, &best_s);
  }

  if (MODE == kModeTopp && P.out_mask) {
    uint8_t* mrow = P.out_mask + (int64_t)r * P.V + c0;
    fill_bytes(mrow, n, (path == kPathFull) ? (uint8_t)1 : (uint8_t)0);
  }

  if (threadIdx.x == 0) {
    ChunkInfo ci;
    ci.count = count;
    ci.cmin = cmin;
    ci.kmax = kmax;
    ci.kmin = kmin;
    ci.kmax_idx = kmax_idx;
    ci.nan = nan;
    ci.best_s = best_s;
    ci.best_idx = best_idx;
    P.info[(int64_t)r * P.chunks + c] = ci;
  }
}

// ------------------------------------------------------------------ leader helpers
struct SegSrc {
  // Candidates of a row: one LDS array, or `chunks` global segments of cap_c slots.
  const uint2* lds;
  uint32_t lds_n;
  const uint2* glob;
  const ChunkInfo* info;
  int chunks;
  int cap;
  bool in_lds;
};

template <class F>
__device__ __forceinline__ void seg_for_each(const SegSrc& src, F f) {
  if (src.in_lds) {
    for (uint32_t i = threadIdx.x; i < src.lds_n; i += kThreads) {
      const uint2 v = src.lds[i];
      f(v.x, v.y);
    }
  } else {
    for (int c = 0; c < src.chunks; ++c) {
      const uint32_t nc = src.info[c].count;
      const uint2* g = src.glob + (int64_t)c * src.cap;
      for (uint32_t i = threadIdx.x; i < nc; i += kThreads) {
        const uint2 v = g[i];
        f(v.x, v.y);
      }
    }
  }
}

template <class Mem, class Out>
__device__ __forceinline__ void seg_emit_ordered(const SegSrc& src, const Mem& mem, const Out& out, Smem& sm) {
  uint32_t run = 0;
  if (src.in_lds) {
    emit_ordered(src.lds_n, [&](uint32_t i, uint32_t& rk, uint32_t& idx) {
      rk = src.lds[i].x; idx = src.lds[i].y; }, mem, out, run, sm);
  } else {
    for (int c = 0; c < src.chunks; ++c) {
      const uint2* g = src.glob + (int64_t)c * src.cap;
      emit_ordered(src.info[c].count, [&](uint32_t i, uint32_t& rk, uint32_t& idx) {
        rk = g[i].x; idx = g[i].y; }, mem, out, run, sm);
    }
  }
}

template <int MODE>
__device__ __forceinline__ void finish_kset(const Params& P, const RowPlan& rp, int r, uint32_t kmax, uint32_t klo,
                            Smem& sm) {
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
    zh = block_sum_u64(zh, sm.red64);
    zl = block_sum_u64(zl, sm.red64);
    const double target = (double)rp.p * mass_to_double(zh, zl, S);
    sp = select_mass(kvis, [&](uint32_t rk) { return weight_of(rk, m, t); }, target, S, nk, kmax,
                     klo, 0u, (uint32_t)(P.V - 1), sm, kept);
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
    const uint64_t sd = P.seed[r];
    const uint32_t k0 = (uint32_t)sd, k1 = (uint32_t)(sd >> 32);
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
__device__ __forceinline__ void leader_phase(const Params& P, const RowPlan& rp, int r, Smem& sm) {
  const ChunkInfo* inf = P.info + (int64_t)r * P.chunks;
  uint32_t nan = 0, kmax = 0, kmin = 0xFFFFFFFFu, cmin = 0xFFFFFFFFu, total = 0;
  for (int c = 0; c < P.chunks; ++c) {
    const ChunkInfo ci = inf[c];
    nan |= ci.nan;
    kmax = max(kmax, ci.kmax);
    kmin = min(kmin, ci.kmin);
    cmin = min(cmin, ci.cmin);
    total += ci.count;
  }
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
      fill_bytes(P.out_mask + (int64_t)r * P.V, P.V, 0);   // chunks had written ones
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
    uint32_t idx = 0xFFFFFFFFu;
    for (int c = 0; c < P.chunks; ++c) {
      if (inf[c].kmax == kmax) { idx = inf[c].kmax_idx; break; }
    }
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
      for (int c = 0; c < P.chunks; ++c) {
        const ChunkInfo ci = inf[c];
        const float adj = ci.best_s + (key2f(ci.kmax) - m) / rp.t;
        if (adj > bs || (adj == bs && ci.best_idx < bi)) { bs = adj; bi = ci.best_idx; }
      }
      if (threadIdx.x == 0) P.out_token[r] = bi;
    }
    return;
  }

  const float* row = P.x + (int64_t)r * P.stride;
  if (path == kPathCand) {
    SegSrc src;
    src.glob = P.cand + (int64_t)r * P.chunks * P.cap_c;
    src.info = inf;
    src.chunks = P.chunks;
    src.cap = P.cap_c;
    src.lds = sm.cand;
    src.in_lds = (total <= (uint32_t)kLdsCand) && !P.leader_global;
    src.lds_n = total;
    if (src.in_lds) {
      uint32_t off = 0;
      for (int c = 0; c < P.chunks; ++c) {
        const uint32_t nc = inf[c].count;
        const uint2* g = src.glob + (int64_t)c * P.cap_c;
        for (uint32_t i = threadIdx.x; i < nc; i += kThreads) sm.cand[off + i] = g[i];
        off += nc;
      }
      bar();
    }
    auto vis = [&](auto f) { seg_for_each(src, f); };
    const uint32_t ke = (uint32_t)rp.k_eff;
    Sel sk = sel_all();
    if (total > ke) {
      sk = select_topk(vis, ke, total, kmax, cmin, 0u, (uint32_t)(P.V - 1), sm);
    }
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
      if (sel_member(sk, rk, idx)) {
        const uint32_t pos = atomicAdd(&sm.kcount, 1u);
        if (pos < (uint32_t)kFastK) sm.kset[pos] = make_uint2(rk, idx);
      }
    });
    bar();
    const uint32_t klo = (sk.lo >= 32) ? cmin : max(cmin, shl(sk.prefix, sk.lo));
    finish_kset<MODE>(P, rp, r, kmax, klo, sm);
    return;
  }

  // STREAM: the leader walks the row in global memory once per pass.
  const uint32_t V = (uint32_t)P.V;
  auto rvis = [&](auto f) {
    for (uint32_t i = threadIdx.x; i < V; i += kThreads) f(f2key(row[i]), i);
  };
  const uint32_t ke = (uint32_t)rp.k_eff;
  Sel sk = sel_all();
  if (ke < V) sk = select_topk(rvis, ke, V, kmax, kmin, 0u, V - 1, sm);
  if (MODE == kModeTopk) {
    int32_t* orow = P.out_idx + (int64_t)r * P.k_max;
    const uint32_t kmx = (uint32_t)P.k_max;
    uint32_t run = 0;
    emit_ordered(V, [&](uint32_t i, uint32_t& rk, uint32_t& idx) { rk = f2key(row[i]); idx = i; },
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
    zh = block_sum_u64(zh, sm.red64);
    zl = block_sum_u64(zl, sm.red64);
    const double target = (double)rp.p * mass_to_double(zh, zl, S);
    const uint32_t klo = (sk.lo >= 32) ? kmin : max(kmin, shl(sk.prefix, sk.lo));
    sp = select_mass(kvis, [&](uint32_t rk) { return weight_of(rk, m, t); }, target, S, ke, kmax,
                     klo, 0u, V - 1, sm, kept);
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
    const uint64_t sd = P.seed[r];
    const uint32_t k0 = (uint32_t)sd, k1 = (uint32_t)(sd >> 32);
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

// ------------------------------------------------------------------ the kernel
template <int MODE>
__global__ __launch_bounds__(kThreads) void ts_rows_kernel(Params P) {
  __shared__ Smem sm;
  const int b = (int)blockIdx.x;
  int L = b;
  if (P.xcd_map) {
    const int per = (P.rows * P.chunks) >> 3;
    L = (b & 7) * per + (b >> 3);
  }
  const int r = L / P.chunks;
  const int c = L - r * P.chunks;
  const RowPlan rp = plan_row(P, MODE, r);
  chunk_phase<MODE>(P, rp, r, c, sm);

  // Publish and elect the row's leader: the last chunk to arrive.
  bar_all();
  if (threadIdx.x == 0) {
    if (P.chunks == 1) {
      sm.is_last = 1;
    } else {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t old = atomicInc(&P.counters[r], (uint32_t)(P.chunks - 1));
      sm.is_last = (old == (uint32_t)(P.chunks - 1)) ? 1u : 0u;
    }
  }
  bar_all();
  if (!sm.is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  leader_phase<MODE>(P, rp, r, sm);
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
  size_t off_counters = 0, off_info = 0, off_cand = 0, total = 0;
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
  pl.cap_c = len < kCapChunk ? len : kCapChunk;
  if (rows * pl.chunks > (int64_t)0x7FFFFFFF) return false;
  size_t b = 0;
  pl.off_counters = b;
  b += align256((size_t)(rows > 0 ? rows : 1) * sizeof(uint32_t));
  pl.off_info = b;
  b += align256((size_t)(rows > 0 ? rows : 1) * pl.chunks * sizeof(ChunkInfo));
  pl.off_cand = b;
  b += align256((size_t)(rows > 0 ? rows : 1) * pl.chunks * pl.cap_c * sizeof(uint2));
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
  P.counters = reinterpret_cast<uint32_t*>(w + pl.off_counters);
  P.info = reinterpret_cast<ChunkInfo*>(w + pl.off_info);
  P.cand = reinterpret_cast<uint2*>(w + pl.off_cand);
  const unsigned grid = (unsigned)(rows * pl.chunks);
  hipLaunchKernelGGL(ts_rows_kernel<MODE>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
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
      if (value != 0 && (value < 4096 || value > kChunkMax || value % 4096 != 0)) return -1;
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
