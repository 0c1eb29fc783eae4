// rejection.hip -- dual-pivot rejection sampling over fp32 logits (gfx950), a sorting-free
// alternative to the Gumbel-max sampler of topselect.hip.
//
// [REJ] mlxcel issue #901 "Sorting-free top-k/top-p/min-p sampling with dual-pivot rejection
// kernels": "Background" (each round draws one candidate by a CDF scan over the entries above
// the lower bound, puts a second pivot halfway between the candidate and the upper bound,
// counts and weighs the entries above both, then accepts the candidate or shrinks the
// interval to whichever pivot still holds the boundary and renormalises; min-p is a filter
// on the row maximum; the joint loop tests top-k and top-p together), "Task" item 2 (a cap
// on the rounds with an exact fallback for the row) and "Regression guard".
//
// Support of a row: the first n_S tokens of the row order (logit descending, id ascending),
// n_S = min(k, n_p, n_m), n_p the shortest prefix whose mass reaches p * Z with Z the mass of
// the whole row, n_m the tokens with w = exp((x - max) / T) >= min_p. Masses are integers
// M_i = floor(w_i * 2^S), S = 63 - bitlen(V), so all sums are exact and order-free.
//
// One 1024-thread workgroup per row. The row is read from global memory once per pass (after
// the first pass mostly from L2 / the last-level cache):
//   pass 1    row maximum, NaN / +inf check, lowest id of the maximum (greedy rows);
//   pass 2    every token's mass: Z, the eligible mass Q (min-p applied) and per-tile
//             eligible masses (a tile is 2^g sub-blocks of 1024 tokens);
//   round j   wave 0 finds the tile where the running eligible mass first exceeds
//             t = floor(word_j * Q / 2^32), then the token inside it: the candidate c. One
//             counting pass then gives the count and mass of the tokens ranked above c and of
//             those above the second pivot, with per-tile masses of both sets, so the next
//             round's CDF scan reads one tile only. The second pivot lies halfway between
//             the candidate's probability and the interval's upper bound (which starts at
//             the maximum's), i.e. at the weight w1 = (w_c + w_hi) / 2; the tokens above it
//             are those whose key reaches K1, the smallest key with weight above w1;
//   fallback  after max_rounds rejections: bisection over the (key, id) order, one counting
//             pass per step (at most 64), finds the support's last token; one CDF draw over
//             the support follows.
#include <float.h>
#include <stdint.h>

#include "topselect.h"
#include "ts_device.hpp"
#include "ts_host.hpp"

using namespace tsd;

namespace {

using tsh::check_device;
using tsh::fail;

constexpr int kJT = 1024;                  // threads per workgroup (one row)
constexpr int kJW = kJT / 64;              // waves
constexpr int kSubQ = 256;                 // quads per sub-block (1024 tokens, 4 quads per lane)
constexpr int kUnroll = 2;                 // sub-blocks per wave with loads in flight
constexpr int kMaxTiles = 2048;            // per-tile masses kept in LDS per set
constexpr int kMaxRejRounds = 64;

struct JParams {
  const float* x;
  int64_t stride;
  int32_t V;
  int32_t rows;
  const int32_t* k;
  const float* p;
  const float* t;
  const float* minp;
  const uint64_t* seed;
  int32_t max_rounds;
  int32_t nsub;            // sub-blocks per row: ceil(V / 1024)
  int32_t tile_shift;      // a tile is 2^tile_shift sub-blocks
  int32_t ntiles;
  int32_t vec;             // rows are 16-byte aligned: float4 loads
  int32_t* out_token;
  int32_t* out_rounds;
  int32_t* status;
};

// A position in the row order: token (key, id) lies above (key_t, id_t) when key > key_t, or
// key == key_t and id < id_t. (key_c, c) is "ranked above token c"; (key, 0) is "key above".
struct Thr {
  uint32_t key;
  uint32_t id;
};
__device__ __forceinline__ bool above(uint32_t key, uint32_t id, Thr t) {
  return key > t.key || (key == t.key && id < t.id);
}
// The same order as one 64-bit number: (key << 32) | ~id.
__device__ __forceinline__ uint64_t thr64(Thr t) { return ((uint64_t)t.key << 32) | (uint32_t)~t.id; }
__device__ __forceinline__ Thr thr_of(uint64_t c) { return Thr{(uint32_t)(c >> 32), ~(uint32_t)c}; }
constexpr Thr kThrAll = {0u, 0u};             // every token of a valid row
constexpr Thr kThrNone = {0xFFFFFFFFu, 0u};   // no token

struct JSmem {
  uint64_t ts[3][kMaxTiles];   // per-tile eligible masses: current set and the two hypotheses
  uint64_t r64[kJW][4];
  uint32_t r32[kJW][4];
  uint32_t cand[2];            // the candidate's id and key
};

struct RowIn {
  const float* p;
  int32_t V;
  bool vec;
  // Tokens 4q .. 4q+3; tokens past the row end read as -inf (callers also test the id).
  __device__ __forceinline__ float4 quad(int32_t q) const {
    const int32_t i = 4 * q;
    if (vec && i + 3 < V) return *reinterpret_cast<const float4*>(p + i);
    float4 r;
    r.x = i < V ? p[i] : -INFINITY;
    r.y = i + 1 < V ? p[i + 1] : -INFINITY;
    r.z = i + 2 < V ? p[i + 2] : -INFINITY;
    r.w = i + 3 < V ? p[i + 3] : -INFINITY;
    return r;
  }
};

__device__ __forceinline__ float qv(const float4& v, int e) {
  return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}
__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) { return readlane64(wave_incl_scan64(v), 63); }
__device__ __forceinline__ uint32_t wave_sum32(uint32_t v) { return wave_total(wave_incl_scan(v)); }
// Workgroup-uniform values read back from LDS, moved to scalar registers.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  return ((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v);
}

// Visits every sub-block of the row once; wave w takes sub-blocks w, w + 16, ... and keeps
// kUnroll of them in flight. f(sb, v) gets the lane's four quads of sub-block sb: quad u holds
// tokens sb * 1024 + 256 u + 4 lane + (0..3).
template <class F>
__device__ __forceinline__ void row_pass(const RowIn& R, int nsub, F f) {
  const int w = wave(), l = lane();
  for (int sb0 = w; sb0 < nsub; sb0 += kJW * kUnroll) {
    float4 v[kUnroll][4];
#pragma unroll
    for (int a = 0; a < kUnroll; ++a) {
      const int sb = sb0 + a * kJW;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[a][u] = sb < nsub ? R.quad(sb * kSubQ + 64 * u + l) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int a = 0; a < kUnroll; ++a) {
      const int sb = sb0 + a * kJW;
      if (sb < nsub) f(sb, v[a]);
    }
  }
}

// Sums over the workgroup (every thread gets the totals). Ends with a barrier, so the LDS it
// uses may be reused at once.
__device__ __forceinline__ void block_sums(uint32_t& a, uint32_t& b, uint64_t& c, uint64_t& d, uint64_t& e,
                                           uint64_t& f, JSmem& sm) {
  a = wave_sum32(a);
  b = wave_sum32(b);
  c = wave_sum64(c);
  d = wave_sum64(d);
  e = wave_sum64(e);
  f = wave_sum64(f);
  if (lane() == 0) {
    sm.r32[wave()][0] = a;
    sm.r32[wave()][1] = b;
    sm.r64[wave()][0] = c;
    sm.r64[wave()][1] = d;
    sm.r64[wave()][2] = e;
    sm.r64[wave()][3] = f;
  }
  bar();
  a = b = 0;
  c = d = e = f = 0;
#pragma unroll
  for (int w = 0; w < kJW; ++w) {
    a += sm.r32[w][0];
    b += sm.r32[w][1];
    c += sm.r64[w][0];
    d += sm.r64[w][1];
    e += sm.r64[w][2];
    f += sm.r64[w][3];
  }
  a = uni(a);
  b = uni(b);
  c = uni64(c);
  d = uni64(d);
  e = uni64(e);
  f = uni64(f);
  bar();
}

struct Weigh {
  float m;
  double c2;
  int S;
  float minp;       // 0 = off
  // Mass of a token and whether min-p keeps it.
  __device__ __forceinline__ uint64_t mass(uint32_t key, bool& ok) const {
    const float w = weight32(key, m, c2);
    ok = !(minp > 0.0f) || w >= minp;
    return mass64_of(w, S);
  }
};

// Counting pass for two positions A and B: counts and masses (all tokens) above each, the
// eligible masses (min-p applied) above each, and, when TILES, per-tile eligible masses
// into tsA / tsB (zeroed by the caller).
struct Counts {
  uint32_t nA, nB;
  uint64_t mA, mB, qA, qB;
};
template <bool TILES>
__device__ __forceinline__ Counts count_pass(const RowIn& R, const JParams& P, const Weigh& W, Thr A, Thr B,
                                             uint64_t* tsA, uint64_t* tsB, JSmem& sm) {
  const uint32_t klow = min(A.key, B.key);
  float xlow = key2f(klow);
  if (!(xlow == xlow)) xlow = -INFINITY;       // keys below -inf's: every token may qualify
  const int l = lane();
  Counts c{0u, 0u, 0ull, 0ull, 0ull, 0ull};
  row_pass(R, P.nsub, [&](int sb, const float4* v) {
    uint64_t sA = 0, sB = 0;
    bool any = false;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float mx = fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w));
      const bool need = mx >= xlow;
      if (__builtin_amdgcn_ballot_w64(need) == 0) continue;
      any = true;
      if (need) {
        const uint32_t id0 = (uint32_t)(sb * 1024 + 256 * u + 4 * l);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t id = id0 + e;
          const uint32_t key = f2key(qv(v[u], e));
          const bool valid = id < (uint32_t)P.V;
          const bool a = valid && above(key, id, A);
          const bool b = valid && above(key, id, B);
          if (a || b) {
            bool ok;
            const uint64_t M = W.mass(key, ok);
            if (a) {
              c.nA += 1;
              c.mA += M;
              if (ok) sA += M;
            }
            if (b) {
              c.nB += 1;
              c.mB += M;
              if (ok) sB += M;
            }
          }
        }
      }
    }
    c.qA += sA;
    c.qB += sB;
    if (TILES && __builtin_amdgcn_ballot_w64(any) != 0) {
      const uint64_t tA = wave_sum64(sA), tB = wave_sum64(sB);
      if (l == 0) {
        const int tile = sb >> P.tile_shift;
        if (tA) atomicAdd((unsigned long long*)&tsA[tile], (unsigned long long)tA);
        if (tB) atomicAdd((unsigned long long*)&tsB[tile], (unsigned long long)tB);
      }
    }
  });
  block_sums(c.nA, c.nB, c.mA, c.mB, c.qA, c.qB, sm);
  return c;
}

// Wave 0: the first eligible token (above E, min-p kept) whose inclusive running mass in id
// order exceeds t, found through the per-tile masses ts. Result in sm.cand.
__device__ __forceinline__ void cdf_draw(const RowIn& R, const JParams& P, const Weigh& W, Thr E,
                                         const uint64_t* ts, uint64_t t, JSmem& sm) {
  const int l = lane();
  uint64_t run = 0;
  int tile = -1;
  for (int base = 0; base < P.ntiles; base += 64) {
    const uint64_t v = base + l < P.ntiles ? ts[base + l] : 0ull;
    const uint64_t incl = wave_incl_scan64(v);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(run + incl > t);
    if (hit) {
      const int L = (int)__builtin_ctzll(hit);
      tile = base + L;
      run += readlane64(incl - v, L);
      break;
    }
    run += readlane64(incl, 63);
  }
  // The tile masses and this scan weigh the same tokens with the same arithmetic, so the
  // crossing exists whenever t < Q.
  uint32_t found = 0xFFFFFFFFu, fkey = 0u;
  if (tile >= 0) {
    const int sb_end = min((tile + 1) << P.tile_shift, P.nsub);
    for (int sb = tile << P.tile_shift; sb < sb_end && found == 0xFFFFFFFFu; ++sb) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = R.quad(sb * kSubQ + 64 * u + l);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint64_t M[4];
        uint64_t s = 0;
        const uint32_t id0 = (uint32_t)(sb * 1024 + 256 * u + 4 * l);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t id = id0 + e;
          const uint32_t key = f2key(qv(v[u], e));
          bool ok = false;
          M[e] = 0;
          if (id < (uint32_t)P.V && above(key, id, E)) {
            const uint64_t mm = W.mass(key, ok);
            M[e] = ok ? mm : 0ull;
          }
          s += M[e];
        }
        const uint64_t incl = wave_incl_scan64(s);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(run + incl > t);
        if (hit) {
          const int L = (int)__builtin_ctzll(hit);
          uint32_t myc = 0xFFFFFFFFu, myk = 0u;
          if (l == L) {
            uint64_t r = run + incl - s;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              r += M[e];
              if (myc == 0xFFFFFFFFu && M[e] != 0 && r > t) {
                myc = id0 + e;
                myk = f2key(qv(v[u], e));
              }
            }
          }
          found = (uint32_t)__builtin_amdgcn_readlane((int)myc, L);
          fkey = (uint32_t)__builtin_amdgcn_readlane((int)myk, L);
          break;
        }
        run += readlane64(incl, 63);
      }
    }
  }
  if (l == 0) {
    sm.cand[0] = found;
    sm.cand[1] = fkey;
  }
}

// The smallest key whose weight exceeds w1 (> 0), or kmax + 1 when none does: the tokens
// "greater than" the second pivot are then exactly those with key >= K1, a prefix of the row
// order whatever the rounding of the weights. Bisection over [key(-inf), kmax]; every key in
// that range decodes to a finite fp32 value <= the row maximum. Uniform over the workgroup.
__device__ __forceinline__ uint32_t first_key_above(float w1, uint32_t kmax, const Weigh& W) {
  if (!(weight32(kmax, W.m, W.c2) > w1)) return kmax + 1u;
  uint32_t lo = kKeyNegInf, hi = kmax;   // weight(lo) = 0 <= w1 < weight(hi)
  while (hi - lo > 1u) {
    const uint32_t mid = lo + (hi - lo) / 2u;
    if (weight32(mid, W.m, W.c2) > w1) hi = mid;
    else lo = mid;
  }
  return hi;
}

__device__ __forceinline__ uint64_t draw_target(uint64_t seed, int r, int j, uint64_t q) {
  const uint32_t word = philox4x32_10((uint32_t)j, (uint32_t)r, (uint32_t)seed, (uint32_t)(seed >> 32), 1u).x;
  return (uint64_t)(((unsigned __int128)word * q) >> 32);
}

__global__ void __launch_bounds__(kJT) ts_rejection_kernel(JParams P) {
  __shared__ JSmem sm;
  const int r = blockIdx.x;
  const RowIn R{P.x + (int64_t)r * P.stride, P.V, P.vec != 0};
  const int32_t kr = P.k ? P.k[r] : P.V;
  const float p = P.p ? P.p[r] : 1.0f;
  const float t = P.t ? P.t[r] : 1.0f;
  const float minp = P.minp ? P.minp[r] : 0.0f;

  // Pass 1: maximum key, NaN and, for greedy rows (T = 0), the lowest id holding the maximum.
  uint32_t bk = 0u, bid = 0xFFFFFFFFu, nan = 0u;
  {
    const int l = lane();
    if (t == 0.0f) {
      row_pass(R, P.nsub, [&](int sb, const float4* v) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t id0 = (uint32_t)(sb * 1024 + 256 * u + 4 * l);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = qv(v[u], e);
            const uint32_t key = f2key(x);
            nan |= (x != x) ? 1u : 0u;
            if (id0 + e < (uint32_t)P.V && key > bk) {
              bk = key;
              bid = id0 + e;
            }
          }
        }
      });
    } else {
      // The IEEE 754-2019 maximum propagates NaN: the running maximum is NaN exactly when the
      // lane read one (tokens past the row end read as -inf).
      float fm = -INFINITY;
      row_pass(R, P.nsub, [&](int, const float4* v) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          fm = __builtin_elementwise_maximum(fm, __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[u].x, v[u].y),
                                                                              __builtin_elementwise_maximum(v[u].z, v[u].w)));
      });
      nan = __builtin_isnan(fm) ? 1u : 0u;
      bk = nan ? 0u : f2key(fm);
    }
    const uint32_t wk = wave_max(bk);
    const uint32_t wi = ~wave_max(bk == wk ? ~bid : 0u);
    const uint32_t wn = wave_max(nan);
    if (lane() == 0) {
      sm.r32[wave()][0] = wk;
      sm.r32[wave()][1] = wi;
      sm.r32[wave()][2] = wn;
    }
    bar();
    bk = 0u;
    bid = 0xFFFFFFFFu;
    nan = 0u;
#pragma unroll
    for (int w = 0; w < kJW; ++w) {
      const uint32_t k2 = sm.r32[w][0], i2 = sm.r32[w][1];
      if (k2 > bk || (k2 == bk && i2 < bid)) {
        bk = k2;
        bid = i2;
      }
      nan |= sm.r32[w][2];
    }
    bar();
  }
  const uint32_t kmax = bk;
  int st = TS_ROW_OK;
  if (nan || kmax >= kKeyPosInf || kmax <= kKeyNegInf) st = TS_ROW_NONFINITE;
  else if (kr < 1) st = TS_ROW_BAD_K;
  else if (!(p > 0.0f && p <= 1.0f)) st = TS_ROW_BAD_P;
  else if (!(t >= 0.0f && t <= FLT_MAX)) st = TS_ROW_BAD_T;
  else if (!(minp >= 0.0f && minp <= 1.0f)) st = TS_ROW_BAD_MINP;
  const bool lead = threadIdx.x == 0;
  if (st != TS_ROW_OK || t == 0.0f) {
    if (lead) {
      P.out_token[r] = st == TS_ROW_OK ? (int32_t)bid : -1;
      if (P.out_rounds) P.out_rounds[r] = 0;
      if (P.status) P.status[r] = st;
    }
    return;
  }
  const uint32_t ke = (uint32_t)min(kr, P.V);
  const bool topp_on = p != 1.0f;
  const uint64_t seed = P.seed[r];
  Weigh W;
  W.m = key2f(kmax);
  W.c2 = kLog2e / (double)t;
  W.S = 63 - bitlen((uint32_t)P.V);
  W.minp = minp;

  // Pass 2: Z over the row, Q and per-tile masses over the min-p set.
  int cur = 0;
  for (int i = threadIdx.x; i < P.ntiles; i += kJT) sm.ts[0][i] = 0ull;
  bar();
  uint64_t Z = 0, Q = 0;
  {
    const int l = lane();
    row_pass(R, P.nsub, [&](int sb, const float4* v) {
      uint64_t s = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t id0 = (uint32_t)(sb * 1024 + 256 * u + 4 * l);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (id0 + e < (uint32_t)P.V) {
            bool ok;
            const uint64_t M = W.mass(f2key(qv(v[u], e)), ok);
            Z += M;
            if (ok) s += M;
          }
        }
      }
      Q += s;
      const uint64_t tot = wave_sum64(s);
      if (l == 0 && tot) atomicAdd((unsigned long long*)&sm.ts[0][sb >> P.tile_shift], (unsigned long long)tot);
    });
    uint32_t d0 = 0, d1 = 0;
    uint64_t d2 = 0, d3 = 0;
    block_sums(d0, d1, Z, Q, d2, d3, sm);   // its barriers also complete the tile atomics
  }
  const uint64_t target = topp_on ? topp_target(p, Z) : 0ull;

  // Rejection rounds.
  Thr E = kThrAll;
  float hi = 1.0f;   // the interval's upper bound, as a weight: the maximum's

  int32_t token = -1, rounds = -1;
  for (int j = 0; j < P.max_rounds; ++j) {
    if (wave() == 0) cdf_draw(R, P, W, E, sm.ts[cur], draw_target(seed, r, j, Q), sm);
    const int iA = cur == 2 ? 0 : cur + 1, iB = iA == 2 ? 0 : iA + 1;
    for (int i = threadIdx.x; i < P.ntiles; i += kJT) {
      sm.ts[iA][i] = 0ull;
      sm.ts[iB][i] = 0ull;
    }
    bar();
    const uint32_t c = uni(sm.cand[0]), kc = uni(sm.cand[1]);
    // second pivot: halfway between the candidate's weight and the upper bound ([REJ]
    // "Background", top-k step (b), in probability space: probabilities are weights / Z)
    const float wc = weight32(kc, W.m, W.c2);
    const float w1 = __fadd_rn(__fmul_rn(0.5f, wc), __fmul_rn(0.5f, hi));
    const Thr A{kc, c}, B{first_key_above(w1, kmax, W), 0xFFFFFFFFu};   // B: key >= K1
    const Counts n = count_pass<true>(R, P, W, A, B, sm.ts[iA], sm.ts[iB], sm);
    if (n.nA < ke && (!topp_on || n.mA < target)) {
      token = (int32_t)c;
      rounds = j + 1;
      break;
    }
    if (n.nB >= ke || (topp_on && n.mB >= target)) {   // the support lies above the second pivot
      E = B;
      Q = n.qB;
      cur = iB;
    } else {                                            // above the candidate, below the pivot
      E = A;
      Q = n.qA;
      cur = iA;
      hi = w1;
    }
  }

  if (token < 0) {
    // Fallback ([REJ] "Task" item 2): the support's last token s lies in (lo, hi64] of the
    // 64-bit order; halve the interval until it is one position wide.
    uint64_t lo = thr64(E), hi64 = ((uint64_t)kmax << 32) | 0xFFFFFFFFull;
    while (hi64 - lo > 1) {
      const uint64_t mid = lo + (hi64 - lo) / 2;
      const Counts n = count_pass<false>(R, P, W, thr_of(mid), kThrNone, nullptr, nullptr, sm);
      if (n.nA >= ke || (topp_on && n.mA >= target)) lo = mid;
      else hi64 = mid;
    }
    const int iA = cur == 2 ? 0 : cur + 1;
    for (int i = threadIdx.x; i < P.ntiles; i += kJT) sm.ts[iA][i] = 0ull;
    bar();
    const Thr F = thr_of(lo);
    const Counts n = count_pass<true>(R, P, W, F, kThrNone, sm.ts[iA], sm.ts[iA], sm);
    if (wave() == 0) cdf_draw(R, P, W, F, sm.ts[iA], draw_target(seed, r, P.max_rounds, n.qA), sm);
    bar();
    token = (int32_t)uni(sm.cand[0]);
    rounds = -1;
  }
  if (lead) {
    P.out_token[r] = token;
    if (P.out_rounds) P.out_rounds[r] = rounds;
    if (P.status) P.status[r] = TS_ROW_OK;
  }
}

}  // namespace

extern "C" int ts_sample_rows_rejection(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                                        const int32_t* top_k, const float* top_p, const float* temperature,
                                        const float* min_p, const uint64_t* seed, int32_t max_rounds,
                                        int32_t* out_token, int32_t* out_rounds, int32_t* row_status,
                                        void* stream) {
  if (rows < 0) return fail(TS_ERR_INVALID_ARG, "rows = %lld < 0", (long long)rows);
  if (vocab < 1 || vocab > TS_MAX_VOCAB)
    return fail(TS_ERR_INVALID_ARG, "vocab = %lld outside [1, 2^30]", (long long)vocab);
  if (row_stride < vocab)
    return fail(TS_ERR_INVALID_ARG, "row_stride %lld < vocab %lld", (long long)row_stride, (long long)vocab);
  if (max_rounds < 0 || max_rounds > kMaxRejRounds)
    return fail(TS_ERR_INVALID_ARG, "max_rounds = %d outside [0, %d]", (int)max_rounds, kMaxRejRounds);
  if (rows == 0) return TS_OK;   // an empty batch: nothing to read or write
  if (!logits) return fail(TS_ERR_INVALID_ARG, "logits pointer is NULL");
  if (rows > 0x7FFFFFFF) return fail(TS_ERR_INVALID_ARG, "rows too large");
  if (!seed || !out_token) return fail(TS_ERR_INVALID_ARG, "seed and out_token are required");
  int dev;
  const int rc = check_device(&dev);
  if (rc != TS_OK) return rc;
  JParams P;
  P.x = logits;
  P.stride = row_stride;
  P.V = (int32_t)vocab;
  P.rows = (int32_t)rows;
  P.k = top_k;
  P.p = top_p;
  P.t = temperature;
  P.minp = min_p;
  P.seed = seed;
  P.max_rounds = max_rounds;
  P.nsub = (int32_t)((vocab + 1023) / 1024);
  int g = 0;
  while (((P.nsub + (1 << g) - 1) >> g) > kMaxTiles) ++g;
  P.tile_shift = g;
  P.ntiles = (P.nsub + (1 << g) - 1) >> g;
  P.vec = (((uintptr_t)logits & 15u) == 0 && row_stride % 4 == 0) ? 1 : 0;
  P.out_token = out_token;
  P.out_rounds = out_rounds;
  P.status = row_status;
  hipLaunchKernelGGL(ts_rejection_kernel, dim3((unsigned)rows), dim3(kJT), 0, (hipStream_t)stream, P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TS_ERR_LAUNCH, "rejection kernel launch failed: %s", hipGetErrorString(e));
  return TS_OK;
}
