// ts_device.hpp -- wave64 / workgroup primitives for the gfx950 sampling kernels.
//
// Block-level helpers take the workgroup's wave count NW as a template argument and must be
// called with workgroup-uniform control flow (every thread reaches every barrier).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsd {

__device__ __forceinline__ int lane() { return (int)__lane_id(); }
__device__ __forceinline__ int wave() { return (int)(threadIdx.x >> 6); }

// Barrier that orders LDS only. Unlike __syncthreads() it does not wait for outstanding
// global loads, so loads issued before it stay in flight across it.
__device__ __forceinline__ void bar() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Barrier that also orders global memory between the threads of the workgroup.
__device__ __forceinline__ void bar_all() { __syncthreads(); }

__device__ __forceinline__ uint32_t shr(uint32_t x, int s) { return s >= 32 ? 0u : (x >> s); }
__device__ __forceinline__ uint32_t shl(uint32_t x, int s) { return s >= 32 ? 0u : (x << s); }

// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ uint32_t mbcnt(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---------------------------------------------------------------- ordered fp32 keys
// Monotone map fp32 -> uint32 (larger float -> larger key) after -0.0 -> +0.0: flip every
// bit of negatives, only the sign bit of non-negatives. Keys are compared as integers, so
// flush-to-zero modes never merge distinct subnormals.
__device__ __forceinline__ uint32_t f2key(float v) {
  uint32_t b = __float_as_uint(v);
  b = (b == 0x80000000u) ? 0u : b;
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}
constexpr uint32_t kKeyPosInf = 0xFF800000u;   // f2key(+inf)
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;   // f2key(-inf)

// ---------------------------------------------------------------- wave scans
// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round trips): Hillis-Steele
// shifts of 1, 2, 4, 8 inside each 16-lane row, then row 0's total is broadcast into row 1
// and row 2's into row 3 (row_bcast:15), then rows 0-1's total into rows 2-3 (row_bcast:31).
// Lanes whose DPP source is outside the row or masked receive 0.
#define TSD_DPP(v, ctrl, rmask, bmask) \
  ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(v), (ctrl), (rmask), (bmask), false))
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += TSD_DPP(v, 0x111, 0xf, 0xf);   // row_shr:1
  v += TSD_DPP(v, 0x112, 0xf, 0xf);   // row_shr:2
  v += TSD_DPP(v, 0x114, 0xf, 0xf);   // row_shr:4
  v += TSD_DPP(v, 0x118, 0xf, 0xf);   // row_shr:8
  v += TSD_DPP(v, 0x142, 0xa, 0xf);   // row_bcast:15 into rows 1 and 3
  v += TSD_DPP(v, 0x143, 0xc, 0xf);   // row_bcast:31 into rows 2 and 3
  return v;
}
// Maximum over the 64 lanes (every lane gets it): the scan pattern with max in place of add
// (lanes without a DPP source receive 0, the identity of an unsigned max).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, TSD_DPP(v, 0x111, 0xf, 0xf));
  v = max(v, TSD_DPP(v, 0x112, 0xf, 0xf));
  v = max(v, TSD_DPP(v, 0x114, 0xf, 0xf));
  v = max(v, TSD_DPP(v, 0x118, 0xf, 0xf));
  v = max(v, TSD_DPP(v, 0x142, 0xa, 0xf));
  v = max(v, TSD_DPP(v, 0x143, 0xc, 0xf));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) { return ~wave_max(~v); }
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= TSD_DPP(v, 0x111, 0xf, 0xf);
  v |= TSD_DPP(v, 0x112, 0xf, 0xf);
  v |= TSD_DPP(v, 0x114, 0xf, 0xf);
  v |= TSD_DPP(v, 0x118, 0xf, 0xf);
  v |= TSD_DPP(v, 0x142, 0xa, 0xf);
  v |= TSD_DPP(v, 0x143, 0xc, 0xf);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Orders this wave's LDS accesses: LDS operations of one wave complete in issue order, so a
// compiler barrier suffices for lanes to read what other lanes of the same wave wrote.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ uint32_t wave_total(uint32_t incl) {
  return (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
}
// Inclusive suffix sums: lane l gets the sum over lanes >= l.
__device__ __forceinline__ uint32_t wave_incl_suffix(uint32_t v) {
  const uint32_t incl = wave_incl_scan(v);
  return wave_total(incl) - incl + v;
}
__device__ __forceinline__ uint64_t wave_incl_suffix64(uint64_t v) {
  // two 32-bit DPP scans with the carry of the low half folded into the high half
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint32_t lo_hi16 = lo >> 16, lo_lo16 = lo & 0xFFFFu;
  // sums of 64 values below 2^16 stay below 2^22, so the split halves cannot overflow
  const uint32_t s_lo16 = wave_incl_suffix(lo_lo16);
  const uint32_t s_hi16 = wave_incl_suffix(lo_hi16);
  const uint32_t s_hi = wave_incl_suffix(hi);
  return ((uint64_t)s_hi << 32) + ((uint64_t)s_hi16 << 16) + (uint64_t)s_lo16;
}

// ---------------------------------------------------------------- block reductions
// `red` is an NW-entry LDS scratch array (NW = waves per workgroup); the function ends with a barrier so it can be
// reused immediately.
template <int NW>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor(v, d, 64));
  if (lane() == 0) red[wave()] = v;
  bar();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = max(r, red[w]);
  bar();
  return r;
}
template <int NW>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, (uint32_t)__shfl_xor(v, d, 64));
  if (lane() == 0) red[wave()] = v;
  bar();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = min(r, red[w]);
  bar();
  return r;
}
template <int NW>
__device__ __forceinline__ uint32_t block_or_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v |= (uint32_t)__shfl_xor(v, d, 64);
  if (lane() == 0) red[wave()] = v;
  bar();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) r |= red[w];
  bar();
  return r;
}
// Workgroup max, min and bitwise-or of three values at once (`red` holds 3 * NW entries).
template <int NW>
__device__ __forceinline__ void block_reduce3(uint32_t& mx, uint32_t& mn, uint32_t& orv, uint32_t* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    mx = max(mx, (uint32_t)__shfl_xor(mx, d, 64));
    mn = min(mn, (uint32_t)__shfl_xor(mn, d, 64));
    orv |= (uint32_t)__shfl_xor(orv, d, 64);
  }
  if (lane() == 0) {
    red[wave()] = mx;
    red[NW + wave()] = mn;
    red[2 * NW + wave()] = orv;
  }
  bar();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mx = max(mx, red[w]);
    mn = min(mn, red[NW + w]);
    orv |= red[2 * NW + w];
  }
  bar();
}
// Workgroup max of two values, min of a third and bitwise-or of a fourth at once (`red` holds
// 4 * NW entries).
template <int NW>
__device__ __forceinline__ void block_reduce4(uint32_t& mx1, uint32_t& mx2, uint32_t& mn, uint32_t& orv,
                                              uint32_t* red) {
  mx1 = wave_max(mx1);
  mx2 = wave_max(mx2);
  mn = wave_min(mn);
  orv = wave_or(orv);
  if (lane() == 0) {
    red[wave()] = mx1;
    red[NW + wave()] = mx2;
    red[2 * NW + wave()] = mn;
    red[3 * NW + wave()] = orv;
  }
  bar();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mx1 = max(mx1, red[w]);
    mx2 = max(mx2, red[NW + w]);
    mn = min(mn, red[2 * NW + w]);
    orv |= red[3 * NW + w];
  }
  bar();
}
template <int NW>
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += (uint64_t)__shfl_xor(v, d, 64);
  if (lane() == 0) red[wave()] = v;
  bar();
  uint64_t r = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) r += red[w];
  bar();
  return r;
}
// Workgroup sums of two 64-bit values at once (`red` holds 2 * NW entries).
template <int NW>
__device__ __forceinline__ void block_sum2_u64(uint64_t& a, uint64_t& b, uint64_t* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    a += (uint64_t)__shfl_xor(a, d, 64);
    b += (uint64_t)__shfl_xor(b, d, 64);
  }
  if (lane() == 0) {
    red[wave()] = a;
    red[NW + wave()] = b;
  }
  bar();
  a = 0;
  b = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    a += red[w];
    b += red[NW + w];
  }
  bar();
}
// Exclusive prefix over the workgroup in thread order; `total` gets the sum of all.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  uint32_t incl = wave_incl_scan(v);
  if (lane() == 63) red[wave()] = incl;
  bar();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint32_t t = red[w];
    base += (w < wave()) ? t : 0u;
    tot += t;
  }
  bar();
  total = tot;
  return base + incl - v;
}

// Argmax over the workgroup of (score, lowest id): every thread gets the winning id and
// (through best_s) its score.
template <int NW>
__device__ __forceinline__ int32_t block_argmax(float s, int32_t id, float* reds, int32_t* redi,
                                                float* best_s = nullptr) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    float os = __shfl_xor(s, d, 64);
    int32_t oi = __shfl_xor(id, d, 64);
    bool take = (os > s) || (os == s && (uint32_t)oi < (uint32_t)id);
    s = take ? os : s;
    id = take ? oi : id;
  }
  if (lane() == 0) { reds[wave()] = s; redi[wave()] = id; }
  bar();
  float bs = reds[0];
  int32_t bi = redi[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    float os = reds[w];
    int32_t oi = redi[w];
    bool take = (os > bs) || (os == bs && (uint32_t)oi < (uint32_t)bi);
    bs = take ? os : bs;
    bi = take ? oi : bi;
  }
  bar();
  if (best_s) *best_s = bs;
  return bi;
}

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11):
// ten rounds of the 4x32 bijection with multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl
// key increments 0x9E3779B9 / 0xBB67AE85. Counter (c0, c1, 0, 0), key (k0, k1).
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1) {
  uint32_t c2 = 0u, c3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint32_t hi_a = __umulhi(0xD2511F53u, c0), lo_a = 0xD2511F53u * c0;
    const uint32_t hi_b = __umulhi(0xCD9E8D57u, c2), lo_b = 0xCD9E8D57u * c2;
    const uint32_t n0 = hi_b ^ c1 ^ k0, n2 = hi_a ^ c3 ^ k1;
    c0 = n0; c1 = lo_b; c2 = n2; c3 = lo_a;
  }
  return make_uint4(c0, c1, c2, c3);
}
__device__ __forceinline__ uint32_t pick_word(uint4 w, uint32_t j) {
  return j == 0 ? w.x : (j == 1 ? w.y : (j == 2 ? w.z : w.w));
}
// u = fp32(word * 2^-32) clamped to [2^-32, 1 - 2^-24]; the conversion rounds to nearest
// and the power-of-two scale is exact, so this is fp32 rounding of word * 2^-32.
__device__ __forceinline__ float uniform_from_word(uint32_t w) {
  const float u = (float)w * 0x1p-32f;
  return fminf(fmaxf(u, 0x1p-32f), 1.0f - 0x1p-24f);
}
// Gumbel noise with the log1p(-u) transform: the large-noise tail maps to u -> 0.
__device__ __forceinline__ float gumbel_from_uniform(float u) { return -logf(-log1pf(-u)); }

// ---------------------------------------------------------------- fixed-point mass
// Probability mass is summed exactly as two unsigned 64-bit integer parts so that
// histograms and totals do not depend on the order of the additions: a weight w in [0,1]
// is represented as floor(w * 2^(2S)) = hi * 2^S + lo with 0 <= lo < 2^S, where S is chosen
// per row so that n weights cannot overflow 64 bits in either part (S = 63 - bitlen(n)).
struct Mass {
  uint64_t hi, lo;
};
__device__ __forceinline__ Mass mass_of(double w, int s) {
  const double t = ldexp(w, s);                 // exact scaling
  const uint64_t hi = (uint64_t)t;              // truncation; t < 2^S + 1
  const double f = t - (double)hi;              // exact fractional part
  const uint64_t lo = (uint64_t)ldexp(f, s);    // exact truncation
  return Mass{hi, lo};
}
__device__ __forceinline__ double mass_to_double(uint64_t hi, uint64_t lo, int s) {
  return ldexp((double)hi, -s) + ldexp((double)lo, -2 * s);
}

}  // namespace tsd
