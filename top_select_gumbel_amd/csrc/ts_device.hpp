// ts_device.hpp -- wave64 / workgroup primitives for the gfx950 sampling kernels.
//
// Block-level helpers take the workgroup's wave count NW as a template argument and must be
// called with workgroup-uniform control flow (every thread reaches every barrier). Wave-level
// reductions and scans use DPP lane moves (a few cycles each) rather than LDS permutes.
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

// Orders this wave's LDS accesses: LDS operations of one wave complete in issue order, so a
// compiler barrier suffices for lanes to read what other lanes of the same wave wrote.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

// ---------------------------------------------------------------- wave scans / reductions
// The lane pattern of an inclusive scan over 64 lanes: Hillis-Steele shifts of 1, 2, 4, 8
// inside each 16-lane row, then row 0's last lane is broadcast into row 1 and row 2's into
// row 3 (row_bcast:15), then row 1's last lane into rows 2-3 (row_bcast:31). A lane whose
// source lies outside its row (or whose row is masked) receives the `identity` operand of
// the combining operation. Lane 63 ends with the combination of all lanes.
template <int CTRL, int RMASK>
__device__ __forceinline__ uint32_t dpp32(uint32_t v, uint32_t identity) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, RMASK, 0xf, false);
}
template <int CTRL, int RMASK>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = dpp32<CTRL, RMASK>((uint32_t)v, 0u);
  const uint32_t hi = dpp32<CTRL, RMASK>((uint32_t)(v >> 32), 0u);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp32<0x111, 0xf>(v, 0u);   // row_shr:1
  v += dpp32<0x112, 0xf>(v, 0u);   // row_shr:2
  v += dpp32<0x114, 0xf>(v, 0u);   // row_shr:4
  v += dpp32<0x118, 0xf>(v, 0u);   // row_shr:8
  v += dpp32<0x142, 0xa>(v, 0u);   // row_bcast:15 into rows 1 and 3
  v += dpp32<0x143, 0xc>(v, 0u);   // row_bcast:31 into rows 2 and 3
  return v;
}
// 64-bit values: the same moves on both halves, added with carry.
__device__ __forceinline__ uint64_t wave_incl_scan64(uint64_t v) {
  v += dpp64<0x111, 0xf>(v);
  v += dpp64<0x112, 0xf>(v);
  v += dpp64<0x114, 0xf>(v);
  v += dpp64<0x118, 0xf>(v);
  v += dpp64<0x142, 0xa>(v);
  v += dpp64<0x143, 0xc>(v);
  return v;
}
__device__ __forceinline__ uint32_t wave_total(uint32_t incl) {
  return (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
}
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
// Inclusive suffix sums: lane l gets the sum over lanes >= l.
__device__ __forceinline__ uint32_t wave_incl_suffix(uint32_t v) {
  const uint32_t incl = wave_incl_scan(v);
  return wave_total(incl) - incl + v;
}
__device__ __forceinline__ uint64_t wave_incl_suffix64(uint64_t v) {
  const uint64_t incl = wave_incl_scan64(v);
  return readlane64(incl, 63) - incl + v;
}
// Maximum / minimum / or over the 64 lanes (every lane gets the result).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, dpp32<0x111, 0xf>(v, 0u));
  v = max(v, dpp32<0x112, 0xf>(v, 0u));
  v = max(v, dpp32<0x114, 0xf>(v, 0u));
  v = max(v, dpp32<0x118, 0xf>(v, 0u));
  v = max(v, dpp32<0x142, 0xa>(v, 0u));
  v = max(v, dpp32<0x143, 0xc>(v, 0u));
  return wave_total(v);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) { return ~wave_max(~v); }
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= dpp32<0x111, 0xf>(v, 0u);
  v |= dpp32<0x112, 0xf>(v, 0u);
  v |= dpp32<0x114, 0xf>(v, 0u);
  v |= dpp32<0x118, 0xf>(v, 0u);
  v |= dpp32<0x142, 0xa>(v, 0u);
  v |= dpp32<0x143, 0xc>(v, 0u);
  return wave_total(v);
}
// Argmax of (score, lowest id) over the wave, every lane gets it: the maximum of the ordered
// score keys, then the minimum id among the lanes holding it -- two plain unsigned DPP
// reductions (a combined compare-and-select per step costs three times as much).
__device__ __forceinline__ void wave_argmax(float& s, int32_t& id) {
  const uint32_t k = f2key(s);
  const uint32_t km = wave_max(k);
  id = (int32_t)wave_min(k == km ? (uint32_t)id : 0xFFFFFFFFu);
  s = key2f(km);
}

// ---------------------------------------------------------------- block reductions
// `red` is LDS scratch (sizes below); each helper ends with a barrier so it can be reused.
template <int NW>   // red: NW entries
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max(v);
  if (lane() == 0) red[wave()] = v;
  bar();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = max(r, red[w]);
  bar();
  return r;
}
template <int NW>   // red: NW entries
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* red) {
  return ~block_max_u32<NW>(~v, red);
}
// Max of two values, min of a third and bitwise-or of a fourth at once (red: 4 * NW).
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
// block_reduce4 together with an exclusive prefix of v over the threads in order (excl) and
// its total: one exchange through LDS for all of them (red: 5 * NW). Ends without the
// barrier that protects `red`: the caller places it (after its own LDS writes).
template <int NW>
__device__ __forceinline__ void block_reduce4_scan(uint32_t& mx1, uint32_t& mx2, uint32_t& mn, uint32_t& orv,
                                                   uint32_t v, uint32_t& excl, uint32_t& total, uint32_t* red) {
  mx1 = wave_max(mx1);
  mx2 = wave_max(mx2);
  mn = wave_min(mn);
  orv = wave_or(orv);
  const uint32_t incl = wave_incl_scan(v);
  if (lane() == 0) {
    red[wave()] = mx1;
    red[NW + wave()] = mx2;
    red[2 * NW + wave()] = mn;
    red[3 * NW + wave()] = orv;
  }
  if (lane() == 63) red[4 * NW + wave()] = incl;
  bar();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mx1 = max(mx1, red[w]);
    mx2 = max(mx2, red[NW + w]);
    mn = min(mn, red[2 * NW + w]);
    orv |= red[3 * NW + w];
    const uint32_t t = red[4 * NW + w];
    base += (w < wave()) ? t : 0u;
    tot += t;
  }
  excl = base + incl - v;
  total = tot;
}
// Sums of two 64-bit values at once (red: 2 * NW).
template <int NW>
__device__ __forceinline__ void block_sum2_u64(uint64_t& a, uint64_t& b, uint64_t* red) {
  a = wave_incl_scan64(a);
  b = wave_incl_scan64(b);
  if (lane() == 63) {
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
// Exclusive prefix over the workgroup in thread order; `total` gets the sum of all (red: NW).
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  const uint32_t incl = wave_incl_scan(v);
  if (lane() == 63) red[wave()] = incl;
  bar();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = red[w];
    base += (w < wave()) ? t : 0u;
    tot += t;
  }
  bar();
  total = tot;
  return base + incl - v;
}
// Argmax over the workgroup of (score, lowest id): every thread gets the winning id and
// (through best_s) its score (reds, redi: NW entries each). A score of -inf loses to every
// Workgroup sum of one double per thread in a fixed tree (lane butterfly, then the waves in
// order): the same bits for every launch. red holds NW doubles. Every thread gets the sum.
template <int NW>
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if (lane() == 0) red[wave()] = v;
  bar();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += red[w];
  bar();
  return s;
}

// finite one; scores are never NaN.
template <int NW>
// `last`: the workgroup's final use of reds / redi, so no barrier needs to protect their reuse.
__device__ __forceinline__ int32_t block_argmax(float s, int32_t id, float* reds, int32_t* redi,
                                                float* best_s = nullptr, bool last = false) {
  wave_argmax(s, id);
  if (lane() == 0) { reds[wave()] = s; redi[wave()] = id; }
  bar();
  uint32_t km = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) km = max(km, f2key(reds[w]));
  uint32_t bi = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < NW; ++w) bi = (f2key(reds[w]) == km) ? min(bi, (uint32_t)redi[w]) : bi;
  if (!last) bar();
  if (best_s) *best_s = key2f(km);
  return (int32_t)bi;
}

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11):
// ten rounds of the 4x32 bijection with multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl
// key increments 0x9E3779B9 / 0xBB67AE85. Counter (c0, c1, c2, 0), key (k0, k1).
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1,
                                               uint32_t c2_in = 0u) {
  uint32_t c2 = c2_in, c3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t pa = (uint64_t)0xD2511F53u * c0;   // one 32x32->64 multiply gives both halves
    const uint64_t pb = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(pb >> 32) ^ c1 ^ k0, n2 = (uint32_t)(pa >> 32) ^ c3 ^ k1;
    c0 = n0; c1 = (uint32_t)pb; c2 = n2; c3 = (uint32_t)pa;
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
// Gumbel noise g = -log(E), E = -log1p(-u): the large-noise tail maps to u -> 0.
// log1p(-u) by Goldberg's compensation ("What every computer scientist should know about
// floating-point arithmetic", ACM Computing Surveys 1991, theorem 4): with y = fl(1 - u) and
// d = 1 - y (exact), log1p(-u) = log(y) * u / d, and -u itself when y == 1; the rounding of y
// cancels in the ratio. Both logarithms come from the hardware base-2 logarithm (v_log_f32,
// normal inputs only here: y >= 2^-24, E >= 2^-32) scaled by ln 2. Error of g within 1e-6 plus
// two fp32 ulps of g over the whole clamped range of u (checked on the GPU against binary64).
__device__ __forceinline__ float gumbel_from_uniform(float u) {
  constexpr float kLn2f = 0.693147180559945309f;
  const float y = 1.0f - u;
  const float d = 1.0f - y;
  const float e = (y == 1.0f) ? u : (-__builtin_amdgcn_logf(y) * kLn2f) * (u * __builtin_amdgcn_rcpf(d));
  return -__builtin_amdgcn_logf(e) * kLn2f;
}

// ---------------------------------------------------------------- fixed-point mass
// Probability mass is summed exactly in unsigned 64-bit fixed point so that histograms and
// totals do not depend on the order of the additions: a weight w in [0, 1] counts as
// floor(w * 2^S), S chosen per row so that n weights cannot overflow (S = 63 - bitlen(n)).
// Computed from the fp32 weight's bits (s <= 62): a normal w is m24 * 2^(E - 150) (E its
// biased exponent), so the product is a shift of m24; zero and subnormals (below 2^-126)
// give 0. Equal to (uint64_t)ldexp((double)w, s) for every such w.
// The same value through binary64 (exact: a power-of-two scale, then truncation). Measured
// faster than the shifts in the rejection kernel's all-token passes, slower elsewhere.
__device__ __forceinline__ uint64_t mass64_of(float w, int s) { return (uint64_t)ldexp((double)w, s); }
// Written with selects only: both shifts are formed and one is kept, so a wave never splits.
__device__ __forceinline__ uint64_t mass32_of(float w, int s) {
  const uint32_t b = __float_as_uint(w);
  const int e = (int)((b >> 23) & 0xFFu);
  const uint64_t m = (uint64_t)((b & 0x7FFFFFu) | 0x800000u);
  const int sh = e - 150 + s;
  const uint64_t up = m << (sh & 63);
  const uint64_t dn = m >> ((-sh) & 63);
  const uint64_t r = sh >= 0 ? up : (sh > -24 ? dn : 0ull);
  return e == 0 ? 0ull : r;
}


// ---------------------------------------------------------------- weights
constexpr double kLog2e = 1.4426950408889634;   // log2(e)

// Unnormalized weight exp((x - m) / T) of a key, about 1.5e-7 relative: the base-2 exponent
// z = (x - m) * log2(e) / T is formed in binary64 (x - m exact, c2 = log2(e) / T rounded
// once), split into integer and fraction, and only 2^fraction is evaluated in fp32.
// -inf logits (and weights below 2^-200) give 0.
// The fraction lies in [0, 1), so the hardware base-2 exponential needs no range reduction.
__device__ __forceinline__ float weightf(float x, float m, double c2) {
  const double z = ((double)x - (double)m) * c2;   // <= 0
  if (!(z > -200.0)) return 0.0f;
  const double n = floor(z);
  return ldexpf(__builtin_amdgcn_exp2f((float)(z - n)), (int)n);
}
__device__ __forceinline__ float weight32(uint32_t key, float m, double c2) { return weightf(key2f(key), m, c2); }

// mass32_of(weightf(x, m, c2), s) in one step: the power of two of the fraction is read as a
// 24-bit significand and shifted once by the exponent's integer part, instead of being scaled
// into a float and taken apart again. Equal bit for bit: a normal weight has that significand
// and exponent; a weight the scaling would make subnormal or zero (exponent below -126) is
// shifted out to 0 here too, as s <= 63.
__device__ __forceinline__ uint64_t massf(float x, float m, double c2, int s) {
  const double z = ((double)x - (double)m) * c2;   // <= 0
  if (!(z > -200.0)) return 0ull;
  const double n = floor(z);
  const uint32_t b = __float_as_uint(__builtin_amdgcn_exp2f((float)(z - n)));   // in [1, 2]
  const uint64_t mant = (uint64_t)((b & 0x7FFFFFu) | 0x800000u);
  const int sh = (int)n + (int)(b >> 23) - 150 + s;
  const uint64_t up = mant << (sh & 63);
  const uint64_t dn = mant >> ((-sh) & 63);
  return sh >= 0 ? up : (sh > -24 ? dn : 0ull);
}

// Natural logarithm of a positive normal binary64 z, fp32-accurate (absolute error below
// 1e-7 for z >= 1): z = f * 2^e with f in [0.5, 1), log z = (e + log2 f) ln 2, log2 f from the
// hardware base-2 logarithm of fp32(f).
__device__ __forceinline__ double log_fast(double z) {
  int e;
  const double f = frexp(z, &e);
  return ((double)e + (double)__builtin_amdgcn_logf((float)f)) * 0.6931471805599453;
}

// ceil(p * Z) for p = fp32 in (0, 1) and a fixed-point total Z: with p = mant * 2^-psh
// (mant < 2^24, read from p's bits: the significand with its hidden bit, or a subnormal's
// bits over 2^149) the product is exact in 128 bits. Callers pass workgroup-uniform values;
// they are moved to scalar registers first, so the integer arithmetic runs once on the scalar
// unit instead of on every lane.
__device__ __forceinline__ uint64_t topp_target(float p, uint64_t z) {
  const uint32_t pb = (uint32_t)__builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, p));
  z = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(z >> 32)) << 32) |
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)z);
  const uint32_t e = (pb >> 23) & 0xFFu;                     // p in (0, 1): e < 127
  const uint64_t mant = e ? ((pb & 0x7FFFFFu) | 0x800000u) : (pb & 0x7FFFFFu);
  const int psh = e ? 150 - (int)e : 149;                   // > 24
  const unsigned __int128 prod = (unsigned __int128)mant * z;
  return psh >= 128 ? (prod != 0 ? 1ull : 0ull)
                    : (uint64_t)((prod + (((unsigned __int128)1 << psh) - 1)) >> psh);
}

__device__ __forceinline__ int bitlen(uint32_t n) { return n ? 32 - __clz((int)n) : 0; }

}  // namespace tsd
