// RMSNorm statistics for gfx950 (MI355X): the normalization in front of the
// W8A8 projections of a DiT block, written as a custom kernel (digipub.cc
// TurboDiffusion article, paragraph on other optimizations: LayerNorm and
// RMSNorm reimplemented for speed).  Per row of bf16 x [R, C]:
//   mu2 = fl32(S / C), S = sum_k x_k^2 exactly (rounded once, nearest-even);
//   r   = fl32(1 / fl32(sqrt(fl32(mu2 + eps)))).
//
// A bf16 value with biased exponent E and significand M (hidden bit
// included) squares to M^2 * 2^e2 units of 2^-266, e2 = 2 max(E, 1) - 2, so
// S is an integer in those units, but one spanning up to 526 bits.
//
// One wave per row (4 rows per 256-thread work-group).  Pass 1 finds the
// row's largest exponent.  Pass 2 adds every square within 2^150 of the
// largest exactly into a 192-bit fixed-point accumulator (unit 2^u0, u0 =
// e2max - 150; squares within 2^40 of the top go through a 64-bit window);
// smaller squares only set a sticky bit.  The lanes' sums are combined
// exactly in-wave, and the kept sum A is divided by C once.
//
// A with the sticky bit rounds like S unless a binary32 rounding midpoint
// lies in (A/C, S/C].  Each left-out square is below 2^14 units and there are
// fewer than C of them, so S < A + C 2^14: if A/C and (A + C 2^14)/C (both
// with the sticky bit) round alike, that is the result, rounding being
// monotone.  Otherwise (a row spanning more than 2^75 in magnitude whose
// A/C lies within a tiny fraction of an ulp, below 2^-100 of one, under a
// midpoint m) the gap g = C m - A (< C 2^14 units) is settled level by level:
// the wave scans the row again for the squares of the next 150 bits down,
// whose exact sum is compared with g 2^150, leaving a smaller gap or a
// decision.  bf16 squares reach at most three levels below the first.
#include "common.h"
#include "exact.h"
#include "kernels.h"

namespace sqattn {

namespace {

constexpr int RMS_WINDOW = 150;            // bits of one level below its top
constexpr int RMS_FAST = RMS_WINDOW - 40;  // fast 64-bit window: shifts 110 .. 150
constexpr int RMS_DROP_BITS = 14;          // a left-out square is below 2^14 units of its level
constexpr int RMS_UNIT_EXP = -266;         // exponent of the units of e2

__device__ __forceinline__ void wave_sum(Acc192& acc, bool& sticky) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    Acc192 t;
    t.w0 = __shfl_xor(acc.w0, o, 64);
    t.w1 = __shfl_xor(acc.w1, o, 64);
    t.w2 = __shfl_xor(acc.w2, o, 64);
    acc192_add(acc, t);
    sticky |= __shfl_xor((int)sticky, o, 64) != 0;
  }
}

// Squares with u <= e2 < u + RMS_WINDOW, exactly, in units of 2^u; a nonzero
// smaller one sets `sticky`.  Wave-wide sums, in every lane.
__device__ void level_sum(const uint16_t* xr, int C, int lane, int u, Acc192& acc, bool& sticky) {
  acc192_zero(acc);
  sticky = false;
  for (int k = lane * 8; k < C; k += 512) {
    const v4i w = *(const v4i*)(xr + k);
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = ((uint32_t)w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      const uint32_t E = (b >> 7) & 0xFF;
      const uint32_t M = (b & 0x7F) | (E ? 0x80u : 0u);
      const int sh = 2 * (int)(E ? E : 1) - 2 - u;
      if (M == 0 || sh >= RMS_WINDOW) continue;
      if (sh < 0)
        sticky = true;
      else
        acc192_add_shifted(acc, M * M, sh, false);
    }
  }
  wave_sum(acc, sticky);
}

// The rounding of S / C when the first level left squares out: `lo` is the
// rounding of A / C (A = a0, units 2^u0) with the sticky bit.  Wave-uniform.
__device__ float settle_rounding(const uint16_t* xr, int C, int lane, const Acc192& a0, int u0, float lo) {
  const uint64_t D = (uint64_t)C << RMS_DROP_BITS;  // bound on the left-out part, units 2^u0
  Acc192 t = a0;
  acc192_add(t, D, 0, 0);
  const float hi = acc192_div_f32(t, (uint32_t)C, u0 + RMS_UNIT_EXP, true);
  const uint32_t lb = __float_as_uint(lo);
  if (__float_as_uint(hi) == lb) return lo;
  // hi is lo's successor; the midpoint between them is (2 m + 1) 2^(q - 1)
  // with m lo's integer significand and 2^q its last bit
  const uint32_t ef = (lb >> 23) & 0xFFu;
  const uint64_t m = (lb & 0x7FFFFFu) | (ef ? 0x800000u : 0u);
  const int q = (int)(ef ? ef : 1u) - 150;
  const int sh = q - 1 - (u0 + RMS_UNIT_EXP);  // the midpoint in units of 2^u0
  // here C m <= A + D < 2^191, and m >= A / C makes sh >= 0
  if (sh < 0 || sh > 191 - 45) return lo;  // not reached (see above)
  Acc192 g;  // g = C m - A: 0 < g <= D
  acc192_zero(g);
  acc192_add_u64_shl(g, (uint64_t)C * (2 * m + 1), sh);
  Acc192 na = a0;
  acc192_neg(na.w0, na.w1, na.w2);
  acc192_add(g, na);
  uint64_t gap = g.w0;
  // S = C m exactly iff the levels below add up to g; more is above the midpoint
  for (int u = u0 - RMS_WINDOW, lvl = 0; lvl < 4; u -= RMS_WINDOW, ++lvl) {
    Acc192 a;
    bool st;
    level_sum(xr, C, lane, u, a, st);
    Acc192 d;  // d = gap 2^150 - a, units 2^u
    d.w0 = 0;
    d.w1 = 0;
    d.w2 = gap << (RMS_WINDOW - 128);
    acc192_neg(a.w0, a.w1, a.w2);
    acc192_add(d, a);
    if (acc192_is_neg(d)) return __uint_as_float(lb + 1);
    if (acc192_is_zero(d)) return (st || (lb & 1u)) ? __uint_as_float(lb + 1) : lo;  // a tie: nearest-even
    if (!st || d.w2 != 0 || d.w1 != 0 || d.w0 >= D) return lo;  // what is left cannot reach d
    gap = d.w0;
  }
  return lo;  // not reached: below the third level no square is left out
}

__device__ __forceinline__ int chunk_emax(const v4i w) {
  int e = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = (uint32_t)w[j];
    e = max(e, max((int)((u >> 7) & 0xFF), (int)((u >> 23) & 0xFF)));
  }
  return e;
}

// The 8 squares of one 16-byte chunk: within 2^40 of the level's top into the
// 64-bit window `win` (each below 2^56), the rest of the level into `acc`,
// below it into the sticky bit.  Zero values add nothing.
__device__ __forceinline__ void chunk_add(const v4i w, int u0, Acc192& acc, uint64_t& win, bool& sticky) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t b = ((uint32_t)w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const uint32_t E = (b >> 7) & 0xFF;
    const uint32_t M = (b & 0x7F) | (E ? 0x80u : 0u);
    const int sh = 2 * (int)(E ? E : 1) - 2 - u0;
    if (sh >= RMS_FAST) {
      win += (uint64_t)(M * M) << (sh - RMS_FAST);
    } else if (M != 0) {
      if (sh < 0)
        sticky = true;
      else
        acc192_add_shifted(acc, M * M, sh, false);
    }
  }
}

// Two passes over the row (the second mostly from cache); the window is
// emptied into the full accumulator every 16 chunks (128 squares, so it
// stays below 2^63).  The pass is bound by the ~14 integer operations per
// square, not by memory: a variant that kept rows of up to 6144 columns in
// registers (one read) needed 170 VGPRs and ran slower.
// Row `row` (of R) starts at x + (row / rn) * sb + (row % rn) * sn.
__global__ __launch_bounds__(256) void rms_inv_kernel(const uint16_t* __restrict__ x, int R, int C, int rn,
                                                      long long sb, long long sn, float eps,
                                                      float* __restrict__ inv_rms) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;  // whole waves leave
  const uint16_t* xr = x + (long long)(row / rn) * sb + (long long)(row % rn) * sn;
  int emax = 0;
  for (int k = lane * 8; k < C; k += 512) emax = max(emax, chunk_emax(*(const v4i*)(xr + k)));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) emax = max(emax, __shfl_xor(emax, o, 64));
  const int u0 = 2 * max(emax, 1) - 2 - RMS_WINDOW;
  Acc192 acc;
  acc192_zero(acc);
  uint64_t win = 0;
  bool sticky = false;
  for (int k = lane * 8, it = 0; k < C; k += 512, ++it) {
    if ((it & 15) == 15) {
      acc192_add_i64_shl(acc, (int64_t)win, RMS_FAST);
      win = 0;
    }
    chunk_add(*(const v4i*)(xr + k), u0, acc, win, sticky);
  }
  acc192_add_i64_shl(acc, (int64_t)win, RMS_FAST);
  wave_sum(acc, sticky);
  float r;
  if (emax == 255) {
    r = __builtin_nanf("");  // Inf or NaN in the row
  } else {
    float mu2 = acc192_div_f32(acc, (uint32_t)C, u0 + RMS_UNIT_EXP, sticky);
    if (sticky) mu2 = settle_rounding(xr, C, lane, acc, u0, mu2);
    r = 1.0f / sqrtf(mu2 + eps);  // binary32, each operation correctly rounded
  }
  if (lane == 0) inv_rms[row] = r;
}

// ---------------------------------------------------------------------------
// LayerNorm statistics (the normalization in front of a DiT block's QKV
// projection; same passage).  Per row of bf16 x [R, C]:
//   mu  = fl32(S1 / C), S1 = sum_k x_k exactly (rounded once);
//   d_k = fl32(x_k - mu);
//   var = fl32(S2 / C), S2 = sum_k d_k^2 exactly (rounded once);
//   r   = fl32(1 / fl32(sqrt(fl32(var + eps)))).
//
// S1: a bf16 value is M * 2^s units of 2^-133 (s = max(E,1) - 1 <= 253,
// M < 2^8), so every row sum fits a 320-bit integer.  Positive and negative
// parts go to two unsigned 320-bit accumulators (the mean is their
// difference); values within 2^40 of the row's largest go through a signed
// 64-bit window first (emptied every 16 loads), smaller ones straight in.
//
// S2: a binary32 d = m 2^(max(E,1) - 150) (m < 2^24, hidden bit included)
// squares to m^2 2^e2 units of 2^-300, e2 = 2 max(E,1).  As for the RMS
// statistics, squares within 2^LN_WINDOW of the largest are summed exactly
// in 192 bits and smaller ones set a sticky bit; a left-out square is below
// 2^46 window units and there are fewer than C of them, so (A + C 2^46) / C
// brackets the result, and a rounding midpoint inside the bracket is settled
// level by level (120-bit levels keep the gap times 2^120 inside 192 bits).
// ---------------------------------------------------------------------------
constexpr int LN_S1_WIN = 40;        // fast window of the mean: 2^40 below the largest value
constexpr int LN_WINDOW = 120;       // bits of one level of the squares
constexpr int LN_DROP_BITS = 46;     // a left-out square is below 2^46 units of its level
constexpr int LN_SQ_UNIT = -300;     // exponent of the units of e2 (squares)
constexpr int LN_S1_UNIT = -133;     // exponent of the units of the sum
constexpr int LN_FAST = LN_WINDOW - 64;  // 128-bit fast window of the squares: shifts 56 .. 120

// a += (hi:lo) * 2^s, 0 <= s < 64, (hi:lo) < 2^120
__device__ __forceinline__ void acc192_add_u128_shl(Acc192& a, uint64_t lo, uint64_t hi, int s) {
  const uint64_t w0 = lo << s;
  const uint64_t w1 = s ? (hi << s) | (lo >> (64 - s)) : hi;
  const uint64_t w2 = s ? hi >> (64 - s) : 0;
  acc192_add(a, w0, w1, w2);
}

struct U320 {
  uint64_t w0, w1, w2, w3, w4;
};

__device__ __forceinline__ void u320_add(U320& a, uint64_t b0, uint64_t b1, uint64_t b2, uint64_t b3, uint64_t b4) {
  uint64_t s, c;
  s = a.w0 + b0; c = s < b0; a.w0 = s;
  s = a.w1 + c; c = s < c; s += b1; c += s < b1; a.w1 = s;
  s = a.w2 + c; c = s < c; s += b2; c += s < b2; a.w2 = s;
  s = a.w3 + c; c = s < c; s += b3; c += s < b3; a.w3 = s;
  a.w4 = a.w4 + c + b4;
}

// a += v * 2^sh, v < 2^63, 0 <= sh < 256 (word index from the shift, no
// indexed registers)
__device__ __forceinline__ void u320_add_shl(U320& a, uint64_t v, int sh) {
  const int wi = sh >> 6, off = sh & 63;
  const uint64_t lo = v << off, hi = off ? v >> (64 - off) : 0;
  u320_add(a, wi == 0 ? lo : 0, wi == 1 ? lo : (wi == 0 ? hi : 0), wi == 2 ? lo : (wi == 1 ? hi : 0),
           wi == 3 ? lo : (wi == 2 ? hi : 0), wi == 3 ? hi : 0);
}

__device__ __forceinline__ void u320_wave_sum(U320& a) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1)
    u320_add(a, __shfl_xor(a.w0, o, 64), __shfl_xor(a.w1, o, 64), __shfl_xor(a.w2, o, 64),
             __shfl_xor(a.w3, o, 64), __shfl_xor(a.w4, o, 64));
}

// fl32((p - n) * 2^unit_exp / N), nearest-even, exact (p, n < 2^319).  The
// difference's magnitude, shifted left by 64 bits, is divided by N in 32-bit
// limbs; the quotient keeps at least 41 significant bits below a nonzero
// result's leading one, and its lower bits and the remainder decide the
// rounding.
__device__ float u320_diff_div_f32(U320 p, U320 n, uint32_t N, int unit_exp) {
  // d = p - n (two's complement)
  U320 d = p;
  u320_add(d, ~n.w0, ~n.w1, ~n.w2, ~n.w3, ~n.w4);
  u320_add(d, 1, 0, 0, 0, 0);
  const bool neg = (d.w4 >> 63) != 0;
  if (neg) {
    U320 z = {~d.w0, ~d.w1, ~d.w2, ~d.w3, ~d.w4};
    u320_add(z, 1, 0, 0, 0, 0);
    d = z;
  }
  uint32_t x[12] = {0u, 0u, (uint32_t)d.w0, (uint32_t)(d.w0 >> 32), (uint32_t)d.w1, (uint32_t)(d.w1 >> 32),
                    (uint32_t)d.w2, (uint32_t)(d.w2 >> 32), (uint32_t)d.w3, (uint32_t)(d.w3 >> 32),
                    (uint32_t)d.w4, (uint32_t)(d.w4 >> 32)};
  uint32_t q[12];
  uint64_t rem = 0;
#pragma unroll
  for (int i = 11; i >= 0; --i) {
    const uint64_t cur = (rem << 32) | x[i];
    q[i] = (uint32_t)(cur / N);
    rem = cur % N;
  }
  int top = 11;
  while (top >= 0 && q[top] == 0) --top;
  if (top < 0) return 0.0f;
  const int nb = 32 * top + (32 - __builtin_clz(q[top]));
  const int e = unit_exp - 64;
  int lsb = e + nb - 24;
  if (lsb < -149) lsb = -149;
  const int sh = lsb - e;  // >= 17
  uint32_t mant = limb_bits(q, 12, sh, 25) & 0x1FFFFFFu;
  const uint32_t rbit = limb_bits(q, 12, sh - 1, 1);
  const bool sticky = (rem != 0) || limb_any_below(q, sh - 1);
  if (rbit && (sticky || (mant & 1u))) mant += 1;
  uint32_t bits = mant + ((uint32_t)(lsb + 149) << 23);
  if (bits >= 0x7F800000u) bits = 0x7F800000u;
  if (neg) bits |= 0x80000000u;
  return __uint_as_float(bits);
}

// square of the binary32 d as (m^2, e2): d = m 2^(max(E,1) - 150)
__device__ __forceinline__ void f32_square(float dv, uint64_t& m2, int& e2) {
  const uint32_t u = __float_as_uint(dv);
  const uint32_t E = (u >> 23) & 0xFF;
  const uint64_t m = (u & 0x7FFFFFu) | (E ? 0x800000u : 0u);
  m2 = m * m;
  e2 = 2 * (int)(E ? E : 1u);
}

// level u of the squares of d_k = fl32(x_k - mu): those with u <= e2 < u +
// LN_WINDOW exactly (units 2^u), smaller nonzero ones into `sticky`
__device__ void ln_level_sum(const uint16_t* xr, int C, int lane, float mu, int u, Acc192& acc, bool& sticky) {
  acc192_zero(acc);
  sticky = false;
  for (int k = lane * 8; k < C; k += 512) {
    const v4i w = *(const v4i*)(xr + k);
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = ((uint32_t)w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      uint64_t m2;
      int e2;
      f32_square(__uint_as_float(b << 16) - mu, m2, e2);
      const int sh = e2 - u;
      if (m2 == 0 || sh >= LN_WINDOW) continue;
      if (sh < 0)
        sticky = true;
      else
        acc192_add_u64_shl(acc, m2, sh);
    }
  }
  wave_sum(acc, sticky);
}

__device__ __forceinline__ bool acc192_ge_u128(const Acc192& a, uint64_t lo, uint64_t hi) {
  if (a.w2 != 0) return true;
  if (a.w1 != hi) return a.w1 > hi;
  return a.w0 >= lo;
}

// the rounding of S2 / C when squares were left out: `lo` rounds A / C (A = a0,
// units 2^u0) with the sticky bit; as settle_rounding with a 128-bit bound
__device__ float ln_settle(const uint16_t* xr, int C, int lane, float mu, const Acc192& a0, int u0, float lo) {
  const uint64_t Dlo = (uint64_t)C << LN_DROP_BITS, Dhi = (uint64_t)C >> (64 - LN_DROP_BITS);
  Acc192 t = a0;
  acc192_add(t, Dlo, Dhi, 0);
  const float hi = acc192_div_f32(t, (uint32_t)C, u0 + LN_SQ_UNIT, true);
  const uint32_t lb = __float_as_uint(lo);
  if (__float_as_uint(hi) == lb) return lo;
  const uint32_t ef = (lb >> 23) & 0xFFu;
  const uint64_t m = (lb & 0x7FFFFFu) | (ef ? 0x800000u : 0u);
  const int q = (int)(ef ? ef : 1u) - 150;
  const int sh = q - 1 - (u0 + LN_SQ_UNIT);  // the midpoint in units of 2^u0
  if (sh < 0 || sh > 191 - 45) return lo;   // not reached: C m <= A + D < 2^191 and m >= A / C
  Acc192 g;  // gap = C m - A, 0 < gap <= D < 2^67
  acc192_zero(g);
  acc192_add_u64_shl(g, (uint64_t)C * (2 * m + 1), sh);
  Acc192 na = a0;
  acc192_neg(na.w0, na.w1, na.w2);
  acc192_add(g, na);
  uint64_t glo = g.w0, ghi = g.w1;
  for (int u = u0 - LN_WINDOW, lvl = 0; lvl < 6; u -= LN_WINDOW, ++lvl) {
    Acc192 a;
    bool st;
    ln_level_sum(xr, C, lane, mu, u, a, st);
    Acc192 d;  // d = gap 2^120 - a, units 2^u
    d.w0 = 0;
    d.w1 = glo << (LN_WINDOW - 64);
    d.w2 = (glo >> (128 - LN_WINDOW)) | (ghi << (LN_WINDOW - 64));
    acc192_neg(a.w0, a.w1, a.w2);
    acc192_add(d, a);
    if (acc192_is_neg(d)) return __uint_as_float(lb + 1);
    if (acc192_is_zero(d)) return (st || (lb & 1u)) ? __uint_as_float(lb + 1) : lo;
    if (!st || acc192_ge_u128(d, Dlo, Dhi)) return lo;
    glo = d.w0;
    ghi = d.w1;
  }
  return lo;  // not reached: below the fifth level no square is left out
}

// One wave per row (4 rows per work-group): pass 1 the exact sum (and the
// row's extreme values), pass 2 the squares of the binary32 differences.
__global__ __launch_bounds__(256) void ln_stats_kernel(const uint16_t* __restrict__ x, int R, int C, float eps,
                                                       float* __restrict__ mean, float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;  // whole waves leave
  const uint16_t* xr = x + (long long)row * C;
  int emax = 0;
  float vmax = -__builtin_inff(), vmin = __builtin_inff();
  for (int k = lane * 8; k < C; k += 512) {
    const v4i w = *(const v4i*)(xr + k);
    emax = max(emax, chunk_emax(w));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = __uint_as_float((((uint32_t)w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu) << 16);
      vmax = fmaxf(vmax, v);
      vmin = fminf(vmin, v);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    emax = max(emax, __shfl_xor(emax, o, 64));
    vmax = fmaxf(vmax, __shfl_xor(vmax, o, 64));
    vmin = fminf(vmin, __shfl_xor(vmin, o, 64));
  }
  if (emax == 255) {  // Inf or NaN in the row
    if (lane == 0) {
      mean[row] = __builtin_nanf("");
      rstd[row] = __builtin_nanf("");
    }
    return;
  }
  // ---- S1: values M 2^s (units 2^-133), window [w0, w0 + 40)
  const int w0 = max(max(emax, 1) - 1 - (LN_S1_WIN - 1), 0);
  U320 pos = {0, 0, 0, 0, 0}, negs = {0, 0, 0, 0, 0};
  int64_t win = 0;
  for (int k = lane * 8, it = 0; k < C; k += 512, ++it) {
    if ((it & 15) == 15) {
      if (win >= 0) u320_add_shl(pos, (uint64_t)win, w0); else u320_add_shl(negs, (uint64_t)(-win), w0);
      win = 0;
    }
    const v4i w = *(const v4i*)(xr + k);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = ((uint32_t)w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      const uint32_t E = (b >> 7) & 0xFF;
      const int64_t M = (int64_t)((b & 0x7F) | (E ? 0x80u : 0u));
      const int sh = (int)(E ? E : 1u) - 1 - w0;
      if (sh >= 0) {
        const int64_t v = M << sh;  // < 2^48
        win += (b & 0x8000u) ? -v : v;
      } else if (M != 0) {
        if (b & 0x8000u) u320_add_shl(negs, (uint64_t)M, sh + w0); else u320_add_shl(pos, (uint64_t)M, sh + w0);
      }
    }
  }
  if (win >= 0) u320_add_shl(pos, (uint64_t)win, w0); else u320_add_shl(negs, (uint64_t)(-win), w0);
  u320_wave_sum(pos);
  u320_wave_sum(negs);
  const float mu = u320_diff_div_f32(pos, negs, (uint32_t)C, LN_S1_UNIT);
  // ---- S2: squares of d = fl32(x - mu); the largest |d| is at the extremes
  uint64_t mm;
  int e2max, e2b;
  f32_square(vmax - mu, mm, e2max);
  f32_square(vmin - mu, mm, e2b);
  e2max = max(e2max, e2b);
  const int u0 = e2max - LN_WINDOW;
  Acc192 acc;
  acc192_zero(acc);
  bool sticky = false;
  // squares within 2^64 of the level's top (shifts LN_FAST .. LN_WINDOW) go
  // to a 128-bit window (each below 2^112; emptied every 16 loads, 128
  // squares, so it stays below 2^119), the rest of the level to the full
  // accumulator, smaller ones to the sticky bit
  uint64_t wlo = 0, whi = 0;
  for (int k = lane * 8, it = 0; k < C; k += 512, ++it) {
    if ((it & 15) == 15) {
      acc192_add_u128_shl(acc, wlo, whi, LN_FAST);
      wlo = whi = 0;
    }
    const v4i w = *(const v4i*)(xr + k);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = ((uint32_t)w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      uint64_t m2;
      int e2;
      f32_square(__uint_as_float(b << 16) - mu, m2, e2);
      const int sh = e2 - u0;
      if (sh >= LN_FAST) {
        const int t = sh - LN_FAST;  // 0 .. 64
        const uint64_t lo = t < 64 ? m2 << t : 0, hi = t ? m2 >> (64 - t) : 0;
        wlo += lo;
        whi += hi + (wlo < lo);
      } else if (m2 != 0) {
        if (sh < 0)
          sticky = true;
        else
          acc192_add_u64_shl(acc, m2, sh);
      }
    }
  }
  acc192_add_u128_shl(acc, wlo, whi, LN_FAST);
  wave_sum(acc, sticky);
  float var = acc192_div_f32(acc, (uint32_t)C, u0 + LN_SQ_UNIT, sticky);
  if (sticky) var = ln_settle(xr, C, lane, mu, acc, u0, var);
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = 1.0f / sqrtf(var + eps);  // binary32, each operation correctly rounded
  }
}

}  // namespace

void launch_rms_inverse(const uint16_t* x, int R, int C, float eps, float* inv_rms, hipStream_t st) {
  hipLaunchKernelGGL(rms_inv_kernel, dim3((R + 3) / 4), dim3(256), 0, st, x, R, C, R, 0LL, (long long)C, eps,
                     inv_rms);
}

void launch_layernorm_stats(const uint16_t* x, int R, int C, float eps, float* mean, float* rstd, hipStream_t st) {
  hipLaunchKernelGGL(ln_stats_kernel, dim3((R + 3) / 4), dim3(256), 0, st, x, R, C, eps, mean, rstd);
}

void launch_rms_inverse_rows(const uint16_t* x, int B, int N, int C, long long sb, long long sn, float eps,
                             float* inv_rms, hipStream_t st) {
  const int R = B * N;
  hipLaunchKernelGGL(rms_inv_kernel, dim3((R + 3) / 4), dim3(256), 0, st, x, R, C, N, sb, sn, eps, inv_rms);
}

}  // namespace sqattn
