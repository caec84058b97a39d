// Exact integer arithmetic of the K-mean step, usable on host and device.
//
// The mean removed from K (the outlier smoothing named in the SageAttention2
// title, GVCLab Video-Generation-101 systems survey, reference [3]) is taken
// here as the binary32 number nearest to the exact mean of the bf16 values.
// Every bf16 value is an integer multiple of 2^-133, so the exact sum is an
// integer in those units; it is held in a 192-bit two's-complement fixed-point
// accumulator and divided by N once, with round-to-nearest-even.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SQ_HD __host__ __device__ __forceinline__
#else
#define SQ_HD static inline
#endif

namespace sqattn {

// value = (w2:w1:w0 as signed 192-bit) * 2^-133
struct Acc192 {
  uint64_t w0, w1, w2;
};

// Units of the accumulator: 2^-133.  A bf16 value with biased exponent E and
// significand M (hidden bit included) is M * 2^(max(E,1) - 1) units.
constexpr int KMEAN_UNIT_EXP = -133;
// A head whose K holds |x| >= 2^33 (biased exponent >= 160, includes Inf/NaN)
// is outside the accumulator's range for N < 2^24.
constexpr uint32_t KMEAN_RANGE_EXP = 160;
// Fast window: values of 2^(W0)..2^(W0+40) units go to a 64-bit accumulator.
constexpr int KMEAN_W0 = 100;
constexpr int KMEAN_WBITS = 40;

SQ_HD void acc192_zero(Acc192& a) { a.w0 = a.w1 = a.w2 = 0; }

SQ_HD void acc192_add(Acc192& a, uint64_t b0, uint64_t b1, uint64_t b2) {
  uint64_t s0 = a.w0 + b0;
  uint64_t c0 = s0 < a.w0;
  uint64_t t1 = a.w1 + b1;
  uint64_t c1 = t1 < a.w1;
  uint64_t s1 = t1 + c0;
  c1 += s1 < t1;
  a.w0 = s0;
  a.w1 = s1;
  a.w2 = a.w2 + b2 + c1;
}

SQ_HD void acc192_add(Acc192& a, const Acc192& b) { acc192_add(a, b.w0, b.w1, b.w2); }

SQ_HD void acc192_neg(uint64_t& v0, uint64_t& v1, uint64_t& v2) {
  v0 = ~v0 + 1;
  uint64_t c = (v0 == 0);
  v1 = ~v1 + c;
  c = c & (v1 == 0);
  v2 = ~v2 + c;
}

// a += (neg ? -1 : 1) * m * 2^s, m < 2^32, 0 <= s < 160.
SQ_HD void acc192_add_shifted(Acc192& a, uint32_t m, int s, bool neg) {
  uint64_t mm = m, v0 = 0, v1 = 0, v2 = 0;
  if (s < 64) {
    v0 = mm << s;
    v1 = (s == 0) ? 0 : (mm >> (64 - s));
  } else if (s < 128) {
    int t = s - 64;
    v1 = mm << t;
    v2 = (t == 0) ? 0 : (mm >> (64 - t));
  } else {
    v2 = mm << (s - 128);
  }
  if (neg) acc192_neg(v0, v1, v2);
  acc192_add(a, v0, v1, v2);
}

// a += v * 2^s for a signed 64-bit v, 64 <= s < 128.
SQ_HD void acc192_add_i64_shl(Acc192& a, int64_t v, int s) {
  uint64_t u = (uint64_t)v;
  uint64_t sx = v < 0 ? ~(uint64_t)0 : 0;
  int t = s - 64;
  uint64_t v1 = (t == 0) ? u : (u << t);
  uint64_t v2 = (t == 0) ? sx : ((sx << t) | (u >> (64 - t)));
  acc192_add(a, 0, v1, v2);
}

// a += v * 2^s for an unsigned 64-bit v, 0 <= s < 192 (bits past 2^192 are lost).
SQ_HD void acc192_add_u64_shl(Acc192& a, uint64_t v, int s) {
  uint64_t w0 = 0, w1 = 0, w2 = 0;
  if (s < 64) {
    w0 = v << s;
    w1 = s ? v >> (64 - s) : 0;
  } else if (s < 128) {
    const int t = s - 64;
    w1 = v << t;
    w2 = t ? v >> (64 - t) : 0;
  } else {
    w2 = v << (s - 128);
  }
  acc192_add(a, w0, w1, w2);
}

SQ_HD bool acc192_is_zero(const Acc192& a) { return (a.w0 | a.w1 | a.w2) == 0; }

SQ_HD bool acc192_is_neg(const Acc192& a) { return (a.w2 >> 63) != 0; }

// Adds one bf16 value (16-bit pattern) to the window or the full accumulator.
// Returns true if the value is out of range (|x| >= 2^33, Inf or NaN).
// A value outside the fast window into the 192-bit accumulator; true if it is
// out of range (biased exponent >= KMEAN_RANGE_EXP: Inf, NaN, |x| >= 2^33).
SQ_HD bool kmean_add_outside(Acc192& acc, uint32_t b) {
  uint32_t E = (b >> 7) & 0xFFu;
  uint32_t M = (b & 0x7Fu) | (E ? 0x80u : 0u);
  int s = (int)(E ? E : 1u) - 1;
  if (E >= KMEAN_RANGE_EXP) return true;
  if (M) acc192_add_shifted(acc, M, s, (b & 0x8000u) != 0);
  return false;
}

SQ_HD bool kmean_accumulate(Acc192& acc, int64_t& win, uint32_t b) {
  uint32_t E = (b >> 7) & 0xFFu;
  uint32_t M = (b & 0x7Fu) | (E ? 0x80u : 0u);
  int s = (int)(E ? E : 1u) - 1;
  bool neg = (b & 0x8000u) != 0;
  int sh = s - KMEAN_W0;
  if ((unsigned)sh < (unsigned)KMEAN_WBITS) {
    int64_t v = (int64_t)((uint64_t)M << sh);
    win += neg ? -v : v;
    return false;
  }
  return kmean_add_outside(acc, b);
}

SQ_HD void kmean_flush_window(Acc192& acc, int64_t& win) {
  acc192_add_i64_shl(acc, win, KMEAN_W0);
  win = 0;
}

// The same window as a binary64 sum.  A bf16 value in the window (biased
// exponent W0 + 1 .. W0 + WBITS) is a multiple of 2^(W0 + UNIT_EXP) = 2^-33
// below 2^14 in magnitude, so a double that has added at most
// KMEAN_F64_ADDS of them holds their exact sum (below 2^20: a multiple of
// 2^-33 with at most 53 significant bits); each add is then exact.
constexpr int KMEAN_F64_ADDS = 64;
SQ_HD bool kmean_in_window(uint32_t b) {
  return ((b >> 7) & 0xFFu) - (uint32_t)(KMEAN_W0 + 1) < (uint32_t)KMEAN_WBITS;
}
// b as a double if it is in the window, else 0 (exact: a normal bf16 widened)
SQ_HD double kmean_window_value(uint32_t b) {
  const uint32_t u = kmean_in_window(b) ? (b << 16) : 0u;
  float f;
  __builtin_memcpy(&f, &u, 4);
  return (double)f;
}
// acc += win, win = 0.  win * 2^33 is an integer below 2^53: split into
// hi * 2^32 + lo with both parts converted exactly.
SQ_HD void kmean_flush_f64(Acc192& acc, double& win) {
  const double v = win * 0x1p33;
  const double hi = __builtin_floor(v * 0x1p-32);
  const double lo = v - hi * 0x1p32;  // in [0, 2^32)
  const int64_t iv = (int64_t)(int32_t)hi * 4294967296LL + (int64_t)(uint32_t)lo;
  acc192_add_i64_shl(acc, iv, KMEAN_W0);
  win = 0.0;
}

// 32-bit limb helpers for the final division (little-endian limbs).
SQ_HD uint32_t limb_bits(const uint32_t* q, int nlimb, int pos, int count) {
  // bits [pos, pos+count) of q, count <= 32, pos >= 0
  int li = pos >> 5, off = pos & 31;
  uint64_t lo = (li < nlimb) ? q[li] : 0;
  uint64_t hi = (li + 1 < nlimb) ? q[li + 1] : 0;
  uint64_t w = (lo | (hi << 32)) >> off;
  return (uint32_t)(w & ((count == 32) ? 0xFFFFFFFFull : ((1ull << count) - 1)));
}

SQ_HD bool limb_any_below(const uint32_t* q, int pos) {
  // any bit set in [0, pos)
  int li = pos >> 5, off = pos & 31;
  for (int i = 0; i < li; ++i)
    if (q[i]) return true;
  if (off && (q[li] & ((1u << off) - 1))) return true;
  return false;
}

// fl32(a * 2^unit_exp / N + tiny), nearest-even, N >= 1, where `sticky`
// says that a positive amount far below the result's last bit was left out
// of a (it can only break ties, upward).  Exact: the accumulator shifted left
// by 64 bits is divided by N in 32-bit limbs; the quotient has at least 41
// significant bits for any nonzero value, so its bits below the 24 kept ones,
// the remainder and `sticky` decide the rounding.  Overflows to +-inf.
SQ_HD float acc192_div_f32(Acc192 a, uint32_t N, int unit_exp, bool sticky_in) {
  bool neg = (a.w2 >> 63) != 0;
  if (neg) acc192_neg(a.w0, a.w1, a.w2);
  uint32_t x[8] = {0u, 0u, (uint32_t)a.w0, (uint32_t)(a.w0 >> 32), (uint32_t)a.w1,
                   (uint32_t)(a.w1 >> 32), (uint32_t)a.w2, (uint32_t)(a.w2 >> 32)};
  uint32_t q[8];
  uint64_t rem = 0;
  for (int i = 7; i >= 0; --i) {
    uint64_t cur = (rem << 32) | x[i];
    q[i] = (uint32_t)(cur / N);
    rem = cur % N;
  }
  int top = 7;
  while (top >= 0 && q[top] == 0) --top;
  if (top < 0) return 0.0f;  // exact zero (a positive sticky rest is below every binary32)
  int nb = 32 * top + (32 - __builtin_clz(q[top]));
  // value = (Q + rem/N) * 2^e
  const int e = unit_exp - 64;
  int lsb = e + nb - 24;
  if (lsb < -149) lsb = -149;
  int sh = lsb - e;  // >= 17
  uint32_t mant = limb_bits(q, 8, sh, 24 + 1);  // may need the 25th bit only if nb - sh == 25 (never)
  mant &= 0x1FFFFFFu;
  uint32_t rbit = limb_bits(q, 8, sh - 1, 1);
  bool sticky = (rem != 0) || limb_any_below(q, sh - 1) || sticky_in;
  if (rbit && (sticky || (mant & 1u))) mant += 1;
  uint32_t bits = mant + ((uint32_t)(lsb + 149) << 23);
  if (bits >= 0x7F800000u) bits = 0x7F800000u;  // past the largest binary32
  if (neg) bits |= 0x80000000u;
  union {
    uint32_t u;
    float f;
  } cvt;
  cvt.u = bits;
  return cvt.f;
}

// fl32(value(a) / N): the K mean (units 2^-133, nothing left out).
SQ_HD float acc192_mean_f32(Acc192 a, uint32_t N) { return acc192_div_f32(a, N, KMEAN_UNIT_EXP, false); }

}  // namespace sqattn
