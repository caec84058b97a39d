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

}  // namespace

void launch_rms_inverse(const uint16_t* x, int R, int C, float eps, float* inv_rms, hipStream_t st) {
  hipLaunchKernelGGL(rms_inv_kernel, dim3((R + 3) / 4), dim3(256), 0, st, x, R, C, R, 0LL, (long long)C, eps,
                     inv_rms);
}

void launch_rms_inverse_rows(const uint16_t* x, int B, int N, int C, long long sb, long long sn, float eps,
                             float* inv_rms, hipStream_t st) {
  const int R = B * N;
  hipLaunchKernelGGL(rms_inv_kernel, dim3((R + 3) / 4), dim3(256), 0, st, x, R, C, N, sb, sn, eps, inv_rms);
}

}  // namespace sqattn
