// Quantization kernels of the sqattn path (gfx950).
//
//   kmean_partial / kmean_finalize : exact per-channel K mean (192-bit fixed
//       point, one rounding), the smoothing step named in the SageAttention2
//       title (GVCLab Video-Generation-101 systems survey, reference [3]).
//   quant_i8 : per-block INT8 codes of Q and of the smoothed K (jefxiong.cn
//       "AIGC weekend special 5.10", section 1.2 item (1): Q/K to low bit so
//       QK^T runs on integer matrix units).  s = fl32(absmax/127),
//       code = clamp(rne(fl32(x/s)), -127, 127).
//   v_tiles_bf16 : V into the attention kernel's tile layout ([d][64 keys]).
//   quant_v_fp8 : per-64-row E4M3 codes of V (GVCLab research log 2026-09-02,
//       section 5.5 table: FP8 P.V), s_v the smallest power of two with
//       absmax <= 448 s_v.
//
// All kernels are HBM-bound streaming passes; loads and stores are 16-byte
// per lane along rows so that each wave touches whole 128-byte lines.
#include "common.h"
#include "e4m3.h"
#include "exact.h"
#include "kernels.h"

namespace sqattn {

// ---------------------------------------------------------------------------
// RMSNorm on load (RowNorm): the q/k normalization over each token's H*d
// features (digipub.cc TurboDiffusion article, paragraph on other
// optimizations), applied to 16-byte chunks of eight bf16 values of one row
// as they are read, with the per-token factor r computed beforehand
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t bf16_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;  // NaN: a quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;                             // nearest even (Inf stays)
}
// bf16(fl32(fl32(x * r) * g)) for the eight values of w (g = 1 without a weight: exact)
__device__ __forceinline__ v4i norm_chunk(v4i w, float r, const float (&g)[8]) {
  v4i o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = (uint32_t)w[j];
    const uint32_t lo = bf16_rne((bf16_bits_to_f32(u & 0xFFFFu) * r) * g[2 * j]);
    const uint32_t hi = bf16_rne((bf16_bits_to_f32(u >> 16) * r) * g[2 * j + 1]);
    o[j] = (int)(lo | (hi << 16));
  }
  return o;
}
// the weights of channels c0 .. c0+7 of head bh % H
__device__ __forceinline__ void norm_weights(const RowNorm& nm, long long bh, int H, int D, int c0, float (&g)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) g[j] = nm.gamma ? nm.gamma[(bh % H) * D + c0 + j] : 1.0f;
}

// ---------------------------------------------------------------------------
// exact K mean
// ---------------------------------------------------------------------------

// grid (S, B*H), 256 threads.  Chunk c of a head covers rows
// [c*rows_per_chunk, min(N, (c+1)*rows_per_chunk)).  Thread t reads channels
// (t % CPR)*8 .. +8 (CPR = D/8 16-byte pieces per row) of rows
// r0 + t/CPR + j*RPP (RPP = 256/CPR rows per pass).
template <int D, bool NORM>
__global__ __launch_bounds__(256) void kmean_partial_kernel(const uint16_t* __restrict__ k, Lay lk, int N,
                                                            int rows_per_chunk,
                                                            uint64_t* __restrict__ partial, RowNorm nm) {
  constexpr int CPR = D / 8;
  constexpr int RPP = 256 / CPR;
  const int chunk = blockIdx.x, S = gridDim.x;
  const long long bh = blockIdx.y;
  const int t = threadIdx.x;
  const int cg = t % CPR, rg = t / CPR;
  const uint16_t* kh = k + lay_row(lk, bh, 0);
  int r0 = chunk * rows_per_chunk;
  int r1 = min(N, r0 + rows_per_chunk);

  Acc192 acc[8];
  double win[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc192_zero(acc[j]);
    win[j] = 0.0;
  }
  bool bad = false;
  float gw[8];
  if constexpr (NORM) norm_weights(nm, bh, lk.H, D, cg * 8, gw);
  const float* rr = NORM ? nm.r + (bh / lk.H) * N : nullptr;
  // values in the fast window add into the doubles (exact for up to
  // KMEAN_F64_ADDS rows, then flushed); a chunk holding any other value
  // sends those into the 192-bit accumulators
  // Rows are loaded KB at a time before any is added, so that the loads are
  // in flight together; rows past the group's end read as zeros, which add
  // nothing (a zero is exact in the window and outside it alike).
  constexpr int KB = 4;
  static_assert(KMEAN_F64_ADDS % KB == 0, "whole batches per window");
  for (int rb = r0 + rg; rb < r1; rb += KMEAN_F64_ADDS * RPP) {
    const int re = min(r1, rb + KMEAN_F64_ADDS * RPP);
    for (int r = rb; r < re; r += KB * RPP) {
      v4i w[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int ru = r + u * RPP;
        w[u] = ru < re ? *(const v4i*)(kh + (long long)ru * lk.sn + cg * 8) : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        if constexpr (NORM) {
          const int ru = r + u * RPP;
          if (ru < re) w[u] = norm_chunk(w[u], rr[ru], gw);
        }
        bool inside = true;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t b = ((uint32_t)w[u][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          inside &= kmean_in_window(b) || (b & 0x7FFFu) == 0;
          win[j] += kmean_window_value(b);
        }
        if (!inside) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t b = ((uint32_t)w[u][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            if (!kmean_in_window(b)) bad |= kmean_add_outside(acc[j], b);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) kmean_flush_f64(acc[j], win[j]);
  }

  // reduce the RPP row groups of each channel: the 64 / CPR groups of a wave
  // by lane exchanges, then the 4 waves through LDS
  const int lane = t & 63, wave = t >> 6;
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint64_t v[3] = {acc[j].w0, acc[j].w1, acc[j].w2};
      uint64_t x[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const uint32_t lo = __shfl_xor((uint32_t)v[i], o, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(v[i] >> 32), o, 64);
        x[i] = ((uint64_t)hi << 32) | lo;
      }
      acc192_add(acc[j], x[0], x[1], x[2]);
    }
  }
  __shared__ Acc192 red[4][D];
  __shared__ int redbad[4];
  const bool wbad = __any(bad);
  if (lane < CPR) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wave][cg * 8 + j] = acc[j];
  }
  if (lane == 0) redbad[wave] = wbad ? 1 : 0;
  __syncthreads();
  if (t < D) {
    Acc192 s = red[0][t];
    for (int g = 1; g < 4; ++g) acc192_add(s, red[g][t]);
    const int anybad = redbad[0] | redbad[1] | redbad[2] | redbad[3];
    uint64_t* p = partial + ((bh * S + chunk) * D + t) * 4;
    p[0] = s.w0;
    p[1] = s.w1;
    p[2] = s.w2;
    p[3] = (uint64_t)anybad;
  }
}

// grid (B*H), D threads: sums the S partials of a channel and rounds the mean.
template <int D>
__global__ __launch_bounds__(D) void kmean_finalize_kernel(const uint64_t* __restrict__ partial,
                                                           int S, int N, float* __restrict__ mean) {
  const long long bh = blockIdx.x;
  const int c = threadIdx.x;
  Acc192 s;
  acc192_zero(s);
  uint64_t bad = 0;
  for (int i = 0; i < S; ++i) {
    const uint64_t* p = partial + ((bh * S + i) * D + c) * 4;
    acc192_add(s, p[0], p[1], p[2]);
    bad |= p[3];
  }
  mean[bh * D + c] = bad ? __builtin_nanf("") : acc192_mean_f32(s, (uint32_t)N);
}

// grid (nq, B*H), D threads: the mean of each Q block from its partial sum
// (the partial pass run with one chunk per block): mu = fl32(sum / rows),
// rounded once; NaN where a value fell outside the exact range.
template <int D>
__global__ __launch_bounds__(D) void qmean_finalize_kernel(const uint64_t* __restrict__ partial, int N,
                                                           int block, float* __restrict__ mean) {
  const long long bh = blockIdx.y;
  const int b = blockIdx.x, nq = gridDim.x, c = threadIdx.x;
  const uint64_t* p = partial + ((bh * nq + b) * D + c) * 4;
  Acc192 s;
  acc192_zero(s);
  acc192_add(s, p[0], p[1], p[2]);
  const int rows = min(N, (b + 1) * block) - b * block;
  mean[(bh * nq + b) * D + c] = p[3] ? __builtin_nanf("") : acc192_mean_f32(s, (uint32_t)rows);
}

// ---------------------------------------------------------------------------
// per-block INT8 quantization
// ---------------------------------------------------------------------------

__device__ __forceinline__ float block_max_256(float v, float* sh) {
  // max over the 256 threads of the work-group (all values >= 0 or NaN-free)
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

// grid (nblocks, B*H), 256 threads.  One work-group per block of `block` rows.
// mean == nullptr: plain Q.  Otherwise x = fl32(X - mean[c]) (IEEE subtract),
// with one mean per head (K, mean_blocks = 0) or per block (Q smoothing,
// mean_blocks = 1).  Q smoothing keeps a block's mean when the smoothed
// block's scale s > 0 and the mean is finite (a NaN mean comes from values
// outside the exact range); otherwise the block is quantized plainly and its
// mean row is set to 0.
// Blocks of at most QCACHE * RPP rows (128 at D = 128, 256 at D = 64) are
// read once and kept in registers between the absmax and the coding pass;
// larger blocks are read twice.
constexpr int QCACHE = 8;
template <int D, bool NORM>
__global__ __launch_bounds__(256) void quant_i8_kernel(const uint16_t* __restrict__ x, Lay lx, int N, int block,
                                                       float* __restrict__ mean, int mean_blocks,
                                                       int8_t* __restrict__ codes,
                                                       float* __restrict__ scales, RowNorm nm) {
  constexpr int CPR = D / 8;
  constexpr int RPP = 256 / CPR;
  __shared__ float sh[4];
  const long long bh = blockIdx.y;
  const int blk = blockIdx.x, nblk = gridDim.x;
  const int t = threadIdx.x, cg = t % CPR, rg = t / CPR;
  const uint16_t* xh = x + lay_row(lx, bh, 0);
  int8_t* ch = codes + bh * (long long)N * D;
  const int r0 = blk * block, r1 = min(N, r0 + block);

  float* mrow = mean ? mean + (mean_blocks ? (bh * nblk + blk) * D : bh * D) : nullptr;
  bool use_mean = mean != nullptr;  // uniform
  float mu[8];
  bool mean_nan = false;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mu[j] = mrow ? mrow[cg * 8 + j] : 0.0f;
    mean_nan |= (mu[j] != mu[j]) && !mean_blocks;
  }

  float gw[8];
  if constexpr (NORM) norm_weights(nm, bh, lx.H, D, cg * 8, gw);
  const float* rr = NORM ? nm.r + (bh / lx.H) * N : nullptr;
  auto chunk_max = [&](v4i w, float m) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t u = (uint32_t)w[j];
      float a = bf16_bits_to_f32(u & 0xFFFFu), b = bf16_bits_to_f32(u >> 16);
      if (use_mean) {
        a = a - mu[2 * j];
        b = b - mu[2 * j + 1];
      }
      m = fmaxf(m, fmaxf(fabsf(a), fabsf(b)));
    }
    return m;
  };
  const bool resident = r1 - r0 <= QCACHE * RPP;  // uniform over the work-group
  v4i cache[QCACHE];
  float amax = 0.0f;
  if (resident) {
#pragma unroll
    for (int i = 0; i < QCACHE; ++i) {
      const int r = r0 + rg + i * RPP;
      cache[i] = r < r1 ? *(const v4i*)(xh + (long long)r * lx.sn + cg * 8) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < QCACHE; ++i) {
      const int r = r0 + rg + i * RPP;
      if (r < r1) {
        if constexpr (NORM) cache[i] = norm_chunk(cache[i], rr[r], gw);
        amax = chunk_max(cache[i], amax);
      }
    }
  } else {
#pragma unroll 4
    for (int r = r0 + rg; r < r1; r += RPP) {
      v4i w = *(const v4i*)(xh + (long long)r * lx.sn + cg * 8);
      if constexpr (NORM) w = norm_chunk(w, rr[r], gw);
      amax = chunk_max(w, amax);
    }
  }
  // a NaN mean (K out of range) poisons the whole block's scale
  float nanflag = block_max_256(mean_nan ? 1.0f : 0.0f, sh);
  amax = block_max_256(amax, sh);
  float s = amax / 127.0f;  // correctly rounded binary32 division
  if (mean_blocks) {
    bool fin = true;
#pragma unroll
    for (int j = 0; j < 8; ++j) fin &= isfinite(mu[j]);
    const bool keep = (s > 0.0f) && __syncthreads_and(fin);  // uniform
    if (!keep) {  // uniform: quantize the block plainly, its mean row 0
      use_mean = false;
      amax = 0.0f;
      if (resident) {
#pragma unroll
        for (int i = 0; i < QCACHE; ++i)
          if (r0 + rg + i * RPP < r1) amax = chunk_max(cache[i], amax);
      } else {
        for (int r = r0 + rg; r < r1; r += RPP) {
          v4i w = *(const v4i*)(xh + (long long)r * lx.sn + cg * 8);
          if constexpr (NORM) w = norm_chunk(w, rr[r], gw);
          amax = chunk_max(w, amax);
        }
      }
      amax = block_max_256(amax, sh);
      s = amax / 127.0f;
      if (t < D) mrow[t] = 0.0f;
    }
  }
  if (t == 0) scales[bh * nblk + blk] = (nanflag > 0.0f) ? __builtin_nanf("") : s;
  const bool zero = !(s > 0.0f) || (nanflag > 0.0f);
  const bool fast = s >= 0x1p-125f;  // 1/s finite
  const float y = 1.0f / s;          // correctly rounded

  auto code_chunk = [&](v4i w, int r) {
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t u = (uint32_t)w[j >> 1];
      float a = bf16_bits_to_f32((j & 1) ? (u >> 16) : (u & 0xFFFFu));
      if (use_mean) a = a - mu[j];
      int c = 0;
      if (!zero) {
        float qv = fast ? rne_quotient(a, s, y) : rintf(a / s);  // rne of the correctly rounded quotient
        qv = fminf(fmaxf(qv, -127.0f), 127.0f);
        c = (int)qv;
      }
      packed[j >> 2] |= ((uint32_t)(c & 0xFF)) << ((j & 3) * 8);
    }
    *(uint2*)(ch + (long long)r * D + cg * 8) = make_uint2(packed[0], packed[1]);
  };
  if (resident) {
#pragma unroll
    for (int i = 0; i < QCACHE; ++i) {
      const int r = r0 + rg + i * RPP;
      if (r < r1) code_chunk(cache[i], r);
    }
  } else {
#pragma unroll 2
    for (int r = r0 + rg; r < r1; r += RPP) {
      v4i w = *(const v4i*)(xh + (long long)r * lx.sn + cg * 8);
      if constexpr (NORM) w = norm_chunk(w, rr[r], gw);
      code_chunk(w, r);
    }
  }
}

// grid (ceil(N / RPW), B*H), 256 threads: one scale per row (block = 1, the
// per-lane granularity of the attention kernel's Q operand: each lane holds
// one query row).  CPR threads own a row (8 channels each), RPW rows per
// work-group; the row's absmax is reduced over its CPR lanes, which lie in
// one wave.  Same rule: s = fl32(absmax/127), code = clamp(rne(fl32(x/s))).
template <int D, bool NORM>
__global__ __launch_bounds__(256) void quant_i8_rows_kernel(const uint16_t* __restrict__ x, Lay lx, int N,
                                                            int8_t* __restrict__ codes,
                                                            float* __restrict__ scales, RowNorm nm) {
  constexpr int CPR = D / 8;
  constexpr int RPW = 256 / CPR;
  const long long bh = blockIdx.y;
  const int t = threadIdx.x, cg = t % CPR;
  const int r = blockIdx.x * RPW + t / CPR;
  const bool ok = r < N;
  const long long base = (bh * N + (ok ? r : 0)) * D + cg * 8;
  v4i w = ok ? *(const v4i*)(x + lay_row(lx, bh, r) + cg * 8) : v4i{0, 0, 0, 0};
  if constexpr (NORM) {
    float gw[8];
    norm_weights(nm, bh, lx.H, D, cg * 8, gw);
    if (ok) w = norm_chunk(w, nm.r[(bh / lx.H) * N + r], gw);
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = (uint32_t)w[j];
    amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(u & 0xFFFFu)), fabsf(bf16_bits_to_f32(u >> 16))));
  }
#pragma unroll
  for (int o = CPR / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float s = amax / 127.0f;  // correctly rounded binary32 division
  if (!ok) return;
  if (cg == 0) scales[bh * N + r] = s;
  const bool zero = !(s > 0.0f);
  const bool fast = s >= 0x1p-125f;  // 1/s finite
  const float y = 1.0f / s;          // correctly rounded
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t u = (uint32_t)w[j >> 1];
    const float a = bf16_bits_to_f32((j & 1) ? (u >> 16) : (u & 0xFFFFu));
    int c = 0;
    if (!zero) c = (int)fminf(fmaxf(fast ? rne_quotient(a, s, y) : rintf(a / s), -127.0f), 127.0f);
    packed[j >> 2] |= ((uint32_t)(c & 0xFF)) << ((j & 3) * 8);
  }
  *(uint2*)(codes + base) = make_uint2(packed[0], packed[1]);
}

// ---------------------------------------------------------------------------
// V layouts for the attention kernel
// ---------------------------------------------------------------------------

// grid (nt, B*H), 256 threads: V bf16 [N][D] -> Vt [nt][D][64] bf16 (tile t,
// channel c, key j) with zeros for keys >= N.
template <int D>
__global__ __launch_bounds__(256) void v_tiles_bf16_kernel(const uint16_t* __restrict__ v, Lay lv, int N,
                                                           uint16_t* __restrict__ vt) {
  __shared__ uint16_t tile[KT][D + 8];
  const long long bh = blockIdx.y;
  const int tt = blockIdx.x, nt = gridDim.x;
  const int t = threadIdx.x;
  const uint16_t* vh = v + lay_row(lv, bh, 0);
  constexpr int CPR = D / 8;
  for (int i = t; i < KT * CPR; i += 256) {
    int r = i / CPR, c8 = (i % CPR) * 8;
    int key = tt * KT + r;
    v4i w = (key < N) ? *(const v4i*)(vh + (long long)key * lv.sn + c8) : v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[r][c8 + 2 * j] = (uint16_t)((uint32_t)w[j] & 0xFFFFu);
      tile[r][c8 + 2 * j + 1] = (uint16_t)((uint32_t)w[j] >> 16);
    }
  }
  __syncthreads();
  uint16_t* out = vt + (bh * nt + tt) * (long long)D * KT;
  for (int i = t; i < D * (KT / 8); i += 256) {
    int c = i / (KT / 8), k8 = (i % (KT / 8)) * 8;
    uint32_t p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      p[j] = (uint32_t)tile[k8 + 2 * j][c] | ((uint32_t)tile[k8 + 2 * j + 1][c] << 16);
    *(v4i*)(out + (long long)c * KT + k8) = v4i{(int)p[0], (int)p[1], (int)p[2], (int)p[3]};
  }
}

// Exponent of the FP8 V block scale: the smallest e >= -127 with
// absmax <= 448 * 2^e, decided on the bits (absmax = f 2^E, 448 = 1.75 2^8:
// e = E - 8 when f <= 1.75, else E - 7; a subnormal absmax clamps to -127).
__device__ __forceinline__ int v_scale_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int e = (int)(b >> 23) - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return max(e, -127);
}

// grid (nt, B*H), 256 threads.  One 64-row block of V: s_v = 2^e (0 for an
// all-zero block), codes E4M3(V / s_v) (an exact product with 2^-e).  The
// power of two is the block-scale form the FP8 matrix instruction applies
// itself, as an E8M0 exponent.  Writes the [N][D] codes (if codes != nullptr)
// and/or the attention tile layout [nt][D][64] with FP8 key positions
// (if vt != nullptr, zero for keys >= N), and the scale.
template <int D>
__global__ __launch_bounds__(256) void quant_v_fp8_kernel(const uint16_t* __restrict__ v, Lay lv, int N,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ vt,
                                                          float* __restrict__ scales) {
  __shared__ float sh[4];
  __shared__ uint8_t tile[KT][D + 16];
  const long long bh = blockIdx.y;
  const int tt = blockIdx.x, nt = gridDim.x;
  const int t = threadIdx.x;
  constexpr int CPR = D / 8;
  constexpr int RPP = 256 / CPR;
  const int cg = t % CPR, rg = t / CPR;
  const uint16_t* vh = v + lay_row(lv, bh, 0);
  const int r0 = tt * KT, r1 = min(N, r0 + KT);
  // the tile's KT / RPP chunks of this thread, read once and kept in
  // registers for the coding pass (rows past N read as zeros, unused)
  constexpr int NCH = KT / RPP;
  static_assert(KT % RPP == 0, "whole passes per tile");
  v4i w[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int r = r0 + rg + i * RPP;
    w[i] = r < r1 ? *(const v4i*)(vh + (long long)r * lv.sn + cg * 8) : v4i{0, 0, 0, 0};
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t u = (uint32_t)w[i][j];
      amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(u & 0xFFFFu)), fabsf(bf16_bits_to_f32(u >> 16))));
    }
  }
  amax = block_max_256(amax, sh);
  const int e = v_scale_exp(amax);
  const bool zero = !(amax > 0.0f);
  // 2^e (2^-127 is the subnormal 0x00400000) and 2^-e (at most 2^127)
  const float s = zero ? 0.0f : __uint_as_float(e >= -126 ? (uint32_t)(e + 127) << 23 : 0x00400000u);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
  if (t == 0) scales[bh * nt + tt] = s;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int r = r0 + rg + i * RPP;
    uint32_t packed[2] = {0u, 0u};
    if (r < r1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t u = (uint32_t)w[i][j >> 1];
        float a = bf16_bits_to_f32((j & 1) ? (u >> 16) : (u & 0xFFFFu));
        uint32_t c = zero ? 0u : e4m3_encode_f32(a * inv);
        packed[j >> 2] |= c << ((j & 3) * 8);
      }
      if (codes)
        *(uint2*)(codes + (bh * (long long)N + r) * D + cg * 8) = make_uint2(packed[0], packed[1]);
    }
    if (vt) {
#pragma unroll
      for (int j = 0; j < 8; ++j) tile[r - r0][cg * 8 + j] = (uint8_t)(packed[j >> 2] >> ((j & 3) * 8));
    }
  }
  if (!vt) return;
  __syncthreads();
  uint8_t* out = vt + (bh * nt + tt) * (long long)D * KT;
  // each thread writes 16 consecutive positions of one channel row
  for (int i = t; i < D * (KT / 16); i += 256) {
    int c = i / (KT / 16), p0 = (i % (KT / 16)) * 16;
    uint32_t p[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      int pos = p0 + j;
      // inverse of fp8_key_pos: pos = g*32 + q*8 + r -> key = q*16 + g*8 + r
      int key = ((pos >> 3) & 3) * 16 + (pos >> 5) * 8 + (pos & 7);
      p[j >> 2] |= (uint32_t)tile[key][c] << ((j & 3) * 8);
    }
    *(v4i*)(out + (long long)c * KT + p0) = v4i{(int)p[0], (int)p[1], (int)p[2], (int)p[3]};
  }
}

// grid (nt, B*H), 256 threads: FP8 codes [N][D] (as written by quant_v_fp8)
// -> attention tile layout.  Used when the caller supplies quantized V.
template <int D>
__global__ __launch_bounds__(256) void v_tiles_fp8_kernel(const uint8_t* __restrict__ codes, int N,
                                                          uint8_t* __restrict__ vt) {
  __shared__ uint8_t tile[KT][D + 16];
  const long long bh = blockIdx.y;
  const int tt = blockIdx.x, nt = gridDim.x;
  const int t = threadIdx.x;
  for (int i = t; i < KT * (D / 16); i += 256) {
    int r = i / (D / 16), c16 = (i % (D / 16)) * 16;
    int key = tt * KT + r;
    v4i w = (key < N) ? *(const v4i*)(codes + (bh * (long long)N + key) * D + c16) : v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 16; ++j) tile[r][c16 + j] = (uint8_t)((uint32_t)w[j >> 2] >> ((j & 3) * 8));
  }
  __syncthreads();
  uint8_t* out = vt + (bh * nt + tt) * (long long)D * KT;
  for (int i = t; i < D * (KT / 16); i += 256) {
    int c = i / (KT / 16), p0 = (i % (KT / 16)) * 16;
    uint32_t p[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      int pos = p0 + j;
      int key = ((pos >> 3) & 3) * 16 + (pos >> 5) * 8 + (pos & 7);
      p[j >> 2] |= (uint32_t)tile[key][c] << ((j & 3) * 8);
    }
    *(v4i*)(out + (long long)c * KT + p0) = v4i{(int)p[0], (int)p[1], (int)p[2], (int)p[3]};
  }
}

// ---------------------------------------------------------------------------
// Q-smoothing bias
// ---------------------------------------------------------------------------

// grid (nt, B*H), 256 threads: thread t owns key j = 64 tile + t % 64 and the
// Q blocks b = t / 64 + 4 i.  For each (b, j) the bias of the logit in units
// of sQ[b] sK[tile]:
//   dS   = mu_b . K'_j, K'_j = fl32(K_j - kmean) (binary32): 16 FMA chains of
//          8 channels each (channel order), summed pairwise
//   beta = fl32(dS / fl32(sQ[b] sK[tile])), 0 when that product is 0
// into bias[(bh nq + b) nt 64 + j], binary32 (0 for blocks whose mean row is
// 0; keys past N repeat key N-1, as the attention kernels' K rows past N do,
// so that the last tile's max over all 64 positions is a real score).  The
// attention kernels add it to their scores in floating point.  The error of
// beta, at most 14 u sum_c |mu_c K'_jc| / (sQ sK) units (u = 2^-24), is part
// of what the oracle's smoothing width charges.
template <int D>
__global__ __launch_bounds__(256) void qbias_kernel(const uint16_t* __restrict__ k, Lay lk, int N,
                                                    const float* __restrict__ kmean,
                                                    const float* __restrict__ qmean,
                                                    const float* __restrict__ sq,
                                                    const float* __restrict__ sk, int nq,
                                                    float* __restrict__ bias) {
  constexpr int NB = 32;  // Q blocks staged in LDS at a time (8 per thread group)
  __shared__ float mus[NB][D];
  const long long bh = blockIdx.y;
  const int tile = blockIdx.x, nt = gridDim.x;
  const int t = threadIdx.x, jl = t & 63, grp = t >> 6;
  const int j = tile * KT + jl;
  float kp[D];
  {
    const uint16_t* kr = k + lay_row(lk, bh, min(j, N - 1));
    const float* km = kmean + bh * D;
#pragma unroll
    for (int c8 = 0; c8 < D / 8; ++c8) {
      const v4i w = *(const v4i*)(kr + c8 * 8);
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const uint32_t u = (uint32_t)w[h >> 1];
        kp[c8 * 8 + h] = bf16_bits_to_f32((h & 1) ? (u >> 16) : (u & 0xFFFFu)) - km[c8 * 8 + h];
      }
    }
  }
  // (a key past N takes key N-1's bias, in units of its own tile's scale:
  // the last tile holds both)
  const float skt = sk[bh * nt + tile];
  const long long row = (long long)nt * KT;
  for (int b0 = 0; b0 < nq; b0 += NB) {
    __syncthreads();
    for (int i = t; i < NB * D / 4; i += 256) {
      const int b = b0 + (4 * i) / D;
      *(v4f*)&mus[(4 * i) / D][(4 * i) % D] =
          b < nq ? *(const v4f*)(qmean + (bh * nq + b) * D + (4 * i) % D) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    __syncthreads();
    for (int bi = grp; bi < NB && b0 + bi < nq; bi += 4) {
      const int b = b0 + bi;
      float part[D / 8];
#pragma unroll
      for (int g = 0; g < D / 8; ++g) {
        const v4f m0 = *(const v4f*)&mus[bi][8 * g];
        const v4f m1 = *(const v4f*)&mus[bi][8 * g + 4];
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = __builtin_fmaf(m0[c], kp[8 * g + c], acc);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = __builtin_fmaf(m1[c], kp[8 * g + 4 + c], acc);
        part[g] = acc;
      }
#pragma unroll
      for (int w = D / 16; w >= 1; w >>= 1)
#pragma unroll
        for (int g = 0; g < w; ++g) part[g] = part[2 * g] + part[2 * g + 1];
      const float den = sq[bh * nq + b] * skt;
      bias[(bh * nq + b) * row + j] = den != 0.0f ? part[0] / den : 0.0f;  // correctly rounded
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

#define SQ_DISPATCH_D(d, KERNEL, GRID, BLOCK, STREAM, ...)                         \
  do {                                                                              \
    if ((d) == 128)                                                                 \
      hipLaunchKernelGGL(KERNEL<128>, GRID, BLOCK, 0, STREAM, __VA_ARGS__);         \
    else                                                                            \
      hipLaunchKernelGGL(KERNEL<64>, GRID, BLOCK, 0, STREAM, __VA_ARGS__);          \
  } while (0)

#define SQ_DISPATCH_DN(d, norm, KERNEL, GRID, BLOCK, STREAM, ...)                  \
  do {                                                                              \
    if ((d) == 128 && (norm))                                                       \
      hipLaunchKernelGGL((KERNEL<128, true>), GRID, BLOCK, 0, STREAM, __VA_ARGS__); \
    else if ((d) == 128)                                                            \
      hipLaunchKernelGGL((KERNEL<128, false>), GRID, BLOCK, 0, STREAM, __VA_ARGS__); \
    else if (norm)                                                                  \
      hipLaunchKernelGGL((KERNEL<64, true>), GRID, BLOCK, 0, STREAM, __VA_ARGS__);  \
    else                                                                            \
      hipLaunchKernelGGL((KERNEL<64, false>), GRID, BLOCK, 0, STREAM, __VA_ARGS__); \
  } while (0)

void launch_kmean(const uint16_t* k, const Lay& lk, int BH, int N, int d, uint64_t* partial, float* mean,
                  hipStream_t st, const RowNorm& nm) {
  int S = kmean_chunks(BH, N);
  int rows = (N + S - 1) / S;
  SQ_DISPATCH_DN(d, nm.r != nullptr, kmean_partial_kernel, dim3(S, BH), dim3(256), st, k, lk, N, rows, partial,
                 nm);
  if (d == 128)
    hipLaunchKernelGGL(kmean_finalize_kernel<128>, dim3(BH), dim3(128), 0, st, partial, S, N, mean);
  else
    hipLaunchKernelGGL(kmean_finalize_kernel<64>, dim3(BH), dim3(64), 0, st, partial, S, N, mean);
}

void launch_quant_i8(const uint16_t* x, const Lay& lx, int BH, int N, int d, int block, float* mean,
                     int8_t* codes, float* scales, hipStream_t st, const RowNorm& nm, bool mean_blocks) {
  const bool norm = nm.r != nullptr;
  if (block == 1 && mean == nullptr) {  // one scale per row
    const int rpw = 256 / (d / 8);
    SQ_DISPATCH_DN(d, norm, quant_i8_rows_kernel, dim3((N + rpw - 1) / rpw, BH), dim3(256), st, x, lx, N, codes,
                   scales, nm);
    return;
  }
  int nb = (N + block - 1) / block;
  SQ_DISPATCH_DN(d, norm, quant_i8_kernel, dim3(nb, BH), dim3(256), st, x, lx, N, block, mean,
                 mean_blocks ? 1 : 0, codes, scales, nm);
}

void launch_qmean(const uint16_t* q, const Lay& lq, int BH, int N, int d, int block, uint64_t* partial,
                  float* mean, hipStream_t st) {
  const int nq = (N + block - 1) / block;
  SQ_DISPATCH_DN(d, false, kmean_partial_kernel, dim3(nq, BH), dim3(256), st, q, lq, N, block, partial,
                 RowNorm{});
  SQ_DISPATCH_D(d, qmean_finalize_kernel, dim3(nq, BH), dim3(d), st, partial, N, block, mean);
}

void launch_qbias(const uint16_t* k, const Lay& lk, int BH, int N, int d, const float* kmean, const float* qmean,
                  const float* q_scale, const float* k_scale, int block, float* bias, hipStream_t st) {
  const int nt = (N + KT - 1) / KT, nq = (N + block - 1) / block;
  SQ_DISPATCH_D(d, qbias_kernel, dim3(nt, BH), dim3(256), st, k, lk, N, kmean, qmean, q_scale, k_scale, nq, bias);
}

void launch_v_tiles_bf16(const uint16_t* v, const Lay& lv, int BH, int N, int d, uint16_t* vt, hipStream_t st) {
  int nt = (N + KT - 1) / KT;
  SQ_DISPATCH_D(d, v_tiles_bf16_kernel, dim3(nt, BH), dim3(256), st, v, lv, N, vt);
}

void launch_quant_v_fp8(const uint16_t* v, const Lay& lv, int BH, int N, int d, uint8_t* codes, uint8_t* vt,
                        float* scales, hipStream_t st) {
  int nt = (N + KT - 1) / KT;
  SQ_DISPATCH_D(d, quant_v_fp8_kernel, dim3(nt, BH), dim3(256), st, v, lv, N, codes, vt, scales);
}

void launch_v_tiles_fp8(const uint8_t* codes, int BH, int N, int d, uint8_t* vt, hipStream_t st) {
  int nt = (N + KT - 1) / KT;
  SQ_DISPATCH_D(d, v_tiles_fp8_kernel, dim3(nt, BH), dim3(256), st, codes, N, vt);
}

}  // namespace sqattn
