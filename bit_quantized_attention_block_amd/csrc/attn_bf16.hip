// Quantized attention kernel, 16-bit P.V path, software-pipelined (gfx950).
//
// Same mathematics and register layouts as the FP8 kernel in attn.hip (INT8
// S^T = K Q^T, lane-local online softmax, O^T = V^T P^T); see that file for
// the layout derivation.  What differs is the schedule.  The unit of the
// pipeline is a half-tile h of 32 keys (half kb = h%2 of 64-key tile h/2):
//
//   iteration h:   MFMA  S(h+1) = K(h+1) Q^T           (8 x i8 32x32x32)
//                  MFMA  O     += V(h-1)^T P(h-1)^T    (16 x bf16 32x32x16)
//                  VALU  P(h)   = softmax step on S(h)
//   with the two MFMA streams interleaved with the VALU stream, so the matrix
//   cores and the vector ALUs work at the same time inside one wave.  Each K
//   and V operand read from LDS feeds both 32-query blocks of the wave.  S and
//   P are double-buffered in registers; the two halves of a tile use them in
//   swapped roles, so no copies are needed.  Tiles move global -> LDS with
//   direct-to-LDS loads issued one tile ahead; one barrier per tile.
//
//   * No rescaling inside the loop: each row's reference max is the max of
//     its first 32 keys, and P = 2^(x - ref) may grow up to 2^HEADROOM (exact
//     in bf16/fp32; O stays finite while |V| * N < 2^(127 - HEADROOM)).  The
//     true running max is tracked; if any row of the work-group exceeds its
//     reference by more than HEADROOM, the work-group recomputes once with the
//     true max as reference (then P <= 1).  So the loop body has no branch.
//   * The row sum is taken on the bf16-rounded P with v_dot2c_f32_bf16, so the
//     normalisation uses exactly the weights the matrix core multiplied.
//   * Only the last, possibly ragged tile carries key masking.  Rows past N in
//     the K tile load row N-1 (in-bounds); their logits are masked.  The packed
//     V tiles are zero past N.
#include "common.h"
#include "kernels.h"

namespace sqattn {

namespace {

__device__ __forceinline__ int perm_key(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128)
    return ((row >> 1) ^ ((row & 1) << 1)) & 7;
  else
    return ((row >> 1) & 1) | ((row >> 2) & 2);
}
__device__ __forceinline__ int swz_v16(int c) { return (c ^ (c >> 3)) & 7; }

constexpr float HEADROOM = 32.0f;  // log2 units

typedef __attribute__((address_space(3))) void lds_void;

// max and sum over lanes l and l^32 (v_permlane32_swap pairs them)
__device__ __forceinline__ int pair_max_i(int v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float pair_sum_f(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

template <int D, int QBW>
struct Ctx {
  static constexpr int WAVES = 8 / QBW;   // 256 query rows per work-group
  static constexpr int NCH = D / 32;
  static constexpr int NCB = D / 32;
  static constexpr int KBYTES = KT * D;
  static constexpr int VBYTES = D * KT * 2;
  uint8_t* lk;     // LDS K tiles [2][KBYTES]
  uint8_t* lv;     // LDS V tiles [2][VBYTES]
  const uint8_t* kh;
  const uint8_t* vth;
  const float* skh;
  int N, nt, tid, lane, wave, g, lr, krow0;
  float cq[QBW];
  v4i qreg[QBW][NCH];
  v16f o[QBW][NCB];
  float m[QBW], l[QBW], mrun[QBW];  // reference max, row sum, running max

  // ---- global -> LDS (direct), tile t of K into buffer b
  __device__ __forceinline__ void load_k(int t, int b) {
    constexpr int CPR = D / 16;  // 16-byte chunks per K row
    constexpr int NINST = KBYTES / 16 / 64;  // 1 KB direct loads per tile
    for (int u = wave; u < NINST; u += WAVES) {
      const int j0 = u * 64;
      const int j = j0 + lane;
      const int row = j / CPR, pc = j % CPR;
      const int key = min(t * KT + row, N - 1);
      const uint8_t* src = kh + (long long)key * D + ((pc ^ swz_k<D>(row)) << 4);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(lk + b * KBYTES + j0 * 16), 16, 0, 0);
    }
  }
  __device__ __forceinline__ void load_v(int t, int b) {
    constexpr int NINST = VBYTES / 16 / 64;
    for (int u = wave; u < NINST; u += WAVES) {
      const int j0 = u * 64;
      const int j = j0 + lane;
      const int c = j >> 3, pc = j & 7;
      const uint8_t* src = vth + (long long)t * VBYTES + c * 128 + ((pc ^ swz_v16(c)) << 4);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(lv + b * VBYTES + j0 * 16), 16, 0, 0);
    }
  }

  // ---- S(h) = K half-tile Q^T for both query blocks (K tile in buffer b, half kb)
  __device__ __forceinline__ void qk(v16i (&s)[QBW], int b, int kb) {
    const int row = kb * 32 + krow0;
    const uint8_t* base = lk + b * KBYTES + row * D;
    const int sw = swz_k<D>(row);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const v4i a = *(const v4i*)(base + (((ch * 2 + g) ^ sw) << 4));
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        if (ch == 0) {
          v16i z;
#pragma unroll
          for (int i = 0; i < 16; ++i) z[i] = 0;
          s[qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[qb][ch], z, 0, 0, 0);
        } else {
          s[qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[qb][ch], s[qb], 0, 0, 0);
        }
      }
    }
  }

  // ---- O^T += V^T P^T over one half-tile (V tile in buffer b, half kb)
  __device__ __forceinline__ void pv(const v4i (&pb)[QBW][2], int b, int kb) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int ks = 2 * kb + k2;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int c = cb * 32 + lr;
        const v8bf a = *(const v8bf*)(lv + b * VBYTES + c * 128 + (((2 * ks + g) ^ swz_v16(c)) << 4));
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb)
          o[qb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, pb[qb][k2]), o[qb][cb], 0,
                                                              0, 0);
      }
    }
  }

  // ---- softmax step on S(h) (half kb of tile t): P(h) = 2^(x - ref) as
  // packed bf16, row-sum and running-max update.  The first half-tile sets
  // the reference.  Keys past N (last tile only) duplicate key N-1, so they
  // never raise the max; fix_tail() removes them afterwards.
  __device__ __forceinline__ void softmax(const v16i (&s)[QBW], v4i (&pb)[QBW][2], int t) {
    const float skt = skh[t];
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      const float c = cq[qb] * skt;
      int d0 = s[qb][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) d0 = max(d0, s[qb][i]);
      const float tmax = (float)pair_max_i(d0) * c;
      mrun[qb] = __builtin_fmaxf(mrun[qb], tmax);
      const float mref = (m[qb] == -__builtin_inff()) ? tmax : m[qb];
      m[qb] = mref;
      float lsum = 0.0f;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        uint32_t w4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 8 * k2 + 2 * j;
          v2bf pk;
          pk[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf((float)s[qb][i], c, -mref));
          pk[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf((float)s[qb][i + 1], c, -mref));
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pk, v2bf{(__bf16)1.0f, (__bf16)1.0f}, lsum, false);
          w4[j] = __builtin_bit_cast(uint32_t, pk);
        }
        pb[qb][k2] = v4i{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
      }
      l[qb] += lsum;
    }
  }

  // ---- last tile, half kb: zero P of keys >= N and take them out of the row sum
  __device__ __forceinline__ void fix_tail(v4i (&pb)[QBW][2], int t, int kb) {
    const int kvalid = N - t * KT - kb * 32;
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      float drop = 0.0f;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k0 = 16 * k2 + 8 * g + 2 * j;
          uint32_t w = (uint32_t)pb[qb][k2][j];
          const uint32_t keep = (k0 >= kvalid ? 0u : 0xFFFFu) | (k0 + 1 >= kvalid ? 0u : 0xFFFF0000u);
          const uint32_t gone = w & ~keep;
          drop = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, gone), v2bf{(__bf16)1.0f, (__bf16)1.0f},
                                                 drop, false);
          pb[qb][k2][j] = (int)(w & keep);
        }
      l[qb] -= drop;
    }
  }

};

// Interleave hint for one pipelined iteration: MFMA, VALU and LDS reads.
// LDS reads run AHEAD reads ahead of the MFMAs that consume them.
template <int NMFMA, int VALU_PER_MFMA, int NREAD, int AHEAD>
__device__ __forceinline__ void interleave() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);              // first LDS reads
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER_MFMA, 0);    // VALU
    if (i * NREAD / NMFMA + AHEAD < NREAD && (i + 1) * NREAD / NMFMA != i * NREAD / NMFMA)
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // next LDS read
  }
}

}  // namespace

template <int D, int QBW>
__global__ __launch_bounds__(64 * (8 / QBW)) void attn_bf16_kernel(AttnParams p) {
  using Cx = Ctx<D, QBW>;
  constexpr int NTHR = 64 * Cx::WAVES;
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2 * KT * D];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2 * D * KT * 2];

  const int w = blockIdx.x;
  const int item = (w & 7) * p.per_xcd + (w >> 3);
  if (item >= p.BH * p.qtiles) return;
  const int bh = item / p.qtiles, qt = item - bh * p.qtiles;

  Cx C;
  C.lk = lds_k;
  C.lv = lds_v;
  C.tid = threadIdx.x;
  C.lane = C.tid & 63;
  C.wave = C.tid >> 6;
  C.g = C.lane >> 5;
  C.lr = C.lane & 31;
  C.krow0 = perm_key(C.lr);
  C.N = p.N;
  C.nt = p.nt;
  const long long hoff = (long long)bh * p.N * D;
  C.kh = (const uint8_t*)p.k + hoff;
  C.vth = (const uint8_t*)p.vt + (long long)bh * p.nt * Cx::VBYTES;
  C.skh = p.sk + (long long)bh * p.nt;
  const int qbase = qt * ATT_QWG + C.wave * 32 * QBW;
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int row = qbase + qb * 32 + C.lr;
    const bool ok = row < p.N;
#pragma unroll
    for (int ch = 0; ch < Cx::NCH; ++ch)
      C.qreg[qb][ch] = ok ? *(const v4i*)(p.q + hoff + (long long)row * D + ch * 32 + C.g * 16) : v4i{0, 0, 0, 0};
    C.cq[qb] = ok ? p.sq[(long long)bh * p.nq + row / p.q_block] * p.scale_log2e : 0.0f;
    C.m[qb] = -__builtin_inff();
    C.mrun[qb] = -__builtin_inff();
  }

  const int nt = p.nt;
  const bool ragged = (p.N & (KT - 1)) != 0;
  v16i S0[QBW], S1[QBW];
  v4i P0[QBW][2], P1[QBW][2];

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      C.l[qb] = 0.0f;
#pragma unroll
      for (int cb = 0; cb < Cx::NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) C.o[qb][cb][i] = 0.0f;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) P1[qb][k2] = v4i{0, 0, 0, 0};
    }

    // prologue: K(0), K(1), V(0) -> LDS, V buffer 1 zeroed (the first
    // iteration multiplies it by P = 0); S(0) from the first half of K(0)
    C.load_k(0, 0);
    C.load_k(nt > 1 ? 1 : 0, 1);
    C.load_v(0, 0);
    for (int i = C.tid; i < Cx::VBYTES / 16; i += NTHR)
      *(v4i*)(lds_v + Cx::VBYTES + i * 16) = v4i{0, 0, 0, 0};
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    C.qk(S0, 0, 0);

    // Half-tile iteration h = 2t + KB: S(h) in SCUR, P(h) into PCUR, S(h+1)
    // into SNEXT, P(h-1) from PPREV.  K(h+1) is half KB^1 of tile t + KB (in
    // the last iteration a stale tile whose S is never used); V(h-1) is half
    // KB^1 of tile t - 1 + KB (for h = 0 the zeroed buffer, with P(-1) = 0).
#define SQ_HALF(KB, SCUR, SNEXT, PPREV, PCUR) \
  do {                                        \
    C.qk(SNEXT, (t + KB) & 1, KB ^ 1);        \
    C.pv(PPREV, (t - 1 + KB) & 1, KB ^ 1);    \
    C.softmax(SCUR, PCUR, t);                 \
    interleave<12 * QBW, 14 / QBW, 12, 3>();  \
  } while (0)

    for (int t = 0; t < nt; ++t) {
      SQ_HALF(0, S0, S1, P1, P0);
      if (ragged && t == nt - 1) C.fix_tail(P0, t, 0);
      // loads of K(t+1), V(t) issued one tile ago have landed and every wave
      // is done with K(t) and V(t-1): refill those buffers with K(t+2), V(t+1)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 2 < nt) C.load_k(t + 2, t & 1);
      if (t + 1 < nt) C.load_v(t + 1, (t + 1) & 1);
      SQ_HALF(1, S1, S0, P0, P1);
      if (ragged && t == nt - 1) C.fix_tail(P1, t, 1);
    }
#undef SQ_HALF
    // the last half-tile's P.V (V(nt-1) half 1)
    C.pv(P1, (nt - 1) & 1, 1);

    // a row whose max outran its reference: redo with the true max
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      over |= C.mrun[qb] > C.m[qb] + HEADROOM;
      C.m[qb] = C.mrun[qb];
    }
    __syncthreads();  // all waves are done with the LDS tiles
    if (!__syncthreads_or(over)) break;
  }

  // epilogue: O = O^T / l, fp32 rows
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const float inv = 1.0f / pair_sum_f(C.l[qb]);
    const int row = qbase + qb * 32 + C.lr;
    if (row < p.N) {
      float* orow = p.out + hoff + (long long)row * D;
#pragma unroll
      for (int cb = 0; cb < Cx::NCB; ++cb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          v4f v = {C.o[qb][cb][4 * i4] * inv, C.o[qb][cb][4 * i4 + 1] * inv, C.o[qb][cb][4 * i4 + 2] * inv,
                   C.o[qb][cb][4 * i4 + 3] * inv};
          *(v4f*)(orow + cb * 32 + i4 * 8 + C.g * 4) = v;
        }
    }
  }
}

// Query blocks per wave: 1 (8 waves, two per SIMD) or 2 (4 waves).
#ifndef SQATTN_BF16_QBW
#define SQATTN_BF16_QBW 1
#endif

void launch_attention_bf16(const AttnParams& q, int d, hipStream_t st) {
  constexpr int QBW = SQATTN_BF16_QBW;
  const dim3 grid(8 * q.per_xcd), block(64 * (8 / QBW));
  if (d == 128)
    hipLaunchKernelGGL((attn_bf16_kernel<128, QBW>), grid, block, 0, st, q);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<64, QBW>), grid, block, 0, st, q);
}

}  // namespace sqattn
