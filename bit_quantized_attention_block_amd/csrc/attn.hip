// Quantized attention kernel for gfx950 (MI355X).
//
// Method: logits from INT8 codes of Q and smoothed K on the integer matrix
// units, softmax, then P.V in bf16 or FP8 with fp32 accumulation
// (jefxiong.cn "AIGC weekend special 5.10", section 1.2 item (1); GVCLab
// research log 2026-09-02, section 5.5 table, SageAttention2 row).  The
// tiling with a running max and running sum is the FlashAttention lineage that
// the same digest names as its baseline.
//
// Work decomposition
//   * A work-group (4 waves) owns 256 query rows of one (b,h) head; each wave
//     owns 64 rows as two 32-row MFMA blocks.  Keys stream in 64-key tiles
//     through double-buffered LDS; the next tile is fetched into registers
//     while the current one is consumed.
//   * Work-group w runs on XCD w % 8 (round-robin dispatch); items are
//     numbered so that each XCD walks consecutive query tiles of the same
//     head, which then share K/V tiles through that XCD's L2.
//
// Register layouts (32x32 MFMA: lane l, accumulator register i holds row
// 8*(i/4) + 4*(l/32) + i%4, column l%32; operand lane-half g = l/32 holds the
// k-slots g*K/2 .. g*K/2 + K/2 - 1)
//   * S^T = K Q^T on v_mfma_i32_32x32x32_i8: A = K tile rows (keys), B = Q
//     rows (held in registers for the whole loop).  Each lane therefore owns
//     one query column; its 16 accumulators are 16 keys.  K rows are loaded in
//     the order pi(r) = r with bits 2 and 3 swapped, which makes the 16 keys
//     of lane-half g in a 32-key block equal to {16h + 8g + j : h<2, j<8}.
//   * O^T = V^T P^T: P^T is the B operand (k = keys, n = queries), built in
//     place from the lane's own softmax values, so no cross-lane movement is
//     needed; V^T (rows = channels) is the A operand read from LDS, where
//     each lane-half's 8 (bf16) or 32 (FP8) keys are contiguous.  Row max and
//     row sum therefore need only one exchange between lanes l and l^32.
//   * LDS rows are XOR-swizzled in 16-byte units so that the 16-byte reads
//     of 8 (and 16) consecutive lanes fall in distinct banks.
#include "common.h"
#include "kernels.h"

namespace sqattn {

__device__ __forceinline__ int perm_key(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128)
    return ((row >> 1) ^ ((row & 1) << 1)) & 7;
  else
    return ((row >> 1) & 1) | ((row >> 2) & 2);
}
__device__ __forceinline__ int swz_v16(int c) { return (c ^ (c >> 3)) & 7; }
__device__ __forceinline__ int swz_v8(int c) { return ((c >> 1) ^ (c >> 3)) & 3; }

__device__ __forceinline__ float xor32_f(float v) { return __shfl_xor(v, 32, 64); }
__device__ __forceinline__ int xor32_i(int v) { return __shfl_xor(v, 32, 64); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  v2bf v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// lazy-rescale threshold of the 16-bit path (log2 units): P may grow to 2^8
constexpr float LAZY_THRESH = 8.0f;

template <int D, int PV>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
  constexpr int NCH = D / 32;                         // 32-byte d chunks (QK k-steps)
  constexpr int NCB = D / 32;                         // 32-channel blocks of O^T
  constexpr int KBYTES = KT * D;                      // one K tile
  constexpr int VROW = (PV == 0) ? KT * 2 : KT;       // bytes per V^T row
  constexpr int VBYTES = D * VROW;                    // one V tile
  constexpr int KCH = KBYTES / 16 / 256;              // 16-byte pieces per thread
  constexpr int VCH = VBYTES / 16 / 256;
  constexpr int VCPR = VROW / 16;                     // 16-byte pieces per V^T row
  constexpr int KCPR = D / 16;

  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][KBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2][VBYTES];

  const int w = blockIdx.x;
  const int item = (w & 7) * p.per_xcd + (w >> 3);
  if (item >= p.BH * p.qtiles) return;
  const int bh = item / p.qtiles, qt = item - bh * p.qtiles;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, lr = lane & 31;
  const int N = p.N, nt = p.nt;
  const long long hoff = (long long)bh * N * D;
  const int qbase = qt * ATT_QWG + wave * ATT_QW;

  // ---- Q operands and per-row logit factors
  v4i qreg[2][NCH];
  float cq[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qbase + qb * 32 + lr;
    const bool ok = row < N;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
      qreg[qb][ch] = ok ? *(const v4i*)(p.q + hoff + (long long)row * D + ch * 32 + g * 16)
                        : v4i{0, 0, 0, 0};
    cq[qb] = ok ? p.sq[(long long)bh * p.nq + row / p.q_block] * p.scale_log2e : 0.0f;
  }

  v16f o[NCB][2];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[cb][qb][i] = 0.0f;
  float m[2] = {-__builtin_inff(), -__builtin_inff()};
  float l[2] = {0.0f, 0.0f};

  const uint8_t* kh = (const uint8_t*)p.k + hoff;
  const uint8_t* vth = (const uint8_t*)p.vt + (long long)bh * nt * VBYTES;

  v4i kst[KCH], vst[VCH];
  auto fetch = [&](int t) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int j = tid + 256 * u, row = j / KCPR, col = j % KCPR;
      const int key = t * KT + row;
      kst[u] = (key < N) ? *(const v4i*)(kh + (long long)key * D + col * 16) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int j = tid + 256 * u;
      vst[u] = *(const v4i*)(vth + (long long)t * VBYTES + j * 16);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int j = tid + 256 * u, row = j / KCPR, col = j % KCPR;
      *(v4i*)(&lds_k[buf][row * D + ((col ^ swz_k<D>(row)) << 4)]) = kst[u];
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int j = tid + 256 * u, c = j / VCPR, col = j % VCPR;
      const int sw = (PV == 0) ? swz_v16(c) : swz_v8(c);
      *(v4i*)(&lds_v[buf][c * VROW + ((col ^ sw) << 4)]) = vst[u];
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();

  const int krow0 = perm_key(lr);
  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) fetch(t + 1);

    // ---- S^T = K Q^T (int32, exact)
    v16i s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][qb][i] = 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = kb * 32 + krow0;
      const uint8_t* base = &lds_k[buf][row * D];
      const int sw = swz_k<D>(row);
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const v4i a = *(const v4i*)(base + (((ch * 2 + g) ^ sw) << 4));
        s[kb][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[0][ch], s[kb][0], 0, 0, 0);
        s[kb][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[1][ch], s[kb][1], 0, 0, 0);
      }
    }

    // ---- online softmax (log2 units)
    const float skt = p.sk[(long long)bh * nt + t];
    const bool tail = (t == nt - 1) && ((N & (KT - 1)) != 0);
    const int kvalid = N - t * KT;  // keys with index < kvalid are valid in this tile
    float pv[2][2][16];
    float cf[2], mref[2], alpha[2];
    bool need_any = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      cf[qb] = cq[qb] * skt;
      int dmax = -0x7FFFFFFF - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          int dv = s[kb][qb][i];
          if (tail) {
            const int key = kb * 32 + 16 * (i >> 3) + 8 * g + (i & 7);
            if (key >= kvalid) dv = -0x7FFFFFFF - 1;
          }
          dmax = max(dmax, dv);
        }
      dmax = max(dmax, xor32_i(dmax));
      const float tmax = (float)dmax * cf[qb];
      float mnew = fmaxf(m[qb], tmax);
      bool need;
      if constexpr (PV == 0) {
        need = mnew > m[qb] + LAZY_THRESH;
      } else {
        need = mnew > m[qb];
      }
      alpha[qb] = need ? __builtin_amdgcn_exp2f(m[qb] - mnew) : 1.0f;
      mref[qb] = need ? mnew : m[qb];
      need_any |= need;
    }
    if (__any(need_any)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        l[qb] *= alpha[qb];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[cb][qb][i] *= alpha[qb];
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      m[qb] = mref[qb];
      float lsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = __builtin_fmaf((float)s[kb][qb][i], cf[qb], -mref[qb]);
          float e = __builtin_amdgcn_exp2f(x);
          if (tail) {
            const int key = kb * 32 + 16 * (i >> 3) + 8 * g + (i & 7);
            if (key >= kvalid) e = 0.0f;
          }
          pv[qb][kb][i] = e;
          lsum += e;
        }
      l[qb] += lsum;
    }

    // ---- O^T += V^T P^T
    if constexpr (PV == 0) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        v8bf pb[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          uint32_t w4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            w4[j] = pack_bf16(pv[qb][ks >> 1][8 * (ks & 1) + 2 * j], pv[qb][ks >> 1][8 * (ks & 1) + 2 * j + 1]);
          v4i wv = {(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
          pb[qb] = __builtin_bit_cast(v8bf, wv);
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int c = cb * 32 + lr;
          const v8bf a = *(const v8bf*)(&lds_v[buf][c * VROW + (((2 * ks + g) ^ swz_v16(c)) << 4)]);
          o[cb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[0], o[cb][0], 0, 0, 0);
          o[cb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[1], o[cb][1], 0, 0, 0);
        }
      }
    } else {
      // FP8: operand bytes 16*kb + i hold E4M3(448 * P~) of key pv[.][kb][i]
      v8i pf[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int kb = r >> 2, i0 = (r & 3) * 4;
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(448.0f * pv[qb][kb][i0], 448.0f * pv[qb][kb][i0 + 1], 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(448.0f * pv[qb][kb][i0 + 2], 448.0f * pv[qb][kb][i0 + 3], word, true);
          pf[qb][r] = word;
        }
      }
      const float fsv = p.sv[(long long)bh * nt + t] * (1.0f / 448.0f);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int c = cb * 32 + lr;
        const int sw = swz_v8(c);
        const v4i a0 = *(const v4i*)(&lds_v[buf][c * VROW + (((2 * g) ^ sw) << 4)]);
        const v4i a1 = *(const v4i*)(&lds_v[buf][c * VROW + (((2 * g + 1) ^ sw) << 4)]);
        const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          v16f z;
#pragma unroll
          for (int i = 0; i < 16; ++i) z[i] = 0.0f;
          const v16f acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf[qb], z, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) o[cb][qb][i] = __builtin_fmaf(acc[i], fsv, o[cb][qb][i]);
        }
      }
    }

    if (t + 1 < nt) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, fp32 rows
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = l[qb] + xor32_f(l[qb]);
    const float inv = 1.0f / lt;
    const int row = qbase + qb * 32 + lr;
    if (row < N) {
      float* orow = p.out + hoff + (long long)row * D;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          v4f v = {o[cb][qb][4 * i4] * inv, o[cb][qb][4 * i4 + 1] * inv, o[cb][qb][4 * i4 + 2] * inv,
                   o[cb][qb][4 * i4 + 3] * inv};
          *(v4f*)(orow + cb * 32 + i4 * 8 + g * 4) = v;
        }
    }
  }
}

void launch_attention(const AttnParams& p, int d, int pv, hipStream_t st) {
  AttnParams q = p;
  q.qtiles = (p.N + ATT_QWG - 1) / ATT_QWG;
  const long long W = (long long)p.BH * q.qtiles;
  q.per_xcd = (int)((W + 7) / 8);
  if (pv == 0) {
    launch_attention_bf16(q, d, st);
    return;
  }
  const dim3 grid(8 * q.per_xcd), block(256);
  if (d == 128)
    hipLaunchKernelGGL((attn_kernel<128, 1>), grid, block, 0, st, q);
  else
    hipLaunchKernelGGL((attn_kernel<64, 1>), grid, block, 0, st, q);
}

}  // namespace sqattn
