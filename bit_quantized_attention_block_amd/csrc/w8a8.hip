// W8A8 block-wise INT8 linear layer for gfx950 (MI355X): y = x W^T (+ b).
//
// Method: the linear layers around attention quantize weights and activations
// to INT8 in blocks of 128x128 and run on the INT8 matrix units (jefxiong.cn
// "AIGC weekend special 5.10", section 1.2 item (4); digipub.cc TurboDiffusion
// article, linear-layer quantization paragraph).  Scale and code rule as for
// the attention's Q/K blocks: s = fl32(absmax/127), code = rne(fl32(v/s)).
//
//   w8a8_quant : one 128x128 block per work-group; the block stays in
//       registers between the absmax reduction and the code pass (one HBM
//       read, one write).
//   w8a8_gemm  : 256x256 output tile per work-group of 8 waves (two per
//       SIMD), each wave 128 rows x 64 columns = 4 x 2 MFMA tiles of 32x32.
//       The reduction axis is walked in 128-wide slices, which are exactly
//       the scale blocks: for one wave and one slice, all its rows lie in one
//       row block of x and all its columns in one row block of W, so the
//       slice's int32 partial (four v_mfma_i32_32x32x32_i8, exact since
//       |partial| < 2^21) is promoted into the fp32 accumulator with ONE
//       wave-uniform factor s = fl32(sx * sw): acc = fma(s, float(partial), acc).
//       That promotion (a convert and an FMA per output per slice) costs as
//       many vector cycles as the slice's matrix cycles, so the two waves of a
//       SIMD overlap one's promotion with the other's MFMAs.
//       Slices stream through a 2-slot LDS ring (x and W tiles, 144-byte
//       padded rows) with direct-to-LDS loads one slice ahead.  Work-groups
//       are numbered so that each XCD walks a compact 8 x 4 patch of output
//       tiles that shares x and W slices in its L2.
#include <mutex>

#include "common.h"
#include "exact.h"
#include "kernels.h"

namespace sqattn {

namespace {

constexpr int QB = 128;                  // scale block edge

// ---------------------------------------------------------------------------
// quantizer
// ---------------------------------------------------------------------------

// grid (C/128, ceil(R/128)), 256 threads.  Thread t holds columns
// 8 (t % 16) .. +8 of rows t/16 + 16 j (j < 8) of the block.  NORM: the
// block of y = fl32(fl32(x * r_row) * gamma_col) (gamma may be null) instead
// of x.
// NORM: 0 plain x; 1 RMSNorm, y = fl32(fl32(x * r_row) * gamma_col); 2
// LayerNorm, y = fl32(fl32(fl32(fl32(x - mean_row) * r_row) * gamma_col) +
// beta_col) (gamma, beta may be null).  The steps are separately rounded
// operations (no contraction into a fused multiply-add).
template <int NORM>
__global__ __launch_bounds__(256) void w8a8_quant_kernel(const uint16_t* __restrict__ x, int R, int C,
                                                         int8_t* __restrict__ codes,
                                                         float* __restrict__ scales,
                                                         const float* __restrict__ inv_rms,
                                                         const float* __restrict__ gamma,
                                                         const float* __restrict__ mean = nullptr,
                                                         const float* __restrict__ beta = nullptr) {
  __shared__ float sh[4];
  const int cb = blockIdx.x, rb = blockIdx.y;
  const int t = threadIdx.x, piece = t & 15, r = t >> 4;
  const long long col = (long long)cb * QB + piece * 8;
  v4i w[8];
  float rr[8], gm[8], bt[8], mr[8];
  if constexpr (NORM != 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) gm[e] = gamma ? gamma[col + e] : 1.0f;
  }
  if constexpr (NORM == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) bt[e] = beta ? beta[col + e] : 0.0f;
  }
  // element e of piece j as the value to quantize
  auto val = [&](int j, int e) {
    const uint32_t u = (uint32_t)w[j][e >> 1];
    float a = bf16_bits_to_f32((e & 1) ? (u >> 16) : (u & 0xFFFFu));
    if constexpr (NORM == 1) {
      a = a * rr[j];                 // fl32(x r)
      if (gamma) a = a * gm[e];      // fl32(. gamma)
    } else if constexpr (NORM == 2) {
      a = __fmul_rn(__fsub_rn(a, mr[j]), rr[j]);  // fl32(fl32(x - mu) r)
      if (gamma) a = __fmul_rn(a, gm[e]);
      if (beta) a = __fadd_rn(a, bt[e]);
    }
    return a;
  };
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = rb * QB + r + 16 * j;
    w[j] = (row < R) ? *(const v4i*)(x + (long long)row * C + col) : v4i{0, 0, 0, 0};
    if constexpr (NORM != 0) rr[j] = (row < R) ? inv_rms[row] : 0.0f;
    if constexpr (NORM == 2) mr[j] = (row < R) ? mean[row] : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(val(j, e)));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((t & 63) == 0) sh[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  const float s = amax / 127.0f;  // correctly rounded binary32 division
  if (t == 0) scales[(long long)rb * gridDim.x + cb] = s;
  const bool zero = !(s > 0.0f);
  const bool fast = s >= 0x1p-125f;  // 1/s finite
  const float y = 1.0f / s;          // correctly rounded
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = rb * QB + r + 16 * j;
    if (row >= R) break;
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = val(j, e);
      int c = 0;
      if (!zero) c = (int)fminf(fmaxf(fast ? rne_quotient(a, s, y) : rintf(a / s), -127.0f), 127.0f);
      packed[e >> 2] |= ((uint32_t)(c & 0xFF)) << ((e & 3) * 8);
    }
    *(uint2*)(codes + (long long)row * C + col) = make_uint2(packed[0], packed[1]);
  }
}

// ---------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------

constexpr int GT = 256;                  // work-group tile edge (rows of x and of W)
constexpr int WAVES = 8, NTHR = 64 * WAVES;
constexpr int ROWC = 9;                  // 16-byte units per LDS row: 8 + 1 pad (odd)
constexpr int ROWB = 16 * ROWC;          // 144
constexpr int TILEB = GT * ROWB;         // one operand tile in LDS
constexpr int SLOTB = 2 * TILEB;         // x tile then W tile
constexpr int SCB = 2 * SLOTB;           // scale rows: [2 chunks][4 rows][64 slices] float
constexpr int LDS_BYTES = SCB + 2 * 4 * 64 * 4;  // 149504 bytes
constexpr int INST = GT * ROWC / 64;     // 1 KB direct loads per tile (36)
constexpr int PER = 2 * INST / WAVES;    // per wave per slice (9)
constexpr int GROUP = 8;                 // M tiles per group of the tile order
constexpr int OUT_STRIDE = GT + 8;       // bf16 elements per staged output row (528 bytes)
static_assert(GT * OUT_STRIDE * 2 <= 2 * SLOTB, "the staged output tile must fit in the ring");
static_assert(2 * INST % WAVES == 0, "loads must split evenly over the waves");

struct GemmParams {
  const int8_t* x;
  const float* sx;
  const int8_t* w;
  const float* sw;
  const float* bias;
  void* out;
  int M, N, K, nkb, mt, nt, per_xcd, out_bf16;
};

__global__ __launch_bounds__(NTHR) void w8a8_gemm_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;

  // tile of this work-group: XCD-major numbering, then groups of GROUP
  // M tiles walked column by column
  const int wg = blockIdx.x;
  const int tix = (wg & 7) * p.per_xcd + (wg >> 3);
  if (tix >= p.mt * p.nt) return;
  const int grp = tix / (GROUP * p.nt);
  const int rem = tix - grp * GROUP * p.nt;
  const int gm = min(GROUP, p.mt - grp * GROUP);
  const int tm = grp * GROUP + rem % gm;
  const int tn = rem / gm;
  const int m0 = tm * GT, n0 = tn * GT;

  // direct loads: instruction u = wave + WAVES i covers LDS units
  // (u % INST) * 64 + lane of the x (u < INST) or W tile; unit q is row q / 9,
  // 16-byte piece q % 9 (the pad piece re-reads piece 7).  Rows past M (N)
  // read the last row.
  uint32_t off[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int u = wave + WAVES * i;
    const int q = (u % INST) * 64 + lane;
    const int row = q / ROWC, piece = min(q % ROWC, 7);
    const int last = (u < INST) ? (p.M - 1 - m0) : (p.N - 1 - n0);
    off[i] = (uint32_t)(min(row, last) * p.K + piece * 16);
  }
  const int8_t* xrow = p.x + (long long)m0 * p.K;
  const int8_t* wrow = p.w + (long long)n0 * p.K;
  const uint32_t lds0 = lds_addr(lds);
  auto load_slice = [&](int j, int slot) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = wave + WAVES * i;
      const bool isx = u < INST;
      lds_dma16((isx ? xrow : wrow) + j * QB, off[i],
                lds0 + slot * SLOTB + (isx ? 0 : TILEB) + (u % INST) * 1024);
    }
  };

  // this wave: rows wm*128 .. +128 (one row block of x), columns wn*64 .. +64
  // (inside one row block of W)
  const int wm = wave & 1, wn = wave >> 1;
  const int mb = min((m0 + wm * 128) / QB, (p.M - 1) / QB);
  const int nb = min((n0 + wn * 64) / QB, (p.N - 1) / QB);
  // Scale factors: the work-group's two row blocks of x (rows 0, 1) and of W
  // (rows 2, 3) are staged in LDS 64 slices at a time by direct dword loads
  // (waves 0-3, one row each), chunk c into half c % 2, issued with slice
  // 64c - 63's tiles.  Slices past the end re-read the last one.
  const int mlast = (p.M - 1) / QB, nlast = (p.N - 1) / QB;
  const float* srow = nullptr;
  if (wave < 4) {
    srow = (wave < 2) ? p.sx + (long long)min(m0 / QB + wave, mlast) * p.nkb
                      : p.sw + (long long)min(n0 / QB + wave - 2, nlast) * p.nkb;
  }
  auto load_scales = [&](int c) {
    if (wave < 4)
      lds_dma4(srow, (uint32_t)(min(64 * c + lane, p.nkb - 1) * 4), lds0 + SCB + ((c & 1) * 4 + wave) * 256);
  };
  const float* scl = (const float*)(lds + SCB);
  const int wrs = wm, wrw = 2 + ((n0 + wn * 64) / QB - n0 / QB);
  const uint32_t abase = (uint32_t)((wm * 128 + (lane & 31)) * ROWB + g * 16);
  const uint32_t bbase = (uint32_t)(TILEB + (wn * 64 + (lane & 31)) * ROWB + g * 16);

  v16f acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.0f;

  const v16i zero = {};
  load_scales(0);
  load_slice(0, 0);
  for (int j = 0; j < p.nkb; ++j) {
    const int slot = j & 1;
    // slice j (and its scale chunk) is in LDS once this wave's direct loads
    // have landed and every wave has passed the barrier; slot slot^1 is free
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < p.nkb) {
      load_slice(j + 1, slot ^ 1);
      if ((j & 63) == 63) load_scales((j + 1) >> 6);
    }
    const float* sc = scl + ((j >> 6) & 1) * 256 + (j & 63);
    const float s = sc[64 * wrs] * sc[64 * wrw];
    const uint8_t* sa = lds + slot * SLOTB + abase;
    const uint8_t* sb = lds + slot * SLOTB + bbase;
    v4i bf[2][4];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bf[n][ks] = *(const v4i*)(sb + n * 32 * ROWB + ks * 32);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v4i af[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) af[ks] = *(const v4i*)(sa + m * 32 * ROWB + ks * 32);
      v16i d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[0], bf[0][0], zero, 0, 0, 0);
      v16i d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[0], bf[1][0], zero, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) {
        d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[ks], bf[0][ks], d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[ks], bf[1][ks], d1, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[m][0][i] = fmaf(s, (float)d0[i], acc[m][0][i]);
        acc[m][1][i] = fmaf(s, (float)d1[i], acc[m][1][i]);
      }
    }
  }

  // epilogue: lane holds column l%32 of each 32x32 tile, rows 8(i/4)+4g+i%4
  const bool full = (m0 + GT <= p.M) && (n0 + GT <= p.N);
  float bcol[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int col = n0 + wn * 64 + n * 32 + (lane & 31);
    bcol[n] = (p.bias && col < p.N) ? p.bias[col] : 0.0f;
  }
  if (p.out_bf16) {
    // The bf16 tile goes through LDS (free once every wave is past the last
    // slice) so that it leaves in 16-byte pieces along whole rows.
    __syncthreads();
    uint16_t* st = (uint16_t*)lds;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wm * 128 + m * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          const int c = wn * 64 + n * 32 + (lane & 31);
          const __bf16 v = (__bf16)(acc[m][n][i] + bcol[n]);
          st[r * OUT_STRIDE + c] = __builtin_bit_cast(uint16_t, v);
        }
    __syncthreads();
    const bool vec = (p.N & 7) == 0;  // rows start 16-byte aligned
    const int piece = threadIdx.x & 31, r0 = threadIdx.x >> 5;
#pragma unroll 4
    for (int r = r0; r < GT; r += NTHR / 32) {
      const int row = m0 + r, col = n0 + piece * 8;
      if (row >= p.M) break;
      const v4i v = *(const v4i*)(st + r * OUT_STRIDE + piece * 8);
      uint16_t* dst = (uint16_t*)p.out + (long long)row * p.N + col;
      if (vec && (full || col + 8 <= p.N)) {
        *(v4i*)dst = v;
      } else {
        for (int e = 0; e < 8 && col + e < p.N; ++e) dst[e] = (uint16_t)(((uint32_t)v[e >> 1]) >> (16 * (e & 1)));
      }
    }
    return;
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int col = n0 + wn * 64 + n * 32 + (lane & 31);
    if (!full && col >= p.N) continue;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m0 + wm * 128 + m * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (!full && row >= p.M) continue;
        ((float*)p.out)[(long long)row * p.N + col] = acc[m][n][i] + bcol[n];
      }
  }
}

}  // namespace

void launch_w8a8_quant(const uint16_t* x, int R, int C, int8_t* codes, float* scales, hipStream_t st) {
  hipLaunchKernelGGL(w8a8_quant_kernel<0>, dim3(C / QB, (R + QB - 1) / QB), dim3(256), 0, st, x, R, C, codes,
                     scales, nullptr, nullptr, nullptr, nullptr);
}

void launch_w8a8_rmsnorm_quant(const uint16_t* x, const float* gamma, float eps, int R, int C, int8_t* codes,
                               float* scales, float* inv_rms, hipStream_t st) {
  launch_rms_inverse(x, R, C, eps, inv_rms, st);
  hipLaunchKernelGGL(w8a8_quant_kernel<1>, dim3(C / QB, (R + QB - 1) / QB), dim3(256), 0, st, x, R, C, codes,
                     scales, inv_rms, gamma, nullptr, nullptr);
}

void launch_w8a8_layernorm_quant(const uint16_t* x, const float* gamma, const float* beta, float eps, int R, int C,
                                 int8_t* codes, float* scales, float* mean, float* rstd, hipStream_t st) {
  launch_layernorm_stats(x, R, C, eps, mean, rstd, st);
  hipLaunchKernelGGL(w8a8_quant_kernel<2>, dim3(C / QB, (R + QB - 1) / QB), dim3(256), 0, st, x, R, C, codes,
                     scales, rstd, gamma, mean, beta);
}

hipError_t launch_w8a8_gemm(const int8_t* x, const float* sx, const int8_t* w, const float* sw, const float* bias,
                            int M, int N, int K, void* out, int out_bf16, hipStream_t st) {
  GemmParams p;
  p.x = x;
  p.sx = sx;
  p.w = w;
  p.sw = sw;
  p.bias = bias;
  p.out = out;
  p.M = M;
  p.N = N;
  p.K = K;
  p.nkb = K / QB;
  p.mt = (M + GT - 1) / GT;
  p.nt = (N + GT - 1) / GT;
  const long long tiles = (long long)p.mt * p.nt;
  p.per_xcd = (int)((tiles + 7) / 8);
  p.out_bf16 = out_bf16;
  // the attribute is per kernel: set once per process (the first status is kept)
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute((const void*)w8a8_gemm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  });
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(w8a8_gemm_kernel, dim3(8 * p.per_xcd), dim3(NTHR), LDS_BYTES, st, p);
  return hipSuccess;
}

}  // namespace sqattn
