// Host-side launchers of the sqattn kernels (all enqueue on the given stream).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqattn {

// Element strides of a [B, H, N, d] operand with d contiguous: row r of head
// (b, h) starts at b*sb + h*sh + r*sn.  Contiguous: {H*N*d, N*d, d, H}.
struct Lay {
  long long sb, sh, sn;
  int H;
};
__host__ __device__ inline Lay contiguous_lay(int H, int N, int d) {
  return Lay{(long long)H * N * d, (long long)N * d, (long long)d, H};
}
__host__ __device__ inline long long lay_row(const Lay& l, long long bh, long long r) {
  return (bh / l.H) * l.sb + (bh % l.H) * l.sh + r * l.sn;
}

// RMSNorm applied on load (the per-token q/k normalization in front of
// attention): a bf16 value x of token n of batch b, head h, channel c is read
// as bf16(fl32(fl32(x * r[b*N + n]) * gamma[h*d + c])) (gamma NULL: weight 1),
// bf16 rounding to nearest even.  Inactive when r is NULL.
struct RowNorm {
  const float* r = nullptr;
  const float* gamma = nullptr;
};

int kmean_chunks(int BH, int N);
void launch_kmean(const uint16_t* k, const Lay& lk, int BH, int N, int d, uint64_t* partial, float* mean,
                  hipStream_t st, const RowNorm& nm = RowNorm{});
void launch_quant_i8(const uint16_t* x, const Lay& lx, int BH, int N, int d, int block, const float* mean,
                     int8_t* codes, float* scales, hipStream_t st, const RowNorm& nm = RowNorm{});
void launch_v_tiles_bf16(const uint16_t* v, const Lay& lv, int BH, int N, int d, uint16_t* vt, hipStream_t st);
void launch_quant_v_fp8(const uint16_t* v, const Lay& lv, int BH, int N, int d, uint8_t* codes, uint8_t* vt,
                        float* scales, hipStream_t st);
void launch_v_tiles_fp8(const uint8_t* codes, int BH, int N, int d, uint8_t* vt, hipStream_t st);

struct AttnParams {
  const int8_t* q;
  const float* sq;
  const int8_t* k;
  const float* sk;
  const void* vt;
  const float* sv;
  void* out;      // fp32, or bf16 (round to nearest even) when out_bf16
  int out_bf16;
  const uint8_t* mask;  // block-sparse mask [BH][mq][nt] (nonzero = computed), or null (dense)
  int mq;               // mask rows per head: ceil(N / 128)
  Lay lo;               // element strides of the output rows
  int N, nq, q_block, nt, BH, qtiles, per_xcd;
  float scale_log2e;
};

void launch_attention(const AttnParams& p, int d, int pv, hipStream_t st);
// 16-bit P.V kernel (software-pipelined); p.qtiles and p.per_xcd must be set.
void launch_attention_bf16(const AttnParams& p, int d, hipStream_t st);
// FP8 P.V kernel (software-pipelined, running max per tile); same requirements.
void launch_attention_fp8(const AttnParams& p, int d, hipStream_t st);

// W8A8 linear layer: 128x128 block quantizer and the block-scaled INT8 GEMM.
// RMSNorm: inv_rms[r] = fl32(1 / fl32(sqrt(fl32(mean_k x[r,k]^2 + eps)))), the mean
// square rounded once from its exact value (norm.hip).
void launch_rms_inverse(const uint16_t* x, int R, int C, float eps, float* inv_rms, hipStream_t st);
// LayerNorm statistics: mean[r] = fl32(sum_k x[r,k] / C) (exact sum rounded once),
// rstd[r] = fl32(1 / fl32(sqrt(fl32(var + eps)))), var = fl32(sum_k d^2 / C) with
// d = fl32(x - mean) (exact sum of the binary32 squares rounded once) (norm.hip).
void launch_layernorm_stats(const uint16_t* x, int R, int C, float eps, float* mean, float* rstd, hipStream_t st);
// the same over B*N token rows of C contiguous values each, row (b, n) at
// x + b*sb + n*sn, into inv_rms[b*N + n]
void launch_rms_inverse_rows(const uint16_t* x, int B, int N, int C, long long sb, long long sn, float eps,
                             float* inv_rms, hipStream_t st);

void launch_w8a8_quant(const uint16_t* x, int R, int C, int8_t* codes, float* scales, hipStream_t st);
// RMSNorm (per-row inverse RMS into inv_rms) fused with the block quantization
void launch_w8a8_rmsnorm_quant(const uint16_t* x, const float* gamma, float eps, int R, int C, int8_t* codes,
                               float* scales, float* inv_rms, hipStream_t st);
// LayerNorm (mean, rstd per row) fused with the block quantization
void launch_w8a8_layernorm_quant(const uint16_t* x, const float* gamma, const float* beta, float eps, int R, int C,
                                 int8_t* codes, float* scales, float* mean, float* rstd, hipStream_t st);
void launch_w8a8_gemm(const int8_t* x, const float* sx, const int8_t* w, const float* sw, const float* bias,
                      int M, int N, int K, void* out, int out_bf16, hipStream_t st);

}  // namespace sqattn
