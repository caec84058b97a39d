/*
 * sqattn.h - low-bit quantized self-attention on AMD Instinct MI355X (gfx950).
 *
 * The operation is the quantized attention step of TurboDiffusion's video-DiT
 * denoiser (SageAttention2++): Q and K are quantized per block to INT8 so that
 * QK^T runs on the integer matrix units, then softmax, then P.V in 16-bit or
 * FP8 (jefxiong.cn "AIGC weekend special 5.10", section 1.2, item (1);
 * digipub.cc TurboDiffusion article, attention-acceleration paragraph; GVCLab
 * research log 2026-09-02, section 5.5 table, SageAttention2 row).  K is first
 * smoothed by removing its per-channel mean over tokens (the outlier smoothing
 * in the SageAttention2 title, GVCLab Video-Generation-101 systems survey,
 * reference [3]).
 *
 * Conventions for every entry point
 *   - Tensors are DEVICE pointers to contiguous [B, H, N, d] row-major data
 *     (BHND), 16-byte aligned.  bf16 data is passed as raw 16-bit patterns.
 *   - Per-block scale arrays are contiguous [B, H, nblocks] float32 with
 *     nblocks = ceil(N / block); block i covers rows [i*block, min(N, (i+1)*block))
 *     and all d channels of one (b, h) head.
 *   - The caller owns every buffer.  The library keeps no pointer after a call
 *     returns and frees nothing it did not allocate.  Its only global state is
 *     a thread-local error message.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *     runs asynchronously; the call returns once it is enqueued.  Output
 *     buffers must not alias inputs.
 *   - Status codes are returned, never thrown.  Argument problems are reported
 *     before anything is enqueued.  There is no fallback path: a request this
 *     library has no kernel for returns SQATTN_ERR_UNSUPPORTED.
 *   - Results are deterministic: identical inputs give bit-identical outputs
 *     (fixed reduction orders, no floating-point atomics).
 *
 * Numerics (where the method statement is silent, these are the readings used)
 *   - K mean: mu[c] = fl32(S_c / N), S_c the exact sum of the bf16 values over
 *     the N tokens (192-bit fixed point, rounded once, nearest-even).  A head
 *     holding any |K| >= 2^33 is outside that accumulator's range: its mu is
 *     set to NaN (and the codes/scales derived from it are meaningless).
 *   - K' = fl32(K - mu) (IEEE binary32, subnormals kept).  Q is not smoothed.
 *   - INT8 scale s = fl32(absmax / 127), correctly rounded; s = 0 for an
 *     all-zero block.  Code = clamp(rne(fl32(x / s)), -127, 127), i.e. the
 *     correctly rounded binary32 quotient rounded half-to-even to an integer;
 *     code = 0 where s = 0.  -128 never occurs.
 *   - FP8 V: s_v = fl32(absmax / 448) per block of 64 rows; code =
 *     E4M3FN(fl32(V / s_v)) (OCP E4M3, bias 7, max 448, nearest-even,
 *     saturating, sign of zero kept); code = 0 where s_v = 0.
 *   - Attention is non-causal over all N keys.  Logits are
 *     D * sQ * sK * scale with D the exact int32 dot product of the codes.
 *     P.V accumulates in fp32; the output is fp32.
 *     With SQATTN_PV_BF16 each row is exponentiated against a reference: the
 *     max logit of its first 32 keys, or, for every row of a 256-row block in
 *     which some row's sum of weights reaches 2^64, the exact row max.  P is
 *     rounded to bf16 for P.V; the row sum adds the fp32 values of P (for the
 *     last, masked tile the bf16 values).  The normalised result is the same
 *     softmax; only roundings differ.
 *     With SQATTN_PV_FP8_E4M3 the kernel rounds 448 * exp(s - m_tile) to E4M3
 *     (m_tile the running max after each 64-key tile) and keeps the unrounded
 *     values in the row sum.
 */
#ifndef SQATTN_H_
#define SQATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SQATTN_VERSION 10100 /* 1.1.0 */

typedef enum {
  SQATTN_OK = 0,
  SQATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad option */
  SQATTN_ERR_UNSUPPORTED = 2, /* valid request with no kernel (e.g. d not in {64,128}) */
  SQATTN_ERR_WORKSPACE = 3,   /* supplied workspace smaller than required */
  SQATTN_ERR_HIP = 4,         /* the HIP runtime reported an error when enqueuing */
  SQATTN_ERR_RANGE = 5        /* sizes whose index arithmetic would overflow */
} sqattn_status;

typedef enum { SQATTN_PV_BF16 = 0, SQATTN_PV_FP8_E4M3 = 1 } sqattn_pv_dtype;

/* Output element type (sqattn_opts.out_dtype). */
typedef enum { SQATTN_OUT_FP32 = 0, SQATTN_OUT_BF16 = 1 } sqattn_out_dtype;

/* Block sizes and output type.  A zero field takes its default.  q_block:
 * any multiple of 16 (default 128), or 1 for one scale per query row (the
 * granularity of the kernel's Q operand, where each lane holds one row; it
 * costs the attention kernel nothing and helps heavy-tailed Q most).  k_block: 64 (the attention tile;
 * default).  v_block: 64 (FP8 only; default).  out_dtype: SQATTN_OUT_FP32
 * (default) or SQATTN_OUT_BF16, the fp32 result rounded to nearest even.
 * smooth_q: 0 (default) or 1, Q smoothing in the forward entry points (dense,
 * without the q/k RMSNorm; q_block 64, 128 or 256): each Q block's exact
 * per-channel mean is removed before the block is quantized and returns as an
 * logit bias mu_b . K'_j in units of sQ sK (binary32), added to the scores
 * (the outlier smoothing of the SageAttention2 title, GVCLab
 * Video-Generation-101 systems survey, reference [3], applied to Q).  A block
 * of equal rows (scale 0) is quantized plainly.  The attend entry points
 * (already quantized Q) refuse it.
 * second_pass_count: NULL (default), or a device pointer to one uint32 that
 * the attention kernel increments (atomically, on the call's stream) once for
 * every work item -- one head's 256 query rows -- that took the rare exact-max
 * second pass of the 16-bit P.V path (a row sum of the one-pass schedule
 * reached its headroom); the caller zeroes it and reads it after the stream
 * has run.  The FP8 path rebases every tile and never takes that pass.
 * Divided by B * H * ceil(N / 256) it is the fallback ratio of the call. */
typedef struct sqattn_opts {
  int q_block;
  int k_block;
  int v_block;
  int out_dtype;
  int smooth_q;
  uint32_t* second_pass_count;
} sqattn_opts;

/* SQATTN_VERSION of the loaded library. */
int sqattn_version(void);

/* Static description of a status code (never NULL). */
const char* sqattn_status_string(int status);

/* Message of the last failing call on this thread ("" if none).  Valid until
 * the next library call on the same thread. */
const char* sqattn_last_error(void);

/*
 * Bytes of device workspace that sqattn_quantize_qk needs for these sizes
 * (the partial sums of the exact K mean).  0 for invalid sizes.
 */
size_t sqattn_quantize_qk_workspace_bytes(int B, int H, int N, int d);

/*
 * Quantize Q and K (smoothing K by its per-channel mean first): the low-bit
 * Q/K of the method (jefxiong.cn "AIGC weekend special 5.10", section 1.2
 * item (1): Q and K to low bit so that QK^T runs on integer matrix units) with
 * the outlier smoothing of K (GVCLab Video-Generation-101 systems survey,
 * reference [3] title); per-block INT8 with absmax/127 scales as read above.
 *   q, k      : bf16 [B,H,N,d] inputs.
 *   q_i8      : int8 [B,H,N,d] codes of Q;  q_scale : float [B,H,ceil(N/q_block)].
 *   k_i8      : int8 [B,H,N,d] codes of K'; k_scale : float [B,H,ceil(N/k_block)].
 *   k_mean    : float [B,H,d], the mean that was removed from K.
 *   q_block   : 1 (one scale per row) or a multiple of 16; k_block :
 *               multiple of 16 (64 for use with sqattn_attend_quantized).
 *   workspace : device memory of at least sqattn_quantize_qk_workspace_bytes();
 *               NULL makes the library allocate it stream-ordered on `stream`
 *               (and free it after use, stream-ordered).
 * B, H, N >= 1; d in {64, 128}; B*H*N*d < 2^40.
 */
int sqattn_quantize_qk(const void* q, const void* k, int B, int H, int N, int d, int q_block,
                       int k_block, int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                       float* k_mean, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sqattn_quantize_qk for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same passes and results, with the K-mean partial sums in a scratch array
 * the library holds in device memory (16 MiB per GPU it runs on, kept until
 * the process ends) instead of a workspace.  Nothing is allocated.
 * Returns SQATTN_ERR_WORKSPACE when the sizes need more scratch than that
 * (sqattn_quantize_qk_workspace_bytes() > 16 MiB, i.e. roughly B*H*S*d > 2^19
 * with S the K-mean chunks per head; every workload of up to 2048 heads at
 * d = 128 fits).  Every entry of the scratch is written before it is read,
 * so the previous call's contents do not matter; calls that overlap in time
 * on one GPU (different streams, or host threads without ordering) share the
 * array and race.
 */
int sqattn_quantize_qk_noalloc(const void* q, const void* k, int B, int H, int N, int d,
                               int q_block, int k_block, int8_t* q_i8, float* q_scale,
                               int8_t* k_i8, float* k_scale, float* k_mean, void* stream);

/*
 * Quantize V to OCP E4M3 per block of v_block (= 64) rows (GVCLab research
 * log 2026-09-02, section 5.5 table, SageAttention2 row: FP8 P.V).  The block
 * scale is a power of two, s = 2^e with e the smallest integer >= -127 such
 * that max|V| <= 448 s (0 for an all-zero block), and code = E4M3(V / s),
 * rounded to nearest even: the E8M0 block-scale form the FP8 matrix
 * instructions apply themselves.
 *   v       : bf16 [B,H,N,d];  v_fp8 : uint8 [B,H,N,d] codes;
 *   v_scale : float [B,H,ceil(N/v_block)].
 */
int sqattn_quantize_v_fp8(const void* v, int B, int H, int N, int d, int v_block, uint8_t* v_fp8,
                          float* v_scale, void* stream);

/*
 * Bytes of device workspace sqattn_forward / sqattn_forward_ex need
 * (INT8 Q and K with their scales, the K mean, V in the kernel's tiled
 * transposed layout, and the K mean partial sums).  opts may be NULL.
 * 0 for invalid arguments.
 */
size_t sqattn_workspace_bytes(int B, int H, int N, int d, int pv_dtype, const sqattn_opts* opts);

/*
 * Full forward: out = softmax(Q K^T * scale) V computed on quantized
 * operands (the steps above), out [B,H,N,d] fp32 (bf16 with
 * opts->out_dtype = SQATTN_OUT_BF16 in sqattn_forward_ex) -- the quantized
 * attention step of the DiT denoiser (digipub.cc TurboDiffusion article,
 * attention-acceleration paragraph: SageAttention2++; jefxiong.cn "AIGC
 * weekend special 5.10", section 1.2 item (1); GVCLab research log
 * 2026-09-02, section 5.5 table: 16-bit or FP8 P.V).
 *   scale     : softmax scale applied to the logits (commonly 1/sqrt(d)),
 *               finite and >= 0.
 *   pv_dtype  : SQATTN_PV_BF16 or SQATTN_PV_FP8_E4M3.
 *   workspace : >= sqattn_workspace_bytes() bytes of device memory, 256-byte
 *               aligned, or NULL for a stream-ordered allocation by the
 *               library on `stream`.
 * Defaults: q_block 128, k_block 64, v_block 64.
 */
int sqattn_forward(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                   float scale, int pv_dtype, void* out, void* workspace, size_t workspace_bytes,
                   void* stream);

/* sqattn_forward with explicit block sizes (opts may be NULL = defaults). */
int sqattn_forward_ex(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                      float scale, int pv_dtype, void* out, void* workspace,
                      size_t workspace_bytes, void* stream, const sqattn_opts* opts);

/*
 * V in the attention kernel's tile layout ("packed V").  Tile t of a head
 * holds keys [64t, 64t+64) transposed, [d][64], zero past N:
 *   SQATTN_PV_BF16     : bf16, element (c, j) at ((bh*nt + t)*d + c)*64 + j.
 *   SQATTN_PV_FP8_E4M3 : E4M3 codes, one byte per element; within each
 *                        64-byte channel row key j sits at position
 *                        32*((j/8)%2) + 8*(j/16) + j%8 (the order the FP8
 *                        matrix instruction consumes keys in).
 * nt = ceil(N/64).  Size: sqattn_packed_v_bytes().
 *   v : bf16 [B,H,N,d] for SQATTN_PV_BF16; E4M3 codes [B,H,N,d] (as written
 *       by sqattn_quantize_v_fp8) for SQATTN_PV_FP8_E4M3.
 */
size_t sqattn_packed_v_bytes(int B, int H, int N, int d, int pv_dtype);
int sqattn_pack_v(const void* v, int B, int H, int N, int d, int pv_dtype, void* v_packed,
                  void* stream);

/*
 * Attention on quantized operands: the logits from the INT8 codes of Q and
 * smoothed K on the integer matrix units, softmax, P.V in bf16 or FP8
 * (jefxiong.cn "AIGC weekend special 5.10", section 1.2 item (1); GVCLab
 * research log 2026-09-02, section 5.5 table, SageAttention2 row), i.e. the
 * forward without its quantization steps.
 *   q_i8/q_scale/k_i8/k_scale : as written by sqattn_quantize_qk with
 *              k_block = 64 and q_block = opts->q_block (default 128).
 *   v        : [B,H,N,d] bf16 for SQATTN_PV_BF16; E4M3 codes (uint8) as
 *              written by sqattn_quantize_v_fp8 for SQATTN_PV_FP8_E4M3.
 *   v_scale  : [B,H,ceil(N/64)] from sqattn_quantize_v_fp8 for FP8; NULL for bf16.
 *              The FP8 kernel applies each scale as its binary exponent (an
 *              E8M0 scale of the matrix instruction): scales must be powers of
 *              two in [2^-127, 2^127], or 0 with all-zero codes, as
 *              sqattn_quantize_v_fp8 writes them; other values act as the
 *              power of two at or below them.
 *   out      : [B,H,N,d], fp32 or bf16 as opts->out_dtype says.
 * V is first laid out in the kernel's tile layout (as sqattn_pack_v) in a
 * temporary of sqattn_packed_v_bytes() allocated and freed stream-ordered on
 * `stream`; arguments are validated before anything is allocated.
 */
int sqattn_attend_quantized(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                            const float* k_scale, const void* v, const float* v_scale,
                            int B, int H, int N, int d, float scale, int pv_dtype,
                            const sqattn_opts* opts, void* out, void* stream);

/*
 * sqattn_attend_quantized on V already in the kernel's tile layout: a single
 * kernel launch (the hot kernel alone, for kernel timing).
 *   v_packed : from sqattn_pack_v with the same pv_dtype.
 * Everything else as sqattn_attend_quantized.
 */
int sqattn_attend_packed(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                         const float* k_scale, const void* v_packed, const float* v_scale, int B,
                         int H, int N, int d, float scale, int pv_dtype, const sqattn_opts* opts,
                         void* out, void* stream);

/*
 * Block-sparse attention: the same step computed only on the (query block,
 * key tile) pairs a caller-supplied mask keeps -- the kernel half of the
 * "sparse + low-bit" composition (digipub.cc TurboDiffusion article, SLA
 * paragraph: sparse attention built on SageAttention, orthogonal to its
 * low-bit arithmetic; GVCLab Video-Generation-101 systems survey,
 * SpargeAttention row: selector, sparse layout, low-bit kernel).  The
 * selector that produces the mask is the caller's.
 *   block_mask : device uint8 [B, H, ceil(N/128), ceil(N/64)], row-major;
 *                entry (b, h, i, j) nonzero = query rows [128i, 128i+128)
 *                attend to keys [64j, 64j+64).  Read only.
 * Keys of a zero entry get zero weight (the softmax runs over the kept keys;
 * quantization, the K mean and every scale are those of the dense step).  A
 * query row whose mask row keeps nothing is written as zeros.  A work-group
 * of 256 query rows visits the union of its two mask rows' tiles, so its
 * work scales with the kept fraction.  Inputs must be finite (a NaN in a
 * dropped tile's V can reach rows of the other query block of the same
 * work-group through 0 * NaN).  N <= 262144 (4096 key tiles), else
 * SQATTN_ERR_UNSUPPORTED.  Everything else as sqattn_forward_ex /
 * sqattn_attend_quantized (raw V) / sqattn_attend_packed (packed V).
 */
int sqattn_forward_sparse(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                          float scale, int pv_dtype, const uint8_t* block_mask, void* out,
                          void* workspace, size_t workspace_bytes, void* stream,
                          const sqattn_opts* opts);
int sqattn_attend_quantized_sparse(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                   const float* k_scale, const void* v, const float* v_scale,
                                   int B, int H, int N, int d, float scale, int pv_dtype,
                                   const uint8_t* block_mask, const sqattn_opts* opts, void* out,
                                   void* stream);
int sqattn_attend_packed_sparse(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                const float* k_scale, const void* v_packed, const float* v_scale,
                                int B, int H, int N, int d, float scale, int pv_dtype,
                                const uint8_t* block_mask, const sqattn_opts* opts, void* out,
                                void* stream);

/*
 * sqattn_forward_ex / sqattn_forward_sparse on strided operands, so that a
 * DiT block can hand over its tensors without layout copies: Q, K and V as
 * views of a fused QKV projection output [B, N, 3, H, d], the output written
 * straight into the [B, N, H, d] (= [B*N, H*d]) input of the output
 * projection.  (The step right before attention in the DiT block:
 * digipub.cc TurboDiffusion article, linear-layer and normalization
 * paragraphs.)
 *   in_strides  : int64 [9], element strides (b, h, n) of q, then k, then v;
 *                 the d channels of a row are contiguous.  Row r of head
 *                 (b, h) of q starts at q + b*s[0] + h*s[1] + r*s[2].
 *   out_strides : int64 [3] (b, h, n) of out, or NULL for contiguous
 *                 [B, H, N, d].  Output rows must not overlap.
 *   block_mask  : as sqattn_forward_sparse, or NULL (dense).
 * Every stride must be a non-negative multiple of 8 elements (16-byte rows)
 * and at most 2^40; base pointers 16-byte aligned.  Results are bit-identical
 * to the contiguous entry points on the same values.
 */
int sqattn_forward_strided(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                           const int64_t* in_strides, const int64_t* out_strides, float scale,
                           int pv_dtype, const uint8_t* block_mask, void* out, void* workspace,
                           size_t workspace_bytes, void* stream, const sqattn_opts* opts);

/*
 * sqattn_forward_strided with the per-token RMSNorm of Q and K fused into
 * their quantization: the q/k normalization a DiT attention block applies
 * over each token's H*d features right after its QKV projection, the step
 * in front of Q/K quantization (digipub.cc TurboDiffusion article, paragraph
 * on other optimizations: RMSNorm rewritten as a custom kernel).  Bit for
 * bit the same as normalizing Q and K into bf16 tensors and calling
 * sqattn_forward_strided on them, without writing them to memory:
 *   q'[b,h,n,c] = bf16(fl32(fl32(q[b,h,n,c] * r_q[b,n]) * gamma_q[h*d + c]))
 *   r_q[b,n]    = fl32(1 / fl32(sqrt(fl32(mu2 + eps)))),
 *   mu2         = fl32(sum over h, c of q[b,h,n,c]^2 / (H*d)), the exact sum
 *                 rounded once (as sqattn_w8a8_rmsnorm_quantize),
 * likewise k' with gamma_k; bf16 rounding is nearest-even (a NaN stays a
 * NaN; a token holding Inf or NaN gets r = NaN).
 *   gamma_q, gamma_k : float32 [H*d] device pointers, or NULL (weight 1).
 *   eps              : finite, > 0.
 *   in_strides       : as sqattn_forward_strided, required when H > 1: each
 *                      token's H*d values of q and of k must be contiguous
 *                      (head stride in_strides[1] = in_strides[4] = d), as in
 *                      a fused QKV projection output [B, N, 3, H, d].
 * V, out_strides, block_mask, opts and the rest as sqattn_forward_strided.
 * workspace: >= sqattn_forward_qknorm_workspace_bytes() bytes (the forward's
 * workspace plus 2*B*N floats), 256-byte aligned, or NULL.
 */
size_t sqattn_forward_qknorm_workspace_bytes(int B, int H, int N, int d, int pv_dtype,
                                             const sqattn_opts* opts);
int sqattn_forward_qknorm(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                          const int64_t* in_strides, const int64_t* out_strides, const float* gamma_q,
                          const float* gamma_k, float eps, float scale, int pv_dtype,
                          const uint8_t* block_mask, void* out, void* workspace,
                          size_t workspace_bytes, void* stream, const sqattn_opts* opts);

/*
 * W8A8 block-wise INT8 linear layer, y = x W^T (+ b): the projections on
 * either side of attention with weights and activations both quantized to
 * INT8 in 128x128 blocks and the products on the INT8 matrix units
 * (jefxiong.cn "AIGC weekend special 5.10", section 1.2 item (4), W8A8;
 * digipub.cc TurboDiffusion article, linear-layer quantization paragraph).
 *
 * Layout (all row-major, device pointers, 16-byte aligned):
 *   x  : [M, K] activations (tokens x in-features), bf16 bits.
 *   W  : [N, K] weights (out-features x in-features), the nn.Linear layout.
 *   codes of a [R, K] matrix : int8 [R, K];  scales : float32
 *        [ceil(R/128), K/128], scale (i, j) for rows [128i, min(R, 128i+128))
 *        and columns [128j, 128j+128).
 *   b  : float32 [N] or NULL;  y : [M, N], fp32 or bf16 (out_dtype).
 * K must be a positive multiple of 128 (the block edge) and at most 2^20;
 * M and N may be 0: then nothing is enqueued and the data pointers are not
 * inspected (they may be NULL); M, N <= 65535 * 128.
 * Inputs must be finite (the result for Inf or NaN inputs is unspecified).
 *
 * Numerics: scale s = fl32(absmax / 127) per block (0 for an all-zero block),
 * code = clamp(rne(fl32(v / s)), -127, 127), as for the attention's Q/K
 * blocks.  For each 128-wide slice j of K the exact int32 partial
 * D_j[m, n] = sum over the slice of cx[m, k] * cw[n, k] is scaled by
 * fl32(sx[m/128, j] * sw[n/128, j]) and added to an fp32 accumulator with
 * one fused multiply-add per slice, in increasing j; then b[n] is added and
 * the sum is stored as fp32 or rounded to nearest-even bf16.
 */

/* Quantize a bf16 [rows, cols] matrix (x or W) to INT8 codes and 128x128
 * block scales.  cols: positive multiple of 128, <= 2^20;
 * 0 <= rows <= 65535 * 128. */
int sqattn_w8a8_quantize(const void* x, int rows, int cols, int8_t* codes, float* scales,
                         void* stream);

/* y = x W^T (+ b) from codes and scales written by sqattn_w8a8_quantize.
 *   bias      : float32 [N] or NULL.
 *   out_dtype : SQATTN_OUT_FP32 or SQATTN_OUT_BF16. */
int sqattn_w8a8_gemm(const int8_t* x_codes, const float* x_scales, const int8_t* w_codes,
                     const float* w_scales, const float* bias, int M, int N, int K, int out_dtype,
                     void* out, void* stream);

/* Bytes of workspace sqattn_w8a8_linear needs (codes and scales of x).
 * 0 for invalid sizes. */
size_t sqattn_w8a8_workspace_bytes(int M, int K);

/* The layer on bf16 activations and pre-quantized weights: quantizes x into
 * the workspace, then sqattn_w8a8_gemm.  workspace: >= sqattn_w8a8_workspace_bytes()
 * bytes, 256-byte aligned, or NULL for a stream-ordered allocation. */
int sqattn_w8a8_linear(const void* x, const int8_t* w_codes, const float* w_scales,
                       const float* bias, int M, int N, int K, int out_dtype, void* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * RMSNorm fused with the W8A8 quantization of the projection input: the
 * normalization in front of the QKV projection of a DiT block, written as a
 * custom kernel (digipub.cc TurboDiffusion article, paragraph on other
 * optimizations: LayerNorm and RMSNorm reimplemented for speed).  Per row of
 * x [rows, cols] (bf16):
 *   mu2 = fl32(S / cols), S = sum of x^2 computed exactly (rounded once);
 *   r   = fl32(1 / fl32(sqrt(fl32(mu2 + eps))))   (binary32 operations);
 *   y   = fl32(fl32(x * r) * gamma)   (gamma fp32 [cols], or NULL: fl32(x * r));
 * then y (binary32, not rounded to bf16) gets the codes and 128x128 block
 * scales of sqattn_w8a8_quantize.
 *   inv_rms : fp32 [rows] output, r per row (NaN for a row holding Inf/NaN).
 *   eps     : finite, > 0.
 * Sizes as sqattn_w8a8_quantize.
 */
int sqattn_w8a8_rmsnorm_quantize(const void* x, const float* gamma, float eps, int rows, int cols,
                                 int8_t* codes, float* scales, float* inv_rms, void* stream);

/* Workspace of sqattn_w8a8_linear_rmsnorm (codes, scales, inverse RMS). */
size_t sqattn_w8a8_rmsnorm_workspace_bytes(int M, int K);

/* y = RMSNorm(x) W^T (+ b) on bf16 x [M, K]: sqattn_w8a8_rmsnorm_quantize
 * into the workspace, then sqattn_w8a8_gemm. */
int sqattn_w8a8_linear_rmsnorm(const void* x, const float* gamma, float eps, const int8_t* w_codes,
                               const float* w_scales, const float* bias, int M, int N, int K,
                               int out_dtype, void* out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * LayerNorm fused with the W8A8 quantization of the projection input: the
 * normalization in front of a DiT block's QKV projection (its modulation,
 * x_norm * (1 + scale) + shift, as gamma = 1 + scale and beta = shift),
 * written as a custom kernel (digipub.cc TurboDiffusion article, paragraph
 * on other optimizations: LayerNorm and RMSNorm reimplemented).  Per row of
 * x [rows, cols] (bf16), every result rounded once and independent of the
 * summation order:
 *   mu   = fl32(sum x / cols)              (exact sum);
 *   d    = fl32(x - mu);
 *   var  = fl32(sum d^2 / cols)            (exact sum of the binary32 squares);
 *   rstd = fl32(1 / fl32(sqrt(fl32(var + eps))));
 *   y    = fl32(fl32(fl32(d * rstd) * gamma) + beta)
 *          (gamma, beta fp32 [cols], each may be NULL: no multiply / no add);
 * then y (binary32) gets the codes and 128x128 block scales of
 * sqattn_w8a8_quantize.
 *   mean, rstd : fp32 [rows] outputs (NaN for a row holding Inf or NaN).
 *   eps        : finite, > 0.
 * Sizes as sqattn_w8a8_quantize.  Inputs are meant to be finite.
 */
int sqattn_w8a8_layernorm_quantize(const void* x, const float* gamma, const float* beta, float eps,
                                   int rows, int cols, int8_t* codes, float* scales, float* mean,
                                   float* rstd, void* stream);

/* Workspace of sqattn_w8a8_linear_layernorm (codes, scales, mean, rstd). */
size_t sqattn_w8a8_layernorm_workspace_bytes(int M, int K);

/* y = LayerNorm(x) W^T (+ b) on bf16 x [M, K]: sqattn_w8a8_layernorm_quantize
 * into the workspace, then sqattn_w8a8_gemm. */
int sqattn_w8a8_linear_layernorm(const void* x, const float* gamma, const float* beta, float eps,
                                 const int8_t* w_codes, const float* w_scales, const float* bias,
                                 int M, int N, int K, int out_dtype, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SQATTN_H_ */
