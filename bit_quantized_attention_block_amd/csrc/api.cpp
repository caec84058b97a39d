// C-ABI of the sqattn library: argument validation, workspace layout and the
// launch sequence of each entry point.  See include/sqattn.h for the contract.
#include "../../include/sqattn.h"
#ifdef SQATTN_DEBUG
#include "../../include/sqattn_debug.h"
#endif

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstdio>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Sizes {
  long long BH, N, d, nq, nk, nt, S;
};

// Common shape checks.  Returns SQATTN_OK or an error (message set).
int check_shape(int B, int H, int N, int d, Sizes* sz) {
  if (B < 1 || H < 1 || N < 1) return fail(SQATTN_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if (d != 64 && d != 128) return fail(SQATTN_ERR_UNSUPPORTED, "head dimension d must be 64 or 128");
  if (N >= (1 << 24)) return fail(SQATTN_ERR_RANGE, "N must be below 2^24");
  long long BH = (long long)B * H;
  if (BH > 65535) return fail(SQATTN_ERR_RANGE, "B*H must be at most 65535");
  if (BH * (long long)N * d >= (1LL << 40)) return fail(SQATTN_ERR_RANGE, "B*H*N*d must be below 2^40");
  sz->BH = BH;
  sz->N = N;
  sz->d = d;
  sz->nt = (N + sqattn::KT - 1) / sqattn::KT;
  sz->S = sqattn::kmean_chunks((int)BH, N);
  return SQATTN_OK;
}

int check_block(int b, const char* name) {
  if (b < 16 || (b % 16) != 0 || b > (1 << 24))
    return fail(SQATTN_ERR_INVALID_ARG, std::string(name) + " must be a positive multiple of 16");
  return SQATTN_OK;
}

// Q blocks: a multiple of 16 rows, or 1 (one scale per query row).
int check_q_block(int b) {
  if (b == 1) return SQATTN_OK;
  if (b < 16 || (b % 16) != 0 || b > (1 << 24))
    return fail(SQATTN_ERR_INVALID_ARG, "q_block must be 1 or a positive multiple of 16");
  return SQATTN_OK;
}

int check_ptr(const void* p, const char* name, size_t align) {
  if (!p) return fail(SQATTN_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned(p, align))
    return fail(SQATTN_ERR_INVALID_ARG, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return SQATTN_OK;
}

struct Opts {
  int q_block, k_block, v_block, out_bf16, smooth_q;
  uint32_t* second_pass;
};

int resolve_opts(const sqattn_opts* o, Opts* r) {
  r->q_block = 128;
  r->k_block = 64;
  r->v_block = 64;
  r->out_bf16 = 0;
  r->smooth_q = 0;
  r->second_pass = nullptr;
  if (!o) return SQATTN_OK;
  if (o->out_dtype != SQATTN_OUT_FP32 && o->out_dtype != SQATTN_OUT_BF16)
    return fail(SQATTN_ERR_INVALID_ARG, "opts.out_dtype must be SQATTN_OUT_FP32 or SQATTN_OUT_BF16");
  r->out_bf16 = o->out_dtype == SQATTN_OUT_BF16;
  if (o->q_block) r->q_block = o->q_block;
  if (o->k_block) r->k_block = o->k_block;
  if (o->v_block) r->v_block = o->v_block;
  if (o->smooth_q != 0 && o->smooth_q != 1) return fail(SQATTN_ERR_INVALID_ARG, "opts.smooth_q must be 0 or 1");
  r->smooth_q = o->smooth_q;
  if (o->second_pass_count && !aligned(o->second_pass_count, 4))
    return fail(SQATTN_ERR_INVALID_ARG, "opts.second_pass_count is not 4-byte aligned");
  r->second_pass = o->second_pass_count;
  int s;
  if ((s = check_q_block(r->q_block))) return s;
  if (r->k_block != sqattn::KT) return fail(SQATTN_ERR_UNSUPPORTED, "k_block must be 64 (the attention tile)");
  if (r->v_block != sqattn::KT) return fail(SQATTN_ERR_UNSUPPORTED, "v_block must be 64");
  if (r->smooth_q && r->q_block != 64 && r->q_block != 128 && r->q_block != 256)
    return fail(SQATTN_ERR_UNSUPPORTED, "Q smoothing needs q_block 64, 128 or 256");
  return SQATTN_OK;
}

// Workspace carving.  Each region is 256-byte aligned.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

struct FwdLayout {
  size_t q_i8, k_i8, q_scale, k_scale, k_mean, partial, vt, v_scale, q_mean, q_bias, total;
};

// smooth: Q smoothing (the block means and the bias; the partial sums serve
// the Q means first, then the K mean)
FwdLayout forward_layout(const Sizes& z, int pv, int q_block, bool smooth = false) {
  FwdLayout L;
  Carve c;
  const long long nq = (z.N + q_block - 1) / q_block;
  L.q_i8 = c.take((size_t)(z.BH * z.N * z.d));
  L.k_i8 = c.take((size_t)(z.BH * z.N * z.d));
  L.q_scale = c.take((size_t)(z.BH * nq) * 4);
  L.k_scale = c.take((size_t)(z.BH * z.nt) * 4);
  L.k_mean = c.take((size_t)(z.BH * z.d) * 4);
  L.partial = c.take((size_t)(z.BH * (smooth && nq > z.S ? nq : z.S) * z.d) * 32);
  L.vt = c.take((size_t)(z.BH * z.nt * z.d * sqattn::KT) * (pv == SQATTN_PV_BF16 ? 2 : 1));
  L.v_scale = c.take(pv == SQATTN_PV_BF16 ? 0 : (size_t)(z.BH * z.nt) * 4);
  L.q_mean = c.take(smooth ? (size_t)(z.BH * nq * z.d) * 4 : 0);
  L.q_bias = c.take(smooth ? (size_t)(z.BH * nq * z.nt * sqattn::KT) * 4 : 0);
  L.total = c.off;
  return L;
}

int hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SQATTN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return SQATTN_OK;
}

// Status of a W8A8 GEMM launch: the one-time attribute setup, then the launch.
int gemm_status(hipError_t attr, const char* what) {
  if (attr != hipSuccess)
    return fail(SQATTN_ERR_HIP, std::string(what) + ": setting the GEMM kernel's LDS size: " + hipGetErrorString(attr));
  return hip_check(what);
}

// The attention kernel of the P.V type.  A work item is (head, 256-row query
// block); work-group w runs on XCD w % 8 (round-robin dispatch) and takes item
// (w % 8) * per_xcd + w / 8, so each XCD walks consecutive query blocks of the
// same head, which share K/V tiles through that XCD's L2.
int launch_attention(sqattn::AttnParams p, int d, int pv, hipStream_t st, const char* what) {
#ifdef SQATTN_DEBUG
  {
    const hipError_t e = sqattn::debug_word(&p.debug);
    if (e != hipSuccess) return fail(SQATTN_ERR_HIP, std::string(what) + ": violation word: " + hipGetErrorString(e));
  }
#endif
  p.qtiles = (p.N + sqattn::ATT_QWG - 1) / sqattn::ATT_QWG;
  const long long W = (long long)p.BH * p.qtiles;
  p.per_xcd = (int)((W + 7) / 8);
  const hipError_t e = pv == SQATTN_PV_BF16 ? sqattn::launch_attention_bf16(p, d, st)
                                            : sqattn::launch_attention_fp8(p, d, st);
  if (e != hipSuccess)
    return fail(SQATTN_ERR_HIP, std::string(what) + ": setting the kernel's LDS size: " + hipGetErrorString(e));
  return hip_check(what);
}

// Provides workspace: the caller's, or a stream-ordered allocation freed by
// the destructor (also stream-ordered).
struct Workspace {
  void* ptr = nullptr;
  bool owned = false;
  hipStream_t st = nullptr;
  int acquire(void* user, size_t user_bytes, size_t need, hipStream_t stream) {
    st = stream;
    if (user) {
      if (user_bytes < need)
        return fail(SQATTN_ERR_WORKSPACE, "workspace has " + std::to_string(user_bytes) + " bytes, " +
                                              std::to_string(need) + " needed");
      if (!aligned(user, kAlign)) return fail(SQATTN_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
      ptr = user;
      return SQATTN_OK;
    }
    if (need == 0) return SQATTN_OK;
    hipError_t e = hipMallocAsync(&ptr, need, stream);
    if (e != hipSuccess) return fail(SQATTN_ERR_HIP, std::string("hipMallocAsync: ") + hipGetErrorString(e));
    owned = true;
    return SQATTN_OK;
  }
  ~Workspace() {
    if (owned && ptr) (void)hipFreeAsync(ptr, st);
  }
  template <class T>
  T* at(size_t off) const {
    return (T*)((char*)ptr + off);
  }
};

const float kLog2e = 1.4426950408889634f;

int validate_forward(const void* q, const void* k, const void* v, int B, int H, int N, int d, float scale,
                     int pv, const void* out, const sqattn_opts* opts, Sizes* z, Opts* o) {
  int s;
  if ((s = check_ptr(q, "q", 16)) || (s = check_ptr(k, "k", 16)) || (s = check_ptr(v, "v", 16)) ||
      (s = check_ptr(out, "out", 16)))
    return s;
  if ((s = check_shape(B, H, N, d, z))) return s;
  if (pv != SQATTN_PV_BF16 && pv != SQATTN_PV_FP8_E4M3) return fail(SQATTN_ERR_INVALID_ARG, "unknown pv_dtype");
  if (!std::isfinite(scale) || scale < 0.0f) return fail(SQATTN_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if ((s = resolve_opts(opts, o))) return s;
  z->nq = (N + o->q_block - 1) / o->q_block;
  z->nk = z->nt;
  return SQATTN_OK;
}

// Block-sparse attention keeps a work-group's list of key tiles in LDS.
int check_sparse(int N) {
  if ((N + sqattn::KT - 1) / sqattn::KT > sqattn::SP_MAXT)
    return fail(SQATTN_ERR_UNSUPPORTED,
                "block-sparse attention supports N <= " + std::to_string(sqattn::SP_MAXT * sqattn::KT));
  return SQATTN_OK;
}

// W8A8 sizes: K a positive multiple of 128 up to 2^20, 0 <= rows <= 65535*128.
int check_w8a8_rows(int rows, const char* name) {
  if (rows < 0) return fail(SQATTN_ERR_INVALID_ARG, std::string(name) + " must be >= 0");
  if (rows > 65535 * 128) return fail(SQATTN_ERR_RANGE, std::string(name) + " must be at most 65535*128");
  return SQATTN_OK;
}

int check_w8a8_k(int K) {
  if (K < 128 || (K % 128) != 0)
    return fail(SQATTN_ERR_INVALID_ARG, "K (columns) must be a positive multiple of 128");
  if (K > (1 << 20)) return fail(SQATTN_ERR_RANGE, "K (columns) must be at most 2^20");
  return SQATTN_OK;
}

int check_out_dtype(int out_dtype) {
  if (out_dtype != SQATTN_OUT_FP32 && out_dtype != SQATTN_OUT_BF16)
    return fail(SQATTN_ERR_INVALID_ARG, "out_dtype must be SQATTN_OUT_FP32 or SQATTN_OUT_BF16");
  return SQATTN_OK;
}

size_t w8a8_scale_bytes(long long rows, long long K) { return (size_t)(((rows + 127) / 128) * (K / 128)) * 4; }

}  // namespace

extern "C" {

int sqattn_version(void) { return SQATTN_VERSION; }

#ifdef SQATTN_DEBUG
uint32_t sqattn_debug_violations(void) {
  uint32_t* w = nullptr;
  uint32_t v = 0xFFFFFFFFu;
  if (sqattn::debug_word(&w) != hipSuccess) return v;
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(&v, w, 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemset(w, 0, 4) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
    return 0xFFFFFFFFu;
  return v;
}
#endif

const char* sqattn_status_string(int s) {
  switch (s) {
    case SQATTN_OK: return "ok";
    case SQATTN_ERR_INVALID_ARG: return "invalid argument";
    case SQATTN_ERR_UNSUPPORTED: return "unsupported";
    case SQATTN_ERR_WORKSPACE: return "workspace too small";
    case SQATTN_ERR_HIP: return "HIP runtime error";
    case SQATTN_ERR_RANGE: return "size out of range";
    default: return "unknown status";
  }
}

const char* sqattn_last_error(void) { return g_err.c_str(); }

size_t sqattn_quantize_qk_workspace_bytes(int B, int H, int N, int d) {
  Sizes z;
  std::string keep = g_err;
  if (check_shape(B, H, N, d, &z)) {
    g_err = keep;
    return 0;
  }
  return align_up((size_t)(z.BH * z.S * z.d) * 32);
}

static int quantize_qk_check(const void* q, const void* k, int B, int H, int N, int d, int q_block, int k_block,
                             const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                             const float* k_mean, Sizes* z) {
  g_err.clear();
  int s;
  if ((s = check_ptr(q, "q", 16)) || (s = check_ptr(k, "k", 16)) || (s = check_ptr(q_i8, "q_i8", 16)) ||
      (s = check_ptr(k_i8, "k_i8", 16)) || (s = check_ptr(q_scale, "q_scale", 4)) ||
      (s = check_ptr(k_scale, "k_scale", 4)) || (s = check_ptr(k_mean, "k_mean", 4)))
    return s;
  if ((s = check_shape(B, H, N, d, z))) return s;
  if ((s = check_q_block(q_block)) || (s = check_block(k_block, "k_block"))) return s;
  return SQATTN_OK;
}

// The three passes on validated arguments; partial: the K-mean partial sums,
// kmean_partial_bytes() of device memory (every entry is written before it is read).
static size_t kmean_partial_bytes(const Sizes& z) { return align_up((size_t)(z.BH * z.S * z.d) * 32); }
static void quantize_qk_launch(const void* q, const void* k, int H, int N, int d, int q_block, int k_block,
                               int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                               uint64_t* partial, const Sizes& z, hipStream_t st) {
  const sqattn::Lay lc = sqattn::contiguous_lay(H, N, d);
  sqattn::launch_quant_i8((const uint16_t*)q, lc, (int)z.BH, N, d, q_block, nullptr, q_i8, q_scale, st);
  sqattn::launch_kmean((const uint16_t*)k, lc, (int)z.BH, N, d, partial, k_mean, st);
  sqattn::launch_quant_i8((const uint16_t*)k, lc, (int)z.BH, N, d, k_block, k_mean, k_i8, k_scale, st);
}

int sqattn_quantize_qk(const void* q, const void* k, int B, int H, int N, int d, int q_block, int k_block,
                       int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int s;
  Sizes z;
  if ((s = quantize_qk_check(q, k, B, H, N, d, q_block, k_block, q_i8, q_scale, k_i8, k_scale, k_mean, &z)))
    return s;
  hipStream_t st = (hipStream_t)stream;
  Workspace ws;
  if ((s = ws.acquire(workspace, workspace_bytes, kmean_partial_bytes(z), st))) return s;
  quantize_qk_launch(q, k, H, N, d, q_block, k_block, q_i8, q_scale, k_i8, k_scale, k_mean, ws.at<uint64_t>(0), z,
                     st);
  return hip_check("sqattn_quantize_qk launch");
}

int sqattn_quantize_qk_noalloc(const void* q, const void* k, int B, int H, int N, int d, int q_block, int k_block,
                               int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                               void* stream) {
  int s;
  Sizes z;
  if ((s = quantize_qk_check(q, k, B, H, N, d, q_block, k_block, q_i8, q_scale, k_i8, k_scale, k_mean, &z)))
    return s;
  const size_t need = kmean_partial_bytes(z);
  if (need > sqattn::kStaticScratchBytes)
    return fail(SQATTN_ERR_WORKSPACE, "these sizes need " + std::to_string(need) +
                                          " bytes of scratch; the library's static scratch holds " +
                                          std::to_string(sqattn::kStaticScratchBytes));
  void* scratch = nullptr;
  const hipError_t e = sqattn::static_scratch(&scratch);
  if (e != hipSuccess)
    return fail(SQATTN_ERR_HIP, std::string("device address of the static scratch: ") + hipGetErrorString(e));
  quantize_qk_launch(q, k, H, N, d, q_block, k_block, q_i8, q_scale, k_i8, k_scale, k_mean, (uint64_t*)scratch, z,
                     (hipStream_t)stream);
  return hip_check("sqattn_quantize_qk_noalloc launch");
}

int sqattn_quantize_v_fp8(const void* v, int B, int H, int N, int d, int v_block, uint8_t* v_fp8,
                          float* v_scale, void* stream) {
  g_err.clear();
  int s;
  Sizes z;
  if ((s = check_ptr(v, "v", 16)) || (s = check_ptr(v_fp8, "v_fp8", 16)) || (s = check_ptr(v_scale, "v_scale", 4)))
    return s;
  if ((s = check_shape(B, H, N, d, &z))) return s;
  if (v_block != sqattn::KT) return fail(SQATTN_ERR_UNSUPPORTED, "v_block must be 64");
  hipStream_t st = (hipStream_t)stream;
  sqattn::launch_quant_v_fp8((const uint16_t*)v, sqattn::contiguous_lay(H, N, d), (int)z.BH, N, d, v_fp8, nullptr,
                             v_scale, st);
  return hip_check("sqattn_quantize_v_fp8 launch");
}

size_t sqattn_workspace_bytes(int B, int H, int N, int d, int pv_dtype, const sqattn_opts* opts) {
  std::string keep = g_err;
  Sizes z;
  Opts o;
  if (check_shape(B, H, N, d, &z) || (pv_dtype != 0 && pv_dtype != 1) || resolve_opts(opts, &o)) {
    g_err = keep;
    return 0;
  }
  return forward_layout(z, pv_dtype, o.q_block, o.smooth_q != 0).total;
}

// q/k RMSNorm fused into the quantization: the per-token factors of q and
// of k, B*N floats each, after the forward's own workspace
struct QkNorm {
  const float* gamma_q;
  const float* gamma_k;
  float eps;
};
size_t qknorm_extra(const Sizes& z, int B) { return align_up((size_t)(2LL * B * z.N) * 4); }

static int forward_impl(const void* q, const void* k, const void* v, int B, int H, int N, int d, float scale,
                        int pv_dtype, const uint8_t* mask, void* out, void* workspace, size_t workspace_bytes,
                        void* stream, const sqattn_opts* opts, const int64_t* in_strides = nullptr,
                        const int64_t* out_strides = nullptr, const QkNorm* qkn = nullptr) {
  g_err.clear();
  int s;
  Sizes z;
  Opts o;
  if ((s = validate_forward(q, k, v, B, H, N, d, scale, pv_dtype, out, opts, &z, &o))) return s;
  if (mask && (s = check_sparse(N))) return s;
  if (o.smooth_q && (mask || qkn))
    return fail(SQATTN_ERR_UNSUPPORTED, "Q smoothing runs on dense attention without the q/k RMSNorm");
  sqattn::Lay lay[4];
  for (int i = 0; i < 4; ++i) lay[i] = sqattn::contiguous_lay(H, N, d);
  for (int i = 0; i < 4; ++i) {
    const int64_t* st = (i < 3) ? (in_strides ? in_strides + 3 * i : nullptr) : out_strides;
    if (!st) continue;
    for (int j = 0; j < 3; ++j)
      if (st[j] < 0 || st[j] % 8 != 0 || st[j] > (1LL << 40))
        return fail(SQATTN_ERR_INVALID_ARG,
                    "strides must be non-negative multiples of 8 elements (16-byte rows), at most 2^40");
    lay[i] = sqattn::Lay{st[0], st[1], st[2], H};
  }
  if (qkn) {
    if (!(qkn->eps > 0.0f) || !std::isfinite(qkn->eps))
      return fail(SQATTN_ERR_INVALID_ARG, "eps must be finite and > 0");
    if ((qkn->gamma_q && (s = check_ptr(qkn->gamma_q, "gamma_q", 4))) ||
        (qkn->gamma_k && (s = check_ptr(qkn->gamma_k, "gamma_k", 4))))
      return s;
    if (H > 1 && (lay[0].sh != d || lay[1].sh != d))
      return fail(SQATTN_ERR_INVALID_ARG,
                  "q/k RMSNorm needs each token's H*d values of q and k contiguous (head stride d)");
  }
  const bool smooth = o.smooth_q != 0;
  const FwdLayout L = forward_layout(z, pv_dtype, o.q_block, smooth);
  hipStream_t st = (hipStream_t)stream;
  Workspace ws;
  if ((s = ws.acquire(workspace, workspace_bytes, L.total + (qkn ? qknorm_extra(z, B) : 0), st))) return s;
  const int BH = (int)z.BH;
  int8_t* qi = ws.at<int8_t>(L.q_i8);
  int8_t* ki = ws.at<int8_t>(L.k_i8);
  float* qs = ws.at<float>(L.q_scale);
  float* ks = ws.at<float>(L.k_scale);
  float* km = ws.at<float>(L.k_mean);
  sqattn::RowNorm nq, nk;
  if (qkn) {
    float* rq = ws.at<float>(L.total);
    float* rk = rq + (size_t)B * N;
    sqattn::launch_rms_inverse_rows((const uint16_t*)q, B, N, H * d, lay[0].sb, lay[0].sn, qkn->eps, rq, st);
    sqattn::launch_rms_inverse_rows((const uint16_t*)k, B, N, H * d, lay[1].sb, lay[1].sn, qkn->eps, rk, st);
    nq = sqattn::RowNorm{rq, qkn->gamma_q};
    nk = sqattn::RowNorm{rk, qkn->gamma_k};
  }
  float* qm = smooth ? ws.at<float>(L.q_mean) : nullptr;
  if (smooth)
    sqattn::launch_qmean((const uint16_t*)q, lay[0], BH, N, d, o.q_block, ws.at<uint64_t>(L.partial), qm, st);
  sqattn::launch_quant_i8((const uint16_t*)q, lay[0], BH, N, d, o.q_block, qm, qi, qs, st, nq, smooth);
  sqattn::launch_kmean((const uint16_t*)k, lay[1], BH, N, d, ws.at<uint64_t>(L.partial), km, st, nk);
  sqattn::launch_quant_i8((const uint16_t*)k, lay[1], BH, N, d, o.k_block, km, ki, ks, st, nk);
  if (smooth)
    sqattn::launch_qbias((const uint16_t*)k, lay[1], BH, N, d, km, qm, qs, ks, o.q_block,
                         ws.at<float>(L.q_bias), st);
  float* vs = nullptr;
  if (pv_dtype == SQATTN_PV_BF16) {
    sqattn::launch_v_tiles_bf16((const uint16_t*)v, lay[2], BH, N, d, ws.at<uint16_t>(L.vt), st);
  } else {
    vs = ws.at<float>(L.v_scale);
    sqattn::launch_quant_v_fp8((const uint16_t*)v, lay[2], BH, N, d, nullptr, ws.at<uint8_t>(L.vt), vs, st);
  }
  sqattn::AttnParams p{};
  p.q = qi;
  p.sq = qs;
  p.k = ki;
  p.sk = ks;
  p.vt = ws.at<void>(L.vt);
  p.sv = vs;
  p.out = out;
  p.out_bf16 = o.out_bf16;
  p.second_pass = o.second_pass;
  p.qbias = smooth ? ws.at<float>(L.q_bias) : nullptr;
  p.N = N;
  p.nq = (int)z.nq;
  p.q_block = o.q_block;
  p.nt = (int)z.nt;
  p.BH = BH;
  p.scale_log2e = scale * kLog2e;
  p.mask = mask;
  p.mq = (N + sqattn::SP_MQ - 1) / sqattn::SP_MQ;
  p.lo = lay[3];
  return launch_attention(p, d, pv_dtype, st,
                          qkn ? "sqattn_forward_qknorm launch"
                              : mask ? "sqattn_forward_sparse launch" : "sqattn_forward launch");
}

int sqattn_forward_ex(const void* q, const void* k, const void* v, int B, int H, int N, int d, float scale,
                      int pv_dtype, void* out, void* workspace, size_t workspace_bytes, void* stream,
                      const sqattn_opts* opts) {
  return forward_impl(q, k, v, B, H, N, d, scale, pv_dtype, nullptr, out, workspace, workspace_bytes, stream, opts);
}

int sqattn_forward_strided(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                           const int64_t* in_strides, const int64_t* out_strides, float scale, int pv_dtype,
                           const uint8_t* block_mask, void* out, void* workspace, size_t workspace_bytes,
                           void* stream, const sqattn_opts* opts) {
  if (!in_strides) {
    g_err.clear();
    return fail(SQATTN_ERR_INVALID_ARG, "in_strides is NULL");
  }
  return forward_impl(q, k, v, B, H, N, d, scale, pv_dtype, block_mask, out, workspace, workspace_bytes, stream,
                      opts, in_strides, out_strides);
}

int sqattn_forward_sparse(const void* q, const void* k, const void* v, int B, int H, int N, int d, float scale,
                          int pv_dtype, const uint8_t* block_mask, void* out, void* workspace, size_t workspace_bytes,
                          void* stream, const sqattn_opts* opts) {
  if (!block_mask) {
    g_err.clear();
    return fail(SQATTN_ERR_INVALID_ARG, "block_mask is NULL");
  }
  return forward_impl(q, k, v, B, H, N, d, scale, pv_dtype, block_mask, out, workspace, workspace_bytes, stream,
                      opts);
}

size_t sqattn_forward_qknorm_workspace_bytes(int B, int H, int N, int d, int pv_dtype, const sqattn_opts* opts) {
  std::string keep = g_err;
  Sizes z;
  Opts o;
  if (check_shape(B, H, N, d, &z) || (pv_dtype != 0 && pv_dtype != 1) || resolve_opts(opts, &o)) {
    g_err = keep;
    return 0;
  }
  return forward_layout(z, pv_dtype, o.q_block).total + qknorm_extra(z, B);
}

int sqattn_forward_qknorm(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                          const int64_t* in_strides, const int64_t* out_strides, const float* gamma_q,
                          const float* gamma_k, float eps, float scale, int pv_dtype, const uint8_t* block_mask,
                          void* out, void* workspace, size_t workspace_bytes, void* stream,
                          const sqattn_opts* opts) {
  if (!in_strides && H > 1) {
    g_err.clear();
    return fail(SQATTN_ERR_INVALID_ARG,
                "q/k RMSNorm needs in_strides with head stride d for q and k (each token's H*d values contiguous)");
  }
  const QkNorm n{gamma_q, gamma_k, eps};
  return forward_impl(q, k, v, B, H, N, d, scale, pv_dtype, block_mask, out, workspace, workspace_bytes, stream,
                      opts, in_strides, out_strides, &n);
}

int sqattn_forward(const void* q, const void* k, const void* v, int B, int H, int N, int d, float scale,
                   int pv_dtype, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return sqattn_forward_ex(q, k, v, B, H, N, d, scale, pv_dtype, out, workspace, workspace_bytes, stream,
                           nullptr);
}

size_t sqattn_packed_v_bytes(int B, int H, int N, int d, int pv_dtype) {
  std::string keep = g_err;
  Sizes z;
  if (check_shape(B, H, N, d, &z) || (pv_dtype != 0 && pv_dtype != 1)) {
    g_err = keep;
    return 0;
  }
  return (size_t)(z.BH * z.nt * z.d * sqattn::KT) * (pv_dtype == SQATTN_PV_BF16 ? 2 : 1);
}

int sqattn_pack_v(const void* v, int B, int H, int N, int d, int pv_dtype, void* v_packed, void* stream) {
  g_err.clear();
  int s;
  Sizes z;
  if ((s = check_ptr(v, "v", 16)) || (s = check_ptr(v_packed, "v_packed", 16))) return s;
  if ((s = check_shape(B, H, N, d, &z))) return s;
  if (pv_dtype != SQATTN_PV_BF16 && pv_dtype != SQATTN_PV_FP8_E4M3)
    return fail(SQATTN_ERR_INVALID_ARG, "unknown pv_dtype");
  hipStream_t st = (hipStream_t)stream;
  if (pv_dtype == SQATTN_PV_BF16)
    sqattn::launch_v_tiles_bf16((const uint16_t*)v, sqattn::contiguous_lay(H, N, d), (int)z.BH, N, d,
                                (uint16_t*)v_packed, st);
  else
    sqattn::launch_v_tiles_fp8((const uint8_t*)v, (int)z.BH, N, d, (uint8_t*)v_packed, st);
  return hip_check("sqattn_pack_v launch");
}

static int attend_impl(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                       const void* v_packed, const float* v_scale, int B, int H, int N, int d, float scale,
                       int pv_dtype, const uint8_t* mask, const sqattn_opts* opts, void* out, void* stream) {
  g_err.clear();
  int s;
  Sizes z;
  Opts o;
  if ((s = check_ptr(q_i8, "q_i8", 16)) || (s = check_ptr(k_i8, "k_i8", 16)) ||
      (s = check_ptr(q_scale, "q_scale", 4)) || (s = check_ptr(k_scale, "k_scale", 4)) ||
      (s = check_ptr(v_packed, "v_packed", 16)) || (s = check_ptr(out, "out", 16)))
    return s;
  if ((s = check_shape(B, H, N, d, &z))) return s;
  if (pv_dtype != SQATTN_PV_BF16 && pv_dtype != SQATTN_PV_FP8_E4M3)
    return fail(SQATTN_ERR_INVALID_ARG, "unknown pv_dtype");
  if (pv_dtype == SQATTN_PV_FP8_E4M3 && (s = check_ptr(v_scale, "v_scale", 4))) return s;
  if (!std::isfinite(scale) || scale < 0.0f) return fail(SQATTN_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if ((s = resolve_opts(opts, &o))) return s;
  if (o.smooth_q) return fail(SQATTN_ERR_UNSUPPORTED, "Q smoothing is a step of the forward (Q is quantized here)");
  sqattn::AttnParams p{};
  p.q = q_i8;
  p.sq = q_scale;
  p.k = k_i8;
  p.sk = k_scale;
  p.vt = v_packed;
  p.sv = v_scale;
  p.out = out;
  p.out_bf16 = o.out_bf16;
  p.second_pass = o.second_pass;
  p.N = N;
  p.nq = (int)((N + o.q_block - 1) / o.q_block);
  p.q_block = o.q_block;
  p.nt = (int)z.nt;
  p.BH = (int)z.BH;
  p.scale_log2e = scale * kLog2e;
  if (mask && (s = check_sparse(N))) return s;
  p.mask = mask;
  p.mq = (N + sqattn::SP_MQ - 1) / sqattn::SP_MQ;
  p.lo = sqattn::contiguous_lay(H, N, d);
  return launch_attention(p, d, pv_dtype, (hipStream_t)stream,
                          mask ? "sqattn_attend_packed_sparse launch" : "sqattn_attend_packed launch");
}

int sqattn_attend_packed(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                         const void* v_packed, const float* v_scale, int B, int H, int N, int d, float scale,
                         int pv_dtype, const sqattn_opts* opts, void* out, void* stream) {
  return attend_impl(q_i8, q_scale, k_i8, k_scale, v_packed, v_scale, B, H, N, d, scale, pv_dtype, nullptr, opts,
                     out, stream);
}

int sqattn_attend_packed_sparse(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                const void* v_packed, const float* v_scale, int B, int H, int N, int d, float scale,
                                int pv_dtype, const uint8_t* block_mask, const sqattn_opts* opts, void* out,
                                void* stream) {
  if (!block_mask) {
    g_err.clear();
    return fail(SQATTN_ERR_INVALID_ARG, "block_mask is NULL");
  }
  return attend_impl(q_i8, q_scale, k_i8, k_scale, v_packed, v_scale, B, H, N, d, scale, pv_dtype, block_mask,
                     opts, out, stream);
}

// Raw V (bf16, or E4M3 codes for FP8) into a stream-ordered temporary in the
// kernel's tile layout, then the kernel.  The temporary is freed
// stream-ordered after the launch.
static int attend_raw(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                      const void* v, const float* v_scale, int B, int H, int N, int d, float scale, int pv_dtype,
                      const uint8_t* mask, const sqattn_opts* opts, void* out, void* stream) {
  g_err.clear();
  int s;
  Sizes z;
  if ((s = check_ptr(v, "v", 16))) return s;
  if ((s = check_shape(B, H, N, d, &z))) return s;
  if (pv_dtype != SQATTN_PV_BF16 && pv_dtype != SQATTN_PV_FP8_E4M3)
    return fail(SQATTN_ERR_INVALID_ARG, "unknown pv_dtype");
  // everything the kernel call checks, before anything is allocated or enqueued
  if ((s = check_ptr(q_i8, "q_i8", 16)) || (s = check_ptr(k_i8, "k_i8", 16)) ||
      (s = check_ptr(q_scale, "q_scale", 4)) || (s = check_ptr(k_scale, "k_scale", 4)) ||
      (s = check_ptr(out, "out", 16)))
    return s;
  if (pv_dtype == SQATTN_PV_FP8_E4M3 && (s = check_ptr(v_scale, "v_scale", 4))) return s;
  if (!std::isfinite(scale) || scale < 0.0f) return fail(SQATTN_ERR_INVALID_ARG, "scale must be finite and >= 0");
  Opts o;
  if ((s = resolve_opts(opts, &o))) return s;
  if (o.smooth_q) return fail(SQATTN_ERR_UNSUPPORTED, "Q smoothing is a step of the forward (Q is quantized here)");
  if (mask && (s = check_sparse(N))) return s;
  hipStream_t st = (hipStream_t)stream;
  Workspace ws;
  const size_t bytes = (size_t)(z.BH * z.nt * z.d * sqattn::KT) * (pv_dtype == SQATTN_PV_BF16 ? 2 : 1);
  if ((s = ws.acquire(nullptr, 0, bytes, st))) return s;
  if (pv_dtype == SQATTN_PV_BF16)
    sqattn::launch_v_tiles_bf16((const uint16_t*)v, sqattn::contiguous_lay(H, N, d), (int)z.BH, N, d,
                                ws.at<uint16_t>(0), st);
  else
    sqattn::launch_v_tiles_fp8((const uint8_t*)v, (int)z.BH, N, d, ws.at<uint8_t>(0), st);
  if ((s = hip_check("V packing launch"))) return s;
  s = attend_impl(q_i8, q_scale, k_i8, k_scale, ws.at<void>(0), v_scale, B, H, N, d, scale, pv_dtype, mask, opts,
                  out, stream);
  return s;
}

int sqattn_attend_quantized(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                            const void* v, const float* v_scale, int B, int H, int N, int d, float scale,
                            int pv_dtype, const sqattn_opts* opts, void* out, void* stream) {
  return attend_raw(q_i8, q_scale, k_i8, k_scale, v, v_scale, B, H, N, d, scale, pv_dtype, nullptr, opts, out,
                    stream);
}

int sqattn_attend_quantized_sparse(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                   const float* k_scale, const void* v, const float* v_scale, int B, int H, int N,
                                   int d, float scale, int pv_dtype, const uint8_t* block_mask,
                                   const sqattn_opts* opts, void* out, void* stream) {
  if (!block_mask) {
    g_err.clear();
    return fail(SQATTN_ERR_INVALID_ARG, "block_mask is NULL");
  }
  return attend_raw(q_i8, q_scale, k_i8, k_scale, v, v_scale, B, H, N, d, scale, pv_dtype, block_mask, opts, out,
                    stream);
}

int sqattn_w8a8_quantize(const void* x, int rows, int cols, int8_t* codes, float* scales, void* stream) {
  g_err.clear();
  int s;
  if ((s = check_w8a8_rows(rows, "rows")) || (s = check_w8a8_k(cols))) return s;
  if (rows == 0) return SQATTN_OK;  // empty: pointers are not inspected
  if ((s = check_ptr(x, "x", 16)) || (s = check_ptr(codes, "codes", 16)) || (s = check_ptr(scales, "scales", 4)))
    return s;
  sqattn::launch_w8a8_quant((const uint16_t*)x, rows, cols, codes, scales, (hipStream_t)stream);
  return hip_check("sqattn_w8a8_quantize launch");
}

int sqattn_w8a8_gemm(const int8_t* x_codes, const float* x_scales, const int8_t* w_codes, const float* w_scales,
                     const float* bias, int M, int N, int K, int out_dtype, void* out, void* stream) {
  g_err.clear();
  int s;
  if ((s = check_w8a8_rows(M, "M")) || (s = check_w8a8_rows(N, "N")) || (s = check_w8a8_k(K)) ||
      (s = check_out_dtype(out_dtype)))
    return s;
  if (M == 0 || N == 0) return SQATTN_OK;  // empty: pointers are not inspected
  if ((s = check_ptr(x_codes, "x_codes", 16)) || (s = check_ptr(w_codes, "w_codes", 16)) ||
      (s = check_ptr(x_scales, "x_scales", 4)) || (s = check_ptr(w_scales, "w_scales", 4)) ||
      (s = check_ptr(out, "out", 16)))
    return s;
  if (bias && (s = check_ptr(bias, "bias", 4))) return s;
  return gemm_status(sqattn::launch_w8a8_gemm(x_codes, x_scales, w_codes, w_scales, bias, M, N, K, out,
                                              out_dtype == SQATTN_OUT_BF16, (hipStream_t)stream),
                     "sqattn_w8a8_gemm launch");
}

size_t sqattn_w8a8_workspace_bytes(int M, int K) {
  std::string keep = g_err;
  if (check_w8a8_rows(M, "M") || check_w8a8_k(K)) {
    g_err = keep;
    return 0;
  }
  return align_up((size_t)M * K) + align_up(w8a8_scale_bytes(M, K));
}

int sqattn_w8a8_linear(const void* x, const int8_t* w_codes, const float* w_scales, const float* bias, int M, int N,
                       int K, int out_dtype, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int s;
  if ((s = check_w8a8_rows(M, "M")) || (s = check_w8a8_rows(N, "N")) || (s = check_w8a8_k(K)) ||
      (s = check_out_dtype(out_dtype)))
    return s;
  if (M == 0 || N == 0) return SQATTN_OK;  // empty: pointers are not inspected
  if ((s = check_ptr(x, "x", 16)) || (s = check_ptr(w_codes, "w_codes", 16)) ||
      (s = check_ptr(w_scales, "w_scales", 4)) || (s = check_ptr(out, "out", 16)))
    return s;
  if (bias && (s = check_ptr(bias, "bias", 4))) return s;
  hipStream_t st = (hipStream_t)stream;
  Workspace ws;
  const size_t codes_bytes = align_up((size_t)M * K);
  if ((s = ws.acquire(workspace, workspace_bytes, codes_bytes + align_up(w8a8_scale_bytes(M, K)), st))) return s;
  int8_t* xc = ws.at<int8_t>(0);
  float* xs = ws.at<float>(codes_bytes);
  sqattn::launch_w8a8_quant((const uint16_t*)x, M, K, xc, xs, st);
  return gemm_status(
      sqattn::launch_w8a8_gemm(xc, xs, w_codes, w_scales, bias, M, N, K, out, out_dtype == SQATTN_OUT_BF16, st),
      "sqattn_w8a8_linear launch");
}

int sqattn_w8a8_rmsnorm_quantize(const void* x, const float* gamma, float eps, int rows, int cols, int8_t* codes,
                                 float* scales, float* inv_rms, void* stream) {
  g_err.clear();
  int s;
  if ((s = check_w8a8_rows(rows, "rows")) || (s = check_w8a8_k(cols))) return s;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return fail(SQATTN_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (rows == 0) return SQATTN_OK;  // empty: pointers are not inspected
  if ((s = check_ptr(x, "x", 16)) || (s = check_ptr(codes, "codes", 16)) || (s = check_ptr(scales, "scales", 4)) ||
      (s = check_ptr(inv_rms, "inv_rms", 4)))
    return s;
  if (gamma && (s = check_ptr(gamma, "gamma", 4))) return s;
  sqattn::launch_w8a8_rmsnorm_quant((const uint16_t*)x, gamma, eps, rows, cols, codes, scales, inv_rms,
                                    (hipStream_t)stream);
  return hip_check("sqattn_w8a8_rmsnorm_quantize launch");
}

size_t sqattn_w8a8_rmsnorm_workspace_bytes(int M, int K) {
  std::string keep = g_err;
  if (check_w8a8_rows(M, "M") || check_w8a8_k(K)) {
    g_err = keep;
    return 0;
  }
  return align_up((size_t)M * K) + align_up(w8a8_scale_bytes(M, K)) + align_up((size_t)M * 4);
}

int sqattn_w8a8_linear_rmsnorm(const void* x, const float* gamma, float eps, const int8_t* w_codes,
                               const float* w_scales, const float* bias, int M, int N, int K, int out_dtype, void* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int s;
  if ((s = check_w8a8_rows(M, "M")) || (s = check_w8a8_rows(N, "N")) || (s = check_w8a8_k(K)) ||
      (s = check_out_dtype(out_dtype)))
    return s;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return fail(SQATTN_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (M == 0 || N == 0) return SQATTN_OK;  // empty: pointers are not inspected
  if ((s = check_ptr(x, "x", 16)) || (s = check_ptr(w_codes, "w_codes", 16)) ||
      (s = check_ptr(w_scales, "w_scales", 4)) || (s = check_ptr(out, "out", 16)))
    return s;
  if (gamma && (s = check_ptr(gamma, "gamma", 4))) return s;
  if (bias && (s = check_ptr(bias, "bias", 4))) return s;
  hipStream_t st = (hipStream_t)stream;
  Workspace ws;
  const size_t cb = align_up((size_t)M * K), sb = align_up(w8a8_scale_bytes(M, K));
  if ((s = ws.acquire(workspace, workspace_bytes, cb + sb + align_up((size_t)M * 4), st))) return s;
  int8_t* xc = ws.at<int8_t>(0);
  float* xs = ws.at<float>(cb);
  float* r = ws.at<float>(cb + sb);
  sqattn::launch_w8a8_rmsnorm_quant((const uint16_t*)x, gamma, eps, M, K, xc, xs, r, st);
  return gemm_status(
      sqattn::launch_w8a8_gemm(xc, xs, w_codes, w_scales, bias, M, N, K, out, out_dtype == SQATTN_OUT_BF16, st),
      "sqattn_w8a8_linear_rmsnorm launch");
}

int sqattn_w8a8_layernorm_quantize(const void* x, const float* gamma, const float* beta, float eps, int rows,
                                   int cols, int8_t* codes, float* scales, float* mean, float* rstd,
                                   void* stream) {
  g_err.clear();
  int s;
  if ((s = check_w8a8_rows(rows, "rows")) || (s = check_w8a8_k(cols))) return s;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return fail(SQATTN_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (rows == 0) return SQATTN_OK;  // empty: pointers are not inspected
  if ((s = check_ptr(x, "x", 16)) || (s = check_ptr(codes, "codes", 16)) || (s = check_ptr(scales, "scales", 4)) ||
      (s = check_ptr(mean, "mean", 4)) || (s = check_ptr(rstd, "rstd", 4)))
    return s;
  if ((gamma && (s = check_ptr(gamma, "gamma", 4))) || (beta && (s = check_ptr(beta, "beta", 4)))) return s;
  sqattn::launch_w8a8_layernorm_quant((const uint16_t*)x, gamma, beta, eps, rows, cols, codes, scales, mean, rstd,
                                      (hipStream_t)stream);
  return hip_check("sqattn_w8a8_layernorm_quantize launch");
}

size_t sqattn_w8a8_layernorm_workspace_bytes(int M, int K) {
  std::string keep = g_err;
  if (check_w8a8_rows(M, "M") || check_w8a8_k(K)) {
    g_err = keep;
    return 0;
  }
  return align_up((size_t)M * K) + align_up(w8a8_scale_bytes(M, K)) + 2 * align_up((size_t)M * 4);
}

int sqattn_w8a8_linear_layernorm(const void* x, const float* gamma, const float* beta, float eps,
                                 const int8_t* w_codes, const float* w_scales, const float* bias, int M, int N, int K,
                                 int out_dtype, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int s;
  if ((s = check_w8a8_rows(M, "M")) || (s = check_w8a8_rows(N, "N")) || (s = check_w8a8_k(K)) ||
      (s = check_out_dtype(out_dtype)))
    return s;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return fail(SQATTN_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (M == 0 || N == 0) return SQATTN_OK;  // empty: pointers are not inspected
  if ((s = check_ptr(x, "x", 16)) || (s = check_ptr(w_codes, "w_codes", 16)) ||
      (s = check_ptr(w_scales, "w_scales", 4)) || (s = check_ptr(out, "out", 16)))
    return s;
  if ((gamma && (s = check_ptr(gamma, "gamma", 4))) || (beta && (s = check_ptr(beta, "beta", 4))) ||
      (bias && (s = check_ptr(bias, "bias", 4))))
    return s;
  hipStream_t st = (hipStream_t)stream;
  Workspace ws;
  const size_t cb = align_up((size_t)M * K), sb = align_up(w8a8_scale_bytes(M, K)), rb = align_up((size_t)M * 4);
  if ((s = ws.acquire(workspace, workspace_bytes, cb + sb + 2 * rb, st))) return s;
  int8_t* xc = ws.at<int8_t>(0);
  float* xs = ws.at<float>(cb);
  float* mu = ws.at<float>(cb + sb);
  float* r = ws.at<float>(cb + sb + rb);
  sqattn::launch_w8a8_layernorm_quant((const uint16_t*)x, gamma, beta, eps, M, K, xc, xs, mu, r, st);
  return gemm_status(
      sqattn::launch_w8a8_gemm(xc, xs, w_codes, w_scales, bias, M, N, K, out, out_dtype == SQATTN_OUT_BF16, st),
      "sqattn_w8a8_linear_layernorm launch");
}

}  // extern "C"
