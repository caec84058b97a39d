// Host-only harness of the C-ABI layer (csrc/api.cpp), built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.
//
// The HIP runtime calls api.cpp makes and the kernel launchers it calls are
// replaced here by recorders that touch no memory: every pointer is a fake
// device address, never dereferenced.  Each launcher records the byte ranges
// its kernels read and write, from the kernels' own indexing (prep.hip,
// attn_*.hip, w8a8.hip, norm.hip).  For every call the harness checks
//   * rejected arguments: the status, and that nothing was launched or
//     allocated (validation precedes every enqueue);
//   * accepted arguments: every range lies inside one buffer the caller
//     passed, the workspace, the static scratch or a stream-ordered
//     allocation; writes never land in an input; within one launch no write
//     overlaps a read of another range (an in-place update of the range it
//     read is declared as such); a write over bytes an earlier launch wrote
//     comes after some launch in between read them (no lost result); every
//     workspace or allocation byte a launch reads was written by an earlier
//     launch of the same call; every allocation is freed, on the call's
//     stream;
//   * the *_workspace_bytes functions: exactly that many bytes are accepted,
//     one 256-byte step less is refused with SQATTN_ERR_WORKSPACE;
//   * HIP errors forced from here (a failed allocation, a failed launch, a
//     failed kernel attribute or static-scratch lookup) come back as
//     SQATTN_ERR_HIP with a message naming the step, and leak nothing.
// The sanitizers add: no out-of-bounds host access, no signed overflow or
// other undefined behaviour in the size and index arithmetic, up to the
// largest sizes the validation accepts.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"
#include "sqattn.h"

namespace {

struct Range {
  uintptr_t a, b;  // [a, b)
};

enum Kind { INPUT, OUTPUT, WORKSPACE, SCRATCH, ALLOC };

struct Buffer {
  std::string name;
  uintptr_t a;
  size_t bytes;
  Kind kind;
  bool freed;
};

struct Access {
  std::string who;
  Range r;
  bool write;
  int launch;
  bool inplace;  // a write of exactly the range this launch read before
};

std::vector<Buffer> g_buf;
std::vector<Access> g_acc;
int g_launches = 0;
int g_failures = 0;
int g_cases = 0;
uintptr_t g_next = (uintptr_t)1 << 44;  // fake device addresses, 2^36 bytes apart
hipStream_t g_stream = (hipStream_t)(uintptr_t)0x5000;
std::string g_case;
// errors forced into the next HIP call of each kind
bool g_fail_malloc = false, g_fail_launch = false, g_fail_attr = false, g_fail_symbol = false;

uintptr_t fresh(size_t bytes) {
  uintptr_t a = g_next;
  g_next += ((uintptr_t)1 << 36) + (((uintptr_t)bytes + 255) & ~(uintptr_t)255);
  return a;
}

void* buffer(const char* name, size_t bytes, Kind kind) {
  uintptr_t a = fresh(bytes);
  g_buf.push_back({name, a, bytes, kind, false});
  return (void*)a;
}

void failf(const std::string& msg) {
  ++g_failures;
  std::fprintf(stderr, "FAIL [%s] %s\n", g_case.c_str(), msg.c_str());
}

void record(const char* who, const void* p, long double bytes, bool write, bool inplace = false) {
  if (bytes <= 0) return;
  if (!p) {
    failf(std::string(who) + ": null pointer with a nonzero extent");
    return;
  }
  const uintptr_t a = (uintptr_t)p;
  g_acc.push_back({who, {a, a + (uintptr_t)bytes}, write, g_launches, inplace});
}

// byte extent of the rows of a [BH, N, d] operand with layout l (element size es)
long double lay_extent(const sqattn::Lay& l, int BH, int N, int d, int es) {
  const long long last = sqattn::lay_row(l, BH - 1, N - 1);
  long long hi = last;
  // the largest row start over the corners of the (b, h, n) box
  const int B = BH / l.H;
  for (int b : {0, B - 1})
    for (int h : {0, l.H - 1})
      for (int n : {0, N - 1}) {
        const long long o = (long long)b * l.sb + (long long)h * l.sh + (long long)n * l.sn;
        if (o > hi) hi = o;
      }
  return (long double)(hi + d) * es;
}

void reset() {
  g_buf.clear();
  g_acc.clear();
  g_launches = 0;
}

const Buffer* owner(const Range& r) {
  for (const Buffer& b : g_buf)
    if (r.a >= b.a && r.b <= b.a + b.bytes) return &b;
  return nullptr;
}

// checks the recorded accesses of one accepted call
void verify() {
  for (const Access& x : g_acc) {
    const Buffer* b = owner(x.r);
    if (!b) {
      failf(x.who + ": range outside every buffer (" + std::to_string(x.r.b - x.r.a) + " bytes)");
      continue;
    }
    if (x.write && b->kind == INPUT) failf(x.who + ": writes into input " + b->name);
    if (x.write) {
      // no read of another range in the same launch overlaps the write
      for (const Access& y : g_acc)
        if (!y.write && y.launch == x.launch && y.r.a < x.r.b && x.r.a < y.r.b &&
            !(x.inplace && y.r.a == x.r.a && y.r.b == x.r.b))
          failf(x.who + " overlaps " + y.who + " in the same launch (" + b->name + ")");
      // a write over an earlier launch's result only after a launch in between read it
      for (const Access& y : g_acc) {
        if (!y.write || y.launch >= x.launch || !(y.r.a < x.r.b && x.r.a < y.r.b)) continue;
        const uintptr_t ia = std::max(x.r.a, y.r.a), ib = std::min(x.r.b, y.r.b);
        bool read = false;
        for (const Access& z : g_acc)
          if (!z.write && z.r.a < ib && ia < z.r.b &&
              ((z.launch > y.launch && z.launch < x.launch) || (x.inplace && z.launch == x.launch)))
            read = true;
        if (!read) failf(x.who + " overwrites " + y.who + " before any launch read it (" + b->name + ")");
      }
    }
    if (b->kind == WORKSPACE || b->kind == ALLOC || b->kind == SCRATCH) {
      if (!x.write) {
        // every byte read was written by an earlier launch: sweep the
        // earlier writes' union over [a, b)
        uintptr_t covered = x.r.a;
        bool progress = true;
        while (covered < x.r.b && progress) {
          progress = false;
          for (const Access& y : g_acc)
            if (y.write && y.launch < x.launch && y.r.a <= covered && y.r.b > covered) {
              covered = y.r.b;
              progress = true;
            }
        }
        if (covered < x.r.b) failf(x.who + ": reads bytes of " + b->name + " that no earlier launch wrote");
      }
    }
  }
  for (const Buffer& b : g_buf)
    if (b.kind == ALLOC && !b.freed) failf("allocation " + b.name + " not freed");
}

void expect(int got, int want, const char* what) {
  ++g_cases;
  if (got != want)
    failf(std::string(what) + ": status " + std::to_string(got) + ", expected " + std::to_string(want) + " (" +
          sqattn_last_error() + ")");
}

void expect_rejected(int got, int want, const char* needle, const char* what) {
  expect(got, want, what);
  if (needle && !std::strstr(sqattn_last_error(), needle))
    failf(std::string(what) + ": message '" + sqattn_last_error() + "' lacks '" + needle + "'");
  if (g_launches) failf(std::string(what) + ": launched kernels before rejecting");
  for (const Buffer& b : g_buf)
    if (b.kind == ALLOC) failf(std::string(what) + ": allocated before rejecting");
}

}  // namespace

// ---- the HIP runtime calls of api.cpp
extern "C" {
hipError_t hipMallocAsync(void** p, size_t n, hipStream_t s) {
  if (s != g_stream) failf("hipMallocAsync on another stream");
  if (g_fail_malloc) {
    g_fail_malloc = false;
    return hipErrorOutOfMemory;
  }
  *p = buffer("stream-ordered allocation", n, ALLOC);
  return hipSuccess;
}
hipError_t hipFreeAsync(void* p, hipStream_t s) {
  if (s != g_stream) failf("hipFreeAsync on another stream");
  for (Buffer& b : g_buf)
    if (b.kind == ALLOC && b.a == (uintptr_t)p) {
      if (b.freed) failf("double hipFreeAsync");
      b.freed = true;
      return hipSuccess;
    }
  failf("hipFreeAsync of an address never allocated");
  return hipErrorInvalidValue;
}
hipError_t hipGetLastError(void) {
  if (g_fail_launch) {
    g_fail_launch = false;
    return hipErrorLaunchFailure;
  }
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "(no HIP runtime in this harness)"; }
}

// ---- the kernel launchers, as ranges read and written
namespace sqattn {

static void launched(hipStream_t st) {
  if (st != g_stream) failf("launch on another stream");
  ++g_launches;
}

static void norm_reads(const char* who, const RowNorm& nm, int BH, int N, int H, int d) {
  if (!nm.r) return;
  record(who, nm.r, (long double)(BH / H) * N * 4, false);
  if (nm.gamma) record(who, nm.gamma, (long double)H * d * 4, false);
}

hipError_t static_scratch(void** ptr) {
  if (g_fail_symbol) {
    g_fail_symbol = false;
    return hipErrorInvalidSymbol;
  }
  for (const Buffer& b : g_buf)
    if (b.kind == SCRATCH) {
      *ptr = (void*)b.a;
      return hipSuccess;
    }
  *ptr = buffer("static scratch", kStaticScratchBytes, SCRATCH);
  return hipSuccess;
}

void launch_kmean(const uint16_t* k, const Lay& lk, int BH, int N, int d, uint64_t* partial, float* mean,
                  hipStream_t st, const RowNorm& nm) {
  const int S = kmean_chunks(BH, N);
  record("kmean: k", k, lay_extent(lk, BH, N, d, 2), false);
  norm_reads("kmean: norm", nm, BH, N, lk.H, d);
  record("kmean: partial", partial, (long double)BH * S * d * 32, true);
  launched(st);
  record("kmean finalize: partial", partial, (long double)BH * S * d * 32, false);
  record("kmean finalize: mean", mean, (long double)BH * d * 4, true);
  launched(st);
}

void launch_quant_i8(const uint16_t* x, const Lay& lx, int BH, int N, int d, int block, float* mean,
                     int8_t* codes, float* scales, hipStream_t st, const RowNorm& nm, bool mean_blocks) {
  const long double nb = (N + block - 1) / block;
  record("quant_i8: x", x, lay_extent(lx, BH, N, d, 2), false);
  norm_reads("quant_i8: norm", nm, BH, N, lx.H, d);
  if (mean) record("quant_i8: mean", mean, (long double)BH * (mean_blocks ? nb : 1) * d * 4, false);
  record("quant_i8: codes", codes, (long double)BH * N * d, true);
  record("quant_i8: scales", scales, (long double)BH * nb * 4, true);
  launched(st);
  // the block means of Q smoothing are rewritten (0 for blocks kept plain):
  // a write of the same launch, after its read
  if (mean && mean_blocks) record("quant_i8: mean rows", mean, (long double)BH * nb * d * 4, true, true);
}

void launch_qmean(const uint16_t* q, const Lay& lq, int BH, int N, int d, int block, uint64_t* partial,
                  float* mean, hipStream_t st) {
  const long double nq = (N + block - 1) / block;
  record("qmean: q", q, lay_extent(lq, BH, N, d, 2), false);
  record("qmean: partial", partial, (long double)BH * nq * d * 32, true);
  launched(st);
  record("qmean finalize: partial", partial, (long double)BH * nq * d * 32, false);
  record("qmean finalize: mean", mean, (long double)BH * nq * d * 4, true);
  launched(st);
}

void launch_qbias(const uint16_t* k, const Lay& lk, int BH, int N, int d, const float* kmean, const float* qmean,
                  const float* q_scale, const float* k_scale, int block, float* bias, hipStream_t st) {
  const long double nq = (N + block - 1) / block, nt = (N + KT - 1) / KT;
  record("qbias: k", k, lay_extent(lk, BH, N, d, 2), false);
  record("qbias: kmean", kmean, (long double)BH * d * 4, false);
  record("qbias: qmean", qmean, (long double)BH * nq * d * 4, false);
  record("qbias: q scales", q_scale, (long double)BH * nq * 4, false);
  record("qbias: k scales", k_scale, (long double)BH * nt * 4, false);
  record("qbias: bias", bias, (long double)BH * nq * nt * KT * 4, true);
  launched(st);
}

void launch_v_tiles_bf16(const uint16_t* v, const Lay& lv, int BH, int N, int d, uint16_t* vt, hipStream_t st) {
  const int nt = (N + KT - 1) / KT;
  record("v_tiles_bf16: v", v, lay_extent(lv, BH, N, d, 2), false);
  record("v_tiles_bf16: vt", vt, (long double)BH * nt * d * KT * 2, true);
  launched(st);
}

void launch_quant_v_fp8(const uint16_t* v, const Lay& lv, int BH, int N, int d, uint8_t* codes, uint8_t* vt,
                        float* scales, hipStream_t st) {
  const int nt = (N + KT - 1) / KT;
  record("quant_v_fp8: v", v, lay_extent(lv, BH, N, d, 2), false);
  if (codes) record("quant_v_fp8: codes", codes, (long double)BH * N * d, true);
  if (vt) record("quant_v_fp8: vt", vt, (long double)BH * nt * d * KT, true);
  record("quant_v_fp8: scales", scales, (long double)BH * nt * 4, true);
  launched(st);
}

void launch_v_tiles_fp8(const uint8_t* codes, int BH, int N, int d, uint8_t* vt, hipStream_t st) {
  const int nt = (N + KT - 1) / KT;
  record("v_tiles_fp8: codes", codes, (long double)BH * N * d, false);
  record("v_tiles_fp8: vt", vt, (long double)BH * nt * d * KT, true);
  launched(st);
}

static hipError_t attention(const AttnParams& p, int d, bool fp8, hipStream_t st) {
  if (g_fail_attr) {
    g_fail_attr = false;
    return hipErrorInvalidValue;  // the kernel attribute setup failed: nothing launched
  }
  const long double BH = p.BH, N = p.N;
  if (p.nt != (p.N + KT - 1) / KT) failf("attention: nt");
  if (p.nq != (p.N + p.q_block - 1) / p.q_block) failf("attention: nq");
  if (p.qtiles != (p.N + ATT_QWG - 1) / ATT_QWG) failf("attention: qtiles");
  if ((long long)p.per_xcd * 8 < (long long)p.BH * p.qtiles) failf("attention: per_xcd does not cover the work");
  record("attention: q", p.q, BH * N * d, false);
  record("attention: q scales", p.sq, BH * p.nq * 4, false);
  record("attention: k", p.k, BH * N * d, false);
  record("attention: k scales", p.sk, BH * p.nt * 4, false);
  record("attention: v tiles", p.vt, BH * p.nt * d * KT * (fp8 ? 1 : 2), false);
  if (fp8) record("attention: v scales", p.sv, BH * p.nt * 4, false);
  if (p.mask) {
    if (p.mq != (p.N + SP_MQ - 1) / SP_MQ) failf("attention: mq");
    record("attention: mask", p.mask, BH * p.mq * p.nt, false);
  }
  record("attention: out", p.out, lay_extent(p.lo, p.BH, p.N, d, p.out_bf16 ? 2 : 4), true);
  if (p.second_pass) record("attention: counter", p.second_pass, 4, true);
  if (p.qbias) {
    if (p.mask) failf("attention: Q smoothing with a block mask");
    if (p.q_block != 64 && p.q_block != 128 && p.q_block != 256) failf("attention: Q smoothing q_block");
    record("attention: q bias", p.qbias, BH * p.nq * p.nt * KT * 4, false);
  }
  launched(st);
  return hipSuccess;
}
hipError_t launch_attention_bf16(const AttnParams& p, int d, hipStream_t st) { return attention(p, d, false, st); }
hipError_t launch_attention_fp8(const AttnParams& p, int d, hipStream_t st) { return attention(p, d, true, st); }

void launch_rms_inverse(const uint16_t*, int, int, float, float*, hipStream_t) { failf("unexpected launcher"); }
void launch_layernorm_stats(const uint16_t*, int, int, float, float*, float*, hipStream_t) {
  failf("unexpected launcher");
}
void launch_rms_inverse_rows(const uint16_t* x, int B, int N, int C, long long sb, long long sn, float,
                             float* inv_rms, hipStream_t st) {
  record("rms rows: x", x, (long double)((long long)(B - 1) * sb + (long long)(N - 1) * sn + C) * 2, false);
  record("rms rows: inv", inv_rms, (long double)B * N * 4, true);
  launched(st);
}
void launch_w8a8_quant(const uint16_t* x, int R, int C, int8_t* codes, float* scales, hipStream_t st) {
  record("w8a8 quant: x", x, (long double)R * C * 2, false);
  record("w8a8 quant: codes", codes, (long double)R * C, true);
  record("w8a8 quant: scales", scales, (long double)((R + 127) / 128) * (C / 128) * 4, true);
  launched(st);
}
void launch_w8a8_rmsnorm_quant(const uint16_t* x, const float* gamma, float, int R, int C, int8_t* codes,
                               float* scales, float* inv_rms, hipStream_t st) {
  record("w8a8 rms: x", x, (long double)R * C * 2, false);
  if (gamma) record("w8a8 rms: gamma", gamma, (long double)C * 4, false);
  record("w8a8 rms: codes", codes, (long double)R * C, true);
  record("w8a8 rms: scales", scales, (long double)((R + 127) / 128) * (C / 128) * 4, true);
  record("w8a8 rms: inv", inv_rms, (long double)R * 4, true);
  launched(st);
}
void launch_w8a8_layernorm_quant(const uint16_t* x, const float* gamma, const float* beta, float, int R, int C,
                                 int8_t* codes, float* scales, float* mean, float* rstd, hipStream_t st) {
  record("w8a8 ln: x", x, (long double)R * C * 2, false);
  if (gamma) record("w8a8 ln: gamma", gamma, (long double)C * 4, false);
  if (beta) record("w8a8 ln: beta", beta, (long double)C * 4, false);
  record("w8a8 ln: codes", codes, (long double)R * C, true);
  record("w8a8 ln: scales", scales, (long double)((R + 127) / 128) * (C / 128) * 4, true);
  record("w8a8 ln: mean", mean, (long double)R * 4, true);
  record("w8a8 ln: rstd", rstd, (long double)R * 4, true);
  launched(st);
}
hipError_t launch_w8a8_gemm(const int8_t* x, const float* sx, const int8_t* w, const float* sw, const float* bias,
                            int M, int N, int K, void* out, int out_bf16, hipStream_t st) {
  record("gemm: x", x, (long double)M * K, false);
  record("gemm: x scales", sx, (long double)((M + 127) / 128) * (K / 128) * 4, false);
  record("gemm: w", w, (long double)N * K, false);
  record("gemm: w scales", sw, (long double)((N + 127) / 128) * (K / 128) * 4, false);
  if (bias) record("gemm: bias", bias, (long double)N * 4, false);
  record("gemm: out", out, (long double)M * N * (out_bf16 ? 2 : 4), true);
  launched(st);
  return hipSuccess;
}

}  // namespace sqattn

// ---- the cases
namespace {

const int kStatusOk = SQATTN_OK;

struct Attn {
  int B, H, N, d, pv;
  int q_block = 128;
  int out_dtype = SQATTN_OUT_FP32;
  bool counter = false;
  int smooth = 0;
};

std::string label(const char* f, const Attn& a) {
  char s[160];
  std::snprintf(s, sizeof s, "%s B=%d H=%d N=%d d=%d pv=%d q_block=%d out=%d smooth=%d", f, a.B, a.H, a.N, a.d,
                a.pv, a.q_block, a.out_dtype, a.smooth);
  return s;
}

size_t elems(const Attn& a) { return (size_t)a.B * a.H * a.N * a.d; }

sqattn_opts opts_of(const Attn& a) {
  sqattn_opts o{};
  o.q_block = a.q_block;
  o.out_dtype = a.out_dtype;
  o.smooth_q = a.smooth;
  if (a.counter) o.second_pass_count = (uint32_t*)buffer("counter", 4, OUTPUT);
  return o;
}

void forward_case(const Attn& a, bool sparse) {
  g_case = label(sparse ? "forward_sparse" : "forward_ex", a);
  reset();
  const size_t n = elems(a);
  void* q = buffer("q", n * 2, INPUT);
  void* k = buffer("k", n * 2, INPUT);
  void* v = buffer("v", n * 2, INPUT);
  void* out = buffer("out", n * (a.out_dtype == SQATTN_OUT_BF16 ? 2 : 4), OUTPUT);
  const size_t nt = (a.N + 63) / 64, mq = (a.N + 127) / 128;
  const uint8_t* mask = sparse ? (const uint8_t*)buffer("mask", (size_t)a.B * a.H * mq * nt, INPUT) : nullptr;
  sqattn_opts o = opts_of(a);
  const size_t wb = sqattn_workspace_bytes(a.B, a.H, a.N, a.d, a.pv, &o);
  if (wb == 0 || wb % 256) failf("workspace size " + std::to_string(wb));
  void* ws = buffer("workspace", wb, WORKSPACE);
  int s = sparse ? sqattn_forward_sparse(q, k, v, a.B, a.H, a.N, a.d, 0.088f, a.pv, mask, out, ws, wb, g_stream, &o)
                 : sqattn_forward_ex(q, k, v, a.B, a.H, a.N, a.d, 0.088f, a.pv, out, ws, wb, g_stream, &o);
  expect(s, kStatusOk, "forward with the reported workspace");
  verify();
  // one 256-byte step less is refused before anything is enqueued
  reset();
  s = sqattn_forward_ex((void*)fresh(n * 2), (void*)fresh(n * 2), (void*)fresh(n * 2), a.B, a.H, a.N, a.d, 0.088f,
                        a.pv, (void*)fresh(n * 4), (void*)fresh(wb), wb - 256, g_stream, &o);
  expect_rejected(s, SQATTN_ERR_WORKSPACE, "needed", "forward with a smaller workspace");
  // no workspace: a stream-ordered allocation, freed
  reset();
  q = buffer("q", n * 2, INPUT);
  k = buffer("k", n * 2, INPUT);
  v = buffer("v", n * 2, INPUT);
  out = buffer("out", n * (a.out_dtype == SQATTN_OUT_BF16 ? 2 : 4), OUTPUT);
  o = opts_of(a);
  s = sqattn_forward_ex(q, k, v, a.B, a.H, a.N, a.d, 0.088f, a.pv, out, nullptr, 0, g_stream, &o);
  expect(s, kStatusOk, "forward with a library allocation");
  verify();
}

void strided_case(const Attn& a, bool qknorm) {
  // q, k, v as views of one [B, N, 3, H, d] projection output; out [B, N, H, d]
  g_case = label(qknorm ? "forward_qknorm" : "forward_strided", a);
  reset();
  const size_t n = elems(a);
  char* qkv = (char*)buffer("qkv", 3 * n * 2, INPUT);
  void* out = buffer("out", n * 4, OUTPUT);
  const int64_t tok = 3LL * a.H * a.d;
  int64_t in[9];
  for (int i = 0; i < 3; ++i) {
    in[3 * i + 0] = (int64_t)a.N * tok;
    in[3 * i + 1] = a.d;
    in[3 * i + 2] = tok;
  }
  const int64_t os[3] = {(int64_t)a.N * a.H * a.d, a.d, (int64_t)a.H * a.d};
  sqattn_opts o = opts_of(a);
  o.out_dtype = SQATTN_OUT_FP32;
  const size_t wb = qknorm ? sqattn_forward_qknorm_workspace_bytes(a.B, a.H, a.N, a.d, a.pv, &o)
                           : sqattn_workspace_bytes(a.B, a.H, a.N, a.d, a.pv, &o);
  void* ws = buffer("workspace", wb, WORKSPACE);
  const size_t hd = (size_t)a.H * a.d * 2;
  int s;
  if (qknorm) {
    const float* gq = (const float*)buffer("gamma_q", (size_t)a.H * a.d * 4, INPUT);
    const float* gk = (const float*)buffer("gamma_k", (size_t)a.H * a.d * 4, INPUT);
    s = sqattn_forward_qknorm(qkv, qkv + hd, qkv + 2 * hd, a.B, a.H, a.N, a.d, in, os, gq, gk, 1e-6f, 0.088f, a.pv,
                              nullptr, out, ws, wb, g_stream, &o);
  } else {
    s = sqattn_forward_strided(qkv, qkv + hd, qkv + 2 * hd, a.B, a.H, a.N, a.d, in, os, 0.088f, a.pv, nullptr, out,
                               ws, wb, g_stream, &o);
  }
  expect(s, kStatusOk, "strided forward");
  verify();
}

void attend_case(const Attn& a, bool packed, bool sparse) {
  g_case = label(packed ? "attend_packed" : "attend_quantized", a);
  reset();
  const size_t n = elems(a), BH = (size_t)a.B * a.H, nt = (a.N + 63) / 64;
  const size_t nq = a.q_block == 1 ? a.N : (a.N + a.q_block - 1) / a.q_block;
  const int8_t* qi = (const int8_t*)buffer("q_i8", n, INPUT);
  const float* qs = (const float*)buffer("q_scale", BH * nq * 4, INPUT);
  const int8_t* ki = (const int8_t*)buffer("k_i8", n, INPUT);
  const float* ks = (const float*)buffer("k_scale", BH * nt * 4, INPUT);
  const size_t vbytes = packed ? sqattn_packed_v_bytes(a.B, a.H, a.N, a.d, a.pv) : n * (a.pv ? 1 : 2);
  const void* v = buffer("v", vbytes, INPUT);
  const float* vs = a.pv ? (const float*)buffer("v_scale", BH * nt * 4, INPUT) : nullptr;
  void* out = buffer("out", n * (a.out_dtype == SQATTN_OUT_BF16 ? 2 : 4), OUTPUT);
  const uint8_t* mask = sparse ? (const uint8_t*)buffer("mask", BH * ((a.N + 127) / 128) * nt, INPUT) : nullptr;
  sqattn_opts o = opts_of(a);
  int s;
  if (packed)
    s = sparse ? sqattn_attend_packed_sparse(qi, qs, ki, ks, v, vs, a.B, a.H, a.N, a.d, 0.088f, a.pv, mask, &o, out,
                                             g_stream)
               : sqattn_attend_packed(qi, qs, ki, ks, v, vs, a.B, a.H, a.N, a.d, 0.088f, a.pv, &o, out, g_stream);
  else
    s = sparse ? sqattn_attend_quantized_sparse(qi, qs, ki, ks, v, vs, a.B, a.H, a.N, a.d, 0.088f, a.pv, mask, &o,
                                                out, g_stream)
               : sqattn_attend_quantized(qi, qs, ki, ks, v, vs, a.B, a.H, a.N, a.d, 0.088f, a.pv, &o, out, g_stream);
  expect(s, kStatusOk, "attend");
  verify();
}

void prep_case(const Attn& a) {
  g_case = label("quantize_qk / quantize_v_fp8 / pack_v", a);
  const size_t n = elems(a), BH = (size_t)a.B * a.H, nt = (a.N + 63) / 64;
  const size_t nq = a.q_block == 1 ? a.N : (a.N + a.q_block - 1) / a.q_block;
  for (int noalloc = 0; noalloc < 2; ++noalloc) {
    reset();
    const void* q = buffer("q", n * 2, INPUT);
    const void* k = buffer("k", n * 2, INPUT);
    int8_t* qi = (int8_t*)buffer("q_i8", n, OUTPUT);
    float* qs = (float*)buffer("q_scale", BH * nq * 4, OUTPUT);
    int8_t* ki = (int8_t*)buffer("k_i8", n, OUTPUT);
    float* ks = (float*)buffer("k_scale", BH * nt * 4, OUTPUT);
    float* km = (float*)buffer("k_mean", BH * a.d * 4, OUTPUT);
    int s;
    if (noalloc) {
      s = sqattn_quantize_qk_noalloc(q, k, a.B, a.H, a.N, a.d, a.q_block, 64, qi, qs, ki, ks, km, g_stream);
      const size_t need = BH * sqattn::kmean_chunks((int)BH, a.N) * a.d * 32;
      if (need > sqattn::kStaticScratchBytes) {
        expect_rejected(s, SQATTN_ERR_WORKSPACE, "static scratch", "quantize_qk_noalloc beyond the scratch");
        continue;
      }
    } else {
      const size_t wb = sqattn_quantize_qk_workspace_bytes(a.B, a.H, a.N, a.d);
      void* ws = buffer("workspace", wb, WORKSPACE);
      s = sqattn_quantize_qk(q, k, a.B, a.H, a.N, a.d, a.q_block, 64, qi, qs, ki, ks, km, ws, wb, g_stream);
    }
    expect(s, kStatusOk, noalloc ? "quantize_qk_noalloc" : "quantize_qk");
    verify();
  }
  reset();
  const void* v = buffer("v", n * 2, INPUT);
  uint8_t* vc = (uint8_t*)buffer("v_fp8", n, OUTPUT);
  float* vs = (float*)buffer("v_scale", BH * nt * 4, OUTPUT);
  expect(sqattn_quantize_v_fp8(v, a.B, a.H, a.N, a.d, 64, vc, vs, g_stream), kStatusOk, "quantize_v_fp8");
  verify();
  for (int pv = 0; pv < 2; ++pv) {
    reset();
    const void* src = buffer("v", n * (pv ? 1 : 2), INPUT);
    void* dst = buffer("v_packed", sqattn_packed_v_bytes(a.B, a.H, a.N, a.d, pv), OUTPUT);
    expect(sqattn_pack_v(src, a.B, a.H, a.N, a.d, pv, dst, g_stream), kStatusOk, "pack_v");
    verify();
  }
}

void w8a8_case(int M, int N, int K, int norm, bool bias, int out_dtype) {
  char lab[96];
  std::snprintf(lab, sizeof lab, "w8a8 M=%d N=%d K=%d norm=%d bias=%d out=%d", M, N, K, norm, (int)bias, out_dtype);
  g_case = lab;
  reset();
  const void* x = buffer("x", (size_t)M * K * 2, INPUT);
  const int8_t* wc = (const int8_t*)buffer("w_codes", (size_t)N * K, INPUT);
  const float* ws = (const float*)buffer("w_scales", (size_t)((N + 127) / 128) * (K / 128) * 4, INPUT);
  const float* b = bias ? (const float*)buffer("bias", (size_t)N * 4, INPUT) : nullptr;
  const float* g = (const float*)buffer("gamma", (size_t)K * 4, INPUT);
  const float* be = (const float*)buffer("beta", (size_t)K * 4, INPUT);
  void* out = buffer("out", (size_t)M * N * (out_dtype ? 2 : 4), OUTPUT);
  const size_t wb = norm == 0   ? sqattn_w8a8_workspace_bytes(M, K)
                    : norm == 1 ? sqattn_w8a8_rmsnorm_workspace_bytes(M, K)
                                : sqattn_w8a8_layernorm_workspace_bytes(M, K);
  void* w = buffer("workspace", wb, WORKSPACE);
  int s = norm == 0 ? sqattn_w8a8_linear(x, wc, ws, b, M, N, K, out_dtype, out, w, wb, g_stream)
          : norm == 1
              ? sqattn_w8a8_linear_rmsnorm(x, g, 1e-6f, wc, ws, b, M, N, K, out_dtype, out, w, wb, g_stream)
              : sqattn_w8a8_linear_layernorm(x, g, be, 1e-6f, wc, ws, b, M, N, K, out_dtype, out, w, wb, g_stream);
  expect(s, kStatusOk, "w8a8 linear");
  verify();
  if (M > 0 && N > 0 && wb >= 256) {
    reset();
    s = sqattn_w8a8_linear((void*)fresh(1), (const int8_t*)fresh(1), (const float*)fresh(1), nullptr, M, N, K,
                           out_dtype, (void*)fresh(1), (void*)fresh(1), sqattn_w8a8_workspace_bytes(M, K) - 256,
                           g_stream);
    expect_rejected(s, SQATTN_ERR_WORKSPACE, "needed", "w8a8 linear with a smaller workspace");
  }
}

void rejections() {
  g_case = "rejected arguments";
  const uintptr_t F = (uintptr_t)1 << 40;
  void* p = (void*)F;
  sqattn_opts bad{};
  struct {
    int B, H, N, d, pv;
    float scale;
    void* q;
    void* out;
    int want;
    const char* needle;
  } t[] = {
      {1, 1, 64, 128, 0, 0.1f, nullptr, p, SQATTN_ERR_INVALID_ARG, "q is NULL"},
      {1, 1, 64, 128, 0, 0.1f, (char*)p + 8, p, SQATTN_ERR_INVALID_ARG, "aligned"},
      {1, 1, 64, 128, 0, 0.1f, p, (char*)p + 4, SQATTN_ERR_INVALID_ARG, "aligned"},
      {0, 1, 64, 128, 0, 0.1f, p, p, SQATTN_ERR_INVALID_ARG, ">= 1"},
      {1, 1, 0, 128, 0, 0.1f, p, p, SQATTN_ERR_INVALID_ARG, ">= 1"},
      {1, 1, 64, 96, 0, 0.1f, p, p, SQATTN_ERR_UNSUPPORTED, "64 or 128"},
      {1, 1, 1 << 24, 128, 0, 0.1f, p, p, SQATTN_ERR_RANGE, "2^24"},
      {256, 256, 64, 128, 0, 0.1f, p, p, SQATTN_ERR_RANGE, "65535"},
      {65535, 1, (1 << 24) - 1, 128, 0, 0.1f, p, p, SQATTN_ERR_RANGE, "2^40"},
      {2147483647, 2147483647, 2147483647, 128, 0, 0.1f, p, p, SQATTN_ERR_RANGE, nullptr},
      {1, 1, 64, 128, 2, 0.1f, p, p, SQATTN_ERR_INVALID_ARG, "pv_dtype"},
      {1, 1, 64, 128, 0, NAN, p, p, SQATTN_ERR_INVALID_ARG, "scale"},
      {1, 1, 64, 128, 0, -1.0f, p, p, SQATTN_ERR_INVALID_ARG, "scale"},
      {1, 1, 64, 128, 0, INFINITY, p, p, SQATTN_ERR_INVALID_ARG, "scale"},
  };
  for (auto& c : t) {
    reset();
    expect_rejected(sqattn_forward_ex(c.q, p, p, c.B, c.H, c.N, c.d, c.scale, c.pv, c.out, p, (size_t)1 << 62,
                                      g_stream, nullptr),
                    c.want, c.needle, "forward_ex");
    reset();
    expect_rejected(sqattn_forward(c.q, p, p, c.B, c.H, c.N, c.d, c.scale, c.pv, c.out, nullptr, 0, g_stream), c.want,
                    c.needle, "forward");
  }
  const int opt_cases[][5] = {{128, 128, 64, 0, SQATTN_ERR_UNSUPPORTED}, {128, 64, 32, 0, SQATTN_ERR_UNSUPPORTED},
                              {24, 64, 64, 0, SQATTN_ERR_INVALID_ARG},   {0x7fffffff, 64, 64, 0, SQATTN_ERR_INVALID_ARG},
                              {-16, 64, 64, 0, SQATTN_ERR_INVALID_ARG},  {128, 64, 64, 2, SQATTN_ERR_INVALID_ARG}};
  for (auto& c : opt_cases) {
    bad = sqattn_opts{};
    bad.q_block = c[0];
    bad.k_block = c[1];
    bad.v_block = c[2];
    bad.out_dtype = c[3];
    reset();
    expect_rejected(sqattn_forward_ex(p, p, p, 1, 2, 300, 64, 0.1f, 0, p, p, (size_t)1 << 40, g_stream, &bad), c[4],
                    nullptr, "forward_ex opts");
    if (sqattn_workspace_bytes(1, 2, 300, 64, 0, &bad) != 0) failf("workspace_bytes of rejected opts is not 0");
  }
  // Q smoothing: its q_block set, dense forward only, not on quantized Q
  for (int qb : {1, 16, 32, 192}) {
    bad = sqattn_opts{};
    bad.q_block = qb;
    bad.smooth_q = 1;
    reset();
    expect_rejected(sqattn_forward_ex(p, p, p, 1, 2, 300, 64, 0.1f, 0, p, p, (size_t)1 << 40, g_stream, &bad),
                    SQATTN_ERR_UNSUPPORTED, "q_block 64, 128 or 256", "forward_ex smoothing q_block");
  }
  bad = sqattn_opts{};
  bad.smooth_q = 2;
  reset();
  expect_rejected(sqattn_forward_ex(p, p, p, 1, 2, 300, 64, 0.1f, 0, p, p, (size_t)1 << 40, g_stream, &bad),
                  SQATTN_ERR_INVALID_ARG, "smooth_q", "forward_ex smooth_q value");
  bad = sqattn_opts{};
  bad.smooth_q = 1;
  reset();
  expect_rejected(sqattn_forward_sparse(p, p, p, 1, 1, 300, 64, 0.1f, 0, (const uint8_t*)p, p, p, (size_t)1 << 40,
                                        g_stream, &bad),
                  SQATTN_ERR_UNSUPPORTED, "dense", "forward_sparse smoothing");
  reset();
  expect_rejected(sqattn_attend_packed((const int8_t*)p, (const float*)p, (const int8_t*)p, (const float*)p, p,
                                       nullptr, 1, 1, 64, 64, 0.1f, 0, &bad, p, g_stream),
                  SQATTN_ERR_UNSUPPORTED, "step of the forward", "attend_packed smoothing");
  reset();
  expect_rejected(sqattn_attend_quantized((const int8_t*)p, (const float*)p, (const int8_t*)p, (const float*)p, p,
                                          nullptr, 1, 1, 64, 64, 0.1f, 0, &bad, p, g_stream),
                  SQATTN_ERR_UNSUPPORTED, "step of the forward", "attend_quantized smoothing");
  bad = sqattn_opts{};
  bad.second_pass_count = (uint32_t*)((char*)p + 2);
  reset();
  expect_rejected(sqattn_forward_ex(p, p, p, 1, 2, 300, 64, 0.1f, 0, p, p, (size_t)1 << 40, g_stream, &bad),
                  SQATTN_ERR_INVALID_ARG, "second_pass_count", "forward_ex counter alignment");
  // strides
  int64_t in[9] = {8, 8, 7, 8, 8, 8, 8, 8, 8}, os[3] = {8, 8, 8};
  reset();
  expect_rejected(sqattn_forward_strided(p, p, p, 1, 1, 64, 64, in, os, 0.1f, 0, nullptr, p, p, (size_t)1 << 40,
                                         g_stream, nullptr),
                  SQATTN_ERR_INVALID_ARG, "strides", "forward_strided odd stride");
  in[2] = (int64_t)1 << 41;
  reset();
  expect_rejected(sqattn_forward_strided(p, p, p, 1, 1, 64, 64, in, os, 0.1f, 0, nullptr, p, p, (size_t)1 << 40,
                                         g_stream, nullptr),
                  SQATTN_ERR_INVALID_ARG, "strides", "forward_strided huge stride");
  // sparse beyond the tile list
  reset();
  expect_rejected(sqattn_forward_sparse(p, p, p, 1, 1, 4096 * 64 + 1, 64, 0.1f, 0, (const uint8_t*)p, p, p,
                                        (size_t)1 << 40, g_stream, nullptr),
                  SQATTN_ERR_UNSUPPORTED, "block-sparse", "forward_sparse N");
  reset();
  expect_rejected(sqattn_attend_quantized_sparse((const int8_t*)p, (const float*)p, (const int8_t*)p,
                                                 (const float*)p, p, nullptr, 1, 1, 64, 64, 0.1f, 0, nullptr, nullptr,
                                                 p, g_stream),
                  SQATTN_ERR_INVALID_ARG, "block_mask", "attend sparse without mask");
  reset();
  expect_rejected(sqattn_attend_quantized((const int8_t*)p, (const float*)p, (const int8_t*)p, (const float*)p, p,
                                          nullptr, 1, 1, 64, 64, 0.1f, 1, nullptr, p, g_stream),
                  SQATTN_ERR_INVALID_ARG, "v_scale", "attend fp8 without v_scale");
  // quantization entry points
  reset();
  expect_rejected(sqattn_quantize_qk(p, p, 1, 1, 64, 64, 8, 64, (int8_t*)p, (float*)p, (int8_t*)p, (float*)p,
                                     (float*)p, p, (size_t)1 << 40, g_stream),
                  SQATTN_ERR_INVALID_ARG, "q_block", "quantize_qk q_block");
  reset();
  expect_rejected(sqattn_quantize_qk(p, p, 1, 1, 64, 64, 128, 64, (int8_t*)p, (float*)p, (int8_t*)p, (float*)p,
                                     (float*)p, p, 1, g_stream),
                  SQATTN_ERR_WORKSPACE, "needed", "quantize_qk workspace");
  reset();
  expect_rejected(sqattn_quantize_qk_noalloc(p, p, 1, 65535, 64, 128, 128, 64, (int8_t*)p, (float*)p, (int8_t*)p,
                                             (float*)p, (float*)p, g_stream),
                  SQATTN_ERR_WORKSPACE, "static scratch", "quantize_qk_noalloc size");
  reset();
  expect_rejected(sqattn_quantize_v_fp8(p, 1, 1, 64, 64, 32, (uint8_t*)p, (float*)p, g_stream), SQATTN_ERR_UNSUPPORTED,
                  "v_block", "quantize_v_fp8 v_block");
  // W8A8
  reset();
  expect_rejected(sqattn_w8a8_gemm((const int8_t*)p, (const float*)p, (const int8_t*)p, (const float*)p, nullptr, 64,
                                   64, 100, 0, p, g_stream),
                  SQATTN_ERR_INVALID_ARG, "multiple of 128", "w8a8 K");
  reset();
  expect_rejected(sqattn_w8a8_gemm((const int8_t*)p, (const float*)p, (const int8_t*)p, (const float*)p, nullptr,
                                   65535 * 128 + 1, 64, 128, 0, p, g_stream),
                  SQATTN_ERR_RANGE, "65535", "w8a8 M");
  reset();
  expect_rejected(sqattn_w8a8_linear_rmsnorm(p, nullptr, 0.0f, (const int8_t*)p, (const float*)p, nullptr, 64, 64,
                                             128, 0, p, p, (size_t)1 << 40, g_stream),
                  SQATTN_ERR_INVALID_ARG, "eps", "w8a8 rmsnorm eps");
  reset();
  expect_rejected(sqattn_w8a8_linear((const void*)p, (const int8_t*)p, (const float*)p, nullptr, 64, 64, 128, 7, p, p,
                                     (size_t)1 << 40, g_stream),
                  SQATTN_ERR_INVALID_ARG, "out_dtype", "w8a8 out_dtype");
  if (sqattn_workspace_bytes(65535, 1, (1 << 24) - 1, 128, 0, nullptr) != 0) failf("workspace_bytes out of range");
  if (sqattn_w8a8_workspace_bytes(65535 * 128 + 1, 128) != 0) failf("w8a8 workspace_bytes out of range");
  if (std::strcmp(sqattn_status_string(12345), "unknown status")) failf("status string");
}

void forced_hip_errors() {
  const Attn a{1, 2, 300, 64, SQATTN_PV_BF16};
  const size_t n = elems(a);
  struct {
    bool* flag;
    const char* needle;
    bool workspace;
  } t[] = {{&g_fail_malloc, "hipMallocAsync", false},
           {&g_fail_launch, "launch", true},
           {&g_fail_attr, "LDS size", true},
           {&g_fail_attr, "LDS size", false}};
  for (auto& c : t) {
    g_case = std::string("forced HIP error: ") + c.needle;
    reset();
    void* q = buffer("q", n * 2, INPUT);
    void* out = buffer("out", n * 4, OUTPUT);
    const size_t wb = sqattn_workspace_bytes(a.B, a.H, a.N, a.d, a.pv, nullptr);
    void* ws = c.workspace ? buffer("workspace", wb, WORKSPACE) : nullptr;
    *c.flag = true;
    const int s = sqattn_forward_ex(q, q, q, a.B, a.H, a.N, a.d, 0.1f, a.pv, out, ws, c.workspace ? wb : 0, g_stream,
                                    nullptr);
    expect(s, SQATTN_ERR_HIP, "forward");
    if (!std::strstr(sqattn_last_error(), c.needle))
      failf(std::string("message '") + sqattn_last_error() + "' lacks '" + c.needle + "'");
    if (*c.flag) failf("the forced error was never reached");
    *c.flag = false;
    for (const Buffer& b : g_buf)
      if (b.kind == ALLOC && !b.freed) failf("allocation not freed after the error");
  }
  g_case = "forced HIP error: static scratch";
  reset();
  g_fail_symbol = true;
  void* p = buffer("p", 1 << 20, OUTPUT);
  expect(sqattn_quantize_qk_noalloc(p, p, 1, 1, 64, 64, 64, 64, (int8_t*)p, (float*)p, (int8_t*)p, (float*)p,
                                    (float*)p, g_stream),
         SQATTN_ERR_HIP, "quantize_qk_noalloc");
  if (!std::strstr(sqattn_last_error(), "static scratch")) failf("static scratch message");
  if (g_launches) failf("launched after a failed scratch lookup");
  g_fail_symbol = false;
}

}  // namespace

int main() {
  rejections();
  forced_hip_errors();
  const int pvs[] = {SQATTN_PV_BF16, SQATTN_PV_FP8_E4M3};
  const int ns[] = {1, 63, 64, 65, 300, 4097};
  for (int pv : pvs)
    for (int d : {64, 128})
      for (int N : ns)
        for (int qb : {1, 16, 128, 192}) {
          Attn a{2, 3, N, d, pv, qb};
          a.out_dtype = (N % 2) ? SQATTN_OUT_BF16 : SQATTN_OUT_FP32;
          a.counter = N == 300;
          forward_case(a, false);
          if (qb == 128 || (qb != 1 && qb != 16 && N > 64)) {
            Attn sm = a;
            sm.smooth = 1;
            sm.q_block = qb == 192 ? 256 : qb;
            forward_case(sm, false);
          }
          if (qb == 128) {
            forward_case(a, true);
            strided_case(a, false);
            strided_case(a, true);
            for (int packed = 0; packed < 2; ++packed)
              for (int sparse = 0; sparse < 2; ++sparse) attend_case(a, packed, sparse);
            prep_case(a);
          }
        }
  // the largest sizes validation accepts: arithmetic only, nothing is touched
  forward_case(Attn{1, 1, (1 << 24) - 1, 128, SQATTN_PV_BF16, 1}, false);
  forward_case(Attn{1, 65535, 32, 128, SQATTN_PV_FP8_E4M3}, false);
  forward_case(Attn{4, 16383, 4096, 64, SQATTN_PV_BF16}, false);
  prep_case(Attn{1, 1, (1 << 24) - 1, 128, SQATTN_PV_BF16});
  prep_case(Attn{2, 8, 40000, 128, SQATTN_PV_BF16});
  for (int norm = 0; norm < 3; ++norm) {
    w8a8_case(300, 260, 384, norm, norm != 1, norm == 2);
    w8a8_case(0, 64, 128, norm, false, 0);
    w8a8_case(65535 * 128, 128, 128, norm, true, 1);
    w8a8_case(128, 3 * 5120, 1 << 20, norm, true, 0);
  }
  std::printf("%d cases, %d failures\n", g_cases, g_failures);
  return g_failures ? 1 : 0;
}
