// Shared device-side definitions of the sqattn HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace sqattn {

// Index checks of the checking build (SQATTN_DEBUG): a failed condition sets
// bit `bit` of the violation word (a vector atomic); nothing in the release
// build.
#ifdef SQATTN_DEBUG
#define SQ_CHECK(word, cond, bit)                                  \
  do {                                                             \
    if ((word) != nullptr && !(cond)) atomicOr((word), 1u << (bit)); \
  } while (0)
#else
#define SQ_CHECK(word, cond, bit) \
  do {                            \
  } while (0)
#endif

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Quantized attention (attn_bf16.hip, attn_fp8.hip): logits from INT8 codes of
// Q and smoothed K on the integer matrix units, softmax, then P.V in bf16 or
// FP8 with fp32 accumulation (jefxiong.cn "AIGC weekend special 5.10",
// section 1.2 item (1); GVCLab research log 2026-09-02, section 5.5 table,
// SageAttention2 row).  The tiling with a running max and running sum is the
// FlashAttention lineage the same digest names as its baseline.
//
// A work-group (8 waves) owns 256 query rows of one (b,h) head; each wave owns
// 32 rows; keys stream in 64-key tiles through an LDS ring.
//
// Register layouts (32x32 MFMA: lane l, accumulator register i holds row
// 8*(i/4) + 4*(l/32) + i%4, column l%32; operand lane-half g = l/32 holds the
// k-slots g*K/2 .. g*K/2 + K/2 - 1)
//   * S^T = K Q^T on v_mfma_i32_32x32x32_i8: A = K tile rows (keys), B = Q
//     rows (held in registers for the whole loop).  Each lane therefore owns
//     one query column; its 16 accumulators are 16 keys.  K rows are read in
//     the order pi(r) = r with bits 2 and 3 swapped, which makes the 16 keys
//     of lane-half g in a 32-key block equal to {16h + 8g + j : h<2, j<8}.
//   * O^T = V^T P^T: P^T is the B operand (k = keys, n = queries), built in
//     place from the lane's own softmax values, so no cross-lane movement is
//     needed; V^T (rows = channels) is the A operand read from LDS, where
//     each lane-half's 8 (bf16) or 32 (FP8) keys are contiguous.  Row max and
//     row sum therefore need only one exchange between lanes l and l^32.

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// rne(fl32(a / s)) with one multiply in the common case.  With y = RN(1/s)
// (a correctly rounded division, once per thread) and q = RN(a y), both
// within 2^-24 relative, |q - fl32(a/s)| < 1.5 * 2^-23 |a/s| < 2^-15 for
// |a/s| <= 128 (every value of a block against its own scale).  Where q is
// farther than 2^-15 from every half-integer, fl32(a/s) lies in the same
// open interval (k - 1/2, k + 1/2) and rounds to the same k; otherwise (ties
// included) the correctly rounded quotient is formed.  Needs a finite 1/s:
// callers take the division for s < 2^-125.
__device__ __forceinline__ float rne_quotient(float a, float s, float y) {
  const float q = a * y;
  const float r = rintf(q);
  if (__builtin_expect(fabsf(q - r) > 0.5f - 0x1p-15f, 0)) return rintf(a / s);
  return r;
}


// Two floats to packed bf16 (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  v2bf v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Direct global -> LDS loads (global_load_lds), each lane's bytes at
// sbase + voff to the LDS address lds_addr + 16 * lane (4 * lane for the
// dword form); lds_addr and sbase are wave-uniform.  Issued from inline
// assembly so that the compiler's LDS-wait bookkeeping is not disturbed: it
// models the compiler-generated form as touching both wait counters and
// then waits for every LDS read in flight at the next use of one.  These
// loads have no register result; their completion is waited for explicitly
// (vmcnt) by the kernels.  M0 carries the LDS address, so the kernels leave
// M0 to these statements alone.
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n s_nop 0\n global_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n s_nop 0\n global_load_lds_dword %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory");
}
// 32-bit LDS address of a pointer into the kernel's dynamic LDS
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Epilogue of the attention kernels: one query row of O = scale * O^T.  Lane
// half g holds channels 32 cb + 8 i4 + 4 g + j in o[cb][4 i4 + j]; the row
// goes out as fp32 or, with bf16, rounded to bf16.
template <int NCB>
__device__ __forceinline__ void store_out_row(void* out, bool bf16, long long base, const v16f (&o)[NCB],
                                              float scale, int g) {
  if (bf16) {
    uint16_t* orow = (uint16_t*)out + base;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const uint2 w = make_uint2(pack_bf16x2(o[cb][4 * i4] * scale, o[cb][4 * i4 + 1] * scale),
                                   pack_bf16x2(o[cb][4 * i4 + 2] * scale, o[cb][4 * i4 + 3] * scale));
        *(uint2*)(orow + cb * 32 + i4 * 8 + g * 4) = w;
      }
  } else {
    float* orow = (float*)out + base;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const v4f v = {o[cb][4 * i4] * scale, o[cb][4 * i4 + 1] * scale, o[cb][4 * i4 + 2] * scale,
                       o[cb][4 * i4 + 3] * scale};
        *(v4f*)(orow + cb * 32 + i4 * 8 + g * 4) = v;
      }
  }
}

// Layout of one 64-key V tile inside the kernel (both in HBM workspace and LDS):
// transposed, [d][64 keys].  For FP8 the 64 key bytes of a row are permuted so
// that the 32 keys one MFMA lane-half consumes are contiguous:
//   pos(key) = g*32 + (key/16)*8 + key%8 with g = (key/8)%2.
__host__ __device__ __forceinline__ int fp8_key_pos(int key) {
  return (((key >> 3) & 1) << 5) | ((key >> 4) << 3) | (key & 7);
}

// Block-sparse attention: the sorted list of key tiles that mask row r0
// (mrow0) or mask row r0 + 1 (mrow1, null past the last row) keeps, built by
// all nthr threads of a work-group.  Entry: tile | row r0 keeps it << 24 |
// row r0 + 1 keeps it << 25.  wcnt: nthr/64 ints of LDS scratch.  Returns
// the count (uniform); list and count are visible to every wave on return.
__device__ __forceinline__ int build_tile_list(const uint8_t* mrow0, const uint8_t* mrow1, int nt, int* list,
                                               int* wcnt, int nthr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = nthr >> 6;
  int base = 0;
  for (int t0 = 0; t0 < nt; t0 += nthr) {
    const int t = t0 + tid;
    const int f0 = (t < nt && mrow0[t] != 0) ? 1 : 0;
    const int f1 = (t < nt && mrow1 != nullptr && mrow1[t] != 0) ? 1 : 0;
    const unsigned long long b = __ballot(f0 | f1);
    const int before = __builtin_popcountll(b & ((1ull << lane) - 1ull));
    if (lane == 0) wcnt[wave] = __builtin_popcountll(b);
    __syncthreads();
    int off = base, tot = 0;
    for (int w = 0; w < nw; ++w) {
      const int c = wcnt[w];
      off += (w < wave) ? c : 0;
      tot += c;
    }
    if (f0 | f1) list[off + before] = t | (f0 << 24) | (f1 << 25);
    base += tot;
    __syncthreads();  // list entries written; wcnt free for the next round
  }
  return base;
}

// Size helpers shared by host code.
__host__ __device__ __forceinline__ long long ceil_div_ll(long long a, long long b) {
  return (a + b - 1) / b;
}

}  // namespace sqattn
