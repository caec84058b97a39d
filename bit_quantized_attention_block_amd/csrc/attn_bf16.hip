// Quantized attention kernel, 16-bit P.V path (gfx950).
//
// INT8 S^T = K Q^T, lane-local softmax, O^T = V^T P^T in the register
// layouts described in common.h.
//
// Work-group: 8 waves, 32 query rows each, 256 rows per work-group, one
// work-group per CU.  Waves w and w + 4 run on the same SIMD.
//
// Ping-pong schedule.  The work of a 64-key tile t is split into two phases:
//
//   V(t)  vector ALU : P(t) = 2^(S(t) c - ref) rounded to bf16, row sum
//   M(t)  matrix core: S(t+1) = K(t+1) Q^T            (2 D/32 x i8 32x32x32)
//                      O^T  += V(t)^T P(t)^T           (4 D/32 x bf16 32x32x16)
//
// Every wave runs V(0) M(0) V(1) M(1) ...; waves 4-7 start one phase later
// than waves 0-3, and a work-group barrier separates consecutive phases.  So
// at any moment one wave of each SIMD issues matrix instructions while the
// other issues the softmax.  On gfx950 a wave's vector instructions overlap
// its own matrix instructions (and those of a wave in the same phase) poorly,
// while two waves in opposite phases overlap almost completely: the tile then
// costs about its matrix-core time.
//
//   * LDS: a ring of NSLOT entries; entry e holds "pair" j = e (mod NSLOT):
//     the K tile j + 1 with its scale, and the V^T tile j.  M(j) reads pair j.
//     Tiles are stored unpadded with the 16-byte units of each row permuted
//     (unit c of row r at position c ^ f(r)), so that the 16 rows 16 lanes
//     read at the same column fall in distinct banks.  V(t) refills the entry
//     of pair t - 2 (read by both wave groups already) with pair t + 3:
//     direct-to-LDS loads, each wave one K and two V 1 KB chunks per pair at
//     d = 128.  Before every barrier a wave waits until at most its two latest
//     refill batches are in flight, which lands each pair before the barrier
//     in front of its first reader.
//   * Softmax without rescaling: each row's exponent reference is the max of
//     its first 32 keys, and P = 2^(x - ref) is exact in bf16/fp32 far above 1.
//     The row sum bounds every P of the row; if some row's sum reaches
//     2^HEADROOM, the work-group takes the exact row max over all keys in a
//     second sweep and recomputes with it as reference (then P <= 1).  So the
//     loop has no branch on data.
//   * Scores come out of the INT8 MFMAs already as float bit patterns (the
//     accumulation starts at the bits of 1.5 * 2^23, and |S| < 2^22 for
//     d <= 128, so the int32 result read as a float is exactly 1.5 * 2^23 + S):
//     a score costs one FMA and one v_exp_f32, then a share of a bf16 pack and
//     one add to the row sum.
//   * Only the last, possibly ragged tile masks keys: K rows past N load row
//     N-1 (in bounds), their P are zeroed; the packed V tiles are zero past N.
//   * Block-sparse (SP): the ring walks the work-group's sorted list of kept
//     tiles (positions index entries, list entries name tiles); a listed tile
//     this wave's mask row drops gets the exponent offset +inf (P = 0), and
//     the reference is taken from the first kept tile.
//   * Q smoothing (SM, dense): the logit bias of the wave's Q block for the K
//     tile's 64 keys (binary32, units of sQ sK) rides in the ring entry with
//     the tile (1 KB, up to four blocks); the vector phase adds it to the
//     float-bits scores before the exponent (the first tile's from global
//     memory), one float add per score rounded at the scores' unit (a c / 2
//     logit error at most where |S + bias| < 2^22, inside the 16-bit path's
//     tolerance); maxima are then taken as floats.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace sqattn {

namespace {

// (1, 1) as a bf16 pair: the row sums' second operand
constexpr v2bf ONE_BF16X2 = {(__bf16)1.0f, (__bf16)1.0f};

__device__ __forceinline__ int perm_key(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

constexpr float HEADROOM = 64.0f;  // log2 units
constexpr int WAVES = 8;
constexpr int NTHR = 64 * WAVES;
constexpr int NSLOT = 5;           // LDS ring depth (pairs)
constexpr int SQ_MAGIC = 0x4B400000;   // bits of 1.5 * 2^23
constexpr float SQ_MAGIC_F = 12582912.0f;

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 field layout:
// vmcnt[3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// max and sum over lanes l and l^32 (v_permlane32_swap pairs them)
__device__ __forceinline__ int pair_max_i(int v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float pair_sum_f(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// uniform load through the scalar cache (the K scales are read-only here)
__device__ __forceinline__ float ld_uniform(const float* p) {
  return *(const __attribute__((address_space(4))) float*)p;
}

// Position of 16-byte unit c of row r in an LDS tile with U units per row:
// r * U + (c ^ f(r)), f(r) = (r / (16 / U)) mod U.  Sixteen consecutive rows
// read at one column c then cover all 16 bank groups of a 256-byte LDS line.
template <int U>
__host__ __device__ __forceinline__ int swz(int r, int c) {
  return r * U + (c ^ ((r / (16 / U)) & (U - 1)));
}

template <int D, bool SM = false>
struct Geo {
  static constexpr int NCH = D / 32;            // INT8 k-steps (32 channels each)
  static constexpr int NCB = D / 32;            // 32-channel blocks of O^T
  static constexpr int KU = D / 16;             // 16-byte units of a K row
  static constexpr int KBYTES = KT * D;         // K tile in LDS
  static constexpr int VU = 8;                  // 16-byte units of a V^T row (64 keys * 2 B)
  static constexpr int VTB = D * 128;           // V^T tile in LDS
  static constexpr int KSC = KBYTES + VTB;      // the K tile's scale (64 copies, one per lane)
  static constexpr int BOFF = KSC + 256;        // the Q-smoothing bias of the K tile (SM)
  static constexpr int ES = BOFF + (SM ? 1024 : 0);  // ring entry: K tile, V^T tile, K scale, bias
  static constexpr int LDS_BYTES = NSLOT * ES;
  static constexpr int KCH = KBYTES / 1024;     // 1 KB direct loads per K tile
  static constexpr int VCH = VTB / 1024;        // ... per V^T tile
  static constexpr int PER = (KCH + VCH + WAVES - 1) / WAVES;  // chunk loads per wave per pair
  static constexpr int VBYTES = D * KT * 2;     // packed V tile in HBM
};

template <int D, bool SP, bool SM = false>
struct Ctx {
  using G = Geo<D, SM>;
  uint8_t* lds;
  const uint8_t* kh;
  const uint8_t* vth;
  const float* skh;
  const uint8_t* qbh;     // SM: the bias rows of the work-group's first Q block
  uint32_t qboff;         // SM: this lane's byte offset in them (block lane / 16, 4 keys)
  uint32_t qbw;           // SM: byte offset of this wave's block in an entry's bias area
  long long qbg;          // SM: byte offset of this wave's block row from qbh (global)
  uint32_t* dbg;          // checking build: the violation word (else null)
  int N, nt, lane, wave, g, lr;
  uint32_t kad[G::NCH];   // per-lane LDS byte offsets of the K operands (k-step ch, half 0)
  uint32_t vad[4];        // ... of the V^T operands (16-key k-step ks, channel block 0)
  float cq;               // sQ(row) * scale * log2(e)
  v4i qreg[G::NCH];       // Q operands
  v16i magic;             // SQ_MAGIC in every element: start of the INT8 accumulation
  v16i s[2];              // S^T of the current tile, two 32-key halves
  v4i pb[4];              // P^T operands of the current tile, four 16-key k-steps
  v16f o[G::NCB];         // O^T accumulators
  float m, l;             // reference max (log2 units), row sum
  float lp[4];            // the row sum's four partials (one per packed pair), kept across tiles
  // block-sparse: the work-group's tile list (LDS), its length, and whether
  // this wave's reference is set (taken from its first kept tile)
  const int* list;
  int cnt;
  bool has_m;

  __device__ __forceinline__ int tile_at(int pos) const {
    // (the list entry is the same for every lane: keep the tile in a scalar register)
    if constexpr (SP) return __builtin_amdgcn_readfirstlane(list[min(pos, cnt - 1)]) & 0xFFFFFF;
    return min(pos, nt - 1);
  }
  __device__ __forceinline__ bool keeps(int e) const { return ((e >> (24 + (wave >> 2))) & 1) != 0; }

  // ---- global -> LDS (direct).  A pair is KCH + VCH 1 KB chunks; chunk u
  // goes to wave u % 8, so each wave issues PER chunk loads per pair (slots
  // past the total wrap around and load a chunk again: the same bytes, so
  // every wave counts the same loads); wave 0 also copies the K scale.  Lane
  // l of a chunk writes LDS unit 64 u + l of the tile, i.e. row (64 u + l) /
  // U, permuted column (64 u + l) % U, and so reads the global unit at the
  // un-permuted column of that row (off[i]).
  uint32_t off[G::PER];  // lane's byte offset of chunk slot i within its global tile
  int chunk[G::PER];     // wave-uniform chunk of slot i: < KCH K, else V

  __device__ __forceinline__ bool is_k(int i) const {
    // at d = 128 slot 0 is the K chunk of every wave, the others V chunks
    if constexpr (G::KCH == WAVES) return i == 0;
    return chunk[i] < G::KCH;
  }
  __device__ __forceinline__ void init_loads() {
#pragma unroll
    for (int i = 0; i < G::PER; ++i) {
      int u = wave + WAVES * i;
      if (u >= G::KCH + G::VCH) u -= G::KCH + G::VCH;
      chunk[i] = u;
      if (u < G::KCH) {
        const int q = u * 64 + lane, r = q / G::KU, p = q % G::KU;
        off[i] = (uint32_t)(r * D + (p ^ ((r / (16 / G::KU)) & (G::KU - 1))) * 16);
      } else {
        const int q = (u - G::KCH) * 64 + lane, r = q / G::VU, p = q % G::VU;
        off[i] = (uint32_t)(r * 128 + (p ^ ((r / (16 / G::VU)) & (G::VU - 1))) * 16);
      }
    }
  }
  // Pair at list position j: K tile of position j + 1 and V tile of position
  // j (both clamped to the last position) into entry j % NSLOT.  K rows past N
  // (last tile) read row N-1: klim is the byte offset of the last row to read.
  struct Refill {
    const uint8_t* kt;
    const uint8_t* vt;
    const float* ks;
    const uint8_t* qb;
    uint32_t klim;
    int entry;
  };
  __device__ __forceinline__ Refill refill(int j) const {
    const int tk = tile_at(j + 1), tv = tile_at(j);
    SQ_CHECK(dbg, tk >= 0 && tk < nt, 0);
    SQ_CHECK(dbg, tv >= 0 && tv < nt, 1);
    SQ_CHECK(dbg, N - 1 - tk * KT >= 0, 2);  // the last K row read exists
    return Refill{kh + (long long)tk * KT * D, vth + (long long)tv * G::VBYTES, skh + tk,
                  SM ? qbh + (long long)tk * KT * 4 : nullptr, (uint32_t)(min(N - 1 - tk * KT, KT) * D),
                  j % NSLOT};
  }
  // chunk slot i of a pair (i == PER: the K scale, wave 0 only, and with SM
  // the tile's bias, wave 1 only).  K rows past the tile's last valid row
  // read that row (same permuted column).
  __device__ __forceinline__ void load_part(const Refill& r, int i) {
    if (i == G::PER) {
      if (wave == 0) lds_dma4(r.ks, 0u, lds_addr(lds + r.entry * G::ES + G::KSC));
      if (SM && wave == 1) lds_dma16(r.qb, qboff, lds_addr(lds + r.entry * G::ES + G::BOFF));
      return;
    }
    const bool isk = is_k(i);  // wave-uniform
    const uint8_t* base = isk ? r.kt : r.vt;
    const uint32_t o = isk ? min(off[i], r.klim + (off[i] & (D - 1))) : off[i];
    const int dst = r.entry * G::ES + (isk ? chunk[i] * 1024 : G::KBYTES + (chunk[i] - G::KCH) * 1024);
    lds_dma16(base, o, lds_addr(lds + dst));
  }
  __device__ __forceinline__ void issue(const Refill& r) {
#pragma unroll
    for (int i = 0; i <= G::PER; ++i) load_part(r, i);
  }

  // Phase boundary: this wave's refill loads older than its two latest
  // batches have landed; then a work-group barrier (a plain s_barrier, since
  // __syncthreads() would also wait for every direct-to-LDS load in flight,
  // which empties the ring).  Wave 0 issues one load more per pair.  LDS
  // reads are not waited for here: the matrix phase consumes its operands
  // itself, and the reads in flight at a barrier (the operands prefetched for
  // the next matrix phase, the next K scale) address entries that no refill
  // touches before both wave groups have passed that phase.
  __device__ __forceinline__ void phase_bar() const {
    __builtin_amdgcn_sched_barrier(0);
#ifdef SQATTN_DEBUG
    // checking build: every load in flight lands before every barrier
    __builtin_amdgcn_s_waitcnt(0);
#else
    if (wave == 0 || (SM && wave == 1))
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (G::PER + 1)));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * G::PER));
#endif
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- S^T of K tile t straight from global memory (rows past N read row N-1)
  __device__ __forceinline__ void qk_global(int t) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(t * KT + kb * 32 + perm_key(lr), N - 1);
#pragma unroll
      for (int ch = 0; ch < G::NCH; ++ch) {
        const v4i a = *(const v4i*)(kh + (long long)key * D + ch * 32 + g * 16);
        s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], ch == 0 ? magic : s[kb], 0, 0, 0);
      }
    }
  }

  // SM: the same over scores held as binary32 bit patterns of any sign, less off
  __device__ __forceinline__ float rowmax_f(const v16i& x, float c, float off) const {
    float d = __builtin_fmaxf(__int_as_float(x[0]), __int_as_float(x[1]));
#pragma unroll
    for (int i = 2; i < 16; ++i) d = __builtin_fmaxf(d, __int_as_float(x[i]));
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(d), __float_as_int(d), false, false);
    return (__builtin_fmaxf(__int_as_float(r[0]), __int_as_float(r[1])) - off) * c;  // c >= 0
  }

  // max over the 32 keys of half kb of S (lanes l and l^32 share a query), in log2 units
  __device__ __forceinline__ float rowmax(const v16i& x, float c, int bias) const {
    int d = max(max(x[0], x[1]), x[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) d = max(max(d, x[i]), x[i + 1]);
    d = max(d, x[15]);
    return (float)(pair_max_i(d) - bias) * c;  // c >= 0
  }

  // ---- SM: add the bias of the tile's keys (64 binary32 values of the
  // wave's block at p, LDS or global) to the scores held as float bits
  // (ints: converted first): register i of half kb is key
  // 32 kb + 16 (i / 8) + 8 g + i % 8
  template <bool FROM_INT = false, class P>
  __device__ __forceinline__ void add_bias(const P* p) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v4f b0 = *(const v4f*)((const uint8_t*)p + (32 * kb + 16 * h + 8 * g) * 4);
        const v4f b1 = *(const v4f*)((const uint8_t*)p + (32 * kb + 16 * h + 8 * g) * 4 + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i0 = 8 * h + r, i1 = 8 * h + 4 + r;
          const float x0 = FROM_INT ? (float)s[kb][i0] : __int_as_float(s[kb][i0]);
          const float x1 = FROM_INT ? (float)s[kb][i1] : __int_as_float(s[kb][i1]);
          s[kb][i0] = __float_as_int(x0 + b0[r]);
          s[kb][i1] = __float_as_int(x1 + b1[r]);
        }
      }
  }

  // ---- V(t): P = 2^(S c - k) with k = 1.5 * 2^23 c + ref, packed to bf16 as
  // the P^T operands, and the row sum of those rounded P.  Register i of half kb holds key
  // 32 kb + 16 (i / 8) + 8 g + i % 8 (perm_key order), which is element
  // i % 8 of lane-half g of 16-key k-step 2 kb + i / 8.  MASK: keys >= kvalid
  // get P = 0.  SM: bias_e is the entry holding the tile's bias (< 0: the
  // bias is in the scores already).
  template <bool MASK>
  __device__ __forceinline__ void vphase(float c, float k, int kvalid, const Refill& rf, int bias_e = -1) {
    if constexpr (SM) {
      if (bias_e >= 0) add_bias(lds + bias_e * G::ES + G::BOFF + qbw);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 8 * (ks & 1) + 2 * j;
        float u0 = __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(s[ks >> 1][i]), c, -k));
        float u1 = __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(s[ks >> 1][i + 1]), c, -k));
        if constexpr (MASK) {
          const int key = 16 * ks + 8 * g + 2 * j;
          u0 = key < kvalid ? u0 : 0.0f;
          u1 = key + 1 < kvalid ? u1 : 0.0f;
        }
        w[j] = pack_bf16x2(u0, u1);
        // the row sum adds the rounded P the matrix cores multiply, a pair
        // per v_dot2_f32_bf16 into one of four partials that are combined
        // only after the last tile (fewer vector instructions and registers
        // than adding the fp32 values per tile)
        lp[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, w[j]), ONE_BF16X2, lp[j], false);
      }
      pb[ks] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      // the refill, spread over the phase
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i <= G::PER; ++i)
        if (i * 4 / (G::PER + 1) == ks) load_part(rf, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- M(t): refill, then S(t+1) from entry t's K tile (QK), then
  // O^T += V(t)^T P(t)^T from entry t's V^T tile.
  // Operand i of M(t) (entry e): the INT8 ones first (K, k-step i / 2, half
  // i % 2), then the bf16 ones (V^T, k-step (i - NK) / NCB, block (i - NK) % NCB).
  template <bool QK>
  __device__ __forceinline__ v4i operand(const uint8_t* e, int i) const {
    constexpr int NK = QK ? 2 * G::NCH : 0;
    if (i < NK) return *(const v4i*)(e + kad[i >> 1] + (i & 1) * 32 * D);
    const int j = i - NK;
    return *(const v4i*)(e + vad[j / G::NCB] + (j % G::NCB) * 32 * 128);
  }
  // operand reads in flight ahead of their MFMA (3 measured 2-3% faster than
  // 2 or 4 on wan14b-480p; 5 spills)
  static constexpr int RD = 3;
  v4i pre[RD];                  // M(t)'s first operands, read at the end of V(t)
  template <bool QK>
  __device__ __forceinline__ void prefetch(int t) {
    const uint8_t* e = lds + (t % NSLOT) * G::ES;
#pragma unroll
    for (int i = 0; i < RD; ++i) pre[i] = operand<QK>(e, i);
  }

  // Returns the scale of K tile t + 1 (kept in the entry), which V(t + 1) needs.
  // Runs at raised wave priority, so that the other wave's vector work does
  // not delay the matrix instructions.
  template <bool QK>
  __device__ __forceinline__ float mphase(int t) {
    __builtin_amdgcn_s_setprio(3);
    const uint8_t* e = lds + (t % NSLOT) * G::ES;
    constexpr int NK = QK ? 2 * G::NCH : 0;  // INT8 MFMAs
    constexpr int NM = NK + 4 * G::NCB;      // all MFMAs of the phase
    v4i a[NM];
#pragma unroll
    for (int i = 0; i < NM; ++i) a[i] = i < RD ? pre[i < RD ? i : 0] : operand<QK>(e, i);
    const float ksc = *(const float*)(e + G::KSC + 4 * lane);
    if constexpr (QK) {
#pragma unroll
      for (int ch = 0; ch < G::NCH; ++ch)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[2 * ch + kb], qreg[ch], ch == 0 ? magic : s[kb], 0, 0, 0);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int cb = 0; cb < G::NCB; ++cb)
        o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[NK + ks * G::NCB + cb]),
                                                        __builtin_bit_cast(v8bf, pb[ks]), o[cb], 0, 0, 0);
    // Issue order: each MFMA followed by the next operand read, so every
    // operand is read RD MFMAs ahead of its use (the first RD were read
    // before the phase; the scale read goes with the first one).
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i > 0 && i + RD < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    return ksc;
  }

  // exponent offset of list position pos (block-sparse): +inf for a tile
  // this wave's mask row drops; the reference is taken lazily from the first
  // 32 keys of the wave's first kept tile
  __device__ __forceinline__ float k_sparse(int pos, float c) {
    const bool act = keeps(list[pos]);
    if (act && !has_m) {
      m = rowmax(s[0], c, SQ_MAGIC);
      has_m = true;
    }
    return act ? __builtin_fmaf(SQ_MAGIC_F, c, m) : __builtin_inff();
  }

  // ---- one pass over the npos listed tiles with the ping-pong schedule
  __device__ __forceinline__ void pipeline(int npos, bool set_ref) {
    init_loads();
#pragma unroll
    for (int j = 0; j < NSLOT - 1; ++j) issue(refill(j));
    qk_global(tile_at(0));
    if constexpr (SM) add_bias(qbh + qbg + (long long)tile_at(0) * KT * 4);
    float c = cq * ld_uniform(skh + tile_at(0));
    if (!SP && set_ref)  // reference: max of the first 32 keys
      m = SM ? rowmax_f(s[0], c, SQ_MAGIC_F) : rowmax(s[0], c, SQ_MAGIC);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (wave >= 4) phase_bar();  // waves 4-7 run one phase behind
    // all positions but the last (only the last can hold the ragged tile)
    for (int t = 0; t < npos - 1; ++t) {
      // V(t) refills the entry of pair t - 2 with pair t + 3, then reads the
      // first operands of M(t)
      vphase<false>(c, SP ? k_sparse(t, c) : __builtin_fmaf(SQ_MAGIC_F, c, m), KT, refill(t + NSLOT - 2),
                    t > 0 ? (t - 1) % NSLOT : -1);
      prefetch<true>(t);
      phase_bar();
      const float ksc = mphase<true>(t);
      phase_bar();
      c = cq * ksc;
    }
    const int t = npos - 1;
    vphase<true>(c, SP ? k_sparse(t, c) : __builtin_fmaf(SQ_MAGIC_F, c, m), N - tile_at(t) * KT,
                 refill(t + NSLOT - 2), t > 0 ? (t - 1) % NSLOT : -1);
    prefetch<false>(t);
    phase_bar();
    mphase<false>(t);
    phase_bar();
    if (wave < 4) phase_bar();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  }

  // ---- exact row max over the listed tiles this wave keeps (the rare second
  // pass): K tiles one at a time through entry 0
  __device__ __forceinline__ float exact_max(int npos) {
    float mx = -__builtin_inff();
    for (int j = 0; j < npos; ++j) {
      const int t = tile_at(j);
      SQ_CHECK(dbg, t >= 0 && t < nt, 4);
      __syncthreads();
      const int kmax = N - 1 - t * KT;
      for (int u = wave; u < G::KCH; u += WAVES) {
        const int q = u * 64 + lane, r = q / G::KU, p = q % G::KU;
        const int pc = p ^ ((r / (16 / G::KU)) & (G::KU - 1));
        lds_dma16(kh + (long long)t * KT * D, (uint32_t)(min(r, kmax) * D + pc * 16), lds_addr(lds + u * 1024));
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const float c = cq * ld_uniform(skh + t);
      v16i z;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ch = 0; ch < G::NCH; ++ch) {
          const v4i a = *(const v4i*)(lds + kad[ch] + kb * 32 * D);
          s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], ch == 0 ? z : s[kb], 0, 0, 0);
        }
      float r;
      if constexpr (SM) {
        add_bias<true>(qbh + qbg + (long long)t * KT * 4);
        r = __builtin_fmaxf(rowmax_f(s[0], c, 0.0f), rowmax_f(s[1], c, 0.0f));
      } else {
        r = __builtin_fmaxf(rowmax(s[0], c, 0), rowmax(s[1], c, 0));
      }
      if (!SP || keeps(list[j])) mx = __builtin_fmaxf(mx, r);
    }
    __syncthreads();
    return mx;
  }
};

}  // namespace

template <int D, bool SP, bool SM>
__global__ __launch_bounds__(NTHR) void attn_bf16_kernel(AttnParams p) {
  using Cx = Ctx<D, SP, SM>;
  using G = Geo<D, SM>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int w = blockIdx.x;
  const int item = (w & 7) * p.per_xcd + (w >> 3);
  if (item >= p.BH * p.qtiles) return;
  const int bh = item / p.qtiles, qt = item - bh * p.qtiles;

  Cx C;
  C.lds = smem;
  const int tid = threadIdx.x;
  C.lane = tid & 63;
  C.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  C.g = C.lane >> 5;
  C.lr = C.lane & 31;
#pragma unroll
  for (int ch = 0; ch < G::NCH; ++ch) C.kad[ch] = swz<G::KU>(perm_key(C.lr), 2 * ch + C.g) * 16;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) C.vad[ks] = G::KBYTES + swz<G::VU>(C.lr, 2 * ks + C.g) * 16;
  C.N = p.N;
  C.nt = p.nt;
  const long long hoff = (long long)bh * p.N * D;
  C.kh = (const uint8_t*)p.k + hoff;
  C.vth = (const uint8_t*)p.vt + (long long)bh * p.nt * G::VBYTES;
  C.skh = p.sk + (long long)bh * p.nt;
  C.dbg = p.debug;
  if constexpr (SM) {
    // blocks of q_block (64, 128 or 256) rows: the work-group's first block
    // and this wave's (a wave whose rows all lie past N takes the last
    // existing block); lane l of the bias load reads block b0 + l / 16 (the
    // last existing one past the end), keys 4 (l % 16) .. + 3
    const int b0 = qt * ATT_QWG / p.q_block, nbw = min(ATT_QWG / p.q_block, p.nq - b0);
    const long long rowb = (long long)p.nt * KT * 4;
    C.qbh = (const uint8_t*)p.qbias + ((long long)bh * p.nq + b0) * rowb;
    C.qboff = (uint32_t)(min(C.lane / 16, nbw - 1) * rowb + (C.lane % 16) * 16);
    const int wb = min(C.wave * ATT_QW / p.q_block, nbw - 1);
    C.qbw = (uint32_t)(wb * 256);
    C.qbg = (long long)wb * rowb;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) C.magic[r] = SQ_MAGIC;
  asm volatile("" : "+v"(C.magic));  // keep the accumulator start in vector registers
  const int row = qt * ATT_QWG + C.wave * ATT_QW + C.lr;
  const bool rok = row < p.N;
#pragma unroll
  for (int ch = 0; ch < G::NCH; ++ch)
    C.qreg[ch] = rok ? *(const v4i*)(p.q + hoff + (long long)row * D + ch * 32 + C.g * 16) : v4i{0, 0, 0, 0};
  C.cq = rok ? p.sq[(long long)bh * p.nq + row / p.q_block] * p.scale_log2e : 0.0f;
  C.m = 0.0f;

  // block-sparse: the list of tiles this work-group visits (a dense pass
  // visits 0 .. nt-1)
  int npos = p.nt;
  if constexpr (SP) {
    int* list = (int*)(smem + G::LDS_BYTES);
    const uint8_t* m0 = p.mask + ((long long)bh * p.mq + 2 * qt) * p.nt;
    const uint8_t* m1 = (2 * qt + 1 < p.mq) ? m0 + p.nt : nullptr;
    npos = build_tile_list(m0, m1, p.nt, list, list + SP_MAXT, NTHR);
    SQ_CHECK(p.debug, npos >= 0 && npos <= SP_MAXT, 3);
    C.list = list;
    C.cnt = npos;
    C.has_m = false;
  }

  for (int pass = 0; pass < 2 && npos > 0; ++pass) {
    if (pass == 1) {
      // Rare path: some row's sum reached 2^HEADROOM.  Take the exact row max
      // over all keys as the reference, so that every P <= 1.
      if (p.second_pass && threadIdx.x == 0) atomicAdd(p.second_pass, 1u);
      C.m = C.exact_max(npos);
      if constexpr (SP) C.has_m = true;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) C.lp[j] = 0.0f;
#pragma unroll
    for (int cb = 0; cb < G::NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) C.o[cb][i] = 0.0f;
    C.pipeline(npos, pass == 0);
    C.l = pair_sum_f((C.lp[0] + C.lp[1]) + (C.lp[2] + C.lp[3]));
    // the sum bounds every P: l < 2^HEADROOM keeps P and O far from overflow
    const bool over = !(C.l < __builtin_exp2f(HEADROOM));
    if (pass == 1 || !__syncthreads_or(over)) break;
  }

  // epilogue: O = O^T / l, fp32 or bf16 rows (block-sparse: rows whose mask
  // keeps no tile have l = 0 and O = 0 and are written as zeros)
  if constexpr (SP) {
    if (npos == 0) {
      C.l = 0.0f;
#pragma unroll
      for (int cb = 0; cb < G::NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) C.o[cb][i] = 0.0f;
    }
  }
  const float inv = (SP && !(C.l > 0.0f)) ? 0.0f : 1.0f / C.l;
  if (rok) store_out_row(p.out, p.out_bf16 != 0, lay_row(p.lo, bh, row), C.o, inv, C.g);
}

template <int D, bool SP, bool SM>
static hipError_t launch_d(const AttnParams& q, hipStream_t st) {
  constexpr int lds = Geo<D, SM>::LDS_BYTES + (SP ? SP_LIST_BYTES : 0);
  // the attribute is per kernel: set once per process (the first status is kept)
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute((const void*)attn_bf16_kernel<D, SP, SM>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((attn_bf16_kernel<D, SP, SM>), dim3(8 * q.per_xcd), dim3(NTHR), lds, st, q);
  return hipSuccess;
}

// Q smoothing (q.qbias) runs on the dense kernels only (the caller checks)
hipError_t launch_attention_bf16(const AttnParams& q, int d, hipStream_t st) {
  const bool sp = q.mask != nullptr, sm = q.qbias != nullptr;
  if (d == 128) {
    if (sm) return launch_d<128, false, true>(q, st);
    return sp ? launch_d<128, true, false>(q, st) : launch_d<128, false, false>(q, st);
  }
  if (sm) return launch_d<64, false, true>(q, st);
  return sp ? launch_d<64, true, false>(q, st) : launch_d<64, false, false>(q, st);
}

}  // namespace sqattn
