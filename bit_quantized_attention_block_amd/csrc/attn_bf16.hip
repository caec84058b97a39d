// Quantized attention kernel, 16-bit P.V path (gfx950).
//
// INT8 S^T = K Q^T, lane-local softmax, O^T = V^T P^T in the register
// layouts described in attn.hip.
//
// Work-group: 8 waves (two per SIMD), 32 query rows each, 256 rows per
// work-group.  The unit of the pipeline is a half-tile h of 32 keys (half
// kb = h%2 of 64-key tile h/2):
//
//   iteration h:   MFMA  S(h+1) = K(h+1) Q^T           (D/32 x i8 32x32x32)
//                  MFMA  O     += V(h-1)^T P(h-1)^T    (D/16 x bf16 32x32x16)
//                  VALU  P(h)   = softmax step on S(h)
//
// The MFMAs and the softmax of an iteration are independent; they are
// interleaved at the finest grain: each MFMA is followed by one softmax pair
// (two scores) in the same inline-assembly statement, and each MFMA operand is
// read from LDS four MFMAs ahead.  The second wave on the SIMD fills what is
// left of the gaps.
//
//   * LDS: a 4-slot ring of K tiles (with the tile's K scale) and of V tiles,
//     refilled with direct-to-LDS loads three tiles ahead; one barrier per
//     tile, waiting only for the loads issued three tiles earlier.  Rows are
//     padded to a stride of 144 bytes (80 for 64-byte K rows): with an odd
//     number of 16-byte units per row, the 16 rows read by 16 consecutive
//     lanes fall in distinct banks, and every operand address is one base
//     register plus an immediate offset.
//   * No rescaling inside the loop: each row's reference is the max of its
//     first 32 keys, and P = 2^(x - ref) is exact in bf16/fp32 far above 1.
//     The row sum bounds every P of the row; if some row's sum reaches
//     2^HEADROOM, the work-group takes the exact row max over all keys in a
//     second sweep and recomputes with it as reference (then P <= 1).  So the
//     loop body has no branch on data.
//   * Scores come out of the INT8 MFMAs already as float bit patterns (the
//     accumulation starts at the bits of 1.5 * 2^23), so a score costs one FMA
//     and one v_exp_f32 before packing; the row sum adds the fp32 P.  (Vector
//     instructions other than transcendentals overlap the matrix core only a
//     little, and v_dot2c stalls it, so the per-score vector work is kept to
//     FMA, exp, a share of one pack and two adds per pair.)
//   * Only the last, possibly ragged tile needs key masking.  Rows past N in
//     the K tile load row N-1 (in bounds, a real score); their P entries are
//     zeroed and taken out of the row sum afterwards.  The packed V tiles are
//     zero past N.
#include "common.h"
#include "kernels.h"

namespace sqattn {

namespace {

__device__ __forceinline__ int perm_key(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

constexpr float HEADROOM = 64.0f;  // log2 units
constexpr int WAVES = 8;
constexpr int NTHR = 64 * WAVES;
constexpr int NSLOT = 4;           // LDS ring depth (tiles)


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

template <int D>
struct Geo {
  static constexpr int NCH = D / 32;            // QK k-steps per half-tile
  static constexpr int NCB = D / 32;            // 32-channel blocks of O^T
  static constexpr int KCPR = D / 16;           // 16-byte chunks of a K row
  static constexpr int KROWC = KCPR + 1;        // ... padded (odd)
  static constexpr int KROW = 16 * KROWC;       // padded K row stride (bytes)
  static constexpr int KSC = KT * KROW;         // offset of the K scale in a K slot
  static constexpr int KS = KSC + 256;          // K slot bytes (64 copies of the scale)
  static constexpr int VROWC = 9;               // V^T row: 64 keys * 2 B = 8 chunks + pad
  static constexpr int VROW = 16 * VROWC;
  static constexpr int VS = D * VROW;           // V slot bytes
  static constexpr int VBASE = NSLOT * KS;      // V ring offset in LDS
  static constexpr int LDS_BYTES = NSLOT * (KS + VS);
  static constexpr int KINST = (KT * KROWC + 63) / 64;   // 1 KB direct loads per K tile
  static constexpr int VINST = (D * VROWC + 63) / 64;     // ... per V tile
  static constexpr int PER = (KINST + VINST + WAVES - 1) / WAVES;  // K+V loads per wave
  static constexpr int LPB = PER + 1;           // direct loads per wave per tile boundary (+ K scale)
  static constexpr int VBYTES = D * KT * 2;     // packed V tile in HBM
};

// ---------------------------------------------------------------------------
// One MFMA followed by one softmax pair, as one inline-assembly statement.
//
// Scores arrive as float bit patterns: the INT8 accumulation starts from the
// bits of 1.5 * 2^23 (SQ_MAGIC) instead of 0, and since |S| < 2^22 the int32
// result read as a float is exactly 1.5 * 2^23 + S.  The pair turns two such
// scores into P = 2^(S c - m) = 2^(x c - k) with k = 1.5 * 2^23 c + m (one
// FMA each, no conversion), rounds the pair to packed bf16 (w), and adds the
// two fp32 values to the row sum (acc).
//
// Only assembly statements read the MFMA results (S, O), so no
// compiler-generated instruction can touch a register an MFMA is still
// writing; the compiler keeps volatile statements in order and does not move
// memory accesses across them ("memory"), so the operand reads written
// between them stay where they are written, with the compiler's own waits.  A
// score of S(h) is read at least one iteration after the MFMA that produced
// it.
// ---------------------------------------------------------------------------
constexpr int SQ_MAGIC = 0x4B400000;   // bits of 1.5 * 2^23
constexpr float SQ_MAGIC_F = 12582912.0f;

// One MFMA and up to two softmax-pair stages as one inline-assembly
// statement.  Stage 1 turns two scores into P = 2^(x c - k) in fp32 (u0, u1);
// stage 2, four MFMAs later, packs such a pair to bf16 (w) and adds it to the
// row sum (acc).  Exponentials overlap the matrix core well, other vector
// instructions much less, so the stages are spread over the iteration's
// MFMAs.  Being one statement, no stage output can share a register with the
// MFMA's sources (early-clobber outputs), which a separate statement could
// reuse while the MFMA has yet to read them.
//   MF: 0 none, 1 first INT8 k-step (accumulator from mg), 2 INT8, 3 bf16 P.V
#define SQ_ST1                                      \
  "\n v_fma_f32 %[u0], %[s0], %[c], -%[k]"          \
  "\n v_fma_f32 %[u1], %[s1], %[c], -%[k]"          \
  "\n v_exp_f32 %[u0], %[u0]"                      \
  "\n v_exp_f32 %[u1], %[u1]"
#define SQ_ST2                                      \
  "\n s_nop 0"                                     \
  "\n v_cvt_pk_bf16_f32 %[w], %[v0], %[v1]"        \
  "\n v_add_f32 %[acc], %[acc], %[v0]"             \
  "\n v_add_f32 %[acc], %[acc], %[v1]"
#define SQ_OUTS [acc] "+v"(acc), [u0] "=&v"(u0), [u1] "=&v"(u1), [w] "=&v"(w)
#define SQ_INS [a] "v"(a), [b] "v"(b), [s0] "v"(s0), [s1] "v"(s1), [c] "v"(c), [k] "v"(k), [v0] "v"(v0), [v1] "v"(v1)
// the statement for MFMA text mf, with the stages this slot holds
#define SQ_SLOT(mf, outs, ins)                                          \
  if constexpr (S1 && S2)                                               \
    asm volatile(mf SQ_ST1 SQ_ST2 : outs : ins : "memory");             \
  else if constexpr (S1)                                                \
    asm volatile(mf SQ_ST1 : outs : ins : "memory");                    \
  else if constexpr (S2)                                                \
    asm volatile(mf SQ_ST2 : outs : ins : "memory");                    \
  else                                                                  \
    asm volatile(mf : outs : ins : "memory");
#define SQ_COMMA ,

template <int MF, bool S1, bool S2>
__device__ __forceinline__ void slot(v16i& sn, v16f& o, v4i a, v4i b, const v16i& mg, int s0, int s1, float c,
                                     float k, float& u0, float& u1, float v0, float v1, uint32_t& w, float& acc) {
  if constexpr (MF == 1) {
    SQ_SLOT("v_mfma_i32_32x32x32_i8 %[sn], %[a], %[b], %[mg]", [sn] "=&v"(sn) SQ_COMMA SQ_OUTS,
            SQ_INS SQ_COMMA [mg] "v"(mg))
  } else if constexpr (MF == 2) {
    SQ_SLOT("v_mfma_i32_32x32x32_i8 %[sn], %[a], %[b], %[sn]", [sn] "+v"(sn) SQ_COMMA SQ_OUTS, SQ_INS)
  } else if constexpr (MF == 3) {
    SQ_SLOT("v_mfma_f32_32x32x16_bf16 %[o], %[a], %[b], %[o]", [o] "+v"(o) SQ_COMMA SQ_OUTS, SQ_INS)
  } else {
    SQ_SLOT("", SQ_OUTS, SQ_INS)
  }
}
#undef SQ_COMMA
#undef SQ_SLOT
#undef SQ_INS
#undef SQ_OUTS
#undef SQ_ST2
#undef SQ_ST1

template <int D, bool SP = false>
struct Ctx {
  using G = Geo<D>;
  uint8_t* lds;
  const uint8_t* kh;
  const uint8_t* vth;
  const float* skh;
  int N, nt, lane, wave, g, lr;
  uint32_t kbase, vbase;  // per-lane LDS operand offsets (slot 0, half 0)
  float cq;               // sQ(row) * scale * log2(e)
  v4i qreg[G::NCH];       // Q operands
  v16i magic;             // SQ_MAGIC in every element: start of the INT8 accumulation
  v16f o[G::NCB];         // O^T accumulators
  float m, l;             // reference max (log2 units), row sum
  // block-sparse only: the work-group's tile list (LDS) and whether this
  // wave's reference is set (it is taken from its first kept tile)
  const int* list;
  int cnt;
  bool has_m;

  // ---- global -> LDS (direct).  One boundary refills a K slot (KINST 1 KB
  // chunks, padded rows) and a V slot (VINST chunks); the KINST + VINST chunks
  // are spread over the waves, PER instructions each (slots past the total
  // wrap around and load a chunk again: the same bytes, so every wave counts
  // the same loads).  Each instruction reads 16 bytes per lane at a fixed
  // per-lane offset (off[i]) from a wave-uniform tile base.  One more
  // instruction per wave copies the K tile's scale into the K slot.
  uint32_t off[G::PER];  // lane's byte offset of chunk slot i within its tile
  int chunk[G::PER];     // wave-uniform chunk of slot i: < KINST K, else V

  __device__ __forceinline__ void init_loads() {
#pragma unroll
    for (int i = 0; i < G::PER; ++i) {
      int u = wave + WAVES * i;
      if (u >= G::KINST + G::VINST) u -= G::KINST + G::VINST;
      chunk[i] = u;
      if (u < G::KINST) {
        const int q = u * 64 + lane;
        off[i] = (uint32_t)(min(q / G::KROWC, KT - 1) * D + min(q % G::KROWC, G::KCPR - 1) * 16);
      } else {
        const int q = (u - G::KINST) * 64 + lane;
        off[i] = (uint32_t)(min(q / G::VROWC, D - 1) * 128 + min(q % G::VROWC, 7) * 16);
      }
    }
  }
  // K rows past N in the last K tile read row N-1 instead.  Refills only move
  // forward and end on the last tile, so from its first refill on the K
  // offsets stay clamped (init_loads restores them).
  __device__ __forceinline__ void clamp_last_k() {
    const uint32_t lim = (uint32_t)((N - 1 - (nt - 1) * KT) * D);
#pragma unroll
    for (int i = 0; i < G::PER; ++i)
      if (chunk[i] < G::KINST) off[i] = min(off[i], lim + (off[i] & (D - 1)));
  }


  // K tile tk into K slot ks and V tile tv into V slot vs.  Instruction i <
  // PER is one chunk; i == PER copies the K scale.
  struct Refill {
    const uint8_t* kt;
    const uint8_t* vt;
    int tk, ks, vs;
  };
  __device__ __forceinline__ Refill refill(int tk, int ks, int tv, int vs) {
    if (tk == nt - 1) clamp_last_k();
    return Refill{kh + (long long)tk * KT * D, vth + (long long)tv * G::VBYTES, tk, ks, vs};
  }
  __device__ __forceinline__ void load_part(const Refill& r, int i) {
    if (i == G::PER) {
      lds_dma4(skh + r.tk, 0u, lds_addr(lds + r.ks * G::KS + G::KSC));
      return;
    }
    const int u = chunk[i];
    const bool isk = u < G::KINST;  // wave-uniform
    const uint8_t* base = isk ? r.kt : r.vt;
    const uint32_t o = off[i];
    const int dst = isk ? r.ks * G::KS + u * 1024 : G::VBASE + r.vs * G::VS + (u - G::KINST) * 1024;
    lds_dma16(base, o, lds_addr(lds + dst));
  }
  __device__ __forceinline__ void load_kv(int tk, int ks, int tv, int vs) {
    const Refill r = refill(tk, ks, tv, vs);
#pragma unroll
    for (int i = 0; i <= G::PER; ++i) load_part(r, i);
  }
  // K tile only, into slot 0 (the exact-max sweep; not on the hot path)
  __device__ __forceinline__ void load_k(int t) {
    const int kmax = N - 1 - t * KT;
    for (int u = wave; u < G::KINST; u += WAVES) {
      const int q = u * 64 + lane;
      const int row = min(min(q / G::KROWC, KT - 1), kmax);
      lds_dma16(kh + (long long)t * KT * D, (uint32_t)(row * D + min(q % G::KROWC, G::KCPR - 1) * 16),
                lds_addr(lds + u * 1024));
    }
  }
  __device__ __forceinline__ float k_scale(int slot) const {
    return *(const float*)(lds + slot * G::KS + G::KSC + 4 * lane);
  }

  // max over the 32 keys of S (lanes l and l^32 share a query), in log2 units
  __device__ __forceinline__ float rowmax(const v16i& s, float c, int bias) const {
    int d = max(max(s[0], s[1]), s[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) d = max(max(d, s[i]), s[i + 1]);
    d = max(d, s[15]);
    return (float)(pair_max_i(d) - bias) * c;  // c >= 0
  }

  // ---- operand i of an iteration (see the MFMA order below); ka/va: lane
  // offsets of the K half / V^T half
  __device__ __forceinline__ v4i operand(int i, uint32_t ka, uint32_t va) const {
    if (i < 2 * G::NCH && (i & 1) == 0) return *(const v4i*)(lds + ka + (i >> 1) * 32);
    const int k2 = (i < 2 * G::NCH) ? 0 : 1;
    const int cb = (i < 2 * G::NCH) ? (i >> 1) : (i - 2 * G::NCH);
    return *(const v4i*)(lds + va + cb * 32 * G::VROW + k2 * 32);
  }

  static constexpr int NMF = G::NCH + 2 * G::NCB;  // MFMAs per half-tile iteration
  static constexpr int RD_AHEAD = 4;                // operand reads ahead of their MFMA

  // ---- slot i of an iteration: MFMA i (if any), stage 1 of pair i (i < 8),
  // stage 2 of pair i - 4 (4 <= i < 12)
  template <int I>
  __device__ __forceinline__ void slot_i(const v16i& scur, v16i& snext, const v4i (&pprev)[2], const v4i (&a)[NMF],
                                         float (&u)[8][2], uint32_t (&w)[8], float c, float k, float& acc) {
    constexpr bool S1 = I < 8, S2 = I >= 4 && I < 12;
    constexpr int MF = I >= NMF ? 0 : (I < 2 * G::NCH && (I & 1) == 0) ? (I == 0 ? 1 : 2) : 3;
    constexpr int K2 = (I < 2 * G::NCH) ? 0 : 1;
    constexpr int CB = I >= NMF ? 0 : (I < 2 * G::NCH) ? (I >> 1) : (I - 2 * G::NCH);
    const v4i av = a[I < NMF ? I : 0];
    const v4i bv = MF == 3 ? pprev[K2] : qreg[MF == 0 ? 0 : ((I >> 1) < G::NCH ? (I >> 1) : 0)];
    float d0, d1;
    uint32_t dw;
    float& u0 = S1 ? u[I < 8 ? I : 0][0] : d0;
    float& u1 = S1 ? u[I < 8 ? I : 0][1] : d1;
    const float v0 = S2 ? u[S2 ? I - 4 : 0][0] : 0.0f;
    const float v1 = S2 ? u[S2 ? I - 4 : 0][1] : 0.0f;
    uint32_t& wr = S2 ? w[S2 ? I - 4 : 0] : dw;
    const int s0 = S1 ? scur[S1 ? 2 * I : 0] : 0, s1 = S1 ? scur[S1 ? 2 * I + 1 : 0] : 0;
    slot<MF, S1, S2>(snext, o[CB], av, bv, magic, s0, s1, c, k, u0, u1, v0, v1, wr, acc);
  }
  template <int I = 0>
  __device__ __forceinline__ void issue_slot(int i, const v16i& scur, v16i& snext, const v4i (&pprev)[2],
                                             const v4i (&a)[NMF], float (&u)[8][2], uint32_t (&w)[8], float c,
                                             float k, float& acc) {
    if (i == I) slot_i<I>(scur, snext, pprev, a, u, w, c, k, acc);
    if constexpr (I + 1 < (NMF > 12 ? NMF : 12)) issue_slot<I + 1>(i, scur, snext, pprev, a, u, w, c, k, acc);
  }

  // ---- one half-tile iteration h = 2t + KB.  K(h+1) is half KB^1 of tile
  // t + KB; V(h-1) is half KB^1 of tile t - 1 + KB (for h = 0 the zeroed slot
  // with P(-1) = 0).  c: the softmax factor of tile t.
  //
  // MFMA order: i < 2 NCH alternates the INT8 chain (k-step i/2) with the
  // first P.V k-step (channel block i/2); then the second P.V k-step.  Each
  // operand is read RD_AHEAD MFMAs ahead; softmax pair j (two scores of S(h),
  // one packed bf16 pair of P(h)) sits between MFMA j and MFMA j+1.
  template <int KB, bool REFILL = false>
  __device__ __forceinline__ void step(const v16i& scur, v16i& snext, const v4i (&pprev)[2], v4i (&pcur)[2],
                                       int t, float c, float k, float& acc, const Refill* rf = nullptr) {
    const uint32_t ka = kbase + ((t + KB) & (NSLOT - 1)) * G::KS + (KB ^ 1) * 32 * G::KROW;
    const uint32_t va = vbase + ((t - 1 + KB) & (NSLOT - 1)) * G::VS + (KB ^ 1) * 64;
    v4i a[NMF];
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < RD_AHEAD; ++i) {
      a[i] = operand(i, ka, va);
      asm volatile("" ::: "memory");  // keep the reads in MFMA order
    }
    float u[8][2];
#pragma unroll
    for (int i = 0; i < (NMF > 12 ? NMF : 12); ++i) {
      issue_slot(i, scur, snext, pprev, a, u, w, c, k, acc);  // MFMA i, pair i stage 1, pair i-4 stage 2
      if (i + RD_AHEAD < NMF) a[i + RD_AHEAD] = operand(i + RD_AHEAD, ka, va);
      // the tile refill, one load after every other MFMA
      if constexpr (REFILL) {
        if ((i & 1) == 1 && (i >> 1) <= G::PER) load_part(*rf, i >> 1);
      }
    }
    // The first INT8 MFMA reads `magic` as its accumulator a few cycles after
    // issue; keep that register block live to the end of the iteration so the
    // compiler cannot hand it to a later statement's outputs meanwhile.
    asm volatile("" ::"v"(magic));
    if constexpr (REFILL) {  // more loads than iterations
#pragma unroll
      for (int j = ((NMF > 12 ? NMF : 12) + 1) / 2; j <= G::PER; ++j) load_part(*rf, j);
    }
    pcur[0] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    pcur[1] = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
  }

  // ---- all tiles of one pass (the loop body is generated once per order)
  __device__ __forceinline__ void tiles(v16i& S0, v16i& S1, v4i (&P0)[2], v4i (&P1)[2], float c) {
    float k = __builtin_fmaf(SQ_MAGIC_F, c, m);
    for (int t = 0; t < nt - 1; ++t) {
      step<0>(S0, S1, P1, P0, t, c, k, l);
      // Tile boundary: every wave is done with K(t) and V(t-1); K(t+1) and
      // V(t) (issued three boundaries ago, or in the prologue) must have
      // landed, the two latest batches may stay in flight.
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * G::LPB));
      __syncthreads();
      // refill the freed slots (past the end: the last tile again, unread),
      // spread over the next iteration's MFMAs
      const Refill rf = refill(min(t + NSLOT, nt - 1), t & (NSLOT - 1), min(t + NSLOT - 1, nt - 1), (t - 1) & (NSLOT - 1));
      const float c_next = cq * k_scale((t + 1) & (NSLOT - 1));
      step<1, true>(S1, S0, P0, P1, t, c, k, l, &rf);
      c = c_next;
      k = __builtin_fmaf(SQ_MAGIC_F, c, m);
    }
    // last tile: keys past N masked; its row-sum terms are taken from the
    // masked bf16 P instead of the pairs' fp32 sums
    const int t = nt - 1;
    float unused = 0.0f;
    step<0>(S0, S1, P1, P0, t, c, k, unused);
    l += tail_sum(P0, t, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    step<1>(S1, S0, P0, P1, t, c, k, unused);
    l += tail_sum(P1, t, 1);
    pv_last(P1, t & (NSLOT - 1));
  }

  // ---- block-sparse: the same pipeline over the work-group's tile list.
  // Slots follow list positions; loads follow tile numbers.  A listed tile
  // that this wave's mask row drops gets k = +inf, so its P is exactly 0
  // (and adds 0 to the row sum); the wave's reference is the max of the first
  // 32 keys of its first kept tile.
  __device__ __forceinline__ bool keeps(int e) const { return ((e >> (24 + (wave >> 2))) & 1) != 0; }
  __device__ __forceinline__ float k_for(int pos, float c, const v16i& s) {
    const bool act = keeps(list[pos]);
    if (act && !has_m) {
      // s was written by MFMAs of the previous iteration's assembly, which
      // the compiler does not track: cover the matrix-core result latency
      asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
      m = rowmax(s, c, SQ_MAGIC);
      has_m = true;
    }
    return act ? __builtin_fmaf(SQ_MAGIC_F, c, m) : __builtin_inff();
  }
  __device__ __forceinline__ void tiles_sparse(v16i& S0, v16i& S1, v4i (&P0)[2], v4i (&P1)[2], float c) {
    float k = k_for(0, c, S0);
    for (int pos = 0; pos < cnt - 1; ++pos) {
      step<0>(S0, S1, P1, P0, pos, c, k, l);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * G::LPB));
      __syncthreads();
      const Refill rf = refill(list[min(pos + NSLOT, cnt - 1)] & 0xFFFFFF, pos & (NSLOT - 1),
                               list[min(pos + NSLOT - 1, cnt - 1)] & 0xFFFFFF, (pos - 1) & (NSLOT - 1));
      const float c_next = cq * k_scale((pos + 1) & (NSLOT - 1));
      step<1, true>(S1, S0, P0, P1, pos, c, k, l, &rf);
      c = c_next;
      k = k_for(pos + 1, c, S0);
    }
    const int pos = cnt - 1, t = list[pos] & 0xFFFFFF;
    float unused = 0.0f;
    step<0>(S0, S1, P1, P0, pos, c, k, unused);
    l += tail_sum(P0, t, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    step<1>(S1, S0, P0, P1, pos, c, k, unused);
    l += tail_sum(P1, t, 1);
    pv_last(P1, pos & (NSLOT - 1));
  }

  // ---- last tile, half kb: zero P of keys >= N; returns the sum of the kept P
  __device__ __forceinline__ float tail_sum(v4i (&pb)[2], int t, int kb) {
    const int kvalid = N - t * KT - kb * 32;
    float kept = 0.0f;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k0 = 16 * k2 + 8 * g + 2 * j;
        const uint32_t keep = (k0 >= kvalid ? 0u : 0xFFFFu) | (k0 + 1 >= kvalid ? 0u : 0xFFFF0000u);
        const uint32_t w = (uint32_t)pb[k2][j] & keep;
        kept += __uint_as_float(w << 16) + __uint_as_float(w & 0xFFFF0000u);
        pb[k2][j] = (int)w;
      }
    return kept;
  }

  // S = half kb of the K tile in slot, accumulated from `init`
  __device__ __forceinline__ void qk_half(v16i& s, int slot, int kb, const v16i& init) const {
#pragma unroll
    for (int ch = 0; ch < G::NCH; ++ch) {
      const v4i a = *(const v4i*)(lds + kbase + slot * G::KS + kb * 32 * G::KROW + ch * 32);
      if (ch == 0) {
        s = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], init, 0, 0, 0);
      } else {
        s = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], s, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void pv_last(const v4i (&pb)[2], int slot) {  // half 1 of V tile in slot
    const uint32_t va = vbase + slot * G::VS + 64;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int cb = 0; cb < G::NCB; ++cb) {
        const v4i a = *(const v4i*)(lds + va + cb * 32 * G::VROW + k2 * 32);
        o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                        __builtin_bit_cast(v8bf, pb[k2]), o[cb], 0, 0, 0);
      }
  }
};

// uniform load through the scalar cache (the K scales are read-only here)
__device__ __forceinline__ float ld_uniform(const float* p) {
  return *(const __attribute__((address_space(4))) float*)p;
}

}  // namespace

template <int D, bool SP>
__global__ __launch_bounds__(NTHR) void attn_bf16_kernel(AttnParams p) {
  using Cx = Ctx<D, SP>;
  using G = Geo<D>;
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
  C.kbase = perm_key(C.lr) * G::KROW + C.g * 16;
  C.vbase = G::VBASE + C.lr * G::VROW + C.g * 16;
  C.N = p.N;
  C.nt = p.nt;
  const long long hoff = (long long)bh * p.N * D;
  C.kh = (const uint8_t*)p.k + hoff;
  C.vth = (const uint8_t*)p.vt + (long long)bh * p.nt * G::VBYTES;
  C.skh = p.sk + (long long)bh * p.nt;
#pragma unroll
  for (int r = 0; r < 16; ++r) C.magic[r] = SQ_MAGIC;
  v16i zero;
#pragma unroll
  for (int r = 0; r < 16; ++r) zero[r] = 0;
  const int row = qt * ATT_QWG + C.wave * ATT_QW + C.lr;
  const bool rok = row < p.N;
#pragma unroll
  for (int ch = 0; ch < G::NCH; ++ch)
    C.qreg[ch] = rok ? *(const v4i*)(p.q + hoff + (long long)row * D + ch * 32 + C.g * 16) : v4i{0, 0, 0, 0};
  C.cq = rok ? p.sq[(long long)bh * p.nq + row / p.q_block] * p.scale_log2e : 0.0f;

  const int nt = p.nt;
  v16i S0, S1;
  v4i P0[2], P1[2];
  // block-sparse: the list of tiles this work-group visits (a dense pass
  // visits 0 .. nt-1)
  int npos = nt;
  int* list = nullptr;
  if constexpr (SP) {
    list = (int*)(smem + G::LDS_BYTES);
    const uint8_t* m0 = p.mask + ((long long)bh * p.mq + 2 * qt) * nt;
    const uint8_t* m1 = (2 * qt + 1 < p.mq) ? m0 + nt : nullptr;
    npos = build_tile_list(m0, m1, nt, list, list + SP_MAXT, NTHR);
    C.list = list;
    C.cnt = npos;
    C.has_m = false;
  }
  auto tile_at = [&](int j) { return SP ? (list[min(j, npos - 1)] & 0xFFFFFF) : min(j, nt - 1); };

  for (int pass = 0; pass < 2 && npos > 0; ++pass) {
    C.init_loads();  // the refills of a pass clamp the K offsets at its end
    if (pass == 1) {
      // Rare path: some row's sum reached 2^HEADROOM.  Take the exact row max
      // over all keys (K tiles one at a time through slot 0) as the reference,
      // so that every P <= 1.
      float mx = -__builtin_inff();
      for (int j = 0; j < npos; ++j) {
        const int t = tile_at(j);
        __syncthreads();
        C.load_k(t);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const float c = C.cq * ld_uniform(C.skh + t);
        C.qk_half(S0, 0, 0, zero);
        C.qk_half(S1, 0, 1, zero);
        const float r = __builtin_fmaxf(C.rowmax(S0, c, 0), C.rowmax(S1, c, 0));
        if (!SP || C.keeps(list[j])) mx = __builtin_fmaxf(mx, r);
      }
      C.m = mx;
      if constexpr (SP) C.has_m = true;
      __syncthreads();
    }
    C.l = 0.0f;
#pragma unroll
    for (int cb = 0; cb < G::NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) C.o[cb][i] = 0.0f;
    P1[0] = P1[1] = v4i{0, 0, 0, 0};

    // Prologue: K(0..3) and V(0..3) into slots 0..3, all landed before the
    // loop.  The first iteration multiplies V slot 3 by P(-1) = 0 (a finite
    // tile, so the product is 0).  In the loop, boundary t waits for the loads
    // of boundary t-3 and lets those of t-2 and t-1 (LPB per wave each) stay
    // in flight.
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) C.load_kv(tile_at(j), j, tile_at(j), j);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    float c = C.cq * C.k_scale(0);
    C.qk_half(S0, 0, 0, C.magic);
    if constexpr (SP) {
      C.tiles_sparse(S0, S1, P0, P1, c);
    } else {
      if (pass == 0) C.m = C.rowmax(S0, c, SQ_MAGIC);  // reference: max of the first 32 keys
      C.tiles(S0, S1, P0, P1, c);
    }
    C.l = pair_sum_f(C.l);
    __syncthreads();  // all waves are done with the LDS tiles
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

template <int D, bool SP>
static void launch_d(const AttnParams& q, hipStream_t st) {
  constexpr int lds = Geo<D>::LDS_BYTES + (SP ? SP_LIST_BYTES : 0);
  static bool configured = false;  // the attribute is per kernel, set once per process
  if (!configured) {
    (void)hipFuncSetAttribute((const void*)attn_bf16_kernel<D, SP>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds);
    configured = true;
  }
  hipLaunchKernelGGL((attn_bf16_kernel<D, SP>), dim3(8 * q.per_xcd), dim3(NTHR), lds, st, q);
}

void launch_attention_bf16(const AttnParams& q, int d, hipStream_t st) {
  const bool sp = q.mask != nullptr;
  if (d == 128)
    sp ? launch_d<128, true>(q, st) : launch_d<128, false>(q, st);
  else
    sp ? launch_d<64, true>(q, st) : launch_d<64, false>(q, st);
}

}  // namespace sqattn
