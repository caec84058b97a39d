// Quantized attention kernel, FP8 P.V path (gfx950).
//
// Same integer logits and register layouts as the 16-bit kernel (INT8
// S^T = K Q^T with K rows in the perm_key order, lane-local softmax, O^T =
// V^T P^T with P^T built in the lane), with the P.V product on
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulation, E8M0
// block scales).  What the FP8 path adds is the online rounding the result
// depends on: P is rounded to E4M3 relative to the running row max of the
// tiles seen so far, so this kernel keeps an exact running max per 64-key
// tile and rescales O when it moves.
//
// Work-group: 8 waves (two per SIMD), 32 query rows each.  The unit of the
// pipeline is a 64-key tile:
//
//   iteration t:   MFMA  O^T += sV(t-1) V(t-1)^T P(t-1)^T (D/32 x fp8 32x32x64)
//                  MFMA  S(t+1) = K(t+1) Q^T             (2 D/32 x i8 32x32x32)
//                  VALU  tile max of S(t) -> m(t); if it moved for some
//                        row of the wave, O and the row sum *= 2^(m(t-1) - m(t))
//                        P(t) = E4M3(448 * 2^(S(t) c(t) - m(t))), row sum
//
// * Tile t's P is relative to m(t), the exact max over tiles 0..t, and so
//   are O and the row sum: the matrix instruction accumulates straight into
//   O.  The rescale is a branch taken by the whole wave when some row's max
//   moved (often on the first tiles, rarely later: a new maximum among t
//   tiles of random scores comes with probability about 1/t per row).
// * The V block scale is a power of two (see the V quantizer) and rides in
//   the instruction as the E8M0 scale of the V operand, so O is held in
//   absolute units with no vector work per tile, also when neighbouring V
//   blocks differ by many orders of magnitude.
// * Scores: the INT8 accumulation starts from the bits of 1.5 * 2^23, so the
//   int32 result read as a float is exactly 1.5 * 2^23 + S (|S| < 2^22) and S
//   is one exact full-rate subtraction away (not the half-rate int-to-float
//   conversion); the tile max is taken on the biased integers.  The bf16
//   kernel's one-FMA form, which folds 1.5 * 2^23 c into the exponent offset,
//   rounds that offset: up to 0.75 c in the exponent, outside the E4M3
//   envelope.
// * 448 is folded into the exponent: y = 2^(x c - (m - log2 448)) = 448 P~,
//   the E4M3 operand is the rounded y and the row sum adds the unrounded y, so
//   O = sum(sV y^ code) / sum(y).
// * LDS ring filled by direct-to-LDS loads: eight slots and one barrier
//   every four tiles in the dense kernel, four slots and a barrier every tile
//   in the block-sparse and Q-smoothing ones (whose tile list or bias leave
//   no room for eight); V^T rows hold 64 one-byte keys padded to 80 bytes
//   (five 16-byte units, odd, so 16 lanes reading 16 bytes of consecutive
//   rows hit distinct banks).  Each slot also carries its tile's scale (64
//   copies, one per lane).  The first K tile is read straight from global
//   memory; K(x) and V(x) sit in slot x mod the ring depth.
// * Keys past N: the K tile reads row N-1 there (a real score of the same
//   tile, so the tile max is unchanged), y is zeroed for them in the last
//   tile, and the packed V tile is zero past N.
// * Q smoothing (SM): the logit bias of the wave's Q block for the tile's 64
//   keys, a binary32 value in units of sQ sK, rides in the V slot of the
//   previous tile (1 KB: up to four blocks of the work-group), which has
//   landed by iteration t and stays put through it; the first tile's comes
//   from global memory.  The scores are converted first and the
//   bias added (fl32(S + bias), one rounding); the tile max and P are taken on
//   those values.  One vector add per score; a rounded integer bias would
//   move logits by up to c / 2, too coarse for the E4M3 rounding of P.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace sqattn {

namespace {

__device__ __forceinline__ int perm_key(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

constexpr int WAVES = 8;
constexpr int NTHR = 64 * WAVES;
// LDS ring: NS slots, one barrier every BE tiles.  The dense kernel takes
// eight slots and a barrier every fourth tile; the block-sparse and
// Q-smoothing kernels, whose tile list or bias leave no room for eight, four
// slots and a barrier every tile (measured faster there than every second).
template <bool SP, bool SM>
constexpr int ring_slots() {
  return (SP || SM) ? 4 : 8;
}
template <bool SP, bool SM>
constexpr int ring_every() {
  return (SP || SM) ? 1 : 4;
}
constexpr float LOG2_448 = 8.80735492205760410f;  // log2(448)
constexpr int E8M0_ONE = 127;                     // E8M0 scale 2^0
constexpr int SQ_MAGIC = 0x4B400000;              // bits of 1.5 * 2^23
constexpr float SQ_MAGIC_F = 12582912.0f;


// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 field layout:
// vmcnt[3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

__device__ __forceinline__ int pair_max_i(int v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float pair_sum_f(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// uniform load through the scalar cache (read-only scales)
__device__ __forceinline__ float ld_uniform(const float* p) {
  return *(const __attribute__((address_space(4))) float*)p;
}

template <int D, bool SM, int NS>
struct Geo {
  static constexpr int NCH = D / 32;            // QK k-steps per 32-key half
  static constexpr int NCB = D / 32;            // 32-channel blocks of O^T
  static constexpr int KCPR = D / 16;           // 16-byte chunks of a K row
  static constexpr int KROWC = KCPR + 1;        // ... padded (odd)
  static constexpr int KROW = 16 * KROWC;       // padded K row stride (bytes)
  static constexpr int KSC = KT * KROW;         // offset of the K scale in a K slot
  static constexpr int KS = KSC + 256;          // K slot bytes
  static constexpr int VROWC = 5;               // V^T row: 64 keys * 1 B = 4 chunks + pad
  static constexpr int VROW = 16 * VROWC;
  static constexpr int VSC = D * VROW;          // offset of the V scale in a V slot
  static constexpr int VQB = VSC + 256;         // offset of the Q-smoothing bias (SM)
  static constexpr int VS = VQB + (SM ? 1024 : 0);  // V slot bytes
  static constexpr int VBASE = NS * KS;         // V ring offset in LDS
  static constexpr int LDS_BYTES = NS * (KS + VS);
  static constexpr int KINST = (KT * KROWC + 63) / 64;   // 1 KB direct loads per K tile
  static constexpr int VINST = (D * VROWC + 63) / 64;     // ... per V tile
  static constexpr int PER = (KINST + VINST + WAVES - 1) / WAVES;  // K+V loads per wave
  static constexpr int LPB = PER + 2 + (SM ? 1 : 0);  // direct loads per wave per boundary (+ 2 scales, bias)
  static constexpr int VBYTES = D * KT;         // packed V tile in HBM
};

template <int D, bool SP = false, bool SM = false>
struct Ctx {
  static constexpr int NS = ring_slots<SP, SM>();
  using G = Geo<D, SM, NS>;
  uint8_t* lds;
  const uint8_t* kh;
  const uint8_t* vth;
  const float* skh;
  const float* svh;
  const uint8_t* qbh;     // SM: the bias rows of the work-group's first Q block
  uint32_t qboff;         // SM: this lane's byte offset in them (block lane / 16, 4 keys)
  uint32_t qbw;           // SM: byte offset of this wave's block in a slot's bias area
  long long qbg;          // SM: byte offset of this wave's block row from qbh (global)
  uint32_t* dbg;          // checking build: the violation word (else null)
  int N, nt, lane, wave, g, lr;
  uint32_t kbase, vbase;  // per-lane LDS operand offsets (slot 0)
  float cq;               // sQ(row) * scale * log2(e)
  v4i qreg[G::NCH];       // Q operands
  v16i magic;             // SQ_MAGIC in every element: start of the INT8 accumulation
  v16f o[G::NCB];         // O^T accumulators (absolute units, relative to m)
  float m;               // running max (log2 units): P, O and l of tile t are relative to m(t)
  float l;               // running sum of 448 P~

  // ---- global -> LDS (direct); see the 16-bit kernel for the scheme.  Chunk
  // slot i < PER of a wave is one 1 KB chunk of the K or V slot; PER and
  // PER + 1 copy the K and V scales.
  uint32_t off[G::PER];    // lane's byte offset of chunk slot i within its tile
  uint32_t kmask[G::PER];  // wave-uniform: all ones for a K chunk, 0 for a V chunk
  uint32_t cofs[G::PER];   // wave-uniform: the chunk's LDS offset in its ring slot (V: past VBASE)

  __device__ __forceinline__ void init_loads() {
#pragma unroll
    for (int i = 0; i < G::PER; ++i) {
      int u = wave + WAVES * i;
      if (u >= G::KINST + G::VINST) u -= G::KINST + G::VINST;
      kmask[i] = u < G::KINST ? ~0u : 0u;
      cofs[i] = u < G::KINST ? (uint32_t)(u * 1024) : (uint32_t)(G::VBASE + (u - G::KINST) * 1024);
      if (u < G::KINST) {
        const int q = u * 64 + lane;
        off[i] = (uint32_t)(min(q / G::KROWC, KT - 1) * D + min(q % G::KROWC, G::KCPR - 1) * 16);
      } else {
        const int q = (u - G::KINST) * 64 + lane;
        off[i] = (uint32_t)(min(q / G::VROWC, D - 1) * KT + min(q % G::VROWC, 3) * 16);
      }
    }
  }
  // K rows past N (last tile) read row N-1 instead: klim is the byte offset
  // of the last row to read (past every offset when the tile is full).
  struct Refill {
    const uint8_t* kt;
    const uint8_t* vt;
    int tk, tv, ks, vs;
    uint32_t klim;
    uint32_t kso, vso;  // LDS offsets of the K slot and of the V slot (from VBASE)
  };
  __device__ __forceinline__ Refill refill(int tk, int ks, int tv, int vs) const {
    SQ_CHECK(dbg, tk >= 0 && tk < nt, 0);
    SQ_CHECK(dbg, tv >= 0 && tv < nt, 1);
    SQ_CHECK(dbg, N - 1 - tk * KT >= 0, 2);  // the last K row read exists
    return Refill{kh + (long long)tk * KT * D, vth + (long long)tv * G::VBYTES, tk, tv, ks, vs,
                  (uint32_t)(min(N - 1 - tk * KT, KT) * D), (uint32_t)(ks * G::KS), (uint32_t)(vs * G::VS)};
  }
  __device__ __forceinline__ void load_part(const Refill& r, int i) {
    if (SM && i == G::PER + 2) {
      // the bias of the tile after V's (dense: tile tv + 1), clamped
      lds_dma16(qbh + (long long)min(r.tv + 1, nt - 1) * KT * 4, qboff,
                lds_addr(lds + G::VBASE + r.vs * G::VS + G::VQB));
      return;
    }
    if (i == G::PER) {
      lds_dma4(skh + r.tk, 0u, lds_addr(lds + r.ks * G::KS + G::KSC));
      return;
    }
    if (i == G::PER + 1) {
      lds_dma4(svh + r.tv, 0u, lds_addr(lds + G::VBASE + r.vs * G::VS + G::VSC));
      return;
    }
    const uint32_t km = kmask[i];
    const bool isk = km != 0;  // wave-uniform
    const uint8_t* base = isk ? r.kt : r.vt;
    const uint32_t o = isk ? min(off[i], r.klim + (off[i] & (D - 1))) : off[i];
    // the slot offset through the masks: written as a select, it compiles to
    // a branch around every load (measured 1-1.5% slower)
    const uint32_t dst = cofs[i] + (r.kso & km) + (r.vso & ~km);
    lds_dma16(base, o, lds_addr(lds) + dst);
  }
  __device__ __forceinline__ void load_kv(int tk, int ks, int tv, int vs) {
    const Refill r = refill(tk, ks, tv, vs);
#pragma unroll
    for (int i = 0; i < G::LPB; ++i) load_part(r, i);
  }
  __device__ __forceinline__ float k_scale(int slot) const {
    return *(const float*)(lds + slot * G::KS + G::KSC + 4 * lane);
  }
  // the V block scale (a power of two) as the E8M0 scale of the instruction:
  // its binary exponent field (2^-127, stored as a subnormal, and 0 give 0)
  __device__ __forceinline__ int v_scale_e8(int slot) const {
    return (int)((*(const uint32_t*)(lds + G::VBASE + slot * G::VS + G::VSC + 4 * lane) >> 23) & 0xFF);
  }

  // ---- SM: the scores of tile t as binary32 values fl32(S + bias), in place
  // (bit patterns in the integer registers); the bias of the 16 keys
  // 32 kb + 16 h + 8 g + j (h < 2, j < 8) of the lane's rows is read from the
  // tile's 64 values of the wave's block at p
  __device__ __forceinline__ void add_bias(v16i (&s)[2], const uint8_t* p) const {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v4f b0 = *(const v4f*)(p + (32 * kb + 16 * h + 8 * g) * 4);
        const v4f b1 = *(const v4f*)(p + (32 * kb + 16 * h + 8 * g) * 4 + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[kb][8 * h + r] = __float_as_int((__int_as_float(s[kb][8 * h + r]) - SQ_MAGIC_F) + b0[r]);
          s[kb][8 * h + 4 + r] = __float_as_int((__int_as_float(s[kb][8 * h + 4 + r]) - SQ_MAGIC_F) + b1[r]);
        }
      }
  }

  // ---- S of K tile t0 straight from global memory (rows past N read row N-1)
  __device__ __forceinline__ void qk_first(v16i (&s)[2], int t0) const {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(t0 * KT + kb * 32 + perm_key(lr), N - 1);
#pragma unroll
      for (int ch = 0; ch < G::NCH; ++ch) {
        const v4i a = *(const v4i*)(kh + (long long)key * D + ch * 32 + g * 16);
        if (ch == 0) {
          s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], magic, 0, 0, 0);
        } else {
          s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], s[kb], 0, 0, 0);
        }
      }
    }
  }

  // ---- SM: the same over binary32 scores held as bit patterns
  __device__ __forceinline__ float tile_max_f(const v16i (&s)[2]) const {
    float d0 = __builtin_fmaxf(__int_as_float(s[0][0]), __int_as_float(s[1][0]));
#pragma unroll
    for (int i = 1; i < 16; ++i)
      d0 = __builtin_fmaxf(d0, __builtin_fmaxf(__int_as_float(s[0][i]), __int_as_float(s[1][i])));
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(d0), __float_as_int(d0), false, false);
    return __builtin_fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
  }

  // ---- row max of S(t) over the tile's 64 keys (lanes l and l^32 share a row)
  __device__ __forceinline__ int tile_max(const v16i (&s)[2]) const {
    int d0 = max(max(s[0][0], s[0][1]), s[0][2]);
    int d1 = max(max(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) {
      d0 = max(max(d0, s[0][i]), s[0][i + 1]);
      d1 = max(max(d1, s[1][i]), s[1][i + 1]);
    }
    d0 = max(max(d0, s[0][15]), max(d1, s[1][15]));
    return pair_max_i(d0);
  }

  // ---- O^T += sV V^T P^T for the V tile at LDS offset va (per lane), its
  // scale as E8M0 exponent sve
  __device__ __forceinline__ void pv(uint32_t va, const v8i& p, int sve, const Refill* rf) {
#pragma unroll
    for (int cb = 0; cb < G::NCB; ++cb) {
      const v4i a0 = *(const v4i*)(lds + va + cb * 32 * G::VROW);
      const v4i a1 = *(const v4i*)(lds + va + cb * 32 * G::VROW + 16);
      const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      // formats 0/0: E4M3 x E4M3; the V operand scaled by 2^(sve - 127)
      o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, p, o[cb], 0, 0, 0, sve, 0, E8M0_ONE);
      if (rf && cb < G::LPB) load_part(*rf, cb);
    }
  }

  // ---- one tile iteration t.  QK: the next tile's scores into sn (when
  // QK); PV: V(t-1) (scale exponent sve) times pprev into O; softmax of sc
  // (tile t, factor c) into pcur.  MASK: last tile, keys >= N excluded.
  // Block-sparse: t is the list position (slots), tile the tile number; a
  // listed tile this wave's mask row drops (act false) leaves the running
  // max alone and gets P = 0 (mp = +inf).
  template <bool QK, bool MASK>
  __device__ __forceinline__ void iter(v16i (&sc)[2], v16i (&sn)[2], const v8i& pprev, v8i& pcur, int t,
                                       float c, int sve, const Refill& rf, int tile = 0, bool act = true) {
    const uint32_t ka = kbase + ((t + 1) & (NS - 1)) * G::KS;
    const uint32_t va = vbase + ((t - 1) & (NS - 1)) * G::VS;

    // Plain scores: the next tile's score MFMAs, then P.V of the previous
    // tile (relative to m(t-1) = m) into O and the rest of the refill, and
    // only then the running max of tile t, so that its vector work runs under
    // the matrix instructions (measured about 2.5% faster than max, P.V,
    // scores).  SM (biased binary32 scores; the bias of tile t > 0 sits in V
    // slot t - 1, landed at boundary t - 1, while this iteration's refill
    // writes V slot t - 2): max, P.V, scores, since the other order needs
    // more registers than the wave has there.
    float mn;
    auto running_max = [&]() {
      if constexpr (SM) {
        if (t > 0) add_bias(sc, lds + G::VBASE + ((t - 1) & (NS - 1)) * G::VS + G::VQB + qbw);
        mn = __builtin_fmaxf(m, tile_max_f(sc) * c);
      } else {
        mn = __builtin_fmaxf(m, (float)(tile_max(sc) - SQ_MAGIC) * c);  // c >= 0
      }
      if constexpr (SP) mn = act ? mn : m;
    };
    auto scores = [&]() {
      if constexpr (QK) {
#pragma unroll
        for (int ch = 0; ch < G::NCH; ++ch)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const v4i a = *(const v4i*)(lds + ka + kb * 32 * G::KROW + ch * 32);
            if (ch == 0) {
              sn[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], magic, 0, 0, 0);
            } else {
              sn[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], sn[kb], 0, 0, 0);
            }
          }
      }
    };
    if constexpr (SM) {
      running_max();
      pv(va, pprev, sve, &rf);
      scores();
    } else {
      scores();
      pv(va, pprev, sve, &rf);
    }
#pragma unroll
    for (int i = G::NCB; i < G::LPB; ++i) load_part(rf, i);
    if constexpr (!SM) running_max();

    // O and l follow the max: rescale when it moved for some row of the
    // wave (always on the first tile, where m = -inf and O = l = 0)
    if (__builtin_amdgcn_ballot_w64(mn > m)) {
      const float f = __builtin_amdgcn_exp2f(m - mn);  // 1 where unmoved; m = -inf: 0
#pragma unroll
      for (int cb = 0; cb < G::NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= f;
      l *= f;
    }
    m = mn;
    float mp = mn - LOG2_448;
    if constexpr (SP) mp = act ? mp : __builtin_inff();

    // P(t) = E4M3(y), y = 448 P~; byte 16 kb + i of the operand is key
    // 32 kb + 16 (i / 8) + 8 g + i % 8, the lane's S(t)[kb][i]
    const int kvalid = N - (SP ? tile : t) * KT;
    float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int kb = r >> 2, i0 = 4 * (r & 3);
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j;
        // exact: 1.5 * 2^23 + S - 1.5 * 2^23 (|S| < 2^22), a full-rate subtract
        const float sv = SM ? __int_as_float(sc[kb][i]) : __int_as_float(sc[kb][i]) - SQ_MAGIC_F;
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, -mp));
        if constexpr (MASK) {
          const int key = 32 * kb + 16 * (i >> 3) + 8 * g + (i & 7);
          if (key >= kvalid) e = 0.0f;
        }
        y[j] = e;
        part[j] += e;
      }
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
      pcur[r] = word;
    }
    l += (part[0] + part[1]) + (part[2] + part[3]);
  }
};

}  // namespace

template <int D, bool SP, bool SM>
__global__ __launch_bounds__(NTHR) void attn_fp8_kernel(AttnParams p) {
  using Cx = Ctx<D, SP, SM>;
  using G = typename Cx::G;
  constexpr int NS = Cx::NS;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int w = blockIdx.x;
  const int item = (w & 7) * p.per_xcd + (w >> 3);
  if (item >= p.BH * p.qtiles) return;
  const int bh = item / p.qtiles, qt = item - bh * p.qtiles;

  Cx C;
  C.lds = smem;
  const int tid = threadIdx.x;
  C.lane = tid & 63;
  C.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  C.g = C.lane >> 5;
  C.lr = C.lane & 31;
  C.kbase = perm_key(C.lr) * G::KROW + C.g * 16;
  C.vbase = G::VBASE + C.lr * G::VROW + C.g * 32;
  C.N = p.N;
  C.nt = p.nt;
  const long long hoff = (long long)bh * p.N * D;
  C.kh = (const uint8_t*)p.k + hoff;
  C.vth = (const uint8_t*)p.vt + (long long)bh * p.nt * G::VBYTES;
  C.skh = p.sk + (long long)bh * p.nt;
  C.svh = p.sv + (long long)bh * p.nt;
  C.dbg = p.debug;
  if constexpr (SM) {
    // blocks of q_block (64, 128 or 256) rows: the work-group's first block
    // and this wave's; lane l of the bias load reads block b0 + l / 16 (the
    // last existing one past the end), keys 4 (l % 16) .. + 3
    const int b0 = qt * ATT_QWG / p.q_block, nbw = min(ATT_QWG / p.q_block, p.nq - b0);
    const long long rowb = (long long)p.nt * KT * 4;
    C.qbh = (const uint8_t*)p.qbias + ((long long)bh * p.nq + b0) * rowb;
    C.qboff = (uint32_t)(min(C.lane / 16, nbw - 1) * rowb + (C.lane % 16) * 16);
    // (a wave whose rows all lie past N takes the last existing block)
    const int wb = min(C.wave * ATT_QW / p.q_block, nbw - 1);
    C.qbw = (uint32_t)(wb * 256);
    C.qbg = (long long)wb * rowb;
  }
  C.init_loads();
  const int row = qt * ATT_QWG + C.wave * ATT_QW + C.lr;
  const bool rok = row < p.N;
#pragma unroll
  for (int ch = 0; ch < G::NCH; ++ch)
    C.qreg[ch] = rok ? *(const v4i*)(p.q + hoff + (long long)row * D + ch * 32 + C.g * 16) : v4i{0, 0, 0, 0};
  C.cq = rok ? p.sq[(long long)bh * p.nq + row / p.q_block] * p.scale_log2e : 0.0f;
  C.m = -__builtin_inff();
  C.l = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) C.magic[r] = SQ_MAGIC;
  asm volatile("" : "+v"(C.magic));  // keep the accumulator start in vector registers
#pragma unroll
  for (int cb = 0; cb < G::NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) C.o[cb][r] = 0.0f;

  const int nt = p.nt;
  // block-sparse: the list of tiles this work-group visits (dense: 0 .. nt-1);
  // positions index slots, list entries the tiles
  int npos = nt;
  int* list = nullptr;
  if constexpr (SP) {
    list = (int*)(smem + G::LDS_BYTES);
    const uint8_t* m0 = p.mask + ((long long)bh * p.mq + 2 * qt) * nt;
    const uint8_t* m1 = (2 * qt + 1 < p.mq) ? m0 + nt : nullptr;
    npos = build_tile_list(m0, m1, nt, list, list + SP_MAXT, NTHR);
    SQ_CHECK(p.debug, npos >= 0 && npos <= SP_MAXT, 3);
  }
  auto tile_at = [&](int j) { return SP ? (list[min(j, npos - 1)] & 0xFFFFFF) : min(j, nt - 1); };
  auto kept = [&](int j) { return SP ? ((list[j] >> (24 + (C.wave >> 2))) & 1) != 0 : true; };
  if (npos == 0) {  // block-sparse: nothing kept for these rows
    if (rok) store_out_row(p.out, p.out_bf16 != 0, lay_row(p.lo, bh, row), C.o, 0.0f, C.g);
    return;
  }
  // The ring: K(x) sits in K slot x mod NS, V(x) in V slot x mod NS, and BE
  // iterations run between two barriers.  Iteration i reads K(i+1) and
  // V(i-1) and refills with K(i+KA) and V(i+VA), KA = NS-BE+1, VA = NS-BE-1,
  // whose slots last held K(i+1-BE) and V(i-1-BE), both read in iteration
  // i-BE, before the last barrier.  The barrier after iteration j needs the
  // tiles of the next BE iterations, loaded in iterations up to j+2BE-NS, so
  // each wave lets its loads of the NS-2BE latest iterations stay in flight.
  // Measured on wan14b-480p-fp8 (interleaved A/B, bit-identical outputs):
  // eight slots with a barrier every fourth tile 12.87 ms against 13.16 ms
  // for four slots with a barrier every tile.
  // Prologue: K(1..NS) and V(0..NS-1) (past the end: the last tile, never
  // read), all landed before the loop; S(0) from global memory meanwhile.
  // The refills of the first iterations rewrite prologue slots with the same
  // bytes, read only after a barrier that waits for them, so every iteration
  // issues the same loads.  The first iteration multiplies V slot NS-1 by
  // P(-1) = 0 (a finite tile, so nothing).
  constexpr int BE = ring_every<SP, SM>(), KA = NS - BE + 1, VA = NS - BE - 1;
  static_assert(NS >= 2 * BE && (BE == 1 || BE % 2 == 0), "ring schedule");
#pragma unroll
  for (int j = 0; j < NS; ++j) C.load_kv(tile_at(j + 1), (j + 1) & (NS - 1), tile_at(j), j);
  v16i S0[2], S1[2];
  v8i P0, P1;
  C.qk_first(S0, tile_at(0));
  if constexpr (SM) C.add_bias(S0, C.qbh + C.qbg + (long long)tile_at(0) * KT * 4);
  float c = C.cq * ld_uniform(C.skh + tile_at(0));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 8; ++r) P1[r] = 0;

  auto refill_for = [&](int i) {
    return C.refill(tile_at(i + KA), (i + KA) & (NS - 1), tile_at(i + VA), (i + VA) & (NS - 1));
  };
  typename Cx::Refill rf = refill_for(0);
  // bar: iteration t ends an interval (t mod BE = BE - 1)
  auto step = [&](v16i (&sc)[2], v16i (&sn)[2], const v8i& pprev, v8i& pcur, int t, bool bar) {
    const float c_next = C.cq * C.k_scale((t + 1) & (NS - 1));
    const int sve = C.v_scale_e8((t - 1) & (NS - 1));
    C.template iter<true, false>(sc, sn, pprev, pcur, t, c, sve, rf, tile_at(t), kept(t));
    if (bar) {
      // Wait for our own loads but those of the NS-2BE latest iterations, and
      // for all LDS reads, then a plain barrier (the "memory" clobber keeps
      // every memory access on its side).  __syncthreads() would add a fence
      // that waits for every direct-to-LDS load in flight, which defeats the
      // ring.
#ifdef SQATTN_DEBUG
      __builtin_amdgcn_s_waitcnt(0);  // checking build: every load in flight lands first
#else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2 * BE) * G::LPB) & ~0x0F00);  // and lgkmcnt(0)
#endif
      asm volatile("s_barrier" ::: "memory");
    }
    rf = refill_for(t + 1);
    c = c_next;
  };
  auto last = [&](v16i (&sc)[2], v16i (&sn)[2], const v8i& pprev, v8i& pcur, int t) {
    const int sve = C.v_scale_e8((t - 1) & (NS - 1));
    C.template iter<false, true>(sc, sn, pprev, pcur, t, c, sve, rf, tile_at(t), kept(t));
    // V(t) may still be in flight (loaded by any wave): wait for every load,
    // then a barrier
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    C.pv(C.vbase + (t & (NS - 1)) * G::VS, pcur, C.v_scale_e8(t & (NS - 1)), nullptr);
  };
  // tiles in pairs, so that the score and P registers alternate without
  // copies (BE is 1 or even: the first of a pair ends an interval only when
  // BE is 1)
  int t = 0;
  for (; t + 2 < npos; t += 2) {
    step(S0, S1, P1, P0, t, BE == 1);
    step(S1, S0, P0, P1, t + 1, BE <= 2 || ((t + 1) & (BE - 1)) == BE - 1);
  }
  if (t + 1 < npos) {
    step(S0, S1, P1, P0, t, BE == 1);
    last(S1, S0, P0, P1, t + 1);
  } else {
    last(S0, S1, P1, P0, t);
  }

  // epilogue: O = O^T / l, fp32 or bf16 rows (block-sparse: rows whose mask
  // keeps no listed tile have l = 0 and O = 0 and are written as zeros)
  const float lsum = pair_sum_f(C.l);
  const float inv = (SP && !(lsum > 0.0f)) ? 0.0f : 1.0f / lsum;
  if (rok) store_out_row(p.out, p.out_bf16 != 0, lay_row(p.lo, bh, row), C.o, inv, C.g);
}

template <int D, bool SP, bool SM>
static hipError_t launch_d(const AttnParams& q, hipStream_t st) {
  constexpr int lds = Geo<D, SM, ring_slots<SP, SM>()>::LDS_BYTES + (SP ? SP_LIST_BYTES : 0);
  // the attribute is per kernel: set once per process (the first status is kept)
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute((const void*)attn_fp8_kernel<D, SP, SM>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((attn_fp8_kernel<D, SP, SM>), dim3(8 * q.per_xcd), dim3(NTHR), lds, st, q);
  return hipSuccess;
}

// Q smoothing (q.qbias) runs on the dense kernels only (the caller checks)
hipError_t launch_attention_fp8(const AttnParams& q, int d, hipStream_t st) {
  const bool sp = q.mask != nullptr, sm = q.qbias != nullptr;
  if (d == 128) {
    if (sm) return launch_d<128, false, true>(q, st);
    return sp ? launch_d<128, true, false>(q, st) : launch_d<128, false, false>(q, st);
  }
  if (sm) return launch_d<64, false, true>(q, st);
  return sp ? launch_d<64, true, false>(q, st) : launch_d<64, false, false>(q, st);
}

}  // namespace sqattn
