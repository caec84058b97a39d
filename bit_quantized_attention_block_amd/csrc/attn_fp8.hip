// Quantized attention kernel, FP8 P.V path (gfx950).
//
// Same integer logits and register layouts as the 16-bit kernel (INT8
// S^T = K Q^T with K rows in the perm_key order, lane-local softmax, O^T =
// V^T P^T with P^T built in the lane), with the P.V product on
// v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulation).  What the FP8
// path adds is the online rounding the result depends on: P is rounded to
// E4M3 relative to the running row max of the tiles seen so far, so this
// kernel keeps an exact running max per 64-key tile and rescales O when it
// moves.
//
// Work-group: 8 waves (two per SIMD), 32 query rows each.  The unit of the
// pipeline is a 64-key tile:
//
//   iteration t:   MFMA  T    = V(t-1)^T P(t-1)^T     (D/32 x fp8 32x32x64)
//                  MFMA  S(t+1) = K(t+1) Q^T          (2 D/32 x i8 32x32x32)
//                  VALU  tile max of S(t) -> m(t)
//                        O += sV(t-1) 2^(m(t-1) - mr) T
//                        P(t) = E4M3(448 * 2^(S(t) c(t) - m(t))), row sum
//
// * Tile t's P is relative to m(t), the exact max over tiles 0..t.  O and
//   the row sum are kept relative to a reference mr <= m that moves up only
//   when some row's max outgrew it by 2^16 (one exp per row and tile, and a
//   vector rescale of O rarely after the first tile).
// * The per-block V scale is applied as O += sV * T with T from an MFMA that
//   starts at zero, so O is held in absolute units (no ratio of scales that
//   could overflow when neighbouring V blocks differ by many orders of
//   magnitude).
// * 448 is folded into the exponent: y = 2^(x c - (m - log2 448)) = 448 P~,
//   the E4M3 operand is the rounded y and the row sum adds the unrounded y, so
//   O = sum(sV y^ code) / sum(y).
// * LDS ring, direct-to-LDS refills three tiles ahead and one barrier per
//   tile as in the 16-bit kernel; V^T rows hold 64 one-byte keys padded to 80
//   bytes (five 16-byte units, odd, so 16 lanes reading 16 bytes of
//   consecutive rows hit distinct banks).  Each slot also carries its tile's
//   scale (64 copies, one per lane).  The first K tile is read straight from
//   global memory, so K slot j holds tiles with index = j mod 4 from tile 1 on
//   and every refill has two tile boundaries to land.
// * Keys past N: the K tile reads row N-1 there (a real score of the same
//   tile, so the tile max is unchanged), y is zeroed for them in the last
//   tile, and the packed V tile is zero past N.
#include "common.h"
#include "kernels.h"

namespace sqattn {

namespace {

__device__ __forceinline__ int perm_key(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

constexpr int WAVES = 8;
constexpr int NTHR = 64 * WAVES;
constexpr int NSLOT = 4;                          // LDS ring depth (tiles)
constexpr float LOG2_448 = 8.80735492205760410f;  // log2(448)
constexpr float REBASE = 16.0f;                   // lazy reference of O: at most 2^16 below the max


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

template <int D>
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
  static constexpr int VS = VSC + 256;          // V slot bytes
  static constexpr int VBASE = NSLOT * KS;      // V ring offset in LDS
  static constexpr int LDS_BYTES = NSLOT * (KS + VS);
  static constexpr int KINST = (KT * KROWC + 63) / 64;   // 1 KB direct loads per K tile
  static constexpr int VINST = (D * VROWC + 63) / 64;     // ... per V tile
  static constexpr int PER = (KINST + VINST + WAVES - 1) / WAVES;  // K+V loads per wave
  static constexpr int LPB = PER + 2;           // direct loads per wave per boundary (+ 2 scales)
  static constexpr int VBYTES = D * KT;         // packed V tile in HBM
};

template <int D, bool SP = false>
struct Ctx {
  using G = Geo<D>;
  uint8_t* lds;
  const uint8_t* kh;
  const uint8_t* vth;
  const float* skh;
  const float* svh;
  int N, nt, lane, wave, g, lr;
  uint32_t kbase, vbase;  // per-lane LDS operand offsets (slot 0)
  float cq;               // sQ(row) * scale * log2(e)
  v4i qreg[G::NCH];       // Q operands
  v16f o[G::NCB];         // O^T accumulators (absolute units, relative to m)
  float m;               // running max (log2 units): P of tile t is relative to m(t)
  float mr;              // reference of O and l (mr <= m, lazily moved up)
  float ep;              // 2^(m - mr) of the latest tile
  float l;               // running sum of 448 P~, relative to mr

  // ---- global -> LDS (direct); see the 16-bit kernel for the scheme.  Chunk
  // slot i < PER of a wave is one 1 KB chunk of the K or V slot; PER and
  // PER + 1 copy the K and V scales.
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
  };
  __device__ __forceinline__ Refill refill(int tk, int ks, int tv, int vs) const {
    return Refill{kh + (long long)tk * KT * D, vth + (long long)tv * G::VBYTES, tk, tv, ks, vs,
                  (uint32_t)(min(N - 1 - tk * KT, KT) * D)};
  }
  __device__ __forceinline__ void load_part(const Refill& r, int i) {
    if (i == G::PER) {
      lds_dma4(skh + r.tk, 0u, lds_addr(lds + r.ks * G::KS + G::KSC));
      return;
    }
    if (i == G::PER + 1) {
      lds_dma4(svh + r.tv, 0u, lds_addr(lds + G::VBASE + r.vs * G::VS + G::VSC));
      return;
    }
    const int u = chunk[i];
    const bool isk = u < G::KINST;  // wave-uniform
    const uint8_t* base = isk ? r.kt : r.vt;
    const uint32_t o = isk ? min(off[i], r.klim + (off[i] & (D - 1))) : off[i];
    const int dst = isk ? r.ks * G::KS + u * 1024 : G::VBASE + r.vs * G::VS + (u - G::KINST) * 1024;
    lds_dma16(base, o, lds_addr(lds + dst));
  }
  __device__ __forceinline__ void load_kv(int tk, int ks, int tv, int vs) {
    const Refill r = refill(tk, ks, tv, vs);
#pragma unroll
    for (int i = 0; i < G::LPB; ++i) load_part(r, i);
  }
  __device__ __forceinline__ float k_scale(int slot) const {
    return *(const float*)(lds + slot * G::KS + G::KSC + 4 * lane);
  }
  __device__ __forceinline__ float v_scale(int slot) const {
    return *(const float*)(lds + G::VBASE + slot * G::VS + G::VSC + 4 * lane);
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
          v16i z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0;
          s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], z, 0, 0, 0);
        } else {
          s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], s[kb], 0, 0, 0);
        }
      }
    }
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

  // ---- one tile iteration t.  QK: the next tile's scores into sn (when
  // QK); PV: V(t-1) (slot vslot, scale svp) times pprev; softmax of sc (tile
  // t, factor c) into pcur.  MASK: last tile, keys >= N excluded.
  // Block-sparse: t is the list position (slots), tile the tile number; a
  // listed tile this wave's mask row drops (act false) leaves the running
  // max alone, gets P = 0 (mp = +inf) and carries weight ep = 0, which also
  // keeps the first kept tile's 2^(m - mr) from meeting m = mr = -inf.
  template <bool QK, bool MASK>
  __device__ __forceinline__ void iter(const v16i (&sc)[2], v16i (&sn)[2], const v8i& pprev, v8i& pcur, int t,
                                       float c, float svp, const Refill& rf, int tile = 0, bool act = true) {
    const uint32_t ka = kbase + ((t + 1) & (NSLOT - 1)) * G::KS;
    const uint32_t va = vbase + ((t - 1) & (NSLOT - 1)) * G::VS;

    // running max of tile t
    float mn = __builtin_fmaxf(m, (float)tile_max(sc) * c);  // c >= 0
    if constexpr (SP) mn = act ? mn : m;
    const float w = svp * ep;  // tile t-1 relative to mr

    // P.V of the previous tile from a zero accumulator, O += w T
#pragma unroll
    for (int cb = 0; cb < G::NCB; ++cb) {
      const v4i a0 = *(const v4i*)(lds + va + cb * 32 * G::VROW);
      const v4i a1 = *(const v4i*)(lds + va + cb * 32 * G::VROW + 16);
      const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      v16f z;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 0.0f;
      const v16f tv = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pprev, z, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) o[cb][r] = __builtin_fmaf(tv[r], w, o[cb][r]);
      if (cb < G::LPB) load_part(rf, cb);
    }
    // scores of the next tile
    if constexpr (QK) {
#pragma unroll
      for (int ch = 0; ch < G::NCH; ++ch)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const v4i a = *(const v4i*)(lds + ka + kb * 32 * G::KROW + ch * 32);
          if (ch == 0) {
            v16i z;
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = 0;
            sn[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], z, 0, 0, 0);
          } else {
            sn[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[ch], sn[kb], 0, 0, 0);
          }
        }
    }
#pragma unroll
    for (int i = G::NCB; i < G::LPB; ++i) load_part(rf, i);

    // move the reference of O and l up once some row's max outgrew it by
    // 2^REBASE (always on the first tile, where mr = -inf)
    if (__builtin_amdgcn_ballot_w64(mn - mr > REBASE)) {
      const float f = __builtin_amdgcn_exp2f(mr - mn);  // mr = -inf: 0
#pragma unroll
      for (int cb = 0; cb < G::NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= f;
      l *= f;
      mr = mn;
    }
    m = mn;
    float mp = mn - LOG2_448;
    ep = __builtin_amdgcn_exp2f(mn - mr);  // tile t relative to mr, <= 2^REBASE
    if constexpr (SP) {
      mp = act ? mp : __builtin_inff();
      ep = act ? ep : 0.0f;
    }

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
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sc[kb][i], c, -mp));
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
    l = __builtin_fmaf(ep, (part[0] + part[1]) + (part[2] + part[3]), l);
  }

  // ---- O += sV(last) 2^(m - mr) V(last)^T P(last)^T
  __device__ __forceinline__ void pv_last(const v8i& p, int slot, float sv) {
    sv *= ep;
    const uint32_t va = vbase + slot * G::VS;
#pragma unroll
    for (int cb = 0; cb < G::NCB; ++cb) {
      const v4i a0 = *(const v4i*)(lds + va + cb * 32 * G::VROW);
      const v4i a1 = *(const v4i*)(lds + va + cb * 32 * G::VROW + 16);
      const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      v16f z;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 0.0f;
      const v16f t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, p, z, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) o[cb][r] = __builtin_fmaf(t[r], sv, o[cb][r]);
    }
  }
};

}  // namespace

template <int D, bool SP>
__global__ __launch_bounds__(NTHR) void attn_fp8_kernel(AttnParams p) {
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
  C.init_loads();
  const int row = qt * ATT_QWG + C.wave * ATT_QW + C.lr;
  const bool rok = row < p.N;
#pragma unroll
  for (int ch = 0; ch < G::NCH; ++ch)
    C.qreg[ch] = rok ? *(const v4i*)(p.q + hoff + (long long)row * D + ch * 32 + C.g * 16) : v4i{0, 0, 0, 0};
  C.cq = rok ? p.sq[(long long)bh * p.nq + row / p.q_block] * p.scale_log2e : 0.0f;
  C.m = -__builtin_inff();
  C.mr = -__builtin_inff();
  C.ep = 0.0f;
  C.l = 0.0f;
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
  }
  auto tile_at = [&](int j) { return SP ? (list[min(j, npos - 1)] & 0xFFFFFF) : min(j, nt - 1); };
  auto kept = [&](int j) { return SP ? ((list[j] >> (24 + (C.wave >> 2))) & 1) != 0 : true; };
  if (npos == 0) {  // block-sparse: nothing kept for these rows
    if (rok) store_out_row(p.out, p.out_bf16 != 0, lay_row(p.lo, bh, row), C.o, 0.0f, C.g);
    return;
  }
  // Prologue: K(1..4) into K slots 1,2,3,0 and V(0..3) into V slots 0..3 (past
  // the end: the last tile, never read), all landed before the loop; S(0)
  // from global memory meanwhile.  The first iteration multiplies V slot 3 by
  // P(-1) = 0 (a finite tile, so T = 0).
#pragma unroll
  for (int j = 0; j < NSLOT; ++j) C.load_kv(tile_at(j + 1), (j + 1) & (NSLOT - 1), tile_at(j), j);
  v16i S0[2], S1[2];
  v8i P0, P1;
  C.qk_first(S0, tile_at(0));
  float c = C.cq * ld_uniform(C.skh + tile_at(0));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 8; ++r) P1[r] = 0;

  // Boundary after iteration t: K(t+2) and V(t) (issued three boundaries ago
  // or in the prologue) must have landed; refill K slot (t+1)%4 with K(t+5)
  // and V slot (t-1)%4 with V(t+3), spread over the next iteration.  The
  // first iteration's refill rewrites K slot 0 and V slot 2 with the bytes
  // the prologue put there (read no earlier than iterations 3 and 2, after
  // boundaries that wait for it), so every iteration issues the same loads.
  typename Cx::Refill rf = C.refill(tile_at(4), 0, tile_at(2), 2);
  auto step = [&](const v16i (&sc)[2], v16i (&sn)[2], const v8i& pprev, v8i& pcur, int t) {
    // K(t+1) and V(t-1) have landed (boundary t-1); their slots are refilled
    // only after this iteration
    const float c_next = C.cq * C.k_scale((t + 1) & (NSLOT - 1));
    const float svp = C.v_scale((t - 1) & (NSLOT - 1));
    C.template iter<true, false>(sc, sn, pprev, pcur, t, c, svp, rf, tile_at(t), kept(t));
    // Wait for our own loads of three boundaries ago and all LDS reads, then
    // a plain barrier (the "memory" clobber keeps every memory access on its
    // side).  __syncthreads() would add a fence that waits for every
    // direct-to-LDS load in flight, which defeats the ring.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * G::LPB) & ~0x0F00);  // and lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    rf = C.refill(tile_at(t + 5), (t + 1) & (NSLOT - 1), tile_at(t + 3), (t - 1) & (NSLOT - 1));
    c = c_next;
  };
  auto last = [&](const v16i (&sc)[2], v16i (&sn)[2], const v8i& pprev, v8i& pcur, int t) {
    const float svp = C.v_scale((t - 1) & (NSLOT - 1));
    C.template iter<false, true>(sc, sn, pprev, pcur, t, c, svp, rf, tile_at(t), kept(t));
    // V(t) may still be in flight (issued up to two boundaries ago, by any
    // wave): wait for every load, then a barrier
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    C.pv_last(pcur, t & (NSLOT - 1), C.v_scale(t & (NSLOT - 1)));
  };
  // tiles in pairs, so that the score and P registers alternate without copies
  int t = 0;
  for (; t + 2 < npos; t += 2) {
    step(S0, S1, P1, P0, t);
    step(S1, S0, P0, P1, t + 1);
  }
  if (t + 1 < npos) {
    step(S0, S1, P1, P0, t);
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

template <int D, bool SP>
static void launch_d(const AttnParams& q, hipStream_t st) {
  constexpr int lds = Geo<D>::LDS_BYTES + (SP ? SP_LIST_BYTES : 0);
  static bool configured = false;  // the attribute is per kernel, set once per process
  if (!configured) {
    (void)hipFuncSetAttribute((const void*)attn_fp8_kernel<D, SP>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds);
    configured = true;
  }
  hipLaunchKernelGGL((attn_fp8_kernel<D, SP>), dim3(8 * q.per_xcd), dim3(NTHR), lds, st, q);
}

void launch_attention_fp8(const AttnParams& q, int d, hipStream_t st) {
  const bool sp = q.mask != nullptr;
  if (d == 128)
    sp ? launch_d<128, true>(q, st) : launch_d<128, false>(q, st);
  else
    sp ? launch_d<64, true>(q, st) : launch_d<64, false>(q, st);
}

}  // namespace sqattn
