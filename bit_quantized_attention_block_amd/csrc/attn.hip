// Quantized attention for gfx950 (MI355X): work decomposition, register
// layouts shared by the two P.V kernels, and the launcher.
//
// Method: logits from INT8 codes of Q and smoothed K on the integer matrix
// units, softmax, then P.V in bf16 or FP8 with fp32 accumulation
// (jefxiong.cn "AIGC weekend special 5.10", section 1.2 item (1); GVCLab
// research log 2026-09-02, section 5.5 table, SageAttention2 row).  The
// tiling with a running max and running sum is the FlashAttention lineage that
// the same digest names as its baseline.
//
// Work decomposition
//   * A work-group (8 waves, two per SIMD) owns 256 query rows of one (b,h)
//     head; each wave owns 32 rows.  Keys stream in 64-key tiles through a
//     4-slot LDS ring filled by direct-to-LDS loads (attn_bf16.hip,
//     attn_fp8.hip).
//   * Work-group w runs on XCD w % 8 (round-robin dispatch); items are
//     numbered so that each XCD walks consecutive query tiles of the same
//     head, which then share K/V tiles through that XCD's L2.
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
#include "common.h"
#include "kernels.h"

namespace sqattn {

void launch_attention(const AttnParams& p, int d, int pv, hipStream_t st) {
  AttnParams q = p;
  q.qtiles = (p.N + ATT_QWG - 1) / ATT_QWG;
  const long long W = (long long)p.BH * q.qtiles;
  q.per_xcd = (int)((W + 7) / 8);
  if (pv == 0)
    launch_attention_bf16(q, d, st);
  else
    launch_attention_fp8(q, d, st);
}

}  // namespace sqattn
