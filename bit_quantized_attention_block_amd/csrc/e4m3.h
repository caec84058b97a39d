// OCP 8-bit floating point E4M3FN encoding (bias 7, largest finite 448, no
// infinities), usable on host and device.  FP8 is the precision the pages give
// for P.V (GVCLab research log 2026-09-02, section 5.5 table, SageAttention2
// row); the bit format itself is the OCP specification's.
#pragma once

#include <math.h>
#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define SQ_HD8 __host__ __device__ __forceinline__
#else
#define SQ_HD8 static inline
#endif

namespace sqattn {

// binary32 -> E4M3FN code, round to nearest even, saturating to +-448; the
// sign bit follows the sign of y (also for zero).  Finite inputs only.
SQ_HD8 uint32_t e4m3_encode_f32(float y) {
  uint32_t u;
  memcpy(&u, &y, 4);
  const uint32_t sign = (u >> 31) << 7;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t mag;
  if (a >= 0x43E80000u) {          // |y| >= 464: nearest-even would leave the format
    mag = 0x7Eu;
  } else if (a < 0x3C800000u) {    // |y| < 2^-6: subnormal quantum 2^-9
    float t;
    memcpy(&t, &a, 4);
    mag = (uint32_t)rintf(t * 512.0f);   // exact scaling, then half-to-even
  } else {                         // normal: keep 3 of 23 fraction bits
    uint32_t keep = (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);
    const uint32_t rem = a & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep += 1;
    mag = keep;
  }
  return sign | mag;
}

}  // namespace sqattn
