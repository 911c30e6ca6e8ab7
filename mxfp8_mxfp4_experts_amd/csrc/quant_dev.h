// MXFP8 quantisation of one 8-element piece per lane, shared by the
// quantisation kernel (quant.hip) and the fused route + quantise + group
// launch (front.hip).
//
// Page 5 (pre-dispatch step): absmax per 32 elements -> UE8M0 scale -> E4M3
// payload; page 1 ("NaN/Inf decision record"): the conversion saturates to a
// finite value and never emits the 0xFF scale.
#pragma once

#include "common.h"

namespace mi355moe {

// Piece gid of the [T, H] activations (H / 8 pieces per row).  Four lanes
// share a 32-element group: each lane loads 8 bf16 (16 bytes), the group
// absmax is two lane-xor max steps, and each lane writes its 8 E4M3 bytes; the
// first lane of the group writes the scale byte.  Every lane must call this
// (pieces past the end repeat the last one and store nothing).
__device__ __forceinline__ void quant_piece(const uint16_t* __restrict__ x, int64_t ld, int T,
                                            int H, uint8_t* __restrict__ xq,
                                            uint8_t* __restrict__ xs, int64_t gid) {
  const int per_row = H / 8;
  const int64_t total = (int64_t)T * per_row;
  const bool valid = gid < total;
  if (!valid) gid = total - 1;   // keep every lane in the shuffles below
  const int t = (int)(gid / per_row), c = (int)(gid % per_row);

  uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)t * ld + (size_t)c * 8);
  float f[8];
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float a = fabsf(f[i]);
    amax = (a > amax) ? a : amax;   // NaN compares false: ignored
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int e = mx8_exponent(amax);

  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= e4m3_encode(ldexpf(f[i], -e)) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= e4m3_encode(ldexpf(f[4 + i], -e)) << (8 * i);
  if (valid) {
    *reinterpret_cast<uint2*>(xq + (size_t)t * H + (size_t)c * 8) = make_uint2(lo, hi);
    if ((c & 3) == 0) xs[(size_t)t * (H / 32) + c / 4] = (uint8_t)(e + 127);
  }
}

}  // namespace mi355moe
