// MXFP8 quantisation of one 8-element piece per lane, shared by the
// quantisation kernel (quant.hip) and the fused route + quantise + group
// launch (front.hip).
//
// Page 5 (pre-dispatch step): absmax per 32 elements -> UE8M0 scale -> E4M3
// payload; page 1 ("NaN/Inf decision record"): the conversion saturates to a
// finite value and never emits the 0xFF scale.
#pragma once

#include "common.h"
#include "fc_common.h"   // e4m3x4_scaled

namespace mi355moe {

// Piece c (8 elements) of row t of the [T, H] activations.  Four lanes share
// a 32-element group: each lane loads 8 bf16 (16 bytes), the group absmax is
// two lane-xor max steps, and each lane writes its 8 E4M3 bytes; the first
// lane of the group writes the scale byte.  A group whose values are all
// finite with a normal scale (e > -127) is converted by the hardware; one
// holding an infinity or a NaN, or whose scale is 2^-127, by the integer
// encoder (NaN -> 0, +-Inf -> +-448, the sign of zero kept).  The four lanes
// of a group must call this together (shuffles); with valid false a lane
// stores nothing.
__device__ __forceinline__ void quant_row_piece(const uint16_t* __restrict__ x, int64_t ld,
                                                int H, uint8_t* __restrict__ xq,
                                                uint8_t* __restrict__ xs, int t, int c,
                                                bool valid) {
  uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)t * ld + (size_t)c * 8);
  float f[8];
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t nonfinite = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    nonfinite |= ((w[i] & 0x7F80u) == 0x7F80u) | ((w[i] & 0x7F800000u) == 0x7F800000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float a = fabsf(f[i]);
    amax = (a > amax) ? a : amax;   // NaN compares false: ignored
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  nonfinite |= __shfl_xor(nonfinite, 1);
  nonfinite |= __shfl_xor(nonfinite, 2);
  const int e = mx8_exponent(amax);

  uint32_t lo = 0, hi = 0;
  if (!nonfinite && e > -127) {
    const float s2 = __uint_as_float((uint32_t)(e + 127) << 23);
    lo = e4m3x4_scaled(f[0], f[1], f[2], f[3], s2);
    hi = e4m3x4_scaled(f[4], f[5], f[6], f[7], s2);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= e4m3_encode(ldexpf(f[i], -e)) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= e4m3_encode(ldexpf(f[4 + i], -e)) << (8 * i);
  }
  if (valid) {
    *reinterpret_cast<uint2*>(xq + (size_t)t * H + (size_t)c * 8) = make_uint2(lo, hi);
    if ((c & 3) == 0) xs[(size_t)t * (H / 32) + c / 4] = (uint8_t)(e + 127);
  }
}

// Piece gid of the [T, H] activations (H / 8 pieces per row).  Every lane
// must call this (pieces past the end repeat the last one and store nothing).
__device__ __forceinline__ void quant_piece(const uint16_t* __restrict__ x, int64_t ld, int T,
                                            int H, uint8_t* __restrict__ xq,
                                            uint8_t* __restrict__ xs, int64_t gid) {
  const int per_row = H / 8;
  const int64_t total = (int64_t)T * per_row;
  const bool valid = gid < total;
  if (!valid) gid = total - 1;   // keep every lane in the shuffles
  quant_row_piece(x, ld, H, xq, xs, (int)(gid / per_row), (int)(gid % per_row), valid);
}

}  // namespace mi355moe
