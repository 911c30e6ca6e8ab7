// Pieces shared by the FC kernels (decode-shaped and prefill-shaped).
#pragma once

#include "common.h"

namespace mi355moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// One 16x16x128 block-scaled MFMA: A = 16 weight rows of E2M1 (cbsz 4), B = 16
// token columns of E4M3 (blgp 0), with this lane's E8M0 scale bytes selected by J.
template <int J>
__device__ __forceinline__ v4f mfma_w4a8(v4i w, v4i a_lo, v4i a_hi, v4f c, int ws, int as) {
  v8i a8 = {w[0], w[1], w[2], w[3], 0, 0, 0, 0};
  v8i b8 = {a_lo[0], a_lo[1], a_lo[2], a_lo[3], a_hi[0], a_hi[1], a_hi[2], a_hi[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 0, J, ws, J, as);
}

struct FcParams {
  const uint8_t* act;        // FC1: xq [T, K]; FC2: hq [R, K]
  const uint8_t* act_s;      // [.., K/32]
  int64_t act_rows;          // rows of act: FC1 T, FC2 R
  const int32_t* gather;     // FC1: sorted_route (grouped row -> route); FC2: unused
  int top_k;
  const uint8_t* w;          // [E_local, N, K/2]
  const uint8_t* w_s;        // [E_local, N, K/32]
  int K, N, I;
  const int32_t* expert_offsets;
  const int32_t* tile_prefix;  // [E_local + 1] for this kernel's tile height
  int E_local;
  int n_units, max_tiles;
  float alpha, beta;
  uint8_t* hq;               // FC1 out [R, I]
  uint8_t* hs;               // FC1 out [R, I/32]
  float* y;                  // FC2 out [R, N]
};

// SiTU(g, u) = alpha tanh(g / alpha) sigmoid(g) * beta tanh(u / beta)
// (page 1, "真实 checkpoint 契约": the SiTU activation with alpha = 4, beta =
// 25), from the hardware base-2 exponential and reciprocal:
//   sigmoid(g) = 1 / (1 + 2^(-g log2 e)),  tanh(y) = 1 - 2 / (1 + 2^(2 y log2 e)).
// Each factor is within a few float32 ulps of its value (the tanh form loses
// only absolute accuracy, ~1e-7, for small |y|), far below the E4M3 rounding
// the result goes through next.  Infinite exponentials give the limits
// (tanh -> +-1, sigmoid -> 0 or 1); NaN propagates.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_tanh(float y) {
  return 1.0f - 2.0f * fast_rcp(1.0f + fast_exp2(y * 2.8853900817779268f));   // 2 log2 e
}
__device__ __forceinline__ float situ(float g, float u, float alpha, float beta) {
  const float sig = fast_rcp(1.0f + fast_exp2(g * -1.4426950408889634f));     // -log2 e
  return alpha * fast_tanh(g * fast_rcp(alpha)) * sig * (beta * fast_tanh(u * fast_rcp(beta)));
}

// Largest expert e with prefix[e] <= tile (the expert owning that tile).
__device__ __forceinline__ int find_expert(const int* prefix, int E_local, int tile) {
  int lo = 0, hi = E_local;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

// The MFMAs read operands from all 64 lanes: make the accumulators live here,
// with every lane active, so no MFMA is moved into per-lane store conditions.
__device__ __forceinline__ void pin_acc(v4f (&acc)[4]) {
#pragma unroll
  for (int bk = 0; bk < 4; ++bk)
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(acc[bk][r]));
}

// The same for accumulators that live in AGPRs (kernels whose accumulators
// fill the architectural VGPRs' counterpart file).
__device__ __forceinline__ void pin_acc_agpr(v4f (&acc)[4]) {
#pragma unroll
  for (int bk = 0; bk < 4; ++bk)
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" : "+a"(acc[bk][r]));
}

// Epilogue of one wavefront unit (64 weight rows) for one 16-token sub-tile.
// Lane (g, li) holds rows 4g..4g+3 of each 16-row block for token column li.
// FC1: blocks 0/1 are gate columns [c0, c0+32), blocks 2/3 the matching up
// columns; SiTU, the 32-column absmax (two lane-xor steps over the lane
// groups), the E8M0 exponent and the E4M3 codes are all computed here.
// FC2: the float rows go to y.  Every lane must call this (shuffles).
template <bool FC1>
__device__ __forceinline__ void store_subtile(const FcParams& p, const v4f (&acc)[4], int row,
                                              bool valid, int u, int g) {
  if (FC1) {
    const int c0 = u * 32;
    float a[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[r] = situ(acc[0][r], acc[2][r], p.alpha, p.beta);       // column c0 + 4g + r
      a[4 + r] = situ(acc[1][r], acc[3][r], p.alpha, p.beta);   // column c0 + 16 + 4g + r
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = fabsf(a[i]);
      amax = v > amax ? v : amax;
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int ex = mx8_exponent(amax);
    uint32_t q0 = 0, q1 = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      q0 |= e4m3_encode(ldexpf(a[r], -ex)) << (8 * r);
      q1 |= e4m3_encode(ldexpf(a[4 + r], -ex)) << (8 * r);
    }
    if (valid) {
      uint8_t* dst = p.hq + (size_t)row * p.I + c0 + 4 * g;
      *reinterpret_cast<uint32_t*>(dst) = q0;
      *reinterpret_cast<uint32_t*>(dst + 16) = q1;
      if (g == 0) p.hs[(size_t)row * (p.I / 32) + c0 / 32] = (uint8_t)(ex + 127);
    }
  } else {
    if (valid) {
      float* dst = p.y + (size_t)row * p.N + u * 64 + 4 * g;
#pragma unroll
      for (int bk = 0; bk < 4; ++bk) *reinterpret_cast<v4f*>(dst + 16 * bk) = acc[bk];
    }
  }
}

}  // namespace mi355moe
