// Pieces shared by the FC kernels (decode-shaped and prefill-shaped).
#pragma once

#include "common.h"

namespace mi355moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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
  int64_t n_routes;          // grouped rows R = T * top_k
  uint32_t* act_st;          // workspace: [K/128][R] scale dwords of the grouped rows
  int32_t* sched;            // workspace: per-XCD work counters (prefill kernels)
  const int32_t* gather;     // FC1: sorted_route (grouped row -> route); FC2: unused
  int top_k;
  const uint8_t* w;          // [E_local, N, K/2]
  const uint8_t* w_s;        // [E_local, N, K/32]
  int K, N, I;
  const int32_t* expert_offsets;
  const int32_t* tile_prefix;  // [E_local + 1] for this kernel's tile height
  const int32_t* tile_map;     // expert of each tile (decode-shaped kernels' tile list)
  int E_local;
  int n_units, max_tiles;
  float alpha, beta;
  uint8_t* hq;               // FC1 out [R, I]
  uint8_t* hs;               // FC1 out [R, I/32]
  uint16_t* y;               // FC2 out [R, N]: fp16 of y / 2^ye (deterministic combine)
  int8_t* ye;                // FC2 out: scale exponent per 64 columns (ye_index)
  // Atomic combine (FC2 only; out_acc == nullptr otherwise): grouped row r
  // adds topk_w[route] * y[r] into out_acc[route / top_k] with
  // route = combine_route[r].
  const int32_t* combine_route;
  const float* topk_w;
  float* out_acc;            // [T, N] float sums
};

// SiTU(g, u) = alpha tanh(g / alpha) sigmoid(g) * beta tanh(u / beta)
// (page 1, "真实 checkpoint 契约": the SiTU activation with alpha = 4, beta =
// 25; alpha, beta > 0), in float32 from hardware base-2 exponentials and
// reciprocals.  With z1 = e^(-2|g|/alpha), z2 = e^(-|g|) and
// w = e^(-2|u|/beta), all in [0, 1]:
//   tanh(g/alpha) = sign(g) (1 - z1) / (1 + z1),
//   sigmoid(g)    = s / (1 + z2), s = 1 for g >= 0 and z2 for g < 0,
//   tanh(u/beta)  = sign(u) (1 - w) / (1 + w),
// so SiTU = alpha beta sign(g)(1 - z1) s sign(u)(1 - w) / ((1 + z1)(1 + z2)(1 + w)),
// where nothing overflows: each denominator lies in [1, 8], so two of them
// share one reciprocal (SiTU values are computed in pairs).  With alpha = 4,
// z2 = z1^2 saves an exponential.  s = max(z2, clamp(g 2^64, 0, 1)) needs no
// per-lane select: 1 for g >= 2^-64, z2 for g <= 0, and z2 (within 2^-64 of
// 1) in between.  The numerators keep the signs of g and u (tanh keeps the
// sign of zero).  1 - z cancels for small |g|/alpha, |u|/beta: the result
// then carries an absolute error of a few float32 ulps of the factor's scale
// (alpha, beta) rather than a relative one.  Measured against float64 on the
// device this flips about 1e-5 of the requantised bytes, against about 5e-4
// that the MFMA's own accumulation flips; a cancellation-free series form
// cost 0.4 ms of the 8K-token prefill FC1, whose epilogue is VALU-bound.  A
// NaN input gives 0 here (the requantisation rule sends NaN to code 0 and
// leaves it out of the block maximum, which is what 0 does).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
struct SituConst {
  float k1, k2, k3, ab;   // -2 log2(e) / alpha, -log2(e), -2 log2(e) / beta, alpha beta
  bool a4;                // alpha == 4: e^(-|g|) = z1^2
};
__device__ __forceinline__ SituConst situ_const(float alpha, float beta) {
  const float l2e = 1.4426950408889634f;
  return SituConst{-2.0f * l2e / alpha, -l2e, -2.0f * l2e / beta, alpha * beta, alpha == 4.0f};
}
// One value's numerator and denominator (see above).
template <bool A4>
__device__ __forceinline__ void situ_parts(float g, float u, const SituConst& c, float& num,
                                           float& den) {
  const float z1 = fast_exp2(fabsf(g) * c.k1);
  const float z2 = A4 ? z1 * z1 : fast_exp2(fabsf(g) * c.k2);
  const float w = fast_exp2(fabsf(u) * c.k3);
  const float s = fmaxf(z2, __builtin_amdgcn_fmed3f(g * 18446744073709551616.0f, 0.0f, 1.0f));
  num = copysignf(1.0f - z1, g) * copysignf(1.0f - w, u) * s;
  den = (1.0f + z1) * (1.0f + z2) * (1.0f + w);
}
template <bool A4>
__device__ __forceinline__ void situ2(float g0, float u0, float g1, float u1, const SituConst& c,
                                      float& v0, float& v1) {
  float n0, d0, n1, d1;
  situ_parts<A4>(g0, u0, c, n0, d0);
  situ_parts<A4>(g1, u1, c, n1, d1);
  const float r = c.ab * fast_rcp(d0 * d1);
  v0 = __builtin_isunordered(g0, u0) ? 0.0f : n0 * d1 * r;
  v1 = __builtin_isunordered(g1, u1) ? 0.0f : n1 * d0 * r;
}
// Four E4M3 codes of x / s (s a normal power of two, |x / s| <= 448), packed
// little-endian, by the hardware scaled conversion.
typedef short v2s __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3x4_scaled(float x0, float x1, float x2, float x3,
                                                  float s) {
  v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, x0, x1, s, false);
  v2s both = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x2, x3, s, true);
  return __builtin_bit_cast(uint32_t, both);
}

// max(v, v of lane l ^ 16) and then with lane l ^ 32, by gfx950's cross-row
// lane swaps (no trip through the LDS crossbar): swapping a register's odd
// 16-lane rows with a copy's even rows leaves each lane holding its own value
// in one result and its xor-16 partner's in the other (the same for halves
// and xor 32).  Every lane must call this.
__device__ __forceinline__ float max_over_lane_groups(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const float m = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const uint32_t c = __float_as_uint(m);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
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
// FC2: the float rows go to y, or with the atomic combine are added, times
// the route's weight, into the token's float sums.  Every lane must call this
// (shuffles).
template <bool FC1>
__device__ __forceinline__ void store_subtile(const FcParams& p, const v4f (&acc)[4], int row,
                                              bool valid, int u, int g) {
  if (FC1) {
    const int c0 = u * 32;
    const SituConst sc = situ_const(p.alpha, p.beta);
    float a[8];   // a[r]: column c0 + 4g + r; a[4 + r]: column c0 + 16 + 4g + r
    if (sc.a4) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        situ2<true>(acc[0][r], acc[2][r], acc[1][r], acc[3][r], sc, a[r], a[4 + r]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        situ2<false>(acc[0][r], acc[2][r], acc[1][r], acc[3][r], sc, a[r], a[4 + r]);
    }
    float amax = 0.0f;   // a NaN value (none: SiTU gives 0 for NaN input) would be skipped
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(a[i]));
    amax = max_over_lane_groups(amax);
    const int ex = mx8_exponent(amax);
    uint32_t q0 = 0, q1 = 0;
    if (ex > -127) {
      // gfx950's scaled conversion divides by the power of two 2^ex and
      // rounds to the nearest E4M3 (ties to even) -- the same code as
      // e4m3_encode for every |value| <= 448, which the scale guarantees.
      const float s2 = __uint_as_float((uint32_t)(ex + 127) << 23);
      q0 = e4m3x4_scaled(a[0], a[1], a[2], a[3], s2);
      q1 = e4m3x4_scaled(a[4], a[5], a[6], a[7], s2);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        q0 |= e4m3_encode(ldexpf(a[r], -ex)) << (8 * r);
        q1 |= e4m3_encode(ldexpf(a[4 + r], -ex)) << (8 * r);
      }
    }
    if (valid) {
      uint8_t* dst = p.hq + (size_t)row * p.I + c0 + 4 * g;
      *reinterpret_cast<uint32_t*>(dst) = q0;
      *reinterpret_cast<uint32_t*>(dst + 16) = q1;
      if (g == 0) p.hs[(size_t)row * (p.I / 32) + c0 / 32] = (uint8_t)(ex + 127);
    }
  } else if (p.out_acc != nullptr) {
    // Atomic combine: this lane's 16 columns of grouped row `row` (columns
    // u 64 + 16 bk + 4 g + r), weighted, into its token's sums.  The adds
    // land in no fixed order, so the sums' rounding varies from run to run.
    if (valid) {
      const int route = p.combine_route[row];
      const float w = p.topk_w[route];
      float* dst = p.out_acc + (size_t)(route / p.top_k) * p.N + u * 64 + 4 * g;
#pragma unroll
      for (int bk = 0; bk < 4; ++bk)
#pragma unroll
        for (int r = 0; r < 4; ++r) unsafeAtomicAdd(dst + 16 * bk + r, w * acc[bk][r]);
    }
  } else {
    // The 64 columns of the unit for this row (16 values in each of the four
    // lanes with this li) share one power-of-two scale 2^e chosen so that the
    // largest finite magnitude lands in [2^14, 2^15): fp16 keeps every value
    // to 2^-11 relative (non-finite values stay non-finite).
    // The largest finite magnitude: a plain maximum (NaN ignored), and the
    // finite-only scan again in the rare lane whose maximum is infinite.
    float amax = 0.0f;
#pragma unroll
    for (int bk = 0; bk < 4; ++bk)
#pragma unroll
      for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(acc[bk][r]));
    if (amax > 3.4028235e38f) {
      amax = 0.0f;
#pragma unroll
      for (int bk = 0; bk < 4; ++bk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = fabsf(acc[bk][r]);
          amax = (v <= 3.4028235e38f && v > amax) ? v : amax;
        }
    }
    amax = max_over_lane_groups(amax);
    const int fe = (int)((__float_as_uint(amax) >> 23) & 0xFF);
    const int e = fe - 141 < -128 ? -128 : fe - 141;
    // fp16 pairs d[bk][h]: columns 16 bk + 4 g + 2 h, +1 of the row.
    uint32_t d[4][2];
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
      // Two values per conversion (round to nearest even, as one at a time).
      const f32x2 lo = {ldexpf(acc[bk][0], -e), ldexpf(acc[bk][1], -e)};
      const f32x2 hi = {ldexpf(acc[bk][2], -e), ldexpf(acc[bk][3], -e)};
      d[bk][0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, f16x2));
      d[bk][1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, f16x2));
    }
    // Rotate the pieces among the four lanes of the row so that lane g ends
    // up with columns 8 g .. 8 g + 7 and 32 + 8 g .. 32 + 8 g + 7: piece
    // (lane group a1 a0, block k1 k0) moves to lane group k0 a1, block
    // k1 a0.  Two exchanges do it: lane-group bit 1 with block bit 0 (32-lane
    // swap), then lane-group bit 0 with block bit 0 (16-lane swap).
#pragma unroll
    for (int k1 = 0; k1 < 2; ++k1)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto r = __builtin_amdgcn_permlane32_swap(d[2 * k1][h], d[2 * k1 + 1][h], false, false);
        d[2 * k1][h] = r[0];
        d[2 * k1 + 1][h] = r[1];
      }
#pragma unroll
    for (int k1 = 0; k1 < 2; ++k1)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto r = __builtin_amdgcn_permlane16_swap(d[2 * k1][h], d[2 * k1 + 1][h], false, false);
        d[2 * k1][h] = r[0];
        d[2 * k1 + 1][h] = r[1];
      }
    if (valid) {
      uint16_t* dst = p.y + (size_t)row * p.N + u * 64 + 8 * g;
#pragma unroll
      for (int s = 0; s < 2; ++s)
        *reinterpret_cast<uint4*>(dst + 32 * s) =
            uint4{d[2 * s][0], d[2 * s][1], d[2 * s + 1][0], d[2 * s + 1][1]};
      if (g == 0) p.ye[ye_index(row, u, p.N / 64)] = (int8_t)e;
    }
  }
}

}  // namespace mi355moe
