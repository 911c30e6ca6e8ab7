// Routing pieces shared by the routing kernels (route.hip) and the fused
// route + quantise + group launch (front.hip).
//
// Page 1, "Serving call chain" and "Key sources" table (routing row): sigmoid
// scores, the correction bias only takes part in choosing experts, the weights
// gather the bias-free scores and are normalised; page 5: routed scaling.
#pragma once

#include "common.h"

namespace mi355moe {

// Order-preserving unsigned image of a float selection key: larger keys map
// to larger values, -inf to 0x007FFFFF.  A NaN key (a NaN logit or bias)
// maps to 1, below every other key, so NaN experts rank last and among
// themselves by lower index (a stable descending sort puts NaN last too).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 1u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Sigmoid evaluated in double and rounded once to float.  Used for both the
// selection keys and the selected scores, so the two agree bit for bit.
__device__ __forceinline__ float sigmoid_score(float logit) {
  return (float)(1.0 / (1.0 + exp(-(double)logit)));
}

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }

// Wavefront maximum / minimum of an unsigned value, uniform result: inclusive
// scans within 16-lane rows (row_shr 1, 2, 4, 8), then row_bcast 15 and 31
// carry the rows' results up to lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = umin32(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x111, 0xf, 0xf, false));
  v = umin32(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x112, 0xf, 0xf, false));
  v = umin32(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x114, 0xf, 0xf, false));
  v = umin32(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x118, 0xf, 0xf, false));
  v = umin32(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xa, 0xf, false));
  v = umin32(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

constexpr int kRegExpertsPerLane = 16;   // register path: E <= 1024

// The lane's best two remaining keys among its experts lane + 64 j with bit j
// of avail set: key descending, expert ascending among equal keys.
struct Top2 {
  uint32_t k0, k1, e0, e1;
  bool has0, has1;
};
__device__ __forceinline__ Top2 lane_top2(const uint32_t (&key)[kRegExpertsPerLane],
                                          uint32_t avail, int lane) {
  Top2 t{0u, 0u, 0xFFFFFFFFu, 0xFFFFFFFFu, false, false};
#pragma unroll
  for (int j = 0; j < kRegExpertsPerLane; ++j) {
    const bool a = (avail >> j) & 1u;
    const uint32_t k = key[j], e = (uint32_t)(lane + 64 * j);
    const bool first = a && (!t.has0 || k > t.k0);
    const bool second = a && !first && (!t.has1 || k > t.k1);
    t.k1 = first ? t.k0 : second ? k : t.k1;
    t.e1 = first ? t.e0 : second ? e : t.e1;
    t.has1 = first ? t.has0 : (second || t.has1);
    t.k0 = first ? k : t.k0;
    t.e0 = first ? e : t.e0;
    t.has0 = t.has0 || first;
  }
  return t;
}

// One wavefront selects the top K of one token (E <= 64 * kRegExpertsPerLane)
// from its keys in LDS.  Lane l holds the keys of experts l, l + 64, ... and a
// cache of its best two remaining ones (key descending, expert ascending).
// Each of the K rounds takes the wavefront maximum of the lanes' best keys
// (DPP row shifts and broadcasts); the expert is read from the one lane
// holding it, or, when several lanes hold that key, is the smallest expert
// among them (a second reduction).  The owning lane retires the winner and
// promotes its second key; only a lane that wins again before its cache is
// refilled rescans its keys.  Lane k < K returns slot k's expert and weight
// (s_k / sum_j s_j in double, times scaling).  Every lane must call this.
__device__ __forceinline__ void select_topk_wave(const uint32_t* keys_s, const float* row, int E,
                                                 int K, float scaling, int lane, int& id_out,
                                                 float& w_out) {
  uint32_t key[kRegExpertsPerLane];
  uint32_t avail = 0;                                // bit j: expert lane + 64 j not yet taken
#pragma unroll
  for (int j = 0; j < kRegExpertsPerLane; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? keys_s[e] : 0u;
    avail |= (e < E ? 1u : 0u) << j;
  }
  // Cache: c0 the best remaining key (has0 iff any remain), c1 the next one
  // (valid while fresh1, until c0 is taken once).
  Top2 c = lane_top2(key, avail, lane);
  uint32_t k0 = c.k0, k1 = c.k1, e0 = c.e0, e1 = c.e1;
  bool has0 = c.has0, has1 = c.has1, fresh1 = true;
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    const uint32_t ck = has0 ? k0 : 0u;
    const uint32_t m = wave_max_u32(ck);
    const bool cand = has0 && ck == m;
    const uint64_t holders = __ballot(cand);
    uint32_t win;
    if (__popcll(holders) == 1)
      win = (uint32_t)__builtin_amdgcn_readlane((int)e0, __ffsll((long long)holders) - 1);
    else
      win = wave_min_u32(cand ? e0 : 0xFFFFFFFFu);   // < E: K <= E
    bool refill = false;
    if ((int)(win & 63) == lane) {
      avail &= ~(1u << (win >> 6));
      if (fresh1) {
        k0 = k1; e0 = e1; has0 = has1;
        fresh1 = false;
      } else {
        refill = true;
      }
    }
    if (__ballot(refill)) {
      if (refill) {
        c = lane_top2(key, avail, lane);
        k0 = c.k0; k1 = c.k1; e0 = c.e0; e1 = c.e1;
        has0 = c.has0; has1 = c.has1; fresh1 = true;
      }
    }
    if (lane == k) my_id = (int)win;
  }
  my_id = (my_id >= 0 && my_id < E) ? my_id : 0;
  const float my_s = lane < K ? sigmoid_score(row[my_id]) : 0.0f;
  double total = 0.0;
  for (int k = 0; k < K; ++k) total += (double)__shfl(my_s, k);   // left to right
  id_out = my_id;
  w_out = (float)(((double)my_s / total) * (double)scaling);
}

}  // namespace mi355moe
