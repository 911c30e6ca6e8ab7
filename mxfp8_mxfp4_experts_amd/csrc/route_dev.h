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

// Top K of one token by rounds (E <= 64 * kRegExpertsPerLane), from its
// keys in LDS.  Lane l holds the keys of experts l, l + 64, ... and a
// cache of its best two remaining ones (key descending, expert ascending).
// Each of the K rounds takes the wavefront maximum of the lanes' best keys
// (DPP row shifts and broadcasts); the expert is read from the one lane
// holding it, or, when several lanes hold that key, is the smallest expert
// among them (a second reduction).  The owning lane retires the winner and
// promotes its second key; only a lane that wins again before its cache is
// refilled rescans its keys.  Lane k < K returns slot k's expert.  Every lane
// must call this.
__device__ __forceinline__ int select_topk_rounds(const uint32_t* keys_s, int E, int K,
                                                  int lane) {
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
  return my_id;
}

// Descending bitonic sort of one value per lane across the wavefront: lane i
// ends with the i-th largest.  In the stage merging blocks of k lanes at
// distance j, lane i keeps the larger of the pair when bit k and bit j of i
// agree (so the final k = 64 stage leaves the larger values in lower lanes).
__device__ __forceinline__ uint32_t wave_sort_desc_u32(uint32_t v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)v, j);
      const bool keep_max = ((lane & k) == 0) == ((lane & j) == 0);
      v = keep_max ? umax32(v, o) : umin32(v, o);
    }
  return v;
}
__device__ __forceinline__ uint64_t wave_sort_desc_u64(uint64_t v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t ohi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), j);
      const uint32_t olo = (uint32_t)__shfl_xor((int)(uint32_t)v, j);
      const uint64_t o = ((uint64_t)ohi << 32) | olo;
      const bool keep_max = ((lane & k) == 0) == ((lane & j) == 0);
      v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
    }
  return v;
}

// The top K of one token by a threshold and two wavefront sorts, for the
// usual case of few keys near the K-th largest.  T0, the K-th largest of the
// 64 lanes' largest keys, is at most the K-th largest key (K lanes hold a key
// of at least T0), so every selected key is at least T0.  Those candidates
// (the key, then the inverted expert index, as one 64-bit value: key
// descending, expert ascending) are gathered through cand (64 entries of LDS
// per wavefront) and sorted, and lane k takes the k-th.  Returns false,
// having selected nothing, when more than 64 keys reach T0 (many equal keys);
// the rounds then select.  Every lane must call this.
__device__ __forceinline__ bool select_topk_threshold(const uint32_t* keys_s, int E, int K,
                                                      int lane, uint64_t* cand, int& my_id) {
  uint32_t key[kRegExpertsPerLane];
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kRegExpertsPerLane; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? keys_s[e] : 0u;   // 0: no expert (every real key is above 0)
    m = umax32(m, key[j]);
  }
  const uint32_t t0 =
      (uint32_t)__builtin_amdgcn_readlane((int)wave_sort_desc_u32(m, lane), K - 1);
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kRegExpertsPerLane; ++j) cnt += key[j] >= t0 && key[j] != 0u ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  const int total = __builtin_amdgcn_readlane(incl, 63);
  if (total > 64) return false;
  int pos = incl - cnt;
#pragma unroll
  for (int j = 0; j < kRegExpertsPerLane; ++j)
    if (key[j] >= t0 && key[j] != 0u)
      cand[pos++] = ((uint64_t)key[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * j));
  // The wavefront's LDS writes before its reads of other lanes' entries.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t c = wave_sort_desc_u64(lane < total ? cand[lane] : 0ull, lane);
  my_id = (int)(0xFFFFFFFFu - (uint32_t)c);
  return true;
}

// One wavefront selects the top K of one token (E <= 64 * kRegExpertsPerLane)
// from its keys in LDS, ordered by key descending with ties to the lower
// expert: by the threshold selection, else by rounds.  Lane k < K returns
// slot k's expert and weight (s_k / sum_j s_j in double, times scaling).
// cand: 64 entries of LDS for this wavefront.  Every lane must call this.
__device__ __forceinline__ void select_topk_wave(const uint32_t* keys_s, const float* row, int E,
                                                 int K, float scaling, int lane, uint64_t* cand,
                                                 int& id_out, float& w_out) {
  int my_id = 0;
  if (!select_topk_threshold(keys_s, E, K, lane, cand, my_id))
    my_id = select_topk_rounds(keys_s, E, K, lane);
  my_id = (my_id >= 0 && my_id < E) ? my_id : 0;
  const float my_s = lane < K ? sigmoid_score(row[my_id]) : 0.0f;
  double total = 0.0;
  for (int k = 0; k < K; ++k) total += (double)__shfl(my_s, k);   // left to right
  id_out = my_id;
  w_out = (float)(((double)my_s / total) * (double)scaling);
}

}  // namespace mi355moe
