// a1: sigmoid + correction-bias top-k routing with renormalised weights.
//
// Page 1, "Serving call chain" and "Key sources" table (routing row): sigmoid
// scores, the correction bias only takes part in choosing experts, the weights
// gather the bias-free scores and are normalised; page 5: routed scaling.
//
// The slots come out ordered by key descending, ties going to the lower
// expert index.
//  * E <= 1024: one workgroup per token computes the keys (as
//    order-preserving unsigned integers) into LDS; then lane l of the first
//    wavefront holds the keys of experts l, l + 64, ... in registers.  Each of
//    the K rounds takes the lane's best remaining key, the wavefront maximum
//    of those (DPP row shifts and broadcasts), then the smallest expert index
//    among the lanes holding that maximum; the owning lane retires the winner.
//  * larger E: the keys sit in LDS and each round takes a wavefront arg-max
//    over a 64-bit key (ordered float key, then inverted expert index)
//    restricted to keys below the previous winner.
#include "common.h"
#include "launch.h"

namespace mi355moe {

namespace {

__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kRouteWaves = 4;

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

// One workgroup per token: its four wavefronts compute the keys (the double
// precision sigmoid is the costly part) into LDS, then the first wavefront
// selects.
__global__ __launch_bounds__(256) void route_reg_kernel(
    const float* __restrict__ logits, int64_t ld, const float* __restrict__ bias, int T, int E,
    int K, float scaling, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  __shared__ uint32_t keys_s[64 * kRegExpertsPerLane];
  const int t = blockIdx.x;
  const float* row = logits + (size_t)t * ld;
  for (int e = threadIdx.x; e < E; e += 256)
    keys_s[e] = ordered_key(sigmoid_score(row[e]) + (bias ? bias[e] : 0.0f));
  __syncthreads();
  if (threadIdx.x >= 64) return;                     // whole wavefronts leave
  const int lane = threadIdx.x;
  uint32_t key[kRegExpertsPerLane];
  uint32_t avail = 0;                                // bit j: expert lane + 64 j not yet taken
#pragma unroll
  for (int j = 0; j < kRegExpertsPerLane; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? keys_s[e] : 0u;
    avail |= (e < E ? 1u : 0u) << j;
  }
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t best = 0, best_e = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < kRegExpertsPerLane; ++j) {
      const bool take = ((avail >> j) & 1u) && (best_e == 0xFFFFFFFFu || key[j] > best);
      best = take ? key[j] : best;
      best_e = take ? (uint32_t)(lane + 64 * j) : best_e;
    }
    const uint32_t m = wave_max_u32(best);
    const uint32_t win = wave_min_u32(best == m ? best_e : 0xFFFFFFFFu);   // < E: K <= E
    if ((int)(win & 63) == lane) avail &= ~(1u << (win >> 6));
    if (lane == k) my_id = (int)win;
  }
  my_id = (my_id >= 0 && my_id < E) ? my_id : 0;
  float my_s = lane < K ? sigmoid_score(row[my_id]) : 0.0f;
  double total = 0.0;
  for (int k = 0; k < K; ++k) total += (double)__shfl(my_s, k);   // left to right
  if (lane < K) {
    topk_idx[(size_t)t * K + lane] = my_id;
    topk_w[(size_t)t * K + lane] = (float)(((double)my_s / total) * (double)scaling);
  }
}

__global__ __launch_bounds__(64 * kRouteWaves) void route_kernel(
    const float* __restrict__ logits, int64_t ld, const float* __restrict__ bias, int T, int E,
    int K, float scaling, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  extern __shared__ float lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteWaves + wave;
  float* key = lds + (size_t)wave * E;
  const float* row = logits + (size_t)(t < T ? t : 0) * ld;
  if (t < T) {
    for (int e = lane; e < E; e += 64) key[e] = sigmoid_score(row[e]) + (bias ? bias[e] : 0.0f);
  }
  __syncthreads();
  if (t >= T) return;

  uint64_t last = ~0ull;
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;
    for (int e = lane; e < E; e += 64) {
      uint64_t p = ((uint64_t)ordered_key(key[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
      best = (p < last && p > best) ? p : best;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      uint64_t o = __shfl_xor(best, off);
      best = o > best ? o : best;
    }
    last = best;
    if (lane == k) my_id = (int)(0xFFFFFFFFu - (uint32_t)best);
  }
  my_id = (my_id >= 0 && my_id < E) ? my_id : 0;   // K <= E always finds K experts
  float my_s = lane < K ? sigmoid_score(row[my_id]) : 0.0f;
  double total = 0.0;
  for (int k = 0; k < K; ++k) total += (double)__shfl(my_s, k);   // left to right
  if (lane < K) {
    topk_idx[(size_t)t * K + lane] = my_id;
    topk_w[(size_t)t * K + lane] = (float)(((double)my_s / total) * (double)scaling);
  }
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t ld, const float* bias, int T, int E, int K,
                        float scaling, int32_t* idx, float* w, hipStream_t stream) {
  int blocks = (T + kRouteWaves - 1) / kRouteWaves;
  if (E <= 64 * kRegExpertsPerLane) {
    hipLaunchKernelGGL(route_reg_kernel, dim3(T), dim3(256), 0, stream, logits, ld, bias, T, E, K,
                       scaling, idx, w);
    return hipGetLastError();
  }
  size_t lds = sizeof(float) * (size_t)E * kRouteWaves;
  hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(64 * kRouteWaves), lds, stream, logits, ld,
                     bias, T, E, K, scaling, idx, w);
  return hipGetLastError();
}

}  // namespace mi355moe
