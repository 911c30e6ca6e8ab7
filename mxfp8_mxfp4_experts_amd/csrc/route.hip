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
//    wavefront holds the keys of experts l, l + 64, ... in registers.  The
//    K-th largest of the lanes' own largest keys bounds the selected keys
//    from below; the keys that reach it (usually few) are sorted across the
//    wavefront (key descending, then expert ascending) and lane k takes the
//    k-th.  With more than 64 such keys (many ties) K rounds select instead:
//    each takes the lane's best remaining key, the wavefront maximum of those
//    (DPP row shifts and broadcasts), then the smallest expert index among
//    the lanes holding that maximum; the owning lane retires the winner.
//  * larger E: the keys sit in LDS and each round takes a wavefront arg-max
//    over a 64-bit key (ordered float key, then inverted expert index)
//    restricted to keys below the previous winner.
#include "common.h"
#include "launch.h"
#include "route_dev.h"

namespace mi355moe {

namespace {

constexpr int kRouteWaves = 4;

__global__ __launch_bounds__(256) void route_reg_kernel(
    const float* __restrict__ logits, int64_t ld, const float* __restrict__ bias, int T, int E,
    int K, float scaling, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  __shared__ uint32_t keys_s[64 * kRegExpertsPerLane];
  __shared__ uint64_t cand_s[64];
  const int t = blockIdx.x;
  const float* row = logits + (size_t)t * ld;
  for (int e = threadIdx.x; e < E; e += 256)
    keys_s[e] = ordered_key(sigmoid_score(row[e]) + (bias ? bias[e] : 0.0f));
  __syncthreads();
  if (threadIdx.x >= 64) return;                     // whole wavefronts leave
  const int lane = threadIdx.x;
  int id;
  float w;
  select_topk_wave(keys_s, row, E, K, scaling, lane, cand_s, id, w);
  if (lane < K) {
    topk_idx[(size_t)t * K + lane] = id;
    topk_w[(size_t)t * K + lane] = w;
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
