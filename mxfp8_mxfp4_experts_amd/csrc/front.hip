// a1 + a2 + a3 in one launch, for decode-sized batches (page 1, "Serving call
// chain": routing, activation quantisation and the expert grouping run before
// the expert GEMMs; the fixed launch costs of these small steps are a visible
// share of a decode step).
//
// Workgroup 0 routes every token and then groups the routes: its sixteen
// wavefronts first compute all T x E selection keys into LDS, then wavefront
// t selects token t's experts (select_topk_wave, exactly as the routing
// kernel does), keeping the ids in LDS, and after a barrier the whole
// workgroup runs the single-workgroup grouping (permute_block) on them.  The
// other workgroups quantise the activations meanwhile (quant_piece), so the
// launch takes about as long as the routing alone.  The results are the bytes
// the three separate calls produce.
#include "common.h"
#include "launch.h"
#include "permute_dev.h"
#include "quant_dev.h"
#include "route_dev.h"

namespace mi355moe {

namespace {

__global__ __launch_bounds__(kPermThreads) void front_kernel(
    const float* __restrict__ logits, int64_t ld, const float* __restrict__ bias, int T, int E,
    int K, float scaling, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    const uint16_t* __restrict__ x, int64_t ld_x, int H, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ xs, int offset, int E_local, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ sorted_route, int32_t* __restrict__ route_row,
    int32_t* __restrict__ tile_prefix) {
  if (blockIdx.x > 0) {
    quant_piece(x, ld_x, T, H, xq, xs, (int64_t)(blockIdx.x - 1) * kPermThreads + threadIdx.x);
    return;
  }
  extern __shared__ __attribute__((aligned(16))) int lds_i[];   // 16-byte aligned base
  uint32_t* keys = reinterpret_cast<uint32_t*>(lds_i);   // [T][E]
  int* ids = lds_i + T * E;                              // [T * K]
  int* cnt = ids + T * K;                                // [E_local]
  int* cursor = cnt + E_local;                           // [E_local]
  // [T][64] selection candidates, 8-byte aligned after the int arrays
  uint64_t* cand = reinterpret_cast<uint64_t*>(lds_i + ((T * E + T * K + 2 * E_local + 1) & ~1));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Up to 16 keys per thread (T * E <= 16 * 1024): all of a thread's logits
  // and biases are loaded before its first sigmoid, so their latencies
  // overlap instead of adding up.
  {
    constexpr int kKeysPerThread = 16;
    float lv[kKeysPerThread], bv[kKeysPerThread];
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
      const int i = tid + j * kPermThreads;
      const int t = i / E, e = i - t * E;
      lv[j] = i < T * E ? logits[(size_t)t * ld + e] : 0.0f;
      bv[j] = i < T * E && bias ? bias[e] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
      const int i = tid + j * kPermThreads;
      if (i < T * E) keys[i] = ordered_key(sigmoid_score(lv[j]) + bv[j]);
    }
  }
  __syncthreads();
  if (wave < T) {
    int id;
    float w;
    select_topk_wave(keys + wave * E, logits + (size_t)wave * ld, E, K, scaling, lane,
                     cand + 64 * wave, id, w);
    if (lane < K) {
      topk_idx[(size_t)wave * K + lane] = id;
      topk_w[(size_t)wave * K + lane] = w;
      ids[wave * K + lane] = id;
    }
  }
  __syncthreads();
  // The grouping's LDS row of local experts reuses ids: each route's entry
  // is read, then overwritten, by the same thread.
  permute_block([&](int r) { return ids[r]; }, T * K, offset, E_local, expert_offsets,
                sorted_route, route_row, tile_prefix, cnt, cursor, ids, nullptr);
}

// a2 + a3 for given top-k ids: workgroup 0 groups the routes (the
// single-workgroup grouping, as permute_kernel), the others quantise.
__global__ __launch_bounds__(kPermThreads) void quant_permute_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, int T, int H, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ xs, const int32_t* __restrict__ idx, int R, int offset, int E_local,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_route,
    int32_t* __restrict__ route_row, int32_t* __restrict__ tile_prefix) {
  if (blockIdx.x > 0) {
    quant_piece(x, ld_x, T, H, xq, xs, (int64_t)(blockIdx.x - 1) * kPermThreads + threadIdx.x);
    return;
  }
  extern __shared__ __attribute__((aligned(16))) int lds_i[];
  permute_block([&](int r) { return idx[r]; }, R, offset, E_local, expert_offsets, sorted_route,
                route_row, tile_prefix, lds_i, lds_i + E_local, lds_i + 2 * E_local,
                E_local <= kPermWaveTableExperts ? lds_i + 2 * E_local + R : nullptr);
}

size_t front_lds_bytes(int T, int E, int K, int E_local) {
  return sizeof(int) * ((((size_t)T * E + (size_t)T * K + 2 * (size_t)E_local + 1) & ~(size_t)1) +
                        2 * 64 * (size_t)T);
}

}  // namespace

bool front_fusable(int T, int E, int K, int E_local) {
  return T >= 1 && T <= kPermWaves && E <= 64 * kRegExpertsPerLane &&
         front_lds_bytes(T, E, K, E_local) <= 64 * 1024;
}

hipError_t launch_front(const float* logits, int64_t ld, const float* bias, int T, int E, int K,
                        float scaling, int32_t* topk_idx, float* topk_w, const uint16_t* x,
                        int64_t ld_x, int H, uint8_t* xq, uint8_t* xs, int offset, int E_local,
                        int32_t* offs, int32_t* sorted_route, int32_t* route_row,
                        int32_t* tile_prefix, hipStream_t stream) {
  const int64_t pieces = (int64_t)T * (H / 8);
  const int blocks = 1 + (int)((pieces + kPermThreads - 1) / kPermThreads);
  hipLaunchKernelGGL(front_kernel, dim3(blocks), dim3(kPermThreads),
                     front_lds_bytes(T, E, K, E_local), stream, logits, ld, bias, T, E, K, scaling,
                     topk_idx, topk_w, x, ld_x, H, xq, xs, offset, E_local, offs, sorted_route,
                     route_row, tile_prefix);
  return hipGetLastError();
}

bool quant_permute_fusable(int64_t R) { return R >= 1 && R <= kPermSingle; }

hipError_t launch_quant_permute(const uint16_t* x, int64_t ld_x, int T, int H, uint8_t* xq,
                                uint8_t* xs, const int32_t* idx, int R, int offset, int E_local,
                                int32_t* offs, int32_t* sorted_route, int32_t* route_row,
                                int32_t* tile_prefix, hipStream_t stream) {
  // LDS of the single-workgroup grouping (as launch_permute sizes it).
  const size_t table = E_local <= kPermWaveTableExperts ? (size_t)kPermWaves * E_local : 0;
  const size_t lds = sizeof(int) * (2 * (size_t)E_local + (size_t)R + table);
  const int64_t pieces = (int64_t)T * (H / 8);
  const int64_t blocks = 1 + (pieces + kPermThreads - 1) / kPermThreads;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quant_permute_kernel, dim3((unsigned)blocks), dim3(kPermThreads), lds, stream,
                     x, ld_x, T, H, xq, xs, idx, R, offset, E_local, offs, sorted_route, route_row,
                     tile_prefix);
  return hipGetLastError();
}

}  // namespace mi355moe
