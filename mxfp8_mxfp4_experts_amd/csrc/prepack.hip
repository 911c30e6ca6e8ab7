// One-time reordering of checkpoint-layout MXFP4 weights into the tiled
// layout (tiled.h).  One workgroup per (expert, column group, stage) block:
// 256 threads copy the block's 2048 sixteen-byte chunks and 512 scale dwords.
//
// w13 may arrive in one of three row orders (page 1, "真实 checkpoint 契约":
// the Kimi checkpoint keeps [gate; up] halves, the CUTLASS runner expects
// [up; gate] halves, the GPT-OSS loader interleaves gate and up rows; page 3:
// the de-interleave takes the even rows as gate and the odd rows as up).  The
// tiled layout always holds [gate; up] order, so the FC kernels are the same
// for all three.
#include "common.h"
#include "launch.h"
#include "tiled.h"

namespace mi355moe {

namespace {

// Source row of logical w13 row L ([gate; up] order: gate j = L < I, up j =
// L - I) in the given row order.
__device__ __forceinline__ int w13_source_row(int L, int I, int layout) {
  if (layout == 1) return L < I ? L + I : L - I;           // [up; gate]
  if (layout == 2) return L < I ? 2 * L : 2 * (L - I) + 1;  // gate j, up j, gate j+1, ...
  return L;                                                 // [gate; up]
}

template <bool FC1>
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t* __restrict__ w,
                                                      const uint8_t* __restrict__ ws, int N, int K,
                                                      int I, int n_cg, int layout,
                                                      uint8_t* __restrict__ tw,
                                                      uint8_t* __restrict__ tws) {
  const int n_st = K / kTileK;
  const int blk = blockIdx.x;
  const int s = blk % n_st, cg = (blk / n_st) % n_cg, e = blk / (n_st * n_cg);
  uint8_t* dst = tw + (size_t)blk * kTileBytes;
  for (int q = threadIdx.x; q < kTileBytes / 16; q += blockDim.x) {
    const int chunk = q >> 6, l = q & 63;
    const int r = 16 * chunk + (l >> 2);              // = 64 w + 16 i + l / 4
    const int c = (l & 3) ^ ((l >> 3) & 3);
    const int lr = tiled_row<FC1>(r, cg, I);
    const size_t row = (size_t)e * N + (FC1 ? w13_source_row(lr, I, layout) : lr);
    *reinterpret_cast<uint4*>(dst + (size_t)q * 16) =
        *reinterpret_cast<const uint4*>(w + row * (K / 2) + (size_t)s * 64 + 16 * c);
  }
  uint32_t* sdst = reinterpret_cast<uint32_t*>(tws + (size_t)blk * kTileScaleBytes);
  for (int r = threadIdx.x; r < kTileRows; r += blockDim.x) {
    const int lr = tiled_row<FC1>(r, cg, I);
    const size_t row = (size_t)e * N + (FC1 ? w13_source_row(lr, I, layout) : lr);
    sdst[r] = *reinterpret_cast<const uint32_t*>(ws + row * (K / 32) + (size_t)s * 4);
  }
}

}  // namespace

hipError_t launch_prepack(bool fc1, const uint8_t* w, const uint8_t* ws, int E_local, int N,
                          int K, int I, int layout, uint8_t* tw, uint8_t* tws,
                          hipStream_t stream) {
  const int n_cg = N / kTileRows, n_st = K / kTileK;
  const int64_t blocks = (int64_t)E_local * n_cg * n_st;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (fc1)
    hipLaunchKernelGGL((prepack_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream, w, ws,
                       N, K, I, n_cg, layout, tw, tws);
  else
    hipLaunchKernelGGL((prepack_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream, w,
                       ws, N, K, I, n_cg, 0, tw, tws);
  return hipGetLastError();
}

}  // namespace mi355moe
