// a2: MXFP8 quantisation of bf16 activations.
//
// Page 5 (pre-dispatch step): absmax per 32 elements -> UE8M0 scale -> E4M3
// payload; page 1 ("NaN/Inf decision record"): the conversion saturates to a
// finite value and never emits the 0xFF scale.  The scale is the smallest
// power of two that keeps the group's absmax within 448, so nothing clips.
//
// Four lanes share a 32-element group: each lane loads 8 bf16 (16 bytes), the
// group absmax is two lane-xor max steps, and each lane writes its 8 E4M3
// bytes; the first lane of the group writes the scale byte.
#include "common.h"
#include "launch.h"
#include "quant_dev.h"

namespace mi355moe {

namespace {

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ x, int64_t ld,
                                                    int T, int H, uint8_t* __restrict__ xq,
                                                    uint8_t* __restrict__ xs) {
  quant_piece(x, ld, T, H, xq, xs, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

}  // namespace

hipError_t launch_quant(const uint16_t* x, int64_t ld, int T, int H, uint8_t* xq, uint8_t* xs,
                        hipStream_t stream) {
  int64_t threads = (int64_t)T * (H / 8);
  int blocks = (int)((threads + 255) / 256);
  hipLaunchKernelGGL(quant_kernel, dim3(blocks), dim3(256), 0, stream, x, ld, T, H, xq, xs);
  return hipGetLastError();
}

}  // namespace mi355moe
