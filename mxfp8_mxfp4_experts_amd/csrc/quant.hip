// a2: MXFP8 quantisation of bf16 activations.
//
// Page 5 (pre-dispatch step): absmax per 32 elements -> UE8M0 scale -> E4M3
// payload; page 1 ("NaN/Inf decision record"): the conversion saturates to a
// finite value and never emits the 0xFF scale.  The scale is the smallest
// power of two that keeps the group's absmax within 448, so nothing clips.
//
// Four lanes share a 32-element group: each lane loads 8 bf16 (16 bytes), the
// group absmax is two lane-xor max steps, and each lane writes its 8 E4M3
// bytes (by the hardware scaled conversion where the group is finite); the
// first lane of the group writes the scale byte.
#include "common.h"
#include "launch.h"
#include "quant_dev.h"

namespace mi355moe {

namespace {

// One workgroup per row: lane i takes pieces i, i + 256, ... (groups of four
// consecutive pieces stay in one wavefront, and H / 8 is a multiple of 4, so
// a group's lanes are active together).
__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ x, int64_t ld,
                                                    int H, uint8_t* __restrict__ xq,
                                                    uint8_t* __restrict__ xs) {
  const int t = blockIdx.x, per_row = H / 8;
  for (int c = threadIdx.x; c < per_row; c += 256) quant_row_piece(x, ld, H, xq, xs, t, c, true);
}

}  // namespace

hipError_t launch_quant(const uint16_t* x, int64_t ld, int T, int H, uint8_t* xq, uint8_t* xs,
                        hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_kernel, dim3(T), dim3(256), 0, stream, x, ld, H, xq, xs);
  return hipGetLastError();
}

}  // namespace mi355moe
