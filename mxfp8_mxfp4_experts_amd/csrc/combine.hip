// a8: top-k weighted combine of the FC2 rows (page 1, "Serving 调用链": the
// finalize step after GEMM2; "对称性约束": the non-fused, deterministic
// finalize).  out[t] = bf16 of the sum over kept slots k, in slot order, of
// w[t,k] * y[route_row[t,k]], accumulated in float32; masked and dropped
// slots contribute nothing, and a token with no kept slot gets zeros.  The
// FC2 rows arrive as fp16 with a power-of-two scale per 64 columns.  The
// fused atomic finalize adds the weighted rows in the FC2 epilogue instead
// and only needs the clear and bf16 passes at the end of this file.
#include "common.h"
#include "fc_common.h"
#include "launch.h"

namespace mi355moe {

namespace {

// out[t] = bf16( sum over kept k, in k order, of w[t,k] * y[route_row[t,k]] ),
// with y = fp16 row * 2^ye.  Workgroup b (one wavefront) covers columns
// [512 x, 512 x + 512) of token t = b / n_x (x = b % n_x), 8 per lane, so
// consecutive workgroups walk each token's row in order and, for H a multiple
// of 512, no lane idles; the token's route rows and weights are the same for
// the whole wavefront, so they are read with scalar loads and the masked slots
// are skipped by uniform branches (with few kept slots per token the per-lane
// copies of those reads were most of the work: EP-share combine 83 -> 54 us).
__global__ __launch_bounds__(64) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int8_t* __restrict__ ye, int H,
                                                      const int32_t* __restrict__ route_row,
                                                      const float* __restrict__ topk_w, int K,
                                                      uint16_t* __restrict__ out,
                                                      int64_t ld_out) {
  const int per_row = H / 8;
  const int n_x = (per_row + 64 - 1) / 64;
  const int t = blockIdx.x / n_x;
  const int c = (blockIdx.x - t * n_x) * 64 + threadIdx.x;
  if (c >= per_row) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // Slots in groups of 16: all route rows and weights of the group first,
  // then all row loads (independent, in flight together), then the sums in
  // slot order.
  for (int k0 = 0; k0 < K; k0 += 16) {
    int rr[16];
    float wk[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int k = k0 + j;
      rr[j] = k < K ? route_row[(size_t)t * K + k] : -1;
      wk[j] = k < K ? topk_w[(size_t)t * K + k] : 0.0f;
    }
    uint4 a[16];
    int ex[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      a[j] = uint4{0u, 0u, 0u, 0u};
      ex[j] = 0;
      if (rr[j] >= 0) {
        // Each row piece is read once: a non-temporal load.
        typedef unsigned int u4v __attribute__((ext_vector_type(4)));
        const u4v v = __builtin_nontemporal_load(
            reinterpret_cast<const u4v*>(y + (size_t)rr[j] * H + (size_t)c * 8));
        a[j] = uint4{v.x, v.y, v.z, v.w};
        ex[j] = ye[ye_index(rr[j], c >> 3, H / 64)];
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (rr[j] < 0) continue;
      const uint32_t h[4] = {a[j].x, a[j].y, a[j].z, a[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)(h[i] & 0xFFFF)), ex[j]);
        const float hi = ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)(h[i] >> 16)), ex[j]);
        acc[2 * i] = fmaf(wk[j], lo, acc[2 * i]);
        acc[2 * i + 1] = fmaf(wk[j], hi, acc[2 * i + 1]);
      }
    }
  }
  uint4 o;
  o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
  o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
  o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
  o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * ld_out + (size_t)c * 8) = o;
}

// Atomic combine, before FC2: the float [T, H] sums start at zero (a plain
// store kernel, so the call chain stays capturable without memset nodes).
// Each lane clears 4 floats; H is a multiple of 128.
__global__ __launch_bounds__(256) void acc_clear_kernel(float4* __restrict__ acc, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) acc[i] = float4{0.f, 0.f, 0.f, 0.f};
}

// Atomic combine, after FC2: out[t] = bf16_rne(acc[t]), 8 columns per lane.
__global__ __launch_bounds__(256) void acc_to_bf16_kernel(const float* __restrict__ acc, int H,
                                                          int64_t n8, uint16_t* __restrict__ out,
                                                          int64_t ld_out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t per_row = H / 8;
  const int64_t t = i / per_row, c = (i - t * per_row) * 8;
  const float4 a = *reinterpret_cast<const float4*>(acc + t * H + c);
  const float4 b = *reinterpret_cast<const float4*>(acc + t * H + c + 4);
  uint4 o;
  o.x = f32_to_bf16(a.x) | (f32_to_bf16(a.y) << 16);
  o.y = f32_to_bf16(a.z) | (f32_to_bf16(a.w) << 16);
  o.z = f32_to_bf16(b.x) | (f32_to_bf16(b.y) << 16);
  o.w = f32_to_bf16(b.z) | (f32_to_bf16(b.w) << 16);
  *reinterpret_cast<uint4*>(out + t * ld_out + c) = o;
}

}  // namespace

hipError_t launch_acc_clear(float* acc, int T, int H, hipStream_t stream) {
  const int64_t n4 = (int64_t)T * H / 4;
  if (n4 <= 0) return hipSuccess;
  const int64_t blocks = (n4 + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(acc_clear_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<float4*>(acc), n4);
  return hipGetLastError();
}

hipError_t launch_acc_to_bf16(const float* acc, int T, int H, uint16_t* out, int64_t ld_out,
                              hipStream_t stream) {
  const int64_t n8 = (int64_t)T * H / 8;
  if (n8 <= 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(acc_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, acc, H, n8,
                     out, ld_out);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y, const int8_t* ye, int H, const int32_t* route_row,
                          const float* topk_w, int T, int K, uint16_t* out, int64_t ld_out,
                          hipStream_t stream) {
  const int64_t blocks = (int64_t)T * ((H / 8 + 64 - 1) / 64);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(64), 0, stream, y, ye, H, route_row, topk_w, K,
                     out, ld_out);
  return hipGetLastError();
}

}  // namespace mi355moe
