// Test-only probe kernels (not part of the library): they run single device
// functions of the FC kernels on inputs the tests choose, so the tests can
// measure the hardware arithmetic those functions rely on against exact
// float64 values:
//   * probe_mfma_w4a8: the block-scaled 16x16x128 MFMA wrapper (E2M1 weights
//     x E4M3 tokens, E8M0 scales per 32 K) accumulated over K as the FC
//     kernels do, raw float32 accumulators out;
//   * probe_situ: the FC1 epilogue's float32 SiTU (in pairs, as there);
//   * probe_e4m3_scaled: the hardware scaled E4M3 conversion (FC1 epilogue,
//     activation quantisation) next to the library's integer encoder.
// Every launch covers exactly the elements the host sizes describe.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../mxfp8_mxfp4_experts_amd/csrc/common.h"
#include "../../mxfp8_mxfp4_experts_amd/csrc/fc_common.h"

using namespace mi355moe;

namespace {

// One wavefront per 16-row weight tile: out[16 tile + row][token] for 16
// tokens, K in 128-K slices in natural order (the checkpoint layout's
// operand reads of the decode-shaped FC kernel).
__global__ __launch_bounds__(64) void mfma_probe_kernel(const uint8_t* __restrict__ w,
                                                        const uint8_t* __restrict__ ws,
                                                        const uint8_t* __restrict__ a,
                                                        const uint8_t* __restrict__ as, int K,
                                                        float* __restrict__ out) {
  const int lane = threadIdx.x, g = lane >> 4, li = lane & 15;
  const size_t row = (size_t)blockIdx.x * 16 + li;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < K / 128; ++s) {
    const v4i wv = *reinterpret_cast<const v4i*>(w + row * (K / 2) + (size_t)s * 64 + 16 * g);
    const int wsv = *reinterpret_cast<const int*>(ws + row * (K / 32) + 4 * s) >> (8 * g);
    const uint8_t* ap = a + (size_t)li * K + (size_t)s * 128 + 16 * g;
    const v4i alo = *reinterpret_cast<const v4i*>(ap);
    const v4i ahi = *reinterpret_cast<const v4i*>(ap + 64);
    const int asv = *reinterpret_cast<const int*>(as + (size_t)li * (K / 32) + 4 * s) >> (8 * g);
    acc = mfma_w4a8<0>(wv, alo, ahi, acc, wsv, asv);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) out[((size_t)blockIdx.x * 16 + 4 * g + r) * 16 + li] = acc[r];
}

// Thread i computes elements 2i and 2i + 1 as one pair (the epilogue's
// shared reciprocal), with the alpha = 4 shortcut where it applies.
__global__ __launch_bounds__(256) void situ_probe_kernel(const float* __restrict__ gv,
                                                         const float* __restrict__ uv, int n2,
                                                         float alpha, float beta,
                                                         float* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n2) return;
  const SituConst c = situ_const(alpha, beta);
  float v0, v1;
  if (c.a4)
    situ2<true>(gv[2 * i], uv[2 * i], gv[2 * i + 1], uv[2 * i + 1], c, v0, v1);
  else
    situ2<false>(gv[2 * i], uv[2 * i], gv[2 * i + 1], uv[2 * i + 1], c, v0, v1);
  out[2 * i] = v0;
  out[2 * i + 1] = v1;
}

// Thread i converts x[4i .. 4i+3] at scale 2^e[i] (a normal power of two).
__global__ __launch_bounds__(256) void e4m3_probe_kernel(const float* __restrict__ x,
                                                         const int* __restrict__ e, int n4,
                                                         uint32_t* __restrict__ hw,
                                                         uint32_t* __restrict__ ref) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const int ex = e[i];
  const float s = __uint_as_float((uint32_t)(ex + 127) << 23);
  const float* p = x + 4 * (size_t)i;
  hw[i] = e4m3x4_scaled(p[0], p[1], p[2], p[3], s);
  uint32_t q = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) q |= e4m3_encode(ldexpf(p[j], -ex)) << (8 * j);
  ref[i] = q;
}

int check(hipError_t e) { return e == hipSuccess ? 0 : 1; }

}  // namespace

extern "C" {

// w [16 n_tiles, K/2], ws [16 n_tiles, K/32], a [16, K], as [16, K/32] ->
// out float [16 n_tiles, 16].  K a multiple of 128.
int probe_mfma_w4a8(const uint8_t* w, const uint8_t* ws, const uint8_t* a, const uint8_t* as,
                    int n_tiles, int K, float* out, hipStream_t stream) {
  if (n_tiles <= 0 || K <= 0 || K % 128 != 0) return 2;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_tiles), dim3(64), 0, stream, w, ws, a, as, K, out);
  return check(hipGetLastError());
}

// n even.
int probe_situ(const float* g, const float* u, int n, float alpha, float beta, float* out,
               hipStream_t stream) {
  if (n <= 0 || n % 2 != 0) return 2;
  const int n2 = n / 2;
  hipLaunchKernelGGL(situ_probe_kernel, dim3((n2 + 255) / 256), dim3(256), 0, stream, g, u, n2,
                     alpha, beta, out);
  return check(hipGetLastError());
}

// x float [4 n4], e int [n4] in [-126, 127] -> hw, ref uint32 [n4] (four codes each).
int probe_e4m3_scaled(const float* x, const int* e, int n4, uint32_t* hw, uint32_t* ref,
                      hipStream_t stream) {
  if (n4 <= 0) return 2;
  hipLaunchKernelGGL(e4m3_probe_kernel, dim3((n4 + 255) / 256), dim3(256), 0, stream, x, e, n4,
                     hw, ref);
  return check(hipGetLastError());
}

}  // extern "C"
