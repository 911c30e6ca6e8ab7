// Achievable-rate probes for the benchmark's roofline (not part of the layer
// library): a streaming HBM read and a register-only loop of the block-scaled
// MFMA the FC kernels issue.  Their rates are reported beside MI355X's
// published peaks (8 TB/s HBM; 5.0 PFLOP/s dense FP8-rate MFMA) as the
// achievable denominators on the box at hand, and the MFMA rate also gives
// the clock the box holds (8192 FLOP per CU and clock at the FP8 rate).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Each workgroup (4 wavefronts) streams one contiguous chunk of `chunk`
// 16-byte vectors, eight loads in flight per lane, and folds them into one
// word so the loads cannot be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const v4i* __restrict__ src,
                                                          int64_t chunk, int64_t n,
                                                          int* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * chunk;
  int acc = 0;
  for (int64_t i = base + threadIdx.x; i < base + chunk; i += 256 * 8) {
    v4i v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t k = i + (int64_t)j * 256;
      v[j] = k < n ? __builtin_nontemporal_load(src + k) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  if (acc == 0x7FFFFFFF) sink[blockIdx.x] = acc;   // practically never; keeps the loads
}

// Eight independent accumulator chains of 16x16x128 E2M1 x E4M3 MFMAs with
// E8M0 scales (the FC kernels' instruction), `iters` rounds.
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  v8i a = {lane, lane + 1, lane + 2, lane + 3, 0, 0, 0, 0};
  v8i b = {lane * 3, lane, 7, 9, 11, 13, 15, 17};
  v4f c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[j], 4, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  if (s == 1234.5f) sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from `src` once, split over `blocks`
// workgroups; `sink` holds at least `blocks` ints.
int rate_stream_read(const void* src, int64_t bytes, int blocks, int* sink, hipStream_t stream) {
  if (bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return 2;
  const int64_t n = bytes / 16;
  // Whole rounds of 256 lanes x 8 loads per chunk; loads past n are skipped.
  const int64_t chunk = ((n + blocks - 1) / blocks + 2047) / 2048 * 2048;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const v4i*>(src), chunk, n, sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// `blocks` workgroups of 4 wavefronts, each wavefront issuing 8 * iters
// MFMAs of 2 * 16 * 16 * 128 FLOP; `sink` holds at least 256 * blocks floats.
int rate_mfma(int blocks, int iters, float* sink, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0) return 2;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
