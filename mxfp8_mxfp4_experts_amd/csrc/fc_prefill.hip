// Prefill-shaped FC1 / FC2: LDS-staged tiles for MFMA operand reuse.
//
// Same method as the decode-shaped kernel (page 1, "Serving 调用链": grouped
// GEMM1 -> gated activation -> GEMM2; "真实 checkpoint 契约": [gate; up] halves,
// SiTU(4, 25); page 5: w13 / w2 and scale layouts), tiled for many rows per
// expert:
//   * a workgroup (8 wavefronts) computes up to 128 grouped rows of one expert
//     against 512 weight rows; wavefront (th, rg) owns token rows
//     [64 th, 64 th + 64) and weight rows [128 rg, 128 rg + 128) = two units
//     (FC1 unit: gate rows [c, c+32) with up rows [I+c, I+c+32));
//   * K advances in 128-wide stages.  Three LDS buffers hold the weight slice
//     (512 rows x 64 bytes), the token slice (128 rows x 128 bytes) and both
//     operands' scale bytes.  They are filled by direct global -> LDS loads
//     (global_load_lds_dwordx4), two stages ahead of the MFMAs, with no
//     staging registers; every wavefront issues exactly 8 such loads per
//     stage, so "s_waitcnt vmcnt(8)" leaves only the next stage in flight;
//   * 16-byte LDS chunks are XOR-swizzled (weights by row bits 1..2, tokens by
//     row bits 0..2) so the eight lanes served together hit eight bank
//     groups; a lane's load source is permuted to match, since each load
//     writes 1 KB of LDS in lane order;
//   * tiles are variable height: the last tile of an expert holds the rest of
//     its rows and wavefronts skip empty 16-row sub-tiles;
//   * persistent grid: each XCD walks a contiguous range of work items
//     (band of `band` column groups, tile, column group), so the tiles of one
//     expert and the column groups of one tile run close together in that
//     XCD's L2.
#include "common.h"
#include "fc_common.h"
#include "launch.h"
#include "tiled.h"

namespace mi355moe {

namespace {

constexpr int kBM = 128;                    // token rows per tile
constexpr int kBN = 512;                    // weight rows per tile (8 units)
constexpr int kKS = 128;                    // K per stage
constexpr int kWBytes = kBN * kKS / 2;      // 32768: E2M1 weight slice
constexpr int kABytes = kBM * kKS;          // 16384: E4M3 token slice
constexpr int kWSBytes = kBN * 4;           // 2048: one scale dword per weight row
constexpr int kASBytes = kBM * 4;           // 512: one scale dword per token row
constexpr int kOffA = kWBytes;
constexpr int kOffWS = kOffA + kABytes;
constexpr int kOffAS = kOffWS + kWSBytes;
constexpr int kStage = kOffAS + kASBytes;   // 51712
constexpr int kNumBuf = 3;
constexpr int kThreads = 512;

static_assert(kBN == kTileRows && kKS == kTileK && kWBytes == kTileBytes, "tile shape");

// Global row of the expert's weight matrix held at LDS row r (0..511) of
// column group cg (the same assignment as the tiled layout).
template <bool FC1>
__device__ __forceinline__ int weight_row(int r, int cg, int I) {
  return tiled_row<FC1>(r, cg, I);
}

__device__ __forceinline__ void dma16(const void* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
}

// TILED: p.w / p.w_s hold the tiled layout (tiled.h), else the checkpoint
// layout.
template <bool FC1, bool TILED>
__global__ __launch_bounds__(kThreads) void fc_prefill_kernel(FcParams p, int n_cg, int band) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kNumBuf * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wavefront
  const int th = wave >> 2, rg = wave & 3, g = lane >> 4, li = lane & 15;
  const int K = p.K;
  const int n_stages = K / kKS;
  const int* prefix = p.tile_prefix;
  const int n_tiles = prefix[p.E_local];
  const int n_bands = (n_cg + band - 1) / band;
  const int per_band = n_tiles * band;
  const int n_items = n_bands * per_band;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
  const int item_lo = (int)((int64_t)n_items * xcd / 8);
  const int item_hi = (int)((int64_t)n_items * (xcd + 1) / 8);

  for (int item = item_lo + slot; item < item_hi; item += per_xcd) {
    const int bnd = item / per_band, rem = item - bnd * per_band;
    const int tile = rem / band, cg = bnd * band + rem % band;
    if (cg >= n_cg) continue;
    const int e = find_expert(prefix, p.E_local, tile);
    const int row_begin = p.expert_offsets[e] + (tile - prefix[e]) * kBM;
    const int n_valid = min(p.expert_offsets[e + 1] - row_begin, kBM);

    // DMA sources of this lane.  Weights: wave w fills rows 64w + 16i + l/4,
    // physical chunk l%4 <- logical chunk (l%4) ^ ((row >> 1) & 3) (in the
    // tiled layout that is simply the next 16 bytes).  Tokens: rows
    // 16w + 8i + l/8, physical chunk l%8 <- logical (l%8) ^ (row & 7).
    // Scales: weight rows 64w + l; token rows 64w + l for waves 0 and 1.
    const uint8_t* wsrc[4];
    const uint8_t* asrc[2];
    size_t wstep, wsstep;
    const uint8_t* wssrc;
    if (TILED) {
      const size_t blk0 = tiled_block(e, cg, 0, n_cg, n_stages);
#pragma unroll
      for (int i = 0; i < 4; ++i) wsrc[i] = p.w + blk0 * kTileBytes + (4 * wave + i) * 1024 + 16 * lane;
      wssrc = p.w_s + blk0 * kTileScaleBytes + (64 * wave + lane) * 4;
      wstep = kTileBytes;
      wsstep = kTileScaleBytes;
    } else {
      const int wc = (lane & 3) ^ ((lane >> 3) & 3);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 64 * wave + 16 * i + (lane >> 2);
        wsrc[i] = p.w + ((size_t)e * p.N + weight_row<FC1>(r, cg, p.I)) * (K / 2) + 16 * wc;
      }
      wssrc = p.w_s + ((size_t)e * p.N + weight_row<FC1>(64 * wave + lane, cg, p.I)) * (K / 32);
      wstep = 64;
      wsstep = 4;
    }
    const int ac = (lane & 7) ^ ((lane >> 3) & 7);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tok = 16 * wave + 8 * i + (lane >> 3);
      const int row = row_begin + min(tok, n_valid - 1);
      const size_t src = FC1 ? (size_t)(p.gather[row] / p.top_k) : (size_t)row;
      asrc[i] = p.act + src * K + 16 * ac;
    }
    const uint8_t* assrc;
    {
      const int tok = 64 * (wave & 1) + lane;
      const int row = row_begin + min(tok, n_valid - 1);
      const size_t src = FC1 ? (size_t)(p.gather[row] / p.top_k) : (size_t)row;
      assrc = p.act_s + src * (K / 32);
    }
    const bool loads_act_scales = wave < 2;
    auto issue = [&](int s) {
      uint8_t* base = lds + (s % kNumBuf) * kStage;
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(wsrc[i] + (size_t)s * wstep, base + wave * 4096 + i * 1024);
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(asrc[i] + (size_t)s * 128, base + kOffA + wave * 2048 + i * 1024);
      dma4(wssrc + (size_t)s * wsstep, base + kOffWS + wave * 256);
      if (loads_act_scales) dma4(assrc + (size_t)s * 4, base + kOffAS + wave * 256);
    };

    const int nsub = max(0, min(4, (n_valid - th * 64 + 15) >> 4));
    v4f acc[4][2][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int uu = 0; uu < 2; ++uu)
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) acc[tt][uu][bk] = v4f{0.f, 0.f, 0.f, 0.f};

    issue(0);
    if (n_stages > 1) issue(1);
    for (int s = 0; s < n_stages; ++s) {
      // This wavefront's loads of stage s are done once at most the next
      // stage's remain (8 loads per stage for waves 0 and 1, 7 for the
      // others); the barrier extends that to every wavefront and also means
      // everyone has finished stage s - 1, whose buffer the loads of stage
      // s + 2 now overwrite.
      if (s + 1 < n_stages) {
        if (loads_act_scales) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      asm volatile("s_barrier" ::: "memory");
      if (s + 2 < n_stages) issue(s + 2);
      const uint8_t* W = lds + (s % kNumBuf) * kStage;
      const uint8_t* A = W + kOffA;
      const int* WS = reinterpret_cast<const int*>(W + kOffWS);
      const int* AS = reinterpret_cast<const int*>(W + kOffAS);
      // Slice K [128 s, +128): slot b is MX block 4 s + b.
      v4i wv[2][4];
      int wsc[2][4];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu)
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
          const int r = 128 * rg + 64 * uu + 16 * bk + li;
          wv[uu][bk] = *reinterpret_cast<const v4i*>(W + r * 64 + 16 * (g ^ ((li >> 1) & 3)));
          wsc[uu][bk] = WS[r] >> (8 * g);
        }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (tt < nsub) {
          const int tok = th * 64 + tt * 16 + li;
          const uint8_t* arow = A + tok * 128;
          const v4i lo = *reinterpret_cast<const v4i*>(arow + 16 * (g ^ (li & 7)));
          const v4i hi = *reinterpret_cast<const v4i*>(arow + 16 * ((4 + g) ^ (li & 7)));
          const int asc = AS[tok] >> (8 * g);
#pragma unroll
          for (int uu = 0; uu < 2; ++uu)
#pragma unroll
            for (int bk = 0; bk < 4; ++bk)
              acc[tt][uu][bk] = mfma_w4a8<0>(wv[uu][bk], lo, hi, acc[tt][uu][bk], wsc[uu][bk], asc);
        }
      }
    }
    // Everyone is done with the LDS buffers before the next item refills them.
    asm volatile("s_barrier" ::: "memory");

#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      pin_acc(acc[tt][0]);
      pin_acc(acc[tt][1]);
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (tt < nsub) {
        const int t_in = th * 64 + tt * 16 + li;
#pragma unroll
        for (int uu = 0; uu < 2; ++uu)
          store_subtile<FC1>(p, acc[tt][uu], row_begin + t_in, t_in < n_valid,
                             cg * 8 + 2 * rg + uu, g);
      }
    }
  }
}

}  // namespace

bool prefill_shape_ok(const FcParams& prm, bool fc1) {
  // FC1: 256 intermediate columns (512 w13 rows) per tile; FC2: 512 output
  // columns.
  return prm.K % kKS == 0 && (fc1 ? prm.I % 256 == 0 : prm.N % kBN == 0);
}

hipError_t launch_fc_prefill(bool fc1, bool tiled, const FcParams& prm, int n_wg,
                             hipStream_t stream) {
  const int n_cg = fc1 ? prm.I / 256 : prm.N / kBN;
  const int band = 2;
  const dim3 grid(n_wg), block(kThreads);
  if (fc1 && tiled)
    hipLaunchKernelGGL((fc_prefill_kernel<true, true>), grid, block, 0, stream, prm, n_cg, band);
  else if (fc1)
    hipLaunchKernelGGL((fc_prefill_kernel<true, false>), grid, block, 0, stream, prm, n_cg, band);
  else if (tiled)
    hipLaunchKernelGGL((fc_prefill_kernel<false, true>), grid, block, 0, stream, prm, n_cg, band);
  else
    hipLaunchKernelGGL((fc_prefill_kernel<false, false>), grid, block, 0, stream, prm, n_cg, band);
  return hipGetLastError();
}

}  // namespace mi355moe
