// Prefill-shaped FC1 / FC2: LDS-staged tiles for MFMA operand reuse.
//
// Same method as the decode-shaped kernel (page 1, "Serving 调用链": grouped
// GEMM1 -> gated activation -> GEMM2; "真实 checkpoint 契约": [gate; up] halves,
// SiTU(4, 25); page 5: w13 / w2 and scale layouts), tiled for many rows per
// expert:
//   * a workgroup (8 wavefronts) computes up to 128 grouped rows of one expert
//     against 256 weight rows; wavefront (th, rq) owns token rows
//     [64 th, 64 th + 64) and weight unit rq (64 rows: for FC1 gate rows
//     [c, c+32) with up rows [I+c, I+c+32));
//   * K advances in 256-wide stages staged through LDS (two buffers, one
//     barrier per stage): the weight slice (256 rows x 128 bytes), the token
//     slice (128 rows x 256 bytes) and both operands' scale bytes; the next
//     stage's global loads are in flight while the current stage's MFMAs issue;
//   * 16-byte LDS chunks are XOR-swizzled by the row's low 3 bits so the eight
//     lanes served together read eight different bank groups;
//   * tiles are variable height: the last tile of an expert holds the rest of
//     its rows and wavefronts skip empty 16-row sub-tiles;
//   * persistent grid: each XCD walks a contiguous range of work items
//     (band of `band` column groups, tile, column group), so the tiles of one
//     expert and the column groups of one tile run close together in that
//     XCD's L2.
#include "common.h"
#include "fc_common.h"
#include "launch.h"

namespace mi355moe {

namespace {

constexpr int kBM = 128;                    // token rows per tile
constexpr int kBN = 256;                    // weight rows per tile
constexpr int kKS = 256;                    // K per LDS stage
constexpr int kWBytes = kBN * kKS / 2;      // 32768: E2M1 weight slice
constexpr int kABytes = kBM * kKS;          // 32768: E4M3 token slice
constexpr int kWSBytes = kBN * (kKS / 32);  // 2048: weight scale bytes
constexpr int kASBytes = kBM * (kKS / 32);  // 1024: token scale bytes
constexpr int kStage = kWBytes + kABytes + kWSBytes + kASBytes;
constexpr int kThreads = 512;

// Global row of the expert's weight matrix held at LDS row r (0..255) of
// column group cg: FC1 unit u = 4 cg + r/64 pairs gate rows [32u, 32u+32)
// with up rows [I+32u, I+32u+32); FC2 takes output rows 256 cg + r.
template <bool FC1>
__device__ __forceinline__ int weight_row(int r, int cg, int I) {
  if (FC1) {
    const int u = cg * 4 + (r >> 6), blk = (r >> 4) & 3, lr = r & 15;
    return (blk < 2 ? 0 : I) + u * 32 + (blk & 1) * 16 + lr;
  }
  return cg * kBN + r;
}

template <bool FC1>
__global__ __launch_bounds__(kThreads) void fc_prefill_kernel(FcParams p, int n_cg, int band) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int th = wave >> 2, rq = wave & 3, g = lane >> 4, li = lane & 15;
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

    // Global -> LDS assignment.  Weights: chunk q = tid + 512 i (16 bytes) of
    // the 256 x 128-byte slice; tokens: chunk q of the 128 x 256-byte slice;
    // scales: threads 0..255 one weight row's 8 bytes, the rest one token
    // row's 8 bytes (threads 384..511 repeat 256..383).
    const uint8_t* wsrc[4];
    const uint8_t* asrc[4];
    int wdst[4], adst[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 64 * i, c = tid & 7;
      wsrc[i] = p.w + ((size_t)e * p.N + weight_row<FC1>(r, cg, p.I)) * (K / 2) + 16 * c;
      wdst[i] = r * 128 + 16 * (c ^ (r & 7));
      const int tok = (tid >> 4) + 32 * i, ca = tid & 15;
      const int row = row_begin + min(tok, n_valid - 1);
      const size_t src = FC1 ? (size_t)(p.gather[row] / p.top_k) : (size_t)row;
      asrc[i] = p.act + src * K + 16 * ca;
      adst[i] = kWBytes + tok * 256 + 16 * (ca ^ (tok & 7));
    }
    const uint8_t* ssrc;
    int sdst;
    if (tid < 256) {
      ssrc = p.w_s + ((size_t)e * p.N + weight_row<FC1>(tid, cg, p.I)) * (K / 32);
      sdst = kWBytes + kABytes + tid * 8;
    } else {
      const int tok = (tid - 256) & 127;
      const int row = row_begin + min(tok, n_valid - 1);
      const size_t src = FC1 ? (size_t)(p.gather[row] / p.top_k) : (size_t)row;
      ssrc = p.act_s + src * (K / 32);
      sdst = kWBytes + kABytes + kWSBytes + tok * 8;
    }

    v4i wreg[4], areg[4];
    uint2 sreg;
    auto load_global = [&](int s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wreg[i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wsrc[i] + (size_t)s * 128));
        areg[i] = *reinterpret_cast<const v4i*>(asrc[i] + (size_t)s * 256);
      }
      sreg = *reinterpret_cast<const uint2*>(ssrc + (size_t)s * 8);
    };
    auto store_lds = [&](int buf) {
      uint8_t* base = lds + buf * kStage;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<v4i*>(base + wdst[i]) = wreg[i];
        *reinterpret_cast<v4i*>(base + adst[i]) = areg[i];
      }
      *reinterpret_cast<uint2*>(base + sdst) = sreg;
    };

    const int nsub = max(0, min(4, (n_valid - th * 64 + 15) >> 4));
    v4f acc[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int bk = 0; bk < 4; ++bk) acc[tt][bk] = v4f{0.f, 0.f, 0.f, 0.f};

    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int s = 0; s < n_stages; ++s) {
      const bool more = s + 1 < n_stages;
      if (more) load_global(s + 1);
      const uint8_t* W = lds + (s & 1) * kStage;
      const uint8_t* A = W + kWBytes;
      const int* WS = reinterpret_cast<const int*>(A + kABytes);
      const int* AS = reinterpret_cast<const int*>(A + kABytes + kWSBytes);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // Slice j = K [256 s + 128 j, +128): slot b is MX block 8 s + 4 j + b.
        v4i wv[4];
        int wsc[4];
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
          const int r = rq * 64 + bk * 16 + li;
          wv[bk] = *reinterpret_cast<const v4i*>(W + r * 128 + 16 * ((4 * j + g) ^ (li & 7)));
          wsc[bk] = WS[r * 2 + j] >> (8 * g);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (tt < nsub) {
            const int tok = th * 64 + tt * 16 + li;
            const uint8_t* arow = A + tok * 256;
            const v4i lo = *reinterpret_cast<const v4i*>(arow + 16 * ((8 * j + g) ^ (li & 7)));
            const v4i hi = *reinterpret_cast<const v4i*>(arow + 16 * ((8 * j + 4 + g) ^ (li & 7)));
            const int asc = AS[tok * 2 + j] >> (8 * g);
#pragma unroll
            for (int bk = 0; bk < 4; ++bk)
              acc[tt][bk] = mfma_w4a8<0>(wv[bk], lo, hi, acc[tt][bk], wsc[bk], asc);
          }
        }
      }
      if (more) store_lds((s + 1) & 1);
      __syncthreads();
    }

#pragma unroll
    for (int tt = 0; tt < 4; ++tt) pin_acc(acc[tt]);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (tt < nsub) {
        const int t_in = th * 64 + tt * 16 + li;
        store_subtile<FC1>(p, acc[tt], row_begin + t_in, t_in < n_valid, cg * 4 + rq, g);
      }
    }
  }
}

}  // namespace

bool prefill_shape_ok(int K, int N_cols, bool fc1) {
  return K % kKS == 0 && (fc1 ? N_cols % 128 == 0 : N_cols % kBN == 0);
}

hipError_t launch_fc_prefill(bool fc1, const FcParams& prm, int n_wg, hipStream_t stream) {
  const int n_cg = fc1 ? prm.I / 128 : prm.N / kBN;
  const int band = 4;
  if (fc1)
    hipLaunchKernelGGL((fc_prefill_kernel<true>), dim3(n_wg), dim3(kThreads), 0, stream, prm, n_cg, band);
  else
    hipLaunchKernelGGL((fc_prefill_kernel<false>), dim3(n_wg), dim3(kThreads), 0, stream, prm, n_cg, band);
  return hipGetLastError();
}

}  // namespace mi355moe
