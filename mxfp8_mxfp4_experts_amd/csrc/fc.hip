// a4..a7: grouped FC1 (+ SiTU + requantisation) and FC2 (writing the per-route
// rows the combine sums) on the gfx950 block-scaled MFMA
// (V_MFMA_SCALE_F32_16X16X128_F8F6F4), for experts holding few grouped rows.
//
// Page 1, "Serving call chain": grouped GEMM1 -> gated activation -> GEMM2 ->
// finalize; "Real checkpoint contract": w13 = [gate; up] halves, SiTU(4, 25);
// page 5: w13 [E, 2I, H/2] + [E, 2I, H/32], w2 [E, H, I/2] + [E, H, I/32].
//
// MFMA operand layout (16x16x128, one wavefront; pinned by a one-hot probe of
// the instruction): A = weights in E2M1 (cbsz 4), B = activations in E4M3
// (blgp 0), out C[weight row][token].
//   * lane l works on A row / B column l % 16; g = l / 16 is its lane group;
//   * E2M1 operand: lane group g holds K [32g, 32g+32) as 16 bytes (low nibble
//     first);
//   * E4M3 operand: lane group g holds K [16g, 16g+16) in bytes 0..15 and
//     K [64+16g, 64+16g+16) in bytes 16..31;
//   * the scale byte of lane group b (selected by opsel) applies to
//     K [32b, 32b+32) of that lane's row (A) or column (B);
//   * C: lane l holds rows 4g .. 4g+3 of column l % 16.
// So with K in natural order, MX block b of a 128-K slice is scaled by lane
// group b on both operands, and each weight-load instruction reads 64
// contiguous bytes of each of 16 rows.
//
// Work decomposition: a workgroup (4 wavefronts) takes one tile of up to 32
// grouped rows of one expert (one or two 16-row subtiles) and a column group
// of 4 units; a unit (one wavefront) is 64 weight rows: for FC1, gate rows
// [c, c+32) with up rows [I+c, I+c+32), so SiTU and the 32-column
// requantisation group are local to the lanes that hold them; for FC2, output
// columns [h, h+64).  The expert of each tile comes from the grouping step's
// tile -> expert map.
#include "common.h"
#include "fc_common.h"
#include "launch.h"
#include "tiled.h"

namespace mi355moe {

namespace {

// 128-K slices per super-step: the operands of two super-steps are in
// registers at a time (about 120 VGPRs for two slices), which leaves room for
// two wavefronts per SIMD.
constexpr int kSJ = 2;

// Tile list of the decode-shaped kernel: 32-row tiles (tile prefix 0), whose
// tile -> expert map the grouping step writes after the prefixes.
constexpr int kDecodeTilePrefixIndex = 0;
constexpr int kDecodeTileRows = tile_rows(kDecodeTilePrefixIndex);
static_assert(kDecodeTileRows == 32, "two 16-row subtiles per tile");
static_assert(kDecodeTilePrefixIndex == kMapTileIndex, "tile map");

// Operands of one super-step (kSJ 128-K slices) for one wavefront.
template <int NT>
struct Stage {
  v4i w[4][kSJ];      // [row block][MFMA j]: 32 E2M1 weights of this lane
  int ws[4][kSJ];     // [row block][MFMA j]: the row's 4 scale bytes of slice j
  v4i alo[NT][kSJ];   // [token tile][MFMA j]: E4M3 K [16g, 16g+16) of the slice
  v4i ahi[NT][kSJ];   //                      E4M3 K [64+16g, 64+16g+16)
  int as[NT][kSJ];    // the token's 4 scale bytes of slice j
};

// Checkpoint layout: wp[bk] points at the lane's row + 16g, wsp[bk] at the
// row's scale bytes.  Tiled layout: wp[bk] points at the lane's 16 bytes in
// stage 0's block and wsp[bk] at the row's scale dword there; stage t adds t
// whole blocks.  STREAM: the weights are read once (the expert has a single
// tile), so they are loaded non-temporally and do not displace lines that
// other tiles will reuse; otherwise they stay cached for the expert's next
// tile.
template <bool STREAM>
__device__ __forceinline__ v4i load_weights(const v4i* p) {
  if (STREAM) return __builtin_nontemporal_load(p);
  return *p;
}

template <int NT, bool TILED, bool STREAM>
__device__ __forceinline__ void load_stage(Stage<NT>& st, const uint8_t* const* wp,
                                           const uint8_t* const* wsp, const uint8_t* const* ap,
                                           const uint8_t* const* asp, int S, int g) {
#pragma unroll
  for (int bk = 0; bk < 4; ++bk) {
    if (TILED) {
#pragma unroll
      for (int j = 0; j < kSJ; ++j) {
        st.w[bk][j] = load_weights<STREAM>(
            reinterpret_cast<const v4i*>(wp[bk] + (size_t)(kSJ * S + j) * kTileBytes));
        st.ws[bk][j] =
            *reinterpret_cast<const int*>(wsp[bk] + (size_t)(kSJ * S + j) * kTileScaleBytes);
      }
    } else {
      const v4i* src = reinterpret_cast<const v4i*>(wp[bk] + (size_t)S * 64 * kSJ);
#pragma unroll
      for (int j = 0; j < kSJ; ++j) {
        st.w[bk][j] = load_weights<STREAM>(src + 4 * j);
        st.ws[bk][j] = *reinterpret_cast<const int*>(wsp[bk] + (size_t)(kSJ * S + j) * 4);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const uint8_t* a = ap[tt] + (size_t)S * 128 * kSJ + 16 * g;
#pragma unroll
    for (int j = 0; j < kSJ; ++j) {
      st.alo[tt][j] = *reinterpret_cast<const v4i*>(a + 128 * j);
      st.ahi[tt][j] = *reinterpret_cast<const v4i*>(a + 128 * j + 64);
      st.as[tt][j] = *reinterpret_cast<const int*>(asp[tt] + (size_t)(kSJ * S + j) * 4);
    }
  }
}

template <int NT>
__device__ __forceinline__ void compute_stage(v4f (&acc)[NT][4], const Stage<NT>& st, int g) {
  const int sh = 8 * g;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
    for (int j = 0; j < kSJ; ++j) {
      const int asv = st.as[tt][j] >> sh;
#pragma unroll
      for (int bk = 0; bk < 4; ++bk)
        acc[tt][bk] = mfma_w4a8<0>(st.w[bk][j], st.alo[tt][j], st.ahi[tt][j], acc[tt][bk],
                                   st.ws[bk][j] >> sh, asv);
    }
  }
}

// The super-step loop over K / (128 kSJ) steps.  No branch inside the loop:
// the wait-count pass then lets the stage just loaded stay in flight while the
// other stage's MFMAs issue.  Tiled layout: the last one or two steps run
// after the loop, so no stage is loaded twice (the load path per CU is the
// bound, and the reload was one super-step in 14 for FC2).  Checkpoint layout
// (whose per-row pointers leave no registers for the peeled steps): the last
// iteration reloads the final stage when n_super is even.
template <int NT, bool TILED, bool STREAM>
__device__ __forceinline__ void super_steps(v4f (&acc)[NT][4], const uint8_t* const* wp,
                                            const uint8_t* const* wsp, const uint8_t* const* ap,
                                            const uint8_t* const* asp, int n_super, int g) {
  if (n_super <= 0) return;
  Stage<NT> st0, st1;
  load_stage<NT, TILED, STREAM>(st0, wp, wsp, ap, asp, 0, g);
  int S = 0;
  if constexpr (!TILED) {
    for (; S + 1 < n_super; S += 2) {
      load_stage<NT, TILED, STREAM>(st1, wp, wsp, ap, asp, S + 1, g);
      __builtin_amdgcn_sched_barrier(0);
      compute_stage<NT>(acc, st0, g);
      __builtin_amdgcn_sched_barrier(0);
      load_stage<NT, TILED, STREAM>(st0, wp, wsp, ap, asp, min(S + 2, n_super - 1), g);
      __builtin_amdgcn_sched_barrier(0);
      compute_stage<NT>(acc, st1, g);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (S < n_super) compute_stage<NT>(acc, st0, g);
    return;
  }
  for (; S + 2 < n_super; S += 2) {
    load_stage<NT, TILED, STREAM>(st1, wp, wsp, ap, asp, S + 1, g);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<NT>(acc, st0, g);
    __builtin_amdgcn_sched_barrier(0);
    load_stage<NT, TILED, STREAM>(st0, wp, wsp, ap, asp, S + 2, g);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<NT>(acc, st1, g);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (S + 1 < n_super) {
    load_stage<NT, TILED, STREAM>(st1, wp, wsp, ap, asp, S + 1, g);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<NT>(acc, st0, g);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<NT>(acc, st1, g);
  } else {
    compute_stage<NT>(acc, st0, g);
  }
}

// One tile of NT 16-row subtiles [row_begin, row_end) of expert e against
// column group cg (one unit per wavefront).  stream_w: the expert has this one
// tile, so its weights are read once and streamed past the caches.
template <bool FC1, int NT, bool TILED>
__device__ __forceinline__ void fc_tile(const FcParams& p, int e, int cg, int row_begin,
                                        int row_end, bool stream_w) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int u = cg * 4 + wave;
  if (u >= p.n_units) return;
  const int g = lane >> 4, li = lane & 15;
  const int K = p.K;

  int wrow[4];
  if (FC1) {
    const int c0 = u * 32;
    wrow[0] = c0 + li; wrow[1] = c0 + 16 + li; wrow[2] = p.I + c0 + li; wrow[3] = p.I + c0 + 16 + li;
  } else {
    const int h0 = u * 64;
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) wrow[bk] = h0 + 16 * bk + li;
  }
  const uint8_t* wp[4];
  const uint8_t* wsp[4];
  if (TILED) {
    // Unit u is rows [64 (u % 8), +64) of column group u / 8; block bk is its
    // 1 KB chunk 4 (u % 8) + bk, where row li's logical chunk g sits at
    // position 4 li + (g ^ ((li >> 1) & 3)).
    const int tcg = u >> 3, wu = u & 7;
    const size_t blk0 = tiled_block(e, tcg, 0, p.N / kTileRows, K / kTileK);
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
      wp[bk] = p.w + blk0 * kTileBytes + (4 * wu + bk) * 1024 + 16 * (4 * li + (g ^ ((li >> 1) & 3)));
      wsp[bk] = p.w_s + blk0 * kTileScaleBytes + (64 * wu + 16 * bk + li) * 4;
    }
  } else {
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
      const size_t r = (size_t)e * p.N + wrow[bk];
      wp[bk] = p.w + r * (K / 2) + 16 * g;
      wsp[bk] = p.w_s + r * (K / 32);
    }
  }
  const uint8_t* ap[NT];
  const uint8_t* asp[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    int row = min(row_begin + tt * 16 + li, row_end - 1);
    size_t src = FC1 ? (size_t)(p.gather[row] / p.top_k) : (size_t)row;
    ap[tt] = p.act + src * K;
    asp[tt] = p.act_s + src * (K / 32);
  }

  v4f acc[NT][4];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) acc[tt][bk] = v4f{0.f, 0.f, 0.f, 0.f};

  // Super-steps of 128 kSJ K: MFMA j takes the 128-K slice
  // [128 (kSJ S + j), +128) in natural order, so slot b holds MX block
  // 4 (kSJ S + j) + b.  Both operands' scales for slice j are one dword per
  // row; lane group g uses byte g of it (a shift by 8g).  The next super-step's
  // operands are loaded before this one's MFMAs are issued (two register
  // stages), keeping a wavefront's weight stream in flight.  The weights of an
  // expert with one tile are streamed past the caches; an expert with several
  // tiles (whose workgroups run at about the same time on one XCD) keeps them
  // in L2 for its other tiles.
  const int n_super = K / (128 * kSJ);
  if (stream_w)
    super_steps<NT, TILED, true>(acc, wp, wsp, ap, asp, n_super, g);
  else
    super_steps<NT, TILED, false>(acc, wp, wsp, ap, asp, n_super, g);
  // Remaining 128-K steps (K not a multiple of 128 kSJ): slot b takes block 4s + b.
  for (int s = n_super * kSJ; s < K / 128; ++s) {
    v4i wv[4];
    int wsv[4];
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
      if (TILED) {
        wv[bk] = *reinterpret_cast<const v4i*>(wp[bk] + (size_t)s * kTileBytes);
        wsv[bk] = *reinterpret_cast<const int*>(wsp[bk] + (size_t)s * kTileScaleBytes) >> (8 * g);
      } else {
        wv[bk] = *reinterpret_cast<const v4i*>(wp[bk] + (size_t)s * 64);
        wsv[bk] = wsp[bk][4 * s + g];
      }
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      v4i alo = *reinterpret_cast<const v4i*>(ap[tt] + (size_t)s * 128 + 16 * g);
      v4i ahi = *reinterpret_cast<const v4i*>(ap[tt] + (size_t)s * 128 + 64 + 16 * g);
      const int asv = asp[tt][4 * s + g];
#pragma unroll
      for (int bk = 0; bk < 4; ++bk) acc[tt][bk] = mfma_w4a8<0>(wv[bk], alo, ahi, acc[tt][bk], wsv[bk], asv);
    }
  }

  // The MFMAs read operands from all 64 lanes: make the accumulators live
  // here, with every lane active, so no MFMA is moved into the per-lane
  // store conditions below.
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) pin_acc(acc[tt]);

#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int row = row_begin + tt * 16 + li;
    store_subtile<FC1>(p, acc[tt], row, row < row_end, u, g);
  }
}

// Tiles of up to 32 grouped rows (the 32-row tile list): a tile holding at
// most 16 rows (every tile of an expert with at most 16) takes the one-subtile
// path, a larger one the two-subtile path, so an expert with 17..32 rows reads
// its weights once and one with fewer does no empty MFMAs.  Two wavefronts per
// SIMD (256 VGPRs at most): one's weight stream is in flight while the
// other's MFMAs issue.
template <bool FC1, bool TILED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fc_kernel(
    FcParams p) {
  // Consecutive block ids land on different XCDs (round robin over 8); remap
  // so that each XCD walks a contiguous range of (column group, tile) items,
  // with the tiles of one expert adjacent and sharing its weights in L2.
  const int nb = gridDim.x, b = blockIdx.x;
  const int logical = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  const int cg = logical / p.max_tiles, tile = logical % p.max_tiles;
  const int* prefix = p.tile_prefix;
  if (tile >= prefix[p.E_local]) return;
  const int e = p.tile_map[tile];
  const int row_begin = p.expert_offsets[e] + (tile - prefix[e]) * kDecodeTileRows;
  const int row_end = min(p.expert_offsets[e + 1], row_begin + kDecodeTileRows);
  const bool stream_w = prefix[e + 1] - prefix[e] == 1;
  if (row_end - row_begin <= 16)
    fc_tile<FC1, 1, TILED>(p, e, cg, row_begin, row_end, stream_w);
  else
    fc_tile<FC1, 2, TILED>(p, e, cg, row_begin, row_end, stream_w);
}

int expected_rows(int R, int E_local) {
  const int touched = R < E_local ? R : E_local;
  return touched > 0 ? R / touched : 1;
}

template <bool FC1>
hipError_t launch_fc(FcParams prm, int R, const int32_t* tile_prefix_all, int n_cu, bool tiled,
                     hipStream_t stream) {
  const int avg = expected_rows(R, prm.E_local);
  if (avg >= 32 && prefill_shape_ok(prm, FC1))
    return launch_fc_prefill(FC1, tiled, prm, tile_prefix_all, n_cu, stream);
  prm.tile_prefix = tile_prefix_all + (size_t)kDecodeTilePrefixIndex * (prm.E_local + 1);
  prm.tile_map = tile_prefix_all + (size_t)kNumTileSizes * (prm.E_local + 1);
  const int touched = R < prm.E_local ? R : prm.E_local;
  prm.max_tiles = R / kDecodeTileRows + touched;
  const int groups = (prm.n_units + 3) / 4;
  const int64_t blocks = (int64_t)groups * prm.max_tiles;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(256);
  if (tiled)
    hipLaunchKernelGGL((fc_kernel<FC1, true>), grid, block, 0, stream, prm);
  else
    hipLaunchKernelGGL((fc_kernel<FC1, false>), grid, block, 0, stream, prm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc1(const uint8_t* xq, const uint8_t* xs, int T, int H, int I, int top_k,
                      int E_local, const int32_t* offs, const int32_t* sorted_route,
                      const uint8_t* w13, const uint8_t* w13_s, float alpha, float beta,
                      uint8_t* hq, uint8_t* hs, const int32_t* tile_prefix_all,
                      uint32_t* act_st, int32_t* sched, int n_cu, bool tiled,
                      hipStream_t stream) {
  FcParams p{};
  p.act = xq; p.act_s = xs; p.act_rows = T; p.gather = sorted_route; p.top_k = top_k;
  p.n_routes = (int64_t)T * top_k; p.act_st = act_st; p.sched = sched;
  p.w = w13; p.w_s = w13_s; p.K = H; p.N = 2 * I; p.I = I;
  p.expert_offsets = offs; p.E_local = E_local;
  p.n_units = I / 32;
  p.alpha = alpha; p.beta = beta; p.hq = hq; p.hs = hs; p.y = nullptr;
  return launch_fc<true>(p, T * top_k, tile_prefix_all, n_cu, tiled, stream);
}

hipError_t launch_fc2(const uint8_t* hq, const uint8_t* hs, int T, int H, int I, int top_k,
                      int E_local, const int32_t* offs, const uint8_t* w2, const uint8_t* w2_s,
                      uint16_t* y, int8_t* ye, const int32_t* sorted_route,
                      const float* topk_w, float* out_acc, const int32_t* tile_prefix_all,
                      uint32_t* act_st, int32_t* sched, int n_cu, bool tiled,
                      hipStream_t stream) {
  FcParams p{};
  p.act = hq; p.act_s = hs; p.act_rows = (int64_t)T * top_k; p.gather = nullptr; p.top_k = top_k;
  p.n_routes = (int64_t)T * top_k; p.act_st = act_st; p.sched = sched;
  p.w = w2; p.w_s = w2_s; p.K = I; p.N = H; p.I = I;
  p.expert_offsets = offs; p.E_local = E_local;
  p.n_units = H / 64;
  p.y = y; p.ye = ye;
  p.combine_route = sorted_route; p.topk_w = topk_w; p.out_acc = out_acc;
  return launch_fc<false>(p, T * top_k, tile_prefix_all, n_cu, tiled, stream);
}

}  // namespace mi355moe
