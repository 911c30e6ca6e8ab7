// a4..a7: grouped FC1 (+ SiTU + requantisation) and FC2 (writing the per-route
// rows the combine sums) on the gfx950 block-scaled MFMA
// (V_MFMA_SCALE_F32_16X16X128_F8F6F4), for experts holding few grouped rows.
//
// Page 1, "Serving call chain": grouped GEMM1 -> gated activation -> GEMM2 ->
// finalize; "Real checkpoint contract": w13 = [gate; up] halves, SiTU(4, 25);
// page 5: w13 [E, 2I, H/2] + [E, 2I, H/32], w2 [E, H, I/2] + [E, H, I/32].
//
// The MFMA operand layout and the tile code (fc_tile) are in decode_tile.h.
//
// Work decomposition: a workgroup (4 wavefronts) takes one tile of up to 32
// grouped rows of one expert (one or two 16-row subtiles) and a column group
// of 4 units; a unit (one wavefront) is 64 weight rows: for FC1, gate rows
// [c, c+32) with up rows [I+c, I+c+32), so SiTU and the 32-column
// requantisation group are local to the lanes that hold them; for FC2, output
// columns [h, h+64).  The expert of each tile comes from the grouping step's
// tile -> expert map.
#include "common.h"
#include "decode_tile.h"
#include "fc_common.h"
#include "launch.h"
#include "tiled.h"

namespace mi355moe {

namespace {

// Tile list of the decode-shaped kernel: 32-row tiles (tile prefix 0), whose
// tile -> expert map the grouping step writes after the prefixes.
constexpr int kDecodeTilePrefixIndex = 0;
constexpr int kDecodeTileRows = tile_rows(kDecodeTilePrefixIndex);
static_assert(kDecodeTileRows == 32, "two 16-row subtiles per tile");
static_assert(kDecodeTilePrefixIndex == kMapTileIndex, "tile map");

// Tiles of up to 32 grouped rows (the 32-row tile list): a tile holding at
// most 16 rows (every tile of an expert with at most 16) takes the one-subtile
// path, a larger one the two-subtile path, so an expert with 17..32 rows reads
// its weights once and one with fewer does no empty MFMAs.  Two wavefronts per
// SIMD (256 VGPRs at most): one's weight stream is in flight while the
// other's MFMAs issue.  WAVES wavefronts per workgroup: 4 (a column group's
// units) or, for a grid that would leave CUs idle, 1 (each unit its own
// workgroup, so the same wavefronts spread over every CU).
template <bool FC1, bool TILED, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2))) void fc_kernel(
    FcParams p) {
  // Consecutive block ids land on different XCDs (round robin over 8).  The
  // items are the (launch group, tile) pairs of the n tiles in use, group by
  // group; XCD x walks items [x W / 8, (x + 1) W / 8) of the W = groups * n,
  // so every XCD gets the same share of the work however many of the grid's
  // max_tiles tiles per group are in use, and the tiles of one expert stay
  // adjacent, sharing its weights in L2.  max_tiles is a multiple of 8 and at
  // least n, so each XCD's nb / 8 workgroups cover its share.
  const int nb = gridDim.x, b = blockIdx.x;
  const int n_groups = nb / p.max_tiles;
  const int* prefix = p.tile_prefix;
  const int n_tiles = prefix[p.E_local];
  const int64_t W = (int64_t)n_groups * n_tiles;
  const int xcd = b & 7, i = b >> 3;
  const int lo = (int)(xcd * W / 8), hi = (int)((xcd + 1) * W / 8);
  if (lo + i >= hi) return;
  const int group = (lo + i) / n_tiles, tile = lo + i - group * n_tiles;
  const int cg = WAVES == 4 ? group : group >> 2;
  const int wave = WAVES == 4 ? (int)(threadIdx.x >> 6) : (group & 3);
  const int e = p.tile_map[tile];
  const int row_begin = p.expert_offsets[e] + (tile - prefix[e]) * kDecodeTileRows;
  const int row_end = min(p.expert_offsets[e + 1], row_begin + kDecodeTileRows);
  const bool stream_w = prefix[e + 1] - prefix[e] == 1;
  if (row_end - row_begin <= 16)
    fc_tile<FC1, 1, TILED>(p, e, cg, wave, row_begin, row_end, stream_w);
  else
    fc_tile<FC1, 2, TILED>(p, e, cg, wave, row_begin, row_end, stream_w);
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
  // A bound on the tiles in use (each touched expert adds at most one partial
  // tile), rounded up to a multiple of the 8 XCDs.
  prm.max_tiles = (R / kDecodeTileRows + touched + 7) & ~7;
  const int groups = (prm.n_units + 3) / 4;
  const int64_t blocks = (int64_t)groups * prm.max_tiles;
  if (blocks <= 0) return hipSuccess;
  if (4 * blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  // Fewer than two four-wavefront workgroups per CU (at most max_tiles
  // tiles, a bound): one workgroup per unit instead.
  if (blocks < 2 * (int64_t)n_cu) {
    const dim3 grid((unsigned)(4 * blocks)), block(64);
    if (tiled)
      hipLaunchKernelGGL((fc_kernel<FC1, true, 1>), grid, block, 0, stream, prm);
    else
      hipLaunchKernelGGL((fc_kernel<FC1, false, 1>), grid, block, 0, stream, prm);
  } else {
    const dim3 grid((unsigned)blocks), block(256);
    if (tiled)
      hipLaunchKernelGGL((fc_kernel<FC1, true, 4>), grid, block, 0, stream, prm);
    else
      hipLaunchKernelGGL((fc_kernel<FC1, false, 4>), grid, block, 0, stream, prm);
  }
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
