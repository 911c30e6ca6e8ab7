// Tiled weight layout shared by the prepack kernel and the tiled FC kernels.
//
// The checkpoint layout keeps an expert's E2M1 weights as [N rows][K/2 bytes]
// and its E8M0 scales as [N rows][K/32 bytes] (page 1, "真实 checkpoint 契约";
// page 5, w13 / w2 shapes).  The tiled layout holds the same bytes, reordered
// once at load time so that the FC kernels read whole contiguous blocks (the
// role the pages give to the weight / scale transforms applied after
// loading, page 5, process_weights_after_loading):
//
//   * rows are grouped 512 at a time (column group cg) and K is cut into
//     stages of 128 elements (64 bytes of E2M1 per row, one scale dword);
//   * data block (e, cg, s), 32 KB: sixteen-byte chunks in the order
//     chunk[(4w + i) * 64 + l] = logical chunk c of row r, with
//     r = 64w + 16i + l/4 and c = (l & 3) ^ ((l >> 3) & 3)  (w < 8, i < 4,
//     l < 64); this is exactly the swizzled LDS image the prefill kernel
//     computes from, so its loads are straight 1 KB copies;
//   * scale block (e, cg, s), 2 KB: dword r = the four scale bytes of row r
//     for MX blocks 4s .. 4s+3;
//   * row r of group cg is the global row tiled_row<FC1>(r, cg): for w13 each
//     64-row unit u = 8 cg + r/64 pairs gate rows [32u, 32u+32) with up rows
//     [I+32u, I+32u+32); for w2 it is 512 cg + r;
//   * blocks are stored [e][cg][s] (data and scales in two arrays of the
//     same sizes as the checkpoint arrays).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mi355moe {

constexpr int kTileRows = 512;           // rows per column group
constexpr int kTileK = 128;              // K per stage
constexpr int kTileBytes = kTileRows * kTileK / 2;   // 32768
constexpr int kTileScaleBytes = kTileRows * 4;        // 2048

template <bool FC1>
__host__ __device__ __forceinline__ int tiled_row(int r, int cg, int I) {
  if (FC1) {
    const int u = cg * 8 + (r >> 6), blk = (r >> 4) & 3, lr = r & 15;
    return (blk < 2 ? 0 : I) + u * 32 + (blk & 1) * 16 + lr;
  }
  return cg * kTileRows + r;
}

// Byte offset of data block (e, cg, s) and of scale block (e, cg, s).
__host__ __device__ __forceinline__ size_t tiled_block(int e, int cg, int s, int n_cg, int n_st) {
  return ((size_t)e * n_cg + cg) * n_st + s;
}

}  // namespace mi355moe
