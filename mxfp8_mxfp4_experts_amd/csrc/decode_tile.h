// One tile of up to 32 grouped rows of one expert against a group of
// 64-row weight units, one unit per wavefront, with the weights streamed
// straight from memory into registers (no LDS): the decode-shaped FC kernel
// (fc.hip) runs one such tile per unit of work (four wavefronts of one
// workgroup, or four one-wavefront workgroups).
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
#pragma once

#include "common.h"
#include "fc_common.h"
#include "tiled.h"

namespace mi355moe {

// Operands of one super-step (SJ 128-K slices) for one wavefront.
template <int NT, int SJ>
struct Stage {
  v4i w[4][SJ];      // [row block][MFMA j]: 32 E2M1 weights of this lane
  int ws[4][SJ];     // [row block][MFMA j]: the row's 4 scale bytes of slice j
  v4i alo[NT][SJ];   // [token tile][MFMA j]: E4M3 K [16g, 16g+16) of the slice
  v4i ahi[NT][SJ];   //                      E4M3 K [64+16g, 64+16g+16)
  int as[NT][SJ];    // the token's 4 scale bytes of slice j
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

template <int NT, int SJ, bool TILED, bool STREAM>
__device__ __forceinline__ void load_stage(Stage<NT, SJ>& st, const uint8_t* const* wp,
                                           const uint8_t* const* wsp, const uint8_t* const* ap,
                                           const uint8_t* const* asp, int S, int g) {
#pragma unroll
  for (int bk = 0; bk < 4; ++bk) {
    if (TILED) {
#pragma unroll
      for (int j = 0; j < SJ; ++j) {
        st.w[bk][j] = load_weights<STREAM>(
            reinterpret_cast<const v4i*>(wp[bk] + (size_t)(SJ * S + j) * kTileBytes));
        st.ws[bk][j] =
            *reinterpret_cast<const int*>(wsp[bk] + (size_t)(SJ * S + j) * kTileScaleBytes);
      }
    } else {
      const v4i* src = reinterpret_cast<const v4i*>(wp[bk] + (size_t)S * 64 * SJ);
#pragma unroll
      for (int j = 0; j < SJ; ++j) {
        st.w[bk][j] = load_weights<STREAM>(src + 4 * j);
        st.ws[bk][j] = *reinterpret_cast<const int*>(wsp[bk] + (size_t)(SJ * S + j) * 4);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const uint8_t* a = ap[tt] + (size_t)S * 128 * SJ + 16 * g;
#pragma unroll
    for (int j = 0; j < SJ; ++j) {
      st.alo[tt][j] = *reinterpret_cast<const v4i*>(a + 128 * j);
      st.ahi[tt][j] = *reinterpret_cast<const v4i*>(a + 128 * j + 64);
      st.as[tt][j] = *reinterpret_cast<const int*>(asp[tt] + (size_t)(SJ * S + j) * 4);
    }
  }
}

template <int NT, int SJ>
__device__ __forceinline__ void compute_stage(v4f (&acc)[NT][4], const Stage<NT, SJ>& st, int g) {
  const int sh = 8 * g;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
    for (int j = 0; j < SJ; ++j) {
      const int asv = st.as[tt][j] >> sh;
#pragma unroll
      for (int bk = 0; bk < 4; ++bk)
        acc[tt][bk] = mfma_w4a8<0>(st.w[bk][j], st.alo[tt][j], st.ahi[tt][j], acc[tt][bk],
                                   st.ws[bk][j] >> sh, asv);
    }
  }
}

// The super-step loop over K / (128 SJ) steps.  No branch inside the loop:
// the wait-count pass then lets the stage just loaded stay in flight while the
// other stage's MFMAs issue.  Tiled layout: the last one or two steps run
// after the loop, so no stage is loaded twice (the load path per CU is the
// bound, and the reload was one super-step in 14 for FC2).  Checkpoint layout
// (whose per-row pointers leave no registers for the peeled steps): the last
// iteration reloads the final stage when n_super is even.
template <int NT, int SJ, bool TILED, bool STREAM>
__device__ __forceinline__ void super_steps(v4f (&acc)[NT][4], const uint8_t* const* wp,
                                            const uint8_t* const* wsp, const uint8_t* const* ap,
                                            const uint8_t* const* asp, int n_super, int g) {
  if (n_super <= 0) return;
  Stage<NT, SJ> st0, st1;
  load_stage<NT, SJ, TILED, STREAM>(st0, wp, wsp, ap, asp, 0, g);
  int S = 0;
  if constexpr (!TILED) {
    for (; S + 1 < n_super; S += 2) {
      load_stage<NT, SJ, TILED, STREAM>(st1, wp, wsp, ap, asp, S + 1, g);
      __builtin_amdgcn_sched_barrier(0);
      compute_stage<NT, SJ>(acc, st0, g);
      __builtin_amdgcn_sched_barrier(0);
      load_stage<NT, SJ, TILED, STREAM>(st0, wp, wsp, ap, asp, min(S + 2, n_super - 1), g);
      __builtin_amdgcn_sched_barrier(0);
      compute_stage<NT, SJ>(acc, st1, g);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (S < n_super) compute_stage<NT, SJ>(acc, st0, g);
    return;
  }
  for (; S + 2 < n_super; S += 2) {
    load_stage<NT, SJ, TILED, STREAM>(st1, wp, wsp, ap, asp, S + 1, g);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<NT, SJ>(acc, st0, g);
    __builtin_amdgcn_sched_barrier(0);
    load_stage<NT, SJ, TILED, STREAM>(st0, wp, wsp, ap, asp, S + 2, g);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<NT, SJ>(acc, st1, g);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (S + 1 < n_super) {
    load_stage<NT, SJ, TILED, STREAM>(st1, wp, wsp, ap, asp, S + 1, g);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<NT, SJ>(acc, st0, g);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<NT, SJ>(acc, st1, g);
  } else {
    compute_stage<NT, SJ>(acc, st0, g);
  }
}

// One tile of NT 16-row subtiles [row_begin, row_end) of expert e against
// unit 4 cg + wave of column group cg (one unit per wavefront; the
// wavefronts of a column group share nothing, so they may sit in one
// workgroup or in four).  stream_w: the expert has this one tile, so its
// weights are read once and streamed past the caches.
template <bool FC1, int NT, bool TILED, int SJ = 2, bool ACC_A = false>
__device__ __forceinline__ void fc_tile(const FcParams& p, int e, int cg, int wave, int row_begin,
                                        int row_end, bool stream_w) {
  const int lane = threadIdx.x & 63;
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
    for (int bk = 0; bk < 4; ++bk) {
      acc[tt][bk] = v4f{0.f, 0.f, 0.f, 0.f};
      if (ACC_A) asm volatile("" : "+a"(acc[tt][bk]));   // accumulators in AGPRs
    }

  // Super-steps of 128 SJ K: MFMA j takes the 128-K slice
  // [128 (SJ S + j), +128) in natural order, so slot b holds MX block
  // 4 (SJ S + j) + b.  Both operands' scales for slice j are one dword per
  // row; lane group g uses byte g of it (a shift by 8g).  The next super-step's
  // operands are loaded before this one's MFMAs are issued (two register
  // stages), keeping a wavefront's weight stream in flight.  The weights of an
  // expert with one tile are streamed past the caches; an expert with several
  // tiles (whose workgroups run at about the same time on one XCD) keeps them
  // in L2 for its other tiles.
  const int n_super = K / (128 * SJ);
  if (stream_w)
    super_steps<NT, SJ, TILED, true>(acc, wp, wsp, ap, asp, n_super, g);
  else
    super_steps<NT, SJ, TILED, false>(acc, wp, wsp, ap, asp, n_super, g);
  // Remaining 128-K steps (K not a multiple of 128 SJ): slot b takes block 4s + b.
  for (int s = n_super * SJ; s < K / 128; ++s) {
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
  for (int tt = 0; tt < NT; ++tt) {
    if (ACC_A)
      pin_acc_agpr(acc[tt]);
    else
      pin_acc(acc[tt]);
  }

#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int row = row_begin + tt * 16 + li;
    store_subtile<FC1>(p, acc[tt], row, row < row_end, u, g);
  }
}


}  // namespace mi355moe
