// Single-workgroup grouping of the kept routes by local expert, shared by the
// grouping kernels (permute.hip) and the fused route + quantise + group launch
// (front.hip).  Page 1, "TP/EP expert mapping": a GPU holds a contiguous block
// of whole experts and maps global ids into it; "Phase 2 correctness harness":
// masked -1 slots and empty experts are part of the contract.
//
// One workgroup of kPermThreads threads:
//  1. histogram of local expert ids in LDS, keeping each route's local
//     expert (or -1) in LDS for step 3;
//  2. block-wide exclusive scans of the counts and of the per-expert tile
//     counts for the FC tile heights (32 and 256 rows), and the expert of
//     every 32-row tile;
//  3. the routes are walked in ascending order, 64 at a time (their local
//     experts read from LDS, so the walk waits on no global load); with a
//     per-wavefront count table (small E_local) each wavefront walks its own
//     contiguous slice from its own cursors, else one wavefront walks all:
//     lanes with the same expert find each other with ballots over the id
//     bits, the lowest such lane reserves their rows from the expert's LDS
//     cursor, and each lane takes base + its rank among them.  This keeps
//     the (token, slot) order inside every expert.
#pragma once

#include "common.h"

namespace mi355moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kScanVals = 1 + kNumTileSizes;
// The per-wavefront count table (kPermWaves x E_local ints) is used up to
// this many local experts (32 KB of LDS).
constexpr int kPermWaveTableExperts = 512;

// idx_of(r): global expert id of route r (r < R).  cnt, cursor: LDS int
// [E_local] each; lrow: LDS int [R]; wtab: LDS int [kPermWaves][E_local], or
// nullptr for the one-wavefront walk.
template <typename IdxFn>
__device__ __forceinline__ void permute_block(const IdxFn& idx_of, int R, int offset, int E_local,
                                              int32_t* __restrict__ expert_offsets,
                                              int32_t* __restrict__ sorted_route,
                                              int32_t* __restrict__ route_row,
                                              int32_t* __restrict__ tile_prefix, int* cnt,
                                              int* cursor, int* lrow, int* wtab) {
  __shared__ int wave_tot[kPermWaves][kScanVals];
  __shared__ int n_kept_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Wavefront w of the walk takes routes [w * slice, (w + 1) * slice).
  const int slice = ((R + kPermWaves - 1) / kPermWaves + 63) & ~63;
  for (int e = tid; e < E_local; e += kPermThreads) cnt[e] = 0;
  if (wtab)
    for (int i = tid; i < kPermWaves * E_local; i += kPermThreads) wtab[i] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += kPermThreads) {
    int g = idx_of(r);
    int l = g - offset;
    const bool kept = g >= 0 && l >= 0 && l < E_local;
    if (kept) {
      atomicAdd(&cnt[l], 1);
      if (wtab) atomicAdd(&wtab[(r / slice) * E_local + l], 1);
    }
    lrow[r] = kept ? l : -1;
  }
  __syncthreads();

  // Each thread owns a contiguous run of experts.
  const int per = (E_local + kPermThreads - 1) / kPermThreads;
  const int e0 = tid * per;
  int local[kScanVals];
#pragma unroll
  for (int v = 0; v < kScanVals; ++v) local[v] = 0;
  for (int e = e0; e < e0 + per && e < E_local; ++e) {
    int c = cnt[e];
    local[0] += c;
#pragma unroll
    for (int i = 0; i < kNumTileSizes; ++i) local[1 + i] += tiles_of(c, i);
  }
  // Inclusive wave scan, then scan of wave totals.
  int incl[kScanVals];
#pragma unroll
  for (int v = 0; v < kScanVals; ++v) {
    int x = local[v];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    incl[v] = x;
    if (lane == 63) wave_tot[wave][v] = x;
  }
  __syncthreads();
  if (tid == 0) {
    int run[kScanVals];
    for (int v = 0; v < kScanVals; ++v) run[v] = 0;
    for (int w = 0; w < kPermWaves; ++w)
      for (int v = 0; v < kScanVals; ++v) {
        int x = wave_tot[w][v];
        wave_tot[w][v] = run[v];
        run[v] += x;
      }
    n_kept_s = run[0];
    expert_offsets[E_local] = run[0];
    for (int i = 0; i < kNumTileSizes; ++i) tile_prefix[i * (E_local + 1) + E_local] = run[1 + i];
  }
  __syncthreads();
  int excl[kScanVals];
#pragma unroll
  for (int v = 0; v < kScanVals; ++v) excl[v] = incl[v] - local[v] + wave_tot[wave][v];
  int32_t* const tile_map = tile_prefix + kNumTileSizes * (E_local + 1);
  for (int e = e0; e < e0 + per && e < E_local; ++e) {
    int c = cnt[e];
    expert_offsets[e] = excl[0];
    cursor[e] = excl[0];
    excl[0] += c;
#pragma unroll
    for (int i = 0; i < kNumTileSizes; ++i) {
      tile_prefix[i * (E_local + 1) + e] = excl[1 + i];
      const int n = tiles_of(c, i);
      if (i == kMapTileIndex)
        for (int t = 0; t < n; ++t) tile_map[excl[1 + i] + t] = e;
      excl[1 + i] += n;
    }
  }
  __syncthreads();
  const int n_kept = n_kept_s;
  for (int r = n_kept + tid; r < R; r += kPermThreads) sorted_route[r] = -1;
  // Per-wavefront cursors: expert e's rows for wavefront w start after its
  // rows from the slices before w.
  if (wtab) {
    for (int e = tid; e < E_local; e += kPermThreads) {
      int run = cursor[e];
      for (int w = 0; w < kPermWaves; ++w) {
        const int c = wtab[w * E_local + e];
        wtab[w * E_local + e] = run;
        run += c;
      }
    }
    __syncthreads();
  }
  int* const cur = wtab ? wtab + wave * E_local : cursor;
  const int r_lo = wtab ? min(R, wave * slice) : 0;
  const int r_hi = wtab ? min(R, r_lo + slice) : R;

  if (wtab || wave == 0) {
    int nbits = 0;
    while ((1 << nbits) < E_local) ++nbits;
    for (int base = r_lo; base < r_hi; base += 64) {
      const int r = base + lane;
      const int l = r < r_hi ? lrow[r] : -1;
      const bool kept = l >= 0;
      uint64_t peers = __ballot(kept);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = kept && ((l >> bit) & 1);
        const uint64_t m = __ballot(set);
        peers &= set ? m : ~m;
      }
      const uint64_t lower = lane ? (~0ull >> (64 - lane)) : 0ull;
      const int rank = __popcll(peers & lower);
      const int leader = kept ? (__ffsll((long long)peers) - 1) : lane;
      int start = 0;
      if (kept && leader == lane) {
        start = cur[l];
        cur[l] = start + __popcll(peers);
      }
      start = __shfl(start, leader);
      if (r < r_hi) {
        if (kept) {
          const int pos = start + rank;
          if (pos < R) sorted_route[pos] = r;   // always true; keeps a stray row in bounds
          route_row[r] = pos;
        } else {
          route_row[r] = -1;
        }
      }
    }
  }
}

}  // namespace mi355moe
