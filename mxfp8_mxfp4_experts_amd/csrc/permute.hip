// a3: grouping of the kept routes by local expert.
//
// Page 1, "TP/EP expert mapping": a GPU holds a contiguous block of whole
// experts and maps global ids into it; "Phase 2 correctness harness": masked
// -1 slots and empty experts are part of the contract.
//
// Result (both paths below give the same bytes): the kept routes of local
// expert e occupy grouped rows [offs[e], offs[e+1]) in ascending route order;
// sorted_route[row] = route, route_row[route] = row or -1; grouped rows past
// the kept count hold -1; tile prefixes for the FC tile heights 32 and 256 and
// the expert of every 32-row tile.
//
// Small batches: one workgroup runs permute_block (permute_dev.h): a
// histogram in LDS, block-wide scans of the counts and tile counts, then the
// routes are ranked 64 at a time with ballots over the id bits (each
// wavefront its own slice when a per-wavefront count table fits in LDS, else
// one wavefront all of them).
// Large batches: the routes are cut into chunks (perm_chunk_size); a count
// kernel writes each chunk's histogram, a column-scan kernel (one workgroup
// per 64 experts) turns each expert's chunk counts into the chunks' first rows
// within the expert and the expert's total, one workgroup scans the totals
// into expert offsets and tile prefixes, and a rank kernel (one wavefront per
// chunk) runs the ballot ranking on its chunk from those starting rows.
#include "common.h"
#include "launch.h"
#include "permute_dev.h"

namespace mi355moe {

namespace {

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ idx, int R, int offset, int E_local,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_route,
    int32_t* __restrict__ route_row, int32_t* __restrict__ tile_prefix) {
  extern __shared__ int lds_i[];
  permute_block([&](int r) { return idx[r]; }, R, offset, E_local, expert_offsets, sorted_route,
                route_row, tile_prefix, lds_i, lds_i + E_local, lds_i + 2 * E_local,
                E_local <= kPermWaveTableExperts ? lds_i + 2 * E_local + R : nullptr);
}

// Local expert of route r, or -1 (masked slot or outside the window).
__device__ __forceinline__ int local_expert(const int32_t* idx, int r, int R, int offset,
                                            int E_local) {
  if (r >= R) return -1;
  const int g = idx[r];
  const int l = g - offset;
  return (g >= 0 && l >= 0 && l < E_local) ? l : -1;
}

// Histogram of one chunk's local expert ids.
__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t* __restrict__ idx, int R,
                                                         int offset, int E_local, int chunk,
                                                         int32_t* __restrict__ counts) {
  extern __shared__ int cnt_s[];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E_local; e += 256) cnt_s[e] = 0;
  __syncthreads();
  const int r0 = c * chunk;
  for (int r = r0 + threadIdx.x; r < r0 + chunk; r += 256) {
    const int l = local_expert(idx, r, R, offset, E_local);
    if (l >= 0) atomicAdd(&cnt_s[l], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E_local; e += 256) counts[(size_t)c * E_local + e] = cnt_s[e];
}

// Chunk histograms -> each chunk's first row within the expert (in place)
// and each expert's total.  Workgroup b takes experts [64 b, 64 b + 64), one
// per lane; each of its kColWaves wavefronts sums its share of the chunks
// (loads of 64 consecutive experts are one coalesced run), the shares' sums
// give each wavefront its starting row, then it rewrites its chunks.
constexpr int kBatch = 16;
constexpr int kColWaves = 16;
__global__ __launch_bounds__(64 * kColWaves) void perm_colscan_kernel(
    int E_local, int n_chunks, int32_t* __restrict__ counts, int32_t* __restrict__ totals) {
  __shared__ int part_s[kColWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const bool ok = e < E_local;
  const int per = (n_chunks + kColWaves - 1) / kColWaves;
  const int c0 = min(w * per, n_chunks), c1 = min(c0 + per, n_chunks);
  int sum = 0;
  for (int c = c0; c < c1; c += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      v[j] = ok && c + j < c1 ? counts[(size_t)(c + j) * E_local + e] : 0;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) sum += v[j];
  }
  part_s[w][lane] = sum;
  __syncthreads();
  int row = 0;
  for (int i = 0; i < w; ++i) row += part_s[i][lane];
  if (w == kColWaves - 1 && ok) totals[e] = row + sum;
  for (int c = c0; c < c1; c += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      v[j] = ok && c + j < c1 ? counts[(size_t)(c + j) * E_local + e] : 0;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (ok && c + j < c1) counts[(size_t)(c + j) * E_local + e] = row;
      row += v[j];
    }
  }
}

// Expert totals -> expert offsets, tile prefixes and the tile -> expert map;
// grouped rows past the kept count get -1.
__global__ __launch_bounds__(kPermThreads) void perm_scan_kernel(
    int R, int E_local, const int32_t* __restrict__ totals,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_route,
    int32_t* __restrict__ tile_prefix) {
  __shared__ int wave_tot[kPermWaves][kScanVals];
  __shared__ int n_kept_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Each thread owns a contiguous run of experts: their totals first.
  const int per = (E_local + kPermThreads - 1) / kPermThreads;
  const int e0 = tid * per;
  int local[kScanVals];
#pragma unroll
  for (int v = 0; v < kScanVals; ++v) local[v] = 0;
  for (int e = e0; e < e0 + per && e < E_local; ++e) {
    const int total = totals[e];
    local[0] += total;
#pragma unroll
    for (int i = 0; i < kNumTileSizes; ++i) local[1 + i] += tiles_of(total, i);
  }
  int incl[kScanVals];
#pragma unroll
  for (int v = 0; v < kScanVals; ++v) {
    int x = local[v];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
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
        const int x = wave_tot[w][v];
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
  // Then each expert's offset, its tile prefixes and its entries of the
  // tile -> expert map.
  int32_t* const tile_map = tile_prefix + kNumTileSizes * (E_local + 1);
  for (int e = e0; e < e0 + per && e < E_local; ++e) {
    expert_offsets[e] = excl[0];
    const int total = totals[e];
    excl[0] += total;
#pragma unroll
    for (int i = 0; i < kNumTileSizes; ++i) {
      tile_prefix[i * (E_local + 1) + e] = excl[1 + i];
      const int n = tiles_of(total, i);
      if (i == kMapTileIndex)
        for (int t = 0; t < n; ++t) tile_map[excl[1 + i] + t] = e;
      excl[1 + i] += n;
    }
  }
  const int n_kept = n_kept_s;
  for (int r = n_kept + tid; r < R; r += kPermThreads) sorted_route[r] = -1;
}

// Step 3 on one chunk, from the chunk's starting rows (within the expert,
// plus the expert's offset).
__global__ __launch_bounds__(64) void perm_rank_kernel(const int32_t* __restrict__ idx, int R,
                                                       int offset, int E_local, int chunk,
                                                       const int32_t* __restrict__ starts,
                                                       const int32_t* __restrict__ expert_offsets,
                                                       int32_t* __restrict__ sorted_route,
                                                       int32_t* __restrict__ route_row) {
  extern __shared__ int cursor_s[];
  const int c = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E_local; e += 64)
    cursor_s[e] = starts[(size_t)c * E_local + e] + expert_offsets[e];
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E_local) ++nbits;
  const int r0 = c * chunk;
  const int r_end = min(r0 + chunk, R);
  for (int base = r0; base < r_end; base += 64) {
    const int r = base + lane;
    const int l = local_expert(idx, r, r_end, offset, E_local);
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
      start = cursor_s[l];
      cursor_s[l] = start + __popcll(peers);
    }
    start = __shfl(start, leader);
    if (r < r_end) {
      if (kept) {
        const int pos = start + rank;
        sorted_route[pos] = r;
        route_row[r] = pos;
      } else {
        route_row[r] = -1;
      }
    }
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* idx, int R, int offset, int E_local, int32_t* offs,
                          int32_t* sorted_route, int32_t* route_row, int32_t* tile_prefix,
                          int32_t* counts, hipStream_t stream) {
  if (R <= kPermSingle) {
    const size_t table = E_local <= kPermWaveTableExperts ? (size_t)kPermWaves * E_local : 0;
    const size_t lds = sizeof(int) * (2 * (size_t)E_local + (size_t)R + table);
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), lds, stream, idx, R, offset,
                       E_local, offs, sorted_route, route_row, tile_prefix);
    return hipGetLastError();
  }
  const int n_chunks = perm_chunks(R), chunk = perm_chunk_size(R);
  const size_t lds = sizeof(int) * (size_t)E_local;
  hipLaunchKernelGGL(perm_count_kernel, dim3(n_chunks), dim3(256), lds, stream, idx, R, offset,
                     E_local, chunk, counts);
  int32_t* const totals = counts + (size_t)n_chunks * E_local;
  hipLaunchKernelGGL(perm_colscan_kernel, dim3((E_local + 63) / 64), dim3(64 * kColWaves), 0, stream,
                     E_local, n_chunks, counts, totals);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kPermThreads), 0, stream, R, E_local,
                     totals, offs, sorted_route, tile_prefix);
  hipLaunchKernelGGL(perm_rank_kernel, dim3(n_chunks), dim3(64), lds, stream, idx, R, offset,
                     E_local, chunk, counts, offs, sorted_route, route_row);
  return hipGetLastError();
}

}  // namespace mi355moe
