// Shared device helpers and host-side layout of the MoE layer library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mi355moe {

// ---------------------------------------------------------------------------
// Limits checked at the C ABI.
constexpr int kMaxExperts = 4096;   // routing width E and local window E_local
constexpr int kMaxTopK = 64;        // one wavefront lane per selected slot
constexpr int kGroup = 32;          // MX block: one E8M0 scale per 32 elements

// FC tile heights (token rows per workgroup tile) for which moe_permute
// writes a tile prefix: 32 << (3 i) for i in [0, kNumTileSizes), i.e. 32
// (the decode-shaped FC kernels) and 256 (the prefill-shaped ones).
constexpr int kNumTileSizes = 2;
__host__ __device__ constexpr int tile_rows(int i) { return 32 << (3 * i); }
__host__ __device__ inline int tiles_of(int rows, int i) {
  return (rows + tile_rows(i) - 1) / tile_rows(i);
}
// After the prefixes it writes the expert of every tile of height
// tile_rows(kMapTileIndex) (the decode-shaped FC kernels' tile list), so a
// workgroup finds its expert with one load: at most R / 32 + E_local tiles
// for R kept routes.
constexpr int kMapTileIndex = 0;
__host__ __device__ inline int64_t tile_map_entries(int64_t R, int E_local) {
  return R / tile_rows(kMapTileIndex) + E_local;
}

// ---------------------------------------------------------------------------
// Workspace layout shared by moe_permute / moe_fc1_situ / moe_fc2_combine.
// Grouping (moe_permute): batches of at most kPermSingle routes take one
// workgroup; larger ones are cut into chunks, one wavefront ranking each --
// 256 routes per chunk up to 16384 routes, 512 above (enough chunks to
// spread the ranking; the per-expert scan over chunks reads them in batches).
constexpr int kPermSingle = 2048;
constexpr int kSchedStride = 64;   // int32 stride between the per-XCD work counters
constexpr int kSchedItemPrefix = 9 * kSchedStride;   // int32 offset of the item prefix
__host__ __device__ inline int perm_chunk_size(int64_t R) { return R <= 16384 ? 256 : 512; }
inline int perm_chunks(int64_t R) {
  return R <= kPermSingle ? 0 : (int)((R + perm_chunk_size(R) - 1) / perm_chunk_size(R));
}

struct WsLayout {
  size_t tile_prefix;   // int32 [kNumTileSizes][E_local + 1], then the tile -> expert map
                        // int32 [tile_map_entries(T * top_k, E_local)]
  size_t perm_counts;   // int32 [perm_chunks(R)][E_local], then [E_local] expert totals
                        // (grouping scratch)
  size_t fc_sched;      // int32 [9][kSchedStride]: per-XCD work counters of the prefill FC
                        // kernels, then their 9 item-range bounds; then int32 [E_local + 1]:
                        // the prefix of the experts' work items
  size_t act_st;        // uint32 [max(H, I) / 128][T * top_k]: an FC input's scale dwords,
                        // stage-major in grouped-row order (prefill-shaped FC kernels)
  size_t y;             // deterministic combine: fp16 [T * top_k][H] (FC2 rows before the
                        // combine, scaled); atomic combine: float [T][H] (the weighted sums)
  size_t ye;            // deterministic combine: int8, the power-of-two scale of each 64
                        // columns of each y row, in blocks of 16 rows (ye_index; atomic
                        // combine: empty)
  size_t total;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Place of the scale exponent of columns [64 u, 64 u + 64) of y row `row`
// (n_u = H / 64 per row): rows in blocks of 16, each block column-major, so
// the 16 rows of an FC2 sub-tile write their exponents of one unit as one
// 16-byte run, and the 8 consecutive units a combine wavefront reads for a
// row lie in one 128-byte line.
__host__ __device__ inline size_t ye_index(int64_t row, int u, int n_u) {
  return ((size_t)(row >> 4) * n_u + u) * 16 + (size_t)(row & 15);
}

inline WsLayout ws_layout(int T, int top_k, int E_local, int H, int I, bool atomic = false) {
  WsLayout l;
  size_t off = 0;
  l.tile_prefix = off;
  off = align256(off + sizeof(int32_t) * (kNumTileSizes * (size_t)(E_local + 1) +
                                          (size_t)tile_map_entries((int64_t)T * top_k, E_local)));
  l.perm_counts = off;
  off = align256(off + sizeof(int32_t) * ((size_t)perm_chunks((int64_t)T * top_k) + 1) * E_local);
  l.fc_sched = off;
  off = align256(off + sizeof(int32_t) * (kSchedItemPrefix + E_local + 1));
  l.act_st = off;
  off = align256(off + (size_t)T * top_k * (size_t)((H > I ? H : I) / 32));
  l.y = off;
  off = atomic ? align256(off + sizeof(float) * (size_t)T * H)
               : align256(off + sizeof(uint16_t) * (size_t)T * top_k * H);
  l.ye = off;
  off = atomic ? off : align256(off + ((size_t)T * top_k + 15) / 16 * 16 * (H / 64));
  l.total = off;
  return l;
}

// ---------------------------------------------------------------------------
// Device helpers: the MX element / scale rules.

// Smallest e with amax <= 448 * 2^e, clamped to [-127, 127].  amax is a
// non-negative float (NaN excluded by the caller).  448 = 1.75 * 2^8, so with
// amax = 1.m * 2^p the rule is e = p - 8, plus one when 1.m > 1.75.
__device__ __forceinline__ int mx8_exponent(float amax) {
  uint32_t b = __float_as_uint(amax);
  uint32_t ex = b >> 23;            // sign is clear
  if (ex == 0) return -127;         // zero or subnormal: 448 * 2^-127 > 2^-126
  if (ex == 255) return 127;        // infinity
  int e = (int)ex - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Nearest E4M3 code to y (ties to even), saturating at +-448, sign of zero
// kept, NaN -> 0x00.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  uint32_t bits = __float_as_uint(y);
  uint32_t sign = (bits >> 24) & 0x80u;
  uint32_t ab = bits & 0x7FFFFFFFu;
  if (ab > 0x7F800000u) return 0u;                     // NaN
  uint32_t code;
  if (ab < 0x3C800000u) {                              // |y| < 2^-6: subnormal grid m * 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(ab) * 512.0f);
  } else {                                             // round 23 mantissa bits to 3 (RNE)
    code = ((ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20) - (120u << 3);
  }
  code = code > 126u ? 126u : code;
  return code | sign;
}

// float -> bf16 bits, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

}  // namespace mi355moe
