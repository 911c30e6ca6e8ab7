// Prefill-shaped FC1 / FC2 (many grouped rows per expert).
//
// Same method as the decode-shaped kernel (page 1, "Serving 调用链": grouped
// GEMM1 -> gated activation -> GEMM2; "真实 checkpoint 契约": [gate; up] halves,
// SiTU(4, 25); page 5: w13 / w2 and scale layouts), organised for experts
// that hold tens to hundreds of grouped rows:
//   * a workgroup of 8 wavefronts (two per SIMD, so one wavefront's waits are
//     covered by the other's MFMAs) computes up to 256 grouped rows of one
//     expert against 256 weight rows.  Wavefront w owns weight half w & 1
//     (two 64-row units: FC1 gate rows [c, c+32) with up rows [I+c, I+c+32),
//     so SiTU pairs stay in one wavefront; FC2 64 output columns each) and
//     token quarter w >> 1 (the 16-row tiles q, q+4, q+8, q+12, so a partly
//     filled tile still spreads over all four SIMDs): 4 tiles x 8 row blocks
//     of 16x16 accumulators, 128 AGPRs;
//   * both operands go through a ring of LDS stages (token rows x 128 bytes,
//     token scale dwords, 256 weight rows x 64 bytes, weight scale dwords),
//     filled by direct buffer -> LDS loads issued ahead: an item with up to
//     256 rows in use has 3 stages of 50 KB and loads 2 ahead; one with up to
//     128 or 64 rows has 4 stages of 34 KB or 5 of 26 KB and loads 3 or 4
//     ahead, since its time is the latency of its weight stream.  Every
//     wavefront issues the same loads per stage (token rows, 2 KB of weights,
//     and the token or the weight scale dwords), so one fixed
//     "s_waitcnt vmcnt" per stage leaves exactly the later stages in flight;
//     past the last stage the final stage is reloaded to keep that count.
//     The loads sit in MFMA slots early in the stage (the longest lead before
//     their wait);
//   * an expert with at most 128 rows takes two column groups per item, so
//     the token rows loaded for a stage feed both weight tiles (the per-CU
//     load path, not HBM, bounds these items; token rows were a third to a
//     half of their bytes), and an item of 128 rows x 512 weight rows has a
//     full tile's accumulators and bytes per MFMA;
//   * the token scale dwords are first restaged (stage_scales_kernel) into a
//     stage-major array in grouped-row order, so a tile's scales for one stage
//     are one contiguous 1 KB run instead of one cache line per row: the
//     per-CU load path is bounded by outstanding cache-line requests, not by
//     bytes;
//   * token 16-byte chunks are XOR-swizzled by row bits 0..2 and weight chunks
//     sit in the tiled layout's order, so the eight lanes served together hit
//     eight bank groups;
//   * an expert with at most 256 rows is one tile, so its weights are read
//     once in total; its token rows are re-read by every column group, which
//     the schedule keeps in one XCD's L2: each XCD owns a contiguous range of
//     items (split by estimated work) and its workgroups take them in order
//     from a shared counter;
//   * per stage a wavefront reads its 8 weight operands once, then per valid
//     token tile 8 MFMAs, each followed by a read of the next tile's operands
//     or one of the stage's global loads.  The stage loop is instantiated per
//     count of valid tiles (0..4), so no accumulator is updated under a
//     condition (which the register allocator handles by copying);
//   * the expert tile prefix and row offsets are copied to LDS once per
//     workgroup (the item lookup is a binary search per item).  The stage
//     ring and this table are one LDS object: with several, the compiler
//     cannot tell the direct-to-LDS loads from the operand reads and waits
//     for every load before each read;
//   * buffer resources keep every per-lane address a 32-bit offset.
#include "common.h"
#include "fc_common.h"
#include "launch.h"
#include "tiled.h"

#include <type_traits>

namespace mi355moe {

namespace {

constexpr int kBM = 256;                     // token rows per tile
constexpr int kBN = 256;                     // weight rows per tile (4 units)
constexpr int kKS = 128;                     // K per stage
constexpr int kThreads = 512;                // 8 wavefronts
constexpr int kTilePrefixIndex = 1;          // tile height 256
constexpr int kMaxLdsExperts = 1024;            // local experts whose metadata LDS holds
static_assert(kKS == kTileK && 2 * kBN == kTileRows, "tile shape");
static_assert(tile_rows(kTilePrefixIndex) == kBM && kTilePrefixIndex < kNumTileSizes, "tile prefix");

// Stage layout of the LDS ring for an item whose used token rows fit in
// 64 P (P = 4, 2 or 1 one-KB token pieces per wavefront and stage):
// [token rows 8P KB][token scale dwords 1 KB][weight operands 16 KB][weight
// scale dwords 1 KB].  A smaller token part leaves room for more stages, so
// an item with few rows, whose time is its weight stream's latency, loads
// further ahead: 2, 3 or 4 stages for P = 4, 2, 1.  Each wavefront issues
// P + 3 direct-to-LDS loads per stage (P token pieces, 2 weight pieces, the
// token or the weight scale dwords); when stage s + 1 is waited for, the
// loads of the kAhead - 1 stages after it stay in flight.
//
// PAIR (P = 1 or 2): the item covers two column groups of an expert with at
// most 64 P rows, so one stage's token rows feed both weight tiles and the
// token bytes per weight byte halve: [token rows 8P KB][token scale dwords
// P/4 KB][weights of both column groups 32 KB][their scale dwords 2 KB], 3
// stages loaded 2 ahead.  Wavefront w works on column group w >> 2 of the
// pair, weight half w & 1 and the token tiles (w >> 1) & 1 + 2 j; it issues
// P + 6 loads per stage (P token pieces, 4 weight pieces, a weight and a
// token scale piece; the token scale pieces of wavefronts w and w + P are
// the same bytes).
template <int P, bool PAIR = false>
struct Ring {
  static_assert(!PAIR || P <= 2, "pairs hold at most 128 rows");
  static constexpr int kCG = PAIR ? 2 : 1;             // column groups per item
  static constexpr int kTokScaleOff = 64 * P * kKS;
  static constexpr int kTokScaleBytes = PAIR ? 256 * P : kBM * 4;
  static constexpr int kWOff = kTokScaleOff + kTokScaleBytes;
  static constexpr int kWScaleOff = kWOff + kCG * kBN * kKS / 2;
  static constexpr int kStage = kWScaleOff + kCG * kBN * 4;
  static constexpr int kNumBuf = PAIR ? 3 : P == 4 ? 3 : P == 2 ? 4 : 5;
  static constexpr int kAhead = kNumBuf - 1;
  static constexpr int kWPieces = 2 * kCG;             // weight pieces per wavefront and stage
  static constexpr int kLoads = P + kWPieces + kCG;
  static constexpr int kTileStep = PAIR ? 2 : 4;       // between a wavefront's token tiles
  static constexpr int kBytes = kNumBuf * kStage;
};
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kRingBytes = cmax(cmax(Ring<4>::kBytes, Ring<2>::kBytes),
                                cmax(cmax(Ring<1>::kBytes, Ring<1, true>::kBytes),
                                     Ring<2, true>::kBytes));   // 155136 (Ring<2, true>)
static_assert((Ring<1>::kAhead - 1) * Ring<1>::kLoads < 64, "vmcnt");
static_assert(Ring<2, true>::kLoads <= 8, "load slots");
constexpr int kLdsBytes = kRingBytes + 8 * (kMaxLdsExperts + 1) + 16;
static_assert(kLdsBytes <= 160 * 1024, "LDS");

// Raw buffer resource: base and byte size in SGPRs.  Sizes stay below 2^31,
// so kOutOfRange (plus any stage offset) is always past the end.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [I, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Largest expert e with prefix[e] <= tile, from the LDS copy.
__device__ __forceinline__ int find_expert_lds(const int* prefix, int E_local, int tile) {
  int lo = 0, hi = E_local;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

typedef __attribute__((address_space(3))) uint8_t lds_t;
typedef __attribute__((address_space(3))) v4i lds_v4i;

// Token operands of one 16-row tile: K [16g, +16) and [64 + 16g, +16) for
// lane group g, and the row's scale byte for MX block g.
struct AOp {
  v4i lo, hi;
  int sc;
};

// Scale dwords of the grouped rows, stage-major: out[s][r] = the four E8M0
// bytes of MX blocks 4s .. 4s+3 of grouped row r's source row (FC1: token
// gather[r] / top_k of act_s; FC2: row r).  The prefill kernels then load a
// tile's scales for a stage as one contiguous run instead of one cache line
// per row.  Only the kept rows [0, offs[E_local]) are written.  Also clears
// the per-XCD work counters of the FC kernel that follows on the stream and
// writes its per-XCD item ranges.
// Items of one FC launch, split over the 8 XCDs by estimated work: an item
// (expert e, column group, 256-row tile) costs about kItemFixedRows + its rows
// rounded up to 16 per stage.  An expert with at most kPairRows rows has
// n_cg / 2 items (each two column groups), one with more n_cg items per
// 256-row tile.
// Workgroup 0 of the pre-pass scans the per-expert work and item counts,
// writes the item prefix over the experts to item_prefix[0..E_local] and the
// first item of each XCD's range (at a column-group boundary) to
// bounds[0..8].
constexpr int kItemFixedRows = 64;
constexpr int kPairRows = 128;  // experts with at most this many rows run as pair items
constexpr int kTileGroup = 4;   // tiles per item group of a multi-tile expert

// Items of an expert with more than kPairRows rows run in groups of
// kTileGroup tiles, the last group (1..kTileGroup tiles) holding the last
// tile; when that tile has at most kPairRows rows it runs as pair items, each
// after the other tiles' items of its two column groups.
__device__ __forceinline__ int expert_items(int rows, int n_tiles, int n_cg) {
  if (rows == 0) return 0;
  if (rows <= kPairRows) return n_cg / 2;
  const int full = (n_tiles - 1) / kTileGroup, rem = n_tiles - full * kTileGroup;
  const bool tail_pair = rows - kBM * (n_tiles - 1) <= kPairRows;
  return full * kTileGroup * n_cg + (tail_pair ? (n_cg / 2) * (2 * rem - 1) : n_cg * rem);
}

__device__ void split_items(const int32_t* __restrict__ offs, const int32_t* __restrict__ prefix,
                            int E_local, int n_cg, int32_t* __restrict__ bounds,
                            int32_t* __restrict__ item_prefix) {
  __shared__ long long cum_s[kMaxLdsExperts + 1];
  __shared__ int items_s[kMaxLdsExperts + 1];
  __shared__ long long wsum_s[4];
  __shared__ int isum_s[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (E_local + 255) / 256, e0 = tid * per;
  long long mine = 0;
  int mine_items = 0;
  for (int e = e0; e < e0 + per && e < E_local; ++e) {
    const int c = offs[e + 1] - offs[e], nt = prefix[e + 1] - prefix[e];
    const long long w = (long long)n_cg * (nt * kItemFixedRows + 16 * ((c + 15) / 16));
    cum_s[e + 1] = w;   // turned into running sums below
    items_s[e + 1] = expert_items(c, nt, n_cg);
    mine += w;
    mine_items += items_s[e + 1];
  }
  // Exclusive scans of the 256 threads' sums: within each wavefront, then
  // plus the totals of the wavefronts before it.
  long long incl = mine;
  int incl_items = mine_items;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long y = __shfl_up(incl, off);
    const int yi = __shfl_up(incl_items, off);
    if (lane >= off) {
      incl += y;
      incl_items += yi;
    }
  }
  if (lane == 63) {
    wsum_s[wv] = incl;
    isum_s[wv] = incl_items;
  }
  if (tid == 0) {
    cum_s[0] = 0;
    items_s[0] = 0;
  }
  __syncthreads();
  long long run = incl - mine;
  int run_items = incl_items - mine_items;
  for (int w = 0; w < wv; ++w) {
    run += wsum_s[w];
    run_items += isum_s[w];
  }
  for (int e = e0; e < e0 + per && e < E_local; ++e) {
    run += cum_s[e + 1];
    cum_s[e + 1] = run;
    run_items += items_s[e + 1];
    items_s[e + 1] = run_items;
  }
  __syncthreads();
  for (int e = tid; e <= E_local; e += 256) item_prefix[e] = items_s[e];
  if (tid <= 8) {
    const long long total = cum_s[E_local];
    const int n_items = items_s[E_local];
    int item = tid == 8 ? n_items : 0;
    if (tid > 0 && tid < 8 && total > 0) {
      const long long target = total * tid / 8;
      int lo = 0, hi = E_local;   // largest e with cum[e] <= target
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cum_s[mid] <= target) lo = mid; else hi = mid;
      }
      const int e = lo, nt = prefix[e + 1] - prefix[e], c = offs[e + 1] - offs[e];
      const long long per_cg = nt > 0 ? (cum_s[e + 1] - cum_s[e]) / n_cg : 1;
      long long cg = per_cg > 0 ? (target - cum_s[e]) / per_cg : 0;
      cg = cg < n_cg ? cg : n_cg;
      // The expert's items in proportion (any item boundary will do).
      item = items_s[e] + (int)((long long)(items_s[e + 1] - items_s[e]) * cg / n_cg);
    }
    bounds[tid] = item;
  }
}

__global__ __launch_bounds__(256) void stage_scales_kernel(const uint8_t* __restrict__ act_s,
                                                           int k32, const int32_t* __restrict__ gather,
                                                           int top_k, const int32_t* __restrict__ offs,
                                                           const int32_t* __restrict__ prefix,
                                                           int E_local, int n_cg, int R,
                                                           int n_stages, uint32_t* __restrict__ out,
                                                           int32_t* __restrict__ sched) {
  // The FC kernel launched next takes its items from these counters and
  // ranges.
  if (blockIdx.x == 0) {
    if (threadIdx.x < 8) sched[threadIdx.x * kSchedStride] = 0;
    split_items(offs, prefix, E_local, n_cg, sched + 8 * kSchedStride, sched + kSchedItemPrefix);
  }
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= offs[E_local]) return;
  const int src = gather ? gather[r] / top_k : r;
  const uint8_t* row = act_s + (size_t)src * k32;
  int s = 0;
  if ((k32 & 15) == 0) {
    // 16-byte rows: four stages per load, all of a row's loads in flight.
    for (; s + 4 <= n_stages; s += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + 4 * s);
      out[(size_t)s * R + r] = v.x;
      out[(size_t)(s + 1) * R + r] = v.y;
      out[(size_t)(s + 2) * R + r] = v.z;
      out[(size_t)(s + 3) * R + r] = v.w;
    }
  }
  for (; s < n_stages; ++s) out[(size_t)s * R + r] = reinterpret_cast<const uint32_t*>(row)[s];
}

// Per-lane constants of a workgroup: wavefront, lane, weight half, token
// quarter, lane group and row, and the LDS read offsets within a stage.
struct LaneGeom {
  int wave, lane, hw, qt, g, li;
  int a_lo, a_hi, a_sc, b_op, b_sc;
};

// One item: column group, first grouped row, valid rows, this wavefront's
// token tiles, rows in use (whole 16-row tiles), stages and K.
struct ItemGeom {
  int cg, row_begin, n_valid, nj, rows_used, n_stages, K;
};

// One item with stage layout Ring<P, PAIR> (rows_used <= 64 P): token row
// offsets, the stage loop and the epilogue.  act_r / w_r / s_r are the
// token-row, weight and scale buffers with this lane's offsets w_voff and
// s_voff, advanced by w_step / s_step bytes per stage (s_r: the wavefront's
// token or weight scale dwords; with PAIR the weight scale dwords, and t_r
// the token scale dwords).  it.cg is the wavefront's column group.
template <bool FC1, bool TILED, int P, bool PAIR>
__device__ __forceinline__ void prefill_item(const FcParams& p, uint8_t* lds, const LaneGeom& lg,
                                             const ItemGeom& it, __amdgpu_buffer_rsrc_t act_r,
                                             __amdgpu_buffer_rsrc_t w_r, __amdgpu_buffer_rsrc_t s_r,
                                             __amdgpu_buffer_rsrc_t t_r, const uint32_t (&w_voff)[4],
                                             uint32_t s_voff, uint32_t t_voff, int w_step,
                                             int s_step, int t_step) {
  using RG = Ring<P, PAIR>;
  lds_t* const lds_base = (lds_t*)lds;
  const int wave = lg.wave, lane = lg.lane, hw = lg.hw, qt = lg.qt, g = lg.g, li = lg.li;
  const int a_lo = lg.a_lo, a_hi = lg.a_hi, a_sc = lg.a_sc, b_op = lg.b_op, b_sc = lg.b_sc;
  const int cg = it.cg, row_begin = it.row_begin, n_valid = it.n_valid, nj = it.nj;
  const int rows_used = it.rows_used, n_stages = it.n_stages, K = it.K;
  // LDS place of this wavefront's scale dwords.
  const int s_lds = PAIR       ? RG::kWScaleOff + 256 * wave
                    : wave < 4 ? RG::kTokScaleOff + 256 * wave
                               : RG::kWScaleOff + 256 * (wave - 4);
  // Token rows: wavefront w fills rows 8 (P w + i) + l / 8 (i < P);
  // physical chunk l % 8 of a row takes logical chunk (l % 8) ^ (row & 7).
  // Source rows are all read before any is used, so the gather latencies
  // overlap; rows past the expert's last repeat that row.  Rows of unused
  // tiles get an offset past the buffer's end, which the buffer unit
  // answers with zeros without touching memory (so every wavefront still
  // issues the same loads).
  int src[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int tok = 8 * (P * wave + i) + (lane >> 3);
    const int row = row_begin + min(tok, n_valid - 1);
    src[i] = FC1 ? p.gather[row] : row;
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
    asm volatile("" : "+v"(src[i]));
    if (FC1) src[i] /= p.top_k;
  }
  uint32_t a_voff[P];
  const int ac = (lane & 7) ^ ((lane >> 3) & 7);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int tok = 8 * (P * wave + i) + (lane >> 3);
    a_voff[i] = tok < rows_used ? (uint32_t)src[i] * K + 16 * ac : kOutOfRange;
  }

  // Load q of stage s_load into stage buffer s_load % kNumBuf: q < P a 1 KB
  // piece of token rows, the next kWPieces a weight piece, then the scale
  // dwords (with PAIR: the weight, then the token scale dwords).
  auto issue_load = [&](int q, int s_load) __attribute__((always_inline)) {
    asm volatile("" : "+s"(s_load));
    const int sc = min(s_load, n_stages - 1);
    uint8_t* base = lds + (s_load % RG::kNumBuf) * RG::kStage;
    constexpr int nw = RG::kWPieces;
    if (q < P)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(act_r, base + 1024 * (P * wave + q), 16,
                                               a_voff[q], kKS * sc, 0, 0);
    else if (q < P + nw)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_r, base + RG::kWOff + 1024 * (nw * wave + q - P),
                                               16, w_voff[q - P], w_step * sc, 0, 0);
    else if (!PAIR || q == P + nw)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_r, base + s_lds, 4, s_voff, s_step * sc, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t_r, base + RG::kTokScaleOff + 256 * (wave % P), 4,
                                               t_voff, t_step * sc, 0, 0);
  };

  // Stage buffer of stage s.  The offset is made opaque so that the compiler
  // cannot prove later tiles' reads in bounds and hoist them.
  auto stage_buf = [&](int s) __attribute__((always_inline)) {
    int off = (s % RG::kNumBuf) * RG::kStage;
    asm volatile("" : "+s"(off));
    return static_cast<const lds_t*>(lds_base) + off;
  };

  // The stage loop for a wavefront holding NJ valid token tiles (a
  // compile-time count, so no accumulator is conditionally updated).
  auto run = [&](auto nji) __attribute__((always_inline)) {
    constexpr int NJ = decltype(nji)::value;
    v4f acc[NJ > 0 ? NJ : 1][2][4];  // [token tile j][unit k][row block i]
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[j][k][i] = v4f{0.f, 0.f, 0.f, 0.f};
          asm volatile("" : "+a"(acc[j][k][i]));   // distinct registers from the start
        }
    AOp abuf[2];
    v4i bw[2][4];   // weight operands of the stage: [unit k][row block i]
    int bs[2][4];

    // Operands of stage s's start: tile 0 and the weights.
    auto read_start = [&](int s) __attribute__((always_inline)) {
      if constexpr (NJ > 0) {
        const lds_t* A = stage_buf(s);
        abuf[0].sc = A[RG::kTokScaleOff + a_sc];
        abuf[0].lo = *reinterpret_cast<const lds_v4i*>(A + a_lo);
        abuf[0].hi = *reinterpret_cast<const lds_v4i*>(A + a_hi);
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bw[k][i] =
                *reinterpret_cast<const lds_v4i*>(A + RG::kWOff + b_op + 4096 * k + 1024 * i);
            bs[k][i] = A[RG::kWScaleOff + b_sc + 256 * k + 64 * i];
          }
      }
      asm volatile("" ::: "memory");
    };
    // Global load slot of MFMA m of tile j: with two or more tiles, the odd
    // MFMAs of tiles 0 and 1 carry loads 0..3 and 4..; with one tile, MFMAs
    // 0.. carry one each.
    auto load_slot = [](int j, int m) constexpr -> int {
      if (NJ == 1) return m < RG::kLoads ? m : -1;
      if (j > 1 || !(m & 1)) return -1;
      const int q = 4 * j + (m >> 1);
      return q < RG::kLoads ? q : -1;
    };
    // One stage: per tile j, 8 MFMAs; after MFMAs 0..2 one read of tile
    // j + 1's operands, and the global loads of stage s + kAhead in their
    // slots.
    auto compute = [&](int s) __attribute__((always_inline)) {
      const lds_t* A = stage_buf(s);
      if constexpr (NJ == 0) {
#pragma unroll
        for (int q = 0; q < RG::kLoads; ++q) issue_load(q, s + RG::kAhead);
      } else {
        auto tile_fn = [&](auto ji) __attribute__((always_inline)) {
          constexpr int j = decltype(ji)::value;
          AOp& cur = abuf[j & 1];
          AOp& nxt = abuf[(j + 1) & 1];
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const int k = m >> 2, i = m & 3;
            acc[j][k][i] = mfma_w4a8<0>(bw[k][i], cur.lo, cur.hi, acc[j][k][i], bs[k][i], cur.sc);
            if constexpr (j + 1 < NJ) {
              constexpr int t1 = RG::kTileStep * (j + 1);   // tiles past the wavefront's first
              if (m == 0) nxt.sc = A[RG::kTokScaleOff + a_sc + 64 * t1];
              if (m == 1) nxt.lo = *reinterpret_cast<const lds_v4i*>(A + a_lo + 2048 * t1);
              if (m == 2) nxt.hi = *reinterpret_cast<const lds_v4i*>(A + a_hi + 2048 * t1);
            }
            if (load_slot(j, m) >= 0) issue_load(load_slot(j, m), s + RG::kAhead);
          }
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
            if (j + 1 < NJ && m < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            if (load_slot(j, m) >= 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        };
        static_for<0, NJ>(tile_fn);
      }
    };

    constexpr int kInFlight = (RG::kAhead - 1) * RG::kLoads;
#pragma unroll
    for (int a = 0; a < RG::kAhead; ++a) {
#pragma unroll
      for (int q = 0; q < RG::kLoads; ++q) issue_load(q, a);
      asm volatile("" ::: "memory");
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kInFlight) : "memory");   // stage 0's loads
    asm volatile("s_barrier" ::: "memory");
    read_start(0);
    // Step s: the stage's MFMAs and stage s + kAhead's loads, the wait for
    // stage s + 1 (issued kAhead - 1 steps back; the loads of the stages
    // after it stay in flight), the barrier (stage s + 1 landed everywhere,
    // stage s's buffer free), and stage s + 1's first operands.
    for (int s = 0; s < n_stages; ++s) {
      compute(s);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kInFlight) : "memory");
      asm volatile("s_barrier" ::: "memory");
      if (s + 1 < n_stages) read_start(s + 1);
    }
    // Drain the reloads issued past the end before the ring is reused.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");

#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      pin_acc_agpr(acc[j][0]);
      pin_acc_agpr(acc[j][1]);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int t_in = 16 * (qt + RG::kTileStep * j) + li;
#pragma unroll
      for (int k = 0; k < 2; ++k)
        store_subtile<FC1>(p, acc[j][k], row_begin + t_in, t_in < n_valid, 4 * cg + 2 * hw + k, g);
    }
  };
  // At most 64 P rows in use make at most 4 P tiles, so a wavefront
  // holds at most P of them (with PAIR, at most 2 P).
  if constexpr (PAIR && P == 1) {
    switch (nj) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      default: run(std::integral_constant<int, 2>{}); break;
    }
  } else if constexpr (PAIR) {
    switch (nj) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      default: run(std::integral_constant<int, 4>{}); break;
    }
  } else if constexpr (P == 1) {
    if (nj == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
  } else if constexpr (P == 2) {
    switch (nj) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      default: run(std::integral_constant<int, 2>{}); break;
    }
  } else {
    switch (nj) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      default: run(std::integral_constant<int, 4>{}); break;
    }
  }
}

template <bool FC1, bool TILED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fc_prefill_kernel(FcParams p, int n_cg) {
  // One LDS object: the stage ring, then the expert tile prefix and row
  // offsets (read once per workgroup), then the current item.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  int* const prefix_s = reinterpret_cast<int*>(lds + kRingBytes);
  int* const offs_s = prefix_s + kMaxLdsExperts + 1;
  int* const item_s = offs_s + kMaxLdsExperts + 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wavefront
  const int hw = wave & 1, qt = wave >> 1;                     // weight half, token quarter
  const int g = lane >> 4, li = lane & 15;
  const int K = p.K;
  const int n_stages = K / kKS;
  for (int i = tid; i <= p.E_local; i += kThreads) {
    prefix_s[i] = p.sched[kSchedItemPrefix + i];
    offs_s[i] = p.expert_offsets[i];
  }
  __syncthreads();
  const int xcd = blockIdx.x & 7;
  // Ranges a workgroup may take items from: its own XCD's, then, when the
  // launch has at least 8 rounds of items, the other XCDs' in turn (below).
  const int32_t* const bounds = p.sched + 8 * kSchedStride;
  const int n_ranges = bounds[8] - bounds[0] >= 8 * (int)gridDim.x ? 8 : 1;
  int victim = 0;   // thread 0: the range it claims from is XCD xcd + victim's
  const __amdgpu_buffer_rsrc_t act_r = rsrc(p.act, (uint32_t)(p.act_rows * K));

  // LDS read offsets within a stage (lane parts; the tile's part and the
  // stage layout's region offsets go into the immediate): token tile
  // tt = qt + 4 j at 2048 tt, its scale bytes at 64 tt; weight operand
  // (unit 2 hw + k, block i) is 1 KB piece 4 (2 hw + k) + i, lane (li, g) at
  // position 4 li + (g ^ ((li >> 1) & 3)); its scale byte is byte g of row
  // 64 (2 hw + k) + 16 i + li's dword.
  const int a_lo = 2048 * qt + li * kKS + 16 * (g ^ (li & 7));
  const int a_hi = 2048 * qt + li * kKS + 16 * ((4 + g) ^ (li & 7));
  const int a_sc = 64 * qt + 4 * li + g;
  const int b_op = 8192 * hw + 16 * (4 * li + (g ^ ((li >> 1) & 3)));
  const int b_sc = 512 * hw + 4 * li + g;

  // The workgroups of one XCD take its items in order from a shared counter,
  // so the items in flight are always a short run of neighbours (the column
  // groups of one tile, reading the same token rows from L2) however long
  // each item takes.  Over many rounds the ranges' estimated work can leave
  // an XCD a round or more behind the rest, so a workgroup whose own range
  // is exhausted goes on to the next XCDs' ranges, one after the other, and
  // takes their next items (each item is still claimed exactly once, by the
  // atomic on its range's counter, and nothing waits).  With fewer rounds
  // every XCD reaches its last round at about the same time, and a taken
  // item would only move to a CU whose L2 lacks its rows: then each
  // workgroup keeps to its own range.
  for (;;) {
    if (tid == 0) {
      int it = -1;
      for (; victim < n_ranges; ++victim) {
        const int x = (xcd + victim) & 7;
        const int lo = bounds[x], hi = bounds[x + 1];
        if (lo >= hi) continue;
        const int c = lo + atomicAdd(p.sched + x * kSchedStride, 1);
        if (c < hi) {
          it = c;
          break;
        }
      }
      item_s[0] = it;
    }
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(item_s[0]);
    if (item < 0) break;
    const int e = __builtin_amdgcn_readfirstlane(find_expert_lds(prefix_s, p.E_local, item));
    const int local = item - __builtin_amdgcn_readfirstlane(prefix_s[e]);
    // An expert with at most kPairRows rows runs as pairs of column groups:
    // its item i takes column groups 2 i and 2 i + 1.
    const int e_rows = __builtin_amdgcn_readfirstlane(offs_s[e + 1]) -
                       __builtin_amdgcn_readfirstlane(offs_s[e]);
    const int nt = (e_rows + kBM - 1) / kBM;
    // Items of a larger expert run in groups of kTileGroup tiles: within a
    // group, column group by column group, tile by tile.  The items in
    // flight then cover about 8 column groups x 4 tiles of a hot expert (its
    // weights shared by 4 tiles, each tile's rows by 8 column groups) instead
    // of 3 column groups x 10 tiles, which needs fewer bytes from memory.
    // The last group (1..kTileGroup tiles) holds the last tile; one of at
    // most kPairRows rows is a pair item after the other tiles' items of its
    // two column groups (their weights still in L2).
    const int full = (nt - 1) / kTileGroup, in_full = n_cg * kTileGroup * full;
    int cg0, t_in_e;   // first column group, tile
    bool pair = e_rows <= kPairRows;
    if (pair) {
      cg0 = 2 * local;
      t_in_e = 0;
    } else if (local < in_full) {
      const int grp = local / (n_cg * kTileGroup), r = local - grp * n_cg * kTileGroup;
      cg0 = r / kTileGroup;
      t_in_e = grp * kTileGroup + (r - cg0 * kTileGroup);
    } else {
      const int rem = nt - full * kTileGroup, r = local - in_full;
      if (e_rows - kBM * (nt - 1) <= kPairRows) {
        const int per = 2 * rem - 1, cgp = r / per, x = r - cgp * per;
        if (x < 2 * (rem - 1)) {
          cg0 = 2 * cgp + x / (rem - 1);
          t_in_e = full * kTileGroup + x % (rem - 1);
        } else {
          cg0 = 2 * cgp;
          t_in_e = nt - 1;
          pair = true;
        }
      } else {
        cg0 = r / rem;
        t_in_e = full * kTileGroup + (r - cg0 * rem);
      }
    }
    const int cg = pair ? cg0 + (wave >> 2) : cg0;   // this wavefront's column group
    const int row_begin = __builtin_amdgcn_readfirstlane(offs_s[e]) + t_in_e * kBM;
    const int n_valid = min(__builtin_amdgcn_readfirstlane(offs_s[e + 1]) - row_begin, kBM);
    const int ntiles = (n_valid + 15) >> 4;                      // 16-row tiles in use
    const int th = (wave >> 1) & 1;                              // token half of a pair item
    const int nj = pair ? (ntiles > th ? (ntiles - th + 1) >> 1 : 0)
                        : (ntiles > qt ? (ntiles - qt + 3) >> 2 : 0);   // this wavefront's tiles
    const int rows_used = 16 * ntiles;

    // Weight pieces: wavefront w copies 1 KB pieces c = 2 w, 2 w + 1 (unit
    // c / 4, row block c % 4); of a pair, pieces c = 4 w .. 4 w + 3 of the
    // two column groups' 32 pieces (column group c / 16).  Scale dwords:
    // wavefronts 0..3 copy token rows 64 w + l, wavefronts 4..7 weight rows
    // 64 (w - 4) + l; of a pair, wavefront w copies weight rows 64 w + l of
    // the two column groups' 512 and token rows 64 (w % P) + l.
    __amdgpu_buffer_rsrc_t w_r, s_r, t_r = act_r;
    uint32_t w_voff[4] = {0u, 0u, 0u, 0u}, s_voff, t_voff = kOutOfRange;
    int w_step, s_step, t_step = 0;
    const int nwp = pair ? 4 : 2;            // weight pieces per wavefront
    if (TILED) {
      const size_t blk0 = tiled_block(e, cg0 >> 1, 0, n_cg >> 1, n_stages);
      w_r = rsrc(p.w + blk0 * kTileBytes + (pair ? 0 : 16384 * (cg & 1)),
                 (uint32_t)n_stages * kTileBytes);
      w_step = kTileBytes;
#pragma unroll
      for (int x = 0; x < 4; ++x) w_voff[x] = 1024 * (nwp * wave + x) + 16 * lane;
    } else {
      const size_t e_rows_off = (size_t)e * p.N;
      w_r = rsrc(p.w + e_rows_off * (K / 2), (uint32_t)p.N * (K / 2));
      w_step = 64;
      // Position l of a piece holds row l / 4 of the block and logical
      // 16-byte chunk (l & 3) ^ ((l >> 3) & 3) (the tiled layout's order).
      const int r = lane >> 2, ch = (lane & 3) ^ ((lane >> 3) & 3);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int c = nwp * wave + x, u = 4 * (cg0 + (c >> 4)) + ((c & 15) >> 2), i = c & 3;
        const int rb = FC1 ? (i < 2 ? 0 : p.I) + 32 * u + 16 * (i & 1) : 64 * u + 16 * i;
        w_voff[x] = (uint32_t)(rb + r) * (K / 2) + 16 * ch;
      }
    }
    // Token scale dwords of stage s: the contiguous run act_st[s][row_begin ..],
    // one coalesced piece per wavefront.
    const __amdgpu_buffer_rsrc_t st_r = rsrc(p.act_st, (uint32_t)(n_stages * p.n_routes * 4));
    const int st_step = (int)(4 * p.n_routes);
    if (pair) {
      t_r = st_r;
      t_step = st_step;
      // Wavefront w copies token rows 64 (w % P) + l (P = 1 or 2 pieces
      // of 64 rows; the wavefronts with equal w % P write the same bytes).
      const int tok = 64 * (wave % (rows_used <= 64 ? 1 : 2)) + lane;
      t_voff = tok < rows_used ? 4u * (uint32_t)(row_begin + tok) : kOutOfRange;
    }
    if (!pair && wave < 4) {
      s_r = st_r;
      s_step = st_step;
      const int tok = 64 * wave + lane;
      s_voff = tok < rows_used ? 4u * (uint32_t)(row_begin + tok) : kOutOfRange;
    } else {
      const int r = pair ? 64 * wave + lane : 64 * (wave - 4) + lane;   // of the item's rows
      if (TILED) {
        const size_t blk0 = tiled_block(e, cg0 >> 1, 0, n_cg >> 1, n_stages);
        s_r = rsrc(p.w_s + blk0 * kTileScaleBytes + (pair ? 0 : 1024 * (cg & 1)),
                   (uint32_t)n_stages * kTileScaleBytes);
        s_step = kTileScaleBytes;
        s_voff = 4 * r;
      } else {
        const size_t e_rows_off = (size_t)e * p.N;
        s_r = rsrc(p.w_s + e_rows_off * (K / 32), (uint32_t)p.N * (K / 32));
        s_step = 4;
        const int rr = r & 255, u = 4 * (cg0 + (r >> 8)) + (rr >> 6), i = (rr >> 4) & 3;
        const int rb = FC1 ? (i < 2 ? 0 : p.I) + 32 * u + 16 * (i & 1) : 64 * u + 16 * i;
        s_voff = (uint32_t)(rb + (rr & 15)) * (K / 32);
      }
    }

    // The rest depends on the stage layout, chosen by the rows in use.
    const ItemGeom it{cg, row_begin, n_valid, nj, rows_used, n_stages, K};
    if (pair) {
      // Token tiles th, th + 2; the weight operands of column group w >> 2.
      const int c = wave >> 2;
      const LaneGeom lg{wave, lane, hw, th, g, li, a_lo - 2048 * (qt - th), a_hi - 2048 * (qt - th),
                        a_sc - 64 * (qt - th), b_op + 16384 * c, b_sc + 1024 * c};
      if (rows_used <= 64)
        prefill_item<FC1, TILED, 1, true>(p, lds, lg, it, act_r, w_r, s_r, t_r, w_voff, s_voff,
                                          t_voff, w_step, s_step, t_step);
      else
        prefill_item<FC1, TILED, 2, true>(p, lds, lg, it, act_r, w_r, s_r, t_r, w_voff, s_voff,
                                          t_voff, w_step, s_step, t_step);
    } else {
      const LaneGeom lg{wave, lane, hw, qt, g, li, a_lo, a_hi, a_sc, b_op, b_sc};
      if (rows_used <= 64)
        prefill_item<FC1, TILED, 1, false>(p, lds, lg, it, act_r, w_r, s_r, t_r, w_voff, s_voff,
                                           t_voff, w_step, s_step, t_step);
      else if (rows_used <= 128)
        prefill_item<FC1, TILED, 2, false>(p, lds, lg, it, act_r, w_r, s_r, t_r, w_voff, s_voff,
                                           t_voff, w_step, s_step, t_step);
      else
        prefill_item<FC1, TILED, 4, false>(p, lds, lg, it, act_r, w_r, s_r, t_r, w_voff, s_voff,
                                           t_voff, w_step, s_step, t_step);
    }
  }
}

}  // namespace

bool prefill_shape_ok(const FcParams& prm, bool fc1) {
  // FC1: 128 intermediate columns (256 w13 rows) per tile and whole 512-row
  // groups of the tiled layout (I % 256); FC2: 256 output columns per tile,
  // whole 512-row groups (H % 512).  Buffer offsets are 32-bit: the
  // activation array and one expert's weights must each stay below 2 GiB.
  // The expert metadata is kept in LDS: at most kMaxLdsExperts local experts.
  // The restaged scales (K/32 bytes per grouped row) need 32-bit offsets too.
  const int64_t K = prm.K;
  return K % kKS == 0 && (fc1 ? prm.I % 256 == 0 : prm.N % 512 == 0) && prm.E_local <= kMaxLdsExperts &&
         prm.act_rows * K < ((int64_t)1 << 31) && (int64_t)prm.N * (K / 2) < ((int64_t)1 << 31) &&
         prm.n_routes * (K / 32) < ((int64_t)1 << 31) && prm.act_st != nullptr &&
         prm.sched != nullptr;
}

hipError_t launch_fc_prefill(bool fc1, bool tiled, FcParams prm, const int32_t* tile_prefix_all,
                             int n_cu, hipStream_t stream) {
  prm.tile_prefix = tile_prefix_all + (size_t)kTilePrefixIndex * (prm.E_local + 1);
  const int n_cg = fc1 ? prm.I / 128 : prm.N / kBN;
  // Persistent grid: one workgroup per CU, a multiple of the 8 XCDs.
  const int n_wg = (n_cu > 8 ? n_cu : 8) & ~7;
  const int n_stages = prm.K / kKS;
  const int R = (int)prm.n_routes;
  if (R > 0) {
    hipLaunchKernelGGL(stage_scales_kernel, dim3((R + 255) / 256), dim3(256), 0, stream, prm.act_s,
                       prm.K / 32, fc1 ? prm.gather : nullptr, prm.top_k, prm.expert_offsets,
                       prm.tile_prefix, prm.E_local, n_cg, R, n_stages, prm.act_st, prm.sched);
  }
  const dim3 grid(n_wg), block(kThreads);
  if (fc1 && tiled)
    hipLaunchKernelGGL((fc_prefill_kernel<true, true>), grid, block, 0, stream, prm, n_cg);
  else if (fc1)
    hipLaunchKernelGGL((fc_prefill_kernel<true, false>), grid, block, 0, stream, prm, n_cg);
  else if (tiled)
    hipLaunchKernelGGL((fc_prefill_kernel<false, true>), grid, block, 0, stream, prm, n_cg);
  else
    hipLaunchKernelGGL((fc_prefill_kernel<false, false>), grid, block, 0, stream, prm, n_cg);
  return hipGetLastError();
}

}  // namespace mi355moe
