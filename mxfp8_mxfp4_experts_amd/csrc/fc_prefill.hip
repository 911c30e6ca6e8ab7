// Prefill-shaped FC1 / FC2 (many grouped rows per expert).
//
// Same method as the decode-shaped kernel (page 1, "Serving 调用链": grouped
// GEMM1 -> gated activation -> GEMM2; "真实 checkpoint 契约": [gate; up] halves,
// SiTU(4, 25); page 5: w13 / w2 and scale layouts), organised for experts
// that hold tens to hundreds of grouped rows:
//   * a workgroup of 4 wavefronts (one per SIMD, each with the whole register
//     file) computes up to 256 grouped rows of one expert against 256 weight
//     rows.  Wavefront w owns one 64-row unit (FC1: gate rows [c, c+32) with
//     up rows [I+c, I+c+32), so SiTU pairs stay in one wavefront; FC2: 64
//     output columns) and all 256 token rows: 4 row blocks x 16 token tiles
//     of 16x16 accumulators, 256 AGPRs;
//   * an expert with at most 256 rows is one tile, so its weights are read
//     once in total; its token rows are re-read by every column group, which
//     the XCD-contiguous schedule keeps in that XCD's L2.  The tiles of a hot
//     expert run side by side on one column group, sharing its weights;
//   * weights go from memory straight to registers: one coalesced 16-byte
//     load per lane per 16-row block and stage (in the tiled layout each
//     block's MFMA operand is one contiguous 1 KB piece in lane order), three
//     stages ahead in four rotating register sets;
//   * token rows go through a ring of 4 LDS stages (256 rows x 128 bytes +
//     one scale dword per row), filled by direct buffer -> LDS loads three
//     stages ahead; 16-byte chunks are XOR-swizzled by row bits 0..2 so the
//     eight lanes served together hit eight bank groups;
//   * token tiles are taken in pairs; pairs past the expert's last row are
//     skipped (at most one empty 16-row tile is computed).  Each of a pair's
//     8 MFMAs is followed by one LDS read of the next pair and, on odd ones,
//     one global load of stage s + 3, so reads and loads issue under the
//     MFMAs rather than in bursts.  Every wavefront issues the same 17 loads
//     per stage (9 direct-to-LDS, then 8 to registers), so one fixed
//     "s_waitcnt vmcnt" per stage leaves exactly the later stages in flight;
//     past the last stage the final stage is reloaded to keep that count;
//   * buffer resources keep every per-lane address a 32-bit offset.
#include "common.h"
#include "fc_common.h"
#include "launch.h"
#include "tiled.h"

#include <type_traits>

namespace mi355moe {

namespace {

constexpr int kBM = 256;                    // token rows per tile
constexpr int kBN = 256;                    // weight rows per tile (4 units)
constexpr int kKS = 128;                    // K per stage
constexpr int kABytes = kBM * kKS;          // 32768: E4M3 token slice
constexpr int kASBytes = kBM * 4;           // 1024: one scale dword per token row
constexpr int kStage = kABytes + kASBytes;  // 33792
constexpr int kNumBuf = 4;                  // LDS ring depth
constexpr int kThreads = 256;
constexpr int kTilePrefixIndex = 4;         // tile height 16 << 4 = 256
constexpr int kNt = 2;                      // nontemporal policy for weight loads
static_assert(kKS == kTileK && 2 * kBN == kTileRows, "tile shape");
static_assert((16 << kTilePrefixIndex) == kBM && kTilePrefixIndex < kNumTileSizes, "tile prefix");

// Loads issued per wavefront and stage: 9 direct-to-LDS (token rows and
// their scales), then 8 to registers (weight blocks and scale bytes).  When
// stage s is waited for (token rows and weights), the loads issued after it
// are the next two stages': 2 * 17 = 34.
constexpr int kActLoads = 9, kWLoads = 8;
constexpr int kLoadsPerStage = kActLoads + kWLoads;
constexpr int kWaitCount = 2 * kLoadsPerStage;   // 34
static_assert(kWaitCount < 64, "vmcnt range");
// First load of each tile pair's share (pair 7 issues none).
constexpr int kLoadStart[9] = {0, 3, 6, 9, 11, 13, 15, 17, 17};

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

typedef __attribute__((address_space(3))) uint8_t lds_t;
typedef __attribute__((address_space(3))) v4i lds_v4i;

// Weight operands of one stage for one wavefront: 4 row blocks.
struct WStage {
  v4i w[4];
  int s[4];
};

// Token operands of one 16-row tile: K [16g, +16) and [64 + 16g, +16) for
// lane group g, and the row's scale byte for MX block g.
struct AOp {
  v4i lo, hi;
  int sc;
};

template <bool FC1, bool TILED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fc_prefill_kernel(FcParams p, int n_cg) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kNumBuf * kStage];
  lds_t* const lds_base = (lds_t*)lds;   // LDS address space: immediate offsets fold
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wavefront
  const int g = lane >> 4, li = lane & 15;
  const int K = p.K;
  const int n_stages = K / kKS;
  const int* prefix = p.tile_prefix;
  const int n_items = prefix[p.E_local] * n_cg;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
  const int item_lo = (int)((int64_t)n_items * xcd / 8);
  const int item_hi = (int)((int64_t)n_items * (xcd + 1) / 8);
  const __amdgpu_buffer_rsrc_t act_r = rsrc(p.act, (uint32_t)(p.act_rows * K));
  const __amdgpu_buffer_rsrc_t acts_r = rsrc(p.act_s, (uint32_t)(p.act_rows * (K / 32)));

  // Items run expert by expert; inside an expert column group by column
  // group, and inside a column group tile by tile: neighbouring items share
  // either the weights (tiles of one hot expert) or the token rows (column
  // groups of one tile).  Expert e owns items [n_cg prefix[e], n_cg prefix[e+1]).
  for (int item = item_lo + slot; item < item_hi; item += per_xcd) {
    const int e = __builtin_amdgcn_readfirstlane(find_expert(prefix, p.E_local, item / n_cg));
    const int nt = prefix[e + 1] - prefix[e];
    const int local = item - prefix[e] * n_cg;
    const int cg = local / nt, t_in_e = local - cg * nt;
    const int row_begin = p.expert_offsets[e] + t_in_e * kBM;
    const int n_valid = min(p.expert_offsets[e + 1] - row_begin, kBM);
    const int npairs = (n_valid + 31) >> 5;                     // token tile pairs in use
    const int unit = 4 * cg + wave;                             // global 64-row unit

    // Weights of row block i of this wavefront's unit (rows 16 i + li):
    // lane offset + SGPR offset per block and stage.  Each lane reads only
    // its scale byte (MX block 4 s + g of its row).
    __amdgpu_buffer_rsrc_t w_r, ws_r;
    uint32_t w_voff, ws_voff;
    int w_soff[4], ws_soff[4], w_step, ws_step;
    if (TILED) {
      // 512-row group cg / 2 holds units 8 (cg / 2) .. + 7; this unit is its
      // (4 (cg & 1) + wave)-th.
      const int u8 = 4 * (cg & 1) + wave;
      const size_t blk0 = tiled_block(e, cg >> 1, 0, n_cg >> 1, n_stages);
      w_r = rsrc(p.w + blk0 * kTileBytes, (uint32_t)n_stages * kTileBytes);
      ws_r = rsrc(p.w_s + blk0 * kTileScaleBytes, (uint32_t)n_stages * kTileScaleBytes);
      w_voff = 4096 * u8 + 16 * (4 * li + (g ^ ((li >> 1) & 3)));
      ws_voff = 4 * (64 * u8 + li) + g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w_soff[i] = 1024 * i;
        ws_soff[i] = 64 * i;
      }
      w_step = kTileBytes;
      ws_step = kTileScaleBytes;
    } else {
      const size_t e_rows = (size_t)e * p.N;
      w_r = rsrc(p.w + e_rows * (K / 2), (uint32_t)p.N * (K / 2));
      ws_r = rsrc(p.w_s + e_rows * (K / 32), (uint32_t)p.N * (K / 32));
      w_voff = li * (K / 2) + 16 * g;
      ws_voff = li * (K / 32) + g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // FC1: blocks 0, 1 are gate rows 32 unit + 16 i, blocks 2, 3 the
        // matching up rows I + 32 unit + 16 (i - 2); FC2: rows 64 unit + 16 i.
        const int rb = FC1 ? (i < 2 ? 0 : p.I) + 32 * unit + 16 * (i & 1) : 64 * unit + 16 * i;
        w_soff[i] = rb * (K / 2);
        ws_soff[i] = rb * (K / 32);
      }
      w_step = 64;
      ws_step = 4;
    }
    // Token rows: wavefront w fills rows 64 w + 8 i + l / 8 (i < 8); physical
    // chunk l % 8 of a row takes logical chunk (l % 8) ^ (row & 7).  Scale
    // dwords: rows 64 w + l.  Rows past the expert's last, inside the last
    // tile pair, repeat that row; rows of skipped pairs get an offset past
    // the buffer's end, which the buffer unit answers with zeros without
    // touching memory (so every wavefront still issues the same loads).
    uint32_t a_voff[8];
    const int ac = (lane & 7) ^ ((lane >> 3) & 7);
    const int rows_used = 32 * npairs;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = 64 * wave + 8 * i + (lane >> 3);
      const int row = row_begin + min(tok, n_valid - 1);
      const int src = FC1 ? p.gather[row] / p.top_k : row;
      a_voff[i] = tok < rows_used ? (uint32_t)src * K + 16 * ac : kOutOfRange;
    }
    uint32_t as_voff;
    {
      const int tok = 64 * wave + lane;
      const int row = row_begin + min(tok, n_valid - 1);
      const int src = FC1 ? p.gather[row] / p.top_k : row;
      as_voff = tok < rows_used ? (uint32_t)src * (K / 32) : kOutOfRange;
    }

    // Load q (0..16) of stage s_load: q < 8 a 1 KB piece of token rows, q = 8
    // the token scale dwords (direct to LDS, stage buffer s_load % 4); q < 13
    // a weight block, q < 17 a weight scale byte (to register set ws).
    auto issue_load = [&](int q, WStage& ws, int s_load) __attribute__((always_inline)) {
      // Recomputed per load (cheap scalar work) rather than kept in scalar
      // registers across the loop.
      asm volatile("" : "+s"(s_load));
      const int sc = min(s_load, n_stages - 1);
      uint8_t* base = lds + (s_load % kNumBuf) * kStage;
      if (q < 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(act_r, base + wave * 8192 + q * 1024, 16,
                                                 a_voff[q], kKS * sc, 0, 0);
      else if (q == 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(acts_r, base + kABytes + wave * 256, 4, as_voff,
                                                 4 * sc, 0, 0);
      else if (q < 13)
        // Weight loads are issued in assembly so that the compiler does not
        // place its own (conservative) waits for them; the stage-end wait
        // covers them and the registers are re-pinned after it.
        asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen nt"
                     : "=v"(ws.w[q - 9])
                     : "v"(w_voff), "s"(w_r), "s"(w_soff[q - 9] + sc * w_step));
      else
        asm volatile("buffer_load_ubyte %0, %1, %2, %3 offen"
                     : "=v"(ws.s[q - 13])
                     : "v"(ws_voff), "s"(ws_r), "s"(ws_soff[q - 13] + sc * ws_step));
    };

    v4f acc[16][4];  // [token tile][row block]
#pragma unroll
    for (int tt = 0; tt < 16; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[tt][i] = v4f{0.f, 0.f, 0.f, 0.f};

    // Token operands of tile tt from stage buffer A: lane parts of the
    // addresses here, the tile's part (2048 tt, or 64 tt for the scale byte)
    // goes into the LDS instructions' immediate offset.
    const int a_lo = li * kKS + 16 * (g ^ (li & 7));
    const int a_hi = li * kKS + 16 * ((4 + g) ^ (li & 7));
    const int a_sc = kABytes + 4 * li + g;
    auto read_a = [&](AOp& o, const lds_t* A, int tt) __attribute__((always_inline)) {
      o.lo = *reinterpret_cast<const lds_v4i*>(A + a_lo + 2048 * tt);
      o.hi = *reinterpret_cast<const lds_v4i*>(A + a_hi + 2048 * tt);
      o.sc = A[a_sc + 64 * tt];
    };
    // Stage buffer of stage s.  The offset is made opaque so that the compiler
    // cannot prove later pairs' reads in bounds and hoist them above the pair
    // conditions (which would hold every pair's operands at once).
    auto stage_buf = [&](int s) __attribute__((always_inline)) {
      int off = (s % kNumBuf) * kStage;
      asm volatile("" : "+s"(off));
      return static_cast<const lds_t*>(lds_base) + off;
    };

    AOp buf[2][2];   // [pair parity][tile of the pair]
    // One stage.  Pair pp: 8 MFMAs; after MFMA j < 6 one LDS read of pair
    // pp + 1, after MFMAs 1, 3, 5 the pair's share of the 17 global loads of
    // stage s + 3 (token rows into the buffer stage s - 1 used, weights into
    // register set nw), so neither the reads nor the loads stall the MFMAs.
    // Skipped pairs still issue their loads: every stage issues the same 17,
    // token rows (0..8) before weights (9..16).  Pair 0's operands were read
    // before the call.
    auto compute = [&](const WStage& ws, WStage& nw, int s) __attribute__((always_inline)) {
      const lds_t* A = stage_buf(s);
      auto pair_fn = [&](auto ppi) __attribute__((always_inline)) {
        constexpr int pp = decltype(ppi)::value;
        constexpr int q0 = kLoadStart[pp], q1 = kLoadStart[pp + 1];
        if (pp < npairs) {
          AOp(&cur)[2] = buf[pp & 1];
          AOp(&nxt)[2] = buf[(pp + 1) & 1];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int h = j >> 2, i = j & 3;
            acc[2 * pp + h][i] =
                mfma_w4a8<0>(ws.w[i], cur[h].lo, cur[h].hi, acc[2 * pp + h][i], ws.s[i], cur[h].sc);
            if constexpr (pp + 1 < 8) {
              // Both scale bytes, then tile 0's operand, then tile 1's (the
              // next pair's first MFMAs wait only for what they use).
              if (j < 2) nxt[j].sc = A[a_sc + 64 * (2 * pp + 2 + j)];
              const int t = 2 * pp + 2 + (j >= 4);
              if (j == 2 || j == 4) nxt[j / 4].lo = *reinterpret_cast<const lds_v4i*>(A + a_lo + 2048 * t);
              if (j == 3 || j == 5) nxt[j / 5].hi = *reinterpret_cast<const lds_v4i*>(A + a_hi + 2048 * t);
            }
            if ((j & 1) && q0 + (j >> 1) < q1) issue_load(q0 + (j >> 1), nw, s + 3);
          }
          // Keep this pair's MFMAs inside its condition (the compiler would
          // otherwise sink them below the later pairs), in the order above.
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) asm volatile("" : "+a"(acc[2 * pp + h][i]));
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
            if (pp + 1 < 8 && j < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            if ((j & 1) && q0 + (j >> 1) < q1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int q = q0; q < q1; ++q) issue_load(q, nw, s + 3);
        }
      };
      static_for<0, 8>(pair_fn);
    };

    // After the stage-end wait the next stage's weights are in their
    // registers: re-define them there so no use can move above the wait.
    auto pin_w = [&](WStage& w) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(w.w[i]), "+v"(w.s[i]));
    };
    // Step s (set cur holds stage s's weights, nw takes stage s + 3's, next
    // holds stage s + 1's): the stage's MFMAs and loads, then the wait for
    // stage s + 1 (its 17 loads were issued two steps back, followed by the 17
    // of each later step: 34), the barrier (stage s + 1 landed everywhere,
    // stage s's buffer free), stage s + 1's first pair.
    auto step = [&](const WStage& cur, WStage& nw, WStage& next, int s) __attribute__((always_inline)) {
      compute(cur, nw, s);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaitCount) : "memory");
      asm volatile("s_barrier" ::: "memory");
      pin_w(next);
      const lds_t* An = stage_buf(s + 1);
      read_a(buf[0][0], An, 0);
      read_a(buf[0][1], An, 1);
      asm volatile("" ::: "memory");
    };
    WStage w0, w1, w2, w3;
#pragma unroll
    for (int q = 0; q < kLoadsPerStage; ++q) issue_load(q, w0, 0);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < kLoadsPerStage; ++q) issue_load(q, w1, 1);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < kLoadsPerStage; ++q) issue_load(q, w2, 2);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaitCount) : "memory");   // stage 0's loads
    asm volatile("s_barrier" ::: "memory");
    pin_w(w0);
    {
      const lds_t* A0 = stage_buf(0);
      read_a(buf[0][0], A0, 0);
      read_a(buf[0][1], A0, 1);
    }
    asm volatile("" ::: "memory");
    // Stage loop, unrolled by 4 so each register set keeps a fixed name.
    int s = 0;
    for (; s + 4 <= n_stages; s += 4) {
      step(w0, w3, w1, s);
      step(w1, w0, w2, s + 1);
      step(w2, w1, w3, s + 2);
      step(w3, w2, w0, s + 3);
    }
    if (s < n_stages) step(w0, w3, w1, s);
    if (s + 1 < n_stages) step(w1, w0, w2, s + 1);
    if (s + 2 < n_stages) step(w2, w1, w3, s + 2);
    // Drain the reloads issued past the end before the ring is reused.  The
    // weight loads are asynchronous writes the compiler does not see: keep
    // every register set allocated until they have landed, so none of them
    // is handed to another value while a load into it is in flight.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    pin_w(w0);
    pin_w(w1);
    pin_w(w2);
    pin_w(w3);
    asm volatile("s_barrier" ::: "memory");

    auto pin = [&](auto tti) __attribute__((always_inline)) {
      pin_acc_agpr(acc[decltype(tti)::value]);
    };
    static_for<0, 16>(pin);
    auto epi = [&](auto tti) __attribute__((always_inline)) {
      constexpr int tt = decltype(tti)::value;
      if (2 * npairs > tt) {
        const int t_in = tt * 16 + li;
        store_subtile<FC1>(p, acc[tt], row_begin + t_in, t_in < n_valid, unit, g);
      }
    };
    static_for<0, 16>(epi);
  }
}

}  // namespace

bool prefill_shape_ok(const FcParams& prm, bool fc1) {
  // FC1: 128 intermediate columns (256 w13 rows) per tile and whole 512-row
  // groups of the tiled layout (I % 256); FC2: 256 output columns per tile,
  // whole 512-row groups (H % 512).  Buffer offsets are 32-bit: the
  // activation array and one expert's weights must each stay below 2 GiB.
  const int64_t K = prm.K;
  return K % kKS == 0 && (fc1 ? prm.I % 256 == 0 : prm.N % 512 == 0) &&
         prm.act_rows * K < ((int64_t)1 << 31) && (int64_t)prm.N * (K / 2) < ((int64_t)1 << 31);
}

hipError_t launch_fc_prefill(bool fc1, bool tiled, FcParams prm, const int32_t* tile_prefix_all,
                             int n_cu, hipStream_t stream) {
  prm.tile_prefix = tile_prefix_all + (size_t)kTilePrefixIndex * (prm.E_local + 1);
  const int n_cg = fc1 ? prm.I / 128 : prm.N / kBN;
  // Persistent grid: one workgroup per CU, a multiple of the 8 XCDs.
  const int n_wg = (n_cu > 8 ? n_cu : 8) & ~7;
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
