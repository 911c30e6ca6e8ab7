/*
 * mi355moe.h -- C ABI of the MXFP8 x MXFP4 fused MoE expert layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (one GPU's share of a Kimi-K3-style routed-expert MoE) is five
 * calls, issued in this order on one HIP stream (the first three can also be
 * issued as one, moe_route_quant_permute; with top-k ids computed elsewhere,
 * the second and third as one, moe_quant_permute):
 *
 *   moe_route        sigmoid + correction-bias top-k routing, renormalised weights
 *   moe_quant_mxfp8  bf16 activations -> MXFP8 (E4M3 + one E8M0 scale per 32)
 *   moe_permute      group the kept routes by local expert (stable)
 *   moe_fc1_situ     grouped FC1 (MXFP8 x MXFP4) + SiTU + requantisation to MXFP8
 *   moe_fc2_combine  grouped FC2 (MXFP8 x MXFP4) + top-k weighted combine to bf16
 *
 * Sources (the pages this library implements): page 1 = the SM120 FlashInfer
 * MXFP4 experiment log for Kimi-K3 (sections "Serving call chain", "Key
 * sources" table, "Real checkpoint contract", "TP/EP expert mapping", "Phase 2
 * correctness harness", "NaN/Inf decision record"); page 5 = the Kimi-K3 MoE
 * path notes (weight/scale layouts, symmetric buffer views, pre-dispatch
 * quantisation).
 *
 * Conventions for every call:
 *  - Every pointer is a DEVICE pointer owned by the caller.  The library never
 *    allocates, frees or synchronises; every call is asynchronous on `stream`
 *    (0 = the null stream) and keeps no state between calls.
 *  - Arguments are validated before anything is launched.  A failed check
 *    returns a status and launches nothing; the pure argument checks make no
 *    HIP call, so they can be exercised on a machine without a GPU.  The
 *    device check (gfx950) runs after them.  A launch failure returns
 *    MOE_ERR_HIP.  Nothing retries or falls back to another path.
 *  - Pointers to byte / bf16 tensors must be 16-byte aligned; float and int32
 *    tensors 4-byte aligned.
 *  - Shapes: H and I multiples of 128; 1 <= top_k <= min(E, 64); E <= 4096;
 *    1 <= E_local <= 4096; T >= 0 (with T = 0 nothing is launched, except
 *    that moe_permute still writes zero expert offsets).
 *  - Byte layouts (little-endian, row-major):
 *      E4M3  OCP 8-bit float "fn": bias 7, max 448, no infinities.
 *      E2M1  4-bit float: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; two per byte,
 *            element 2j in the low nibble of byte j (page 1: packed FP4,
 *            two elements per byte; shapes [rows, K/2]).
 *      E8M0  byte b is 2^(b-127); 0xFF is NaN (page 1, NaN/Inf record).
 *    One scale per 32 consecutive elements along the contraction axis,
 *    stored [rows, K/32] (page 1 checkpoint shapes; page 5 w13 scale
 *    [E, 2I, H/32]).  The activation scale bytes [T, H/32] are the same bytes
 *    as page 5's x_sf view [T, H/128] of int32 words.
 */
#ifndef MI355MOE_H
#define MI355MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

/* Status codes have fixed values (page 1 records a Python/C++ enum mismatch
 * that silently turned SiTU into a non-gated activation; these values never
 * change within an ABI version). */
typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,            /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,           /* a size or stride is out of range */
  MOE_ERR_ALIGN = 3,           /* a pointer or stride is misaligned */
  MOE_ERR_ENUM = 4,            /* an enum argument has no defined value */
  MOE_ERR_WORKSPACE = 5,       /* workspace too small */
  MOE_ERR_HIP = 6,             /* a HIP runtime call or launch failed */
  MOE_ERR_UNSUPPORTED_DEVICE = 7, /* current device is not gfx950 */
  MOE_ERR_SCRATCH_LIMIT = 8    /* sizes need more than the library's static scratch
                                  (moe_permute_noalloc only) */
} moe_status_t;

/* How moe_fc2_combine sums the top-k FC2 rows of a token (fixed values).
 * Page 1 ("Serving call chain": finalize after GEMM2; "Phase 2 correctness
 * harness" / symmetry constraints) describes both: a fused finalize that
 * accumulates with atomics, whose order and so whose float rounding vary
 * from run to run, and the non-fused finalize kept for bitwise-repeatable
 * results.
 *   MOE_COMBINE_DETERMINISTIC  FC2 writes each kept route's row to the
 *       workspace; a second kernel sums a token's rows in slot order.
 *       Bitwise repeatable.  The default.
 *   MOE_COMBINE_ATOMIC  the FC2 epilogue adds topk_w * row into a float
 *       [T, H] sum in the workspace with atomic adds (cleared first in the
 *       same call), then one pass rounds it to bf16.  Same bar against the
 *       definition, not bitwise repeatable. */
typedef enum moe_combine {
  MOE_COMBINE_DETERMINISTIC = 0,
  MOE_COMBINE_ATOMIC = 1
} moe_combine_t;

/* MOE_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

/* Static description of a status code (never NULL). */
const char* moe_strerror(int status);

/* Bytes of workspace that moe_permute, moe_fc1_situ and moe_fc2_combine need
 * for a layer call with these sizes and combine mode (one buffer serves all
 * three; moe_permute writes the FC kernels' tile schedule into it and
 * moe_fc2_combine keeps the per-route FC2 rows, or with MOE_COMBINE_ATOMIC the
 * float [T, H] sums, there, so pass the same buffer to all three).
 * Returns 0 for invalid sizes or an unknown mode. */
size_t moe_workspace_size(int T, int top_k, int E_local, int H, int I, int mode);

/* a1 -- routing (page 1 "Serving call chain": sigmoid + correction bias +
 * top-k + renormalise; "Key sources" routing row: the bias only selects, the
 * weights come from the bias-free sigmoid scores, normalised; page 5: routed
 * scaling factor).
 *   logits  float [T, E], row stride ld_logits (>= E) elements.
 *   bias    float [E] correction bias, or NULL for none.
 *   s_e = float(sigmoid(logit) evaluated in double); key_e = s_e + bias_e in
 *   float; the top_k largest keys, equal keys ranked by lower expert index,
 *   slots ordered by key descending; w_k = s_k / sum_j s_j (double) times
 *   routed_scaling, rounded to float.
 *   topk_idx int32 [T, top_k] global expert ids; topk_w float [T, top_k].
 *   A NaN logit (or bias) gives a NaN key, which ranks below every other key
 *   (NaN experts are chosen last, lower index first); if one is chosen, the
 *   token's weights are NaN. */
moe_status_t moe_route(const float* logits, int64_t ld_logits, const float* bias,
                       int T, int E, int top_k, float routed_scaling,
                       int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* a2 -- MXFP8 quantisation of bf16 activations (page 5 pre-dispatch step:
 * absmax per 32 elements -> UE8M0 scale -> E4M3; page 1 NaN/Inf record:
 * saturating finite conversion).
 *   x   bf16 bits [T, H], row stride ld_x (>= H, multiple of 8) elements.
 *   Per 32-element group: scale exponent e = the smallest integer with
 *   absmax <= 448 * 2^e, clamped to [-127, 127] (0 for an all-zero group
 *   gives e = -127); element = nearest E4M3 to x * 2^-e, ties to even,
 *   saturating at +-448, sign of zero kept; NaN elements are ignored by the
 *   absmax and encode as 0x00; a group holding +-Inf gets e = 127.
 *   xq  uint8 E4M3 [T, H]; xs  uint8 E8M0 [T, H/32].  H % 32 == 0 suffices
 *   for this call. */
moe_status_t moe_quant_mxfp8(const uint16_t* x, int64_t ld_x, int T, int H,
                             uint8_t* xq, uint8_t* xs, hipStream_t stream);

/* a3 -- grouping by local expert (page 1 "TP/EP expert mapping": a GPU holds
 * the contiguous experts [expert_offset, expert_offset + E_local) and maps
 * global ids into that window; "Phase 2" coverage: -1 masked slots, empty
 * experts).
 *   topk_idx       int32 [T, top_k] global ids (-1 = masked slot).
 *   Route r = t * top_k + k is kept iff its id lies in the window.
 *   expert_offsets int32 [E_local + 1]: rows of local expert e are
 *                  [expert_offsets[e], expert_offsets[e+1]).
 *   sorted_route   int32 [T * top_k]: kept routes in grouped order, ascending
 *                  r within an expert; entries past the kept count are -1.
 *   route_row      int32 [T * top_k]: grouped row of route r, or -1 if dropped.
 *   workspace      >= moe_workspace_size(...) bytes, 256-byte aligned; also
 *                  receives the tile schedule read by the FC calls. */
moe_status_t moe_permute(const int32_t* topk_idx, int T, int top_k, int expert_offset,
                         int E_local, int32_t* expert_offsets, int32_t* sorted_route,
                         int32_t* route_row, void* workspace, size_t ws_bytes,
                         hipStream_t stream);

/* moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments as moe_permute minus the workspace, and
 * the same expert_offsets / sorted_route / route_row bytes.  It allocates
 * nothing: the grouping's tile schedule and chunked histogram go to a
 * library-owned device array of 4 MiB (4194304 bytes) that every GPU the
 * library runs on holds until the process ends.
 * Sizes whose schedule does not fit (the schedule part of
 * moe_workspace_size: about 4 * (3 * E_local + T * top_k / 32) bytes plus
 * 4 * E_local bytes per 256 or 512 routes above 2048 routes) return
 * MOE_ERR_SCRATCH_LIMIT before anything is launched.  Every call on one GPU
 * shares that GPU's array, so calls that overlap on one GPU (several streams
 * or threads) race; the FC calls cannot use this call's schedule (they read
 * the one moe_permute writes into their workspace). */
moe_status_t moe_permute_noalloc(const int32_t* topk_idx, int T, int top_k, int expert_offset,
                                 int E_local, int32_t* expert_offsets, int32_t* sorted_route,
                                 int32_t* route_row, hipStream_t stream);

/* a1 + a2 + a3 in one call (decode latency: page 1 "Serving call chain" runs
 * routing, quantisation and grouping before the expert GEMMs; their fixed
 * launch costs are a visible share of a decode step).  Computes exactly what
 * moe_route, then moe_quant_mxfp8, then moe_permute compute with the same
 * arguments (same bytes in every output and in the workspace), and accepts
 * what those three accept together (every check of each; xs needs only
 * 4-byte alignment as in moe_quant_mxfp8).  For T <= 16, E <= 1024 and small
 * enough E_local it is a single launch; otherwise it issues the three
 * launches in order on `stream`. */
moe_status_t moe_route_quant_permute(const float* logits, int64_t ld_logits, const float* bias,
                                     int T, int E, int top_k, float routed_scaling,
                                     const uint16_t* x, int64_t ld_x, int H, int expert_offset,
                                     int E_local, int32_t* topk_idx, float* topk_w, uint8_t* xq,
                                     uint8_t* xs, int32_t* expert_offsets, int32_t* sorted_route,
                                     int32_t* route_row, void* workspace, size_t ws_bytes,
                                     hipStream_t stream);

/* a2 + a3 in one call, for top-k ids and weights computed before the expert
 * layer (page 1 "Serving call chain": the fused MoE call receives the router's
 * top-k ids and weights; its Phase 4 benchmark feeds them in directly).
 * Computes exactly what moe_quant_mxfp8 and then moe_permute compute with the
 * same arguments (same bytes in every output and in the workspace), and
 * accepts what those two accept together (every check of each).  When the
 * grouping runs as one workgroup (T * top_k <= 2048) it is a single launch,
 * workgroup 0 grouping while the others quantise; otherwise it issues the two
 * calls' launches in order on `stream`. */
moe_status_t moe_quant_permute(const uint16_t* x, int64_t ld_x, int T, int H,
                               const int32_t* topk_idx, int top_k, int expert_offset,
                               int E_local, uint8_t* xq, uint8_t* xs, int32_t* expert_offsets,
                               int32_t* sorted_route, int32_t* route_row, void* workspace,
                               size_t ws_bytes, hipStream_t stream);

/* a4 + a5 + a6 -- FC1 grouped GEMM, SiTU, requantisation (page 1 "Serving call
 * chain": grouped GEMM1 then gated activation; "Real checkpoint contract": w13
 * holds [gate; up] in two contiguous halves, SiTU gate' = alpha *
 * tanh(gate/alpha) * sigmoid(gate), up' = beta * tanh(up/beta), out = gate' *
 * up' with alpha = 4, beta = 25; page 5: w13 [E, 2I, H/2], scales
 * [E, 2I, H/32]).
 *   xq, xs          MXFP8 activations from moe_quant_mxfp8 ([T, H], [T, H/32]).
 *   expert_offsets, sorted_route   from moe_permute; grouped row j of expert e
 *                   multiplies token sorted_route[j] / top_k.
 *   w13, w13_s      uint8 [E_local, 2I, H/2], [E_local, 2I, H/32] (local window).
 *   hq, hs          uint8 [T*top_k, I], [T*top_k, I/32]: the SiTU output of
 *                   each kept grouped row, requantised with the moe_quant_mxfp8
 *                   rule from the float accumulators (rows past the kept count
 *                   are not written).
 *   workspace       the buffer moe_permute filled. */
moe_status_t moe_fc1_situ(const uint8_t* xq, const uint8_t* xs, int T, int H, int I, int top_k,
                          int E_local, const int32_t* expert_offsets,
                          const int32_t* sorted_route, const uint8_t* w13,
                          const uint8_t* w13_s, float situ_alpha, float situ_beta,
                          uint8_t* hq, uint8_t* hs, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/* a7 + a8 -- FC2 grouped GEMM and top-k combine (page 1 "Serving call chain":
 * GEMM2 then finalize; "Phase 2": the non-fused finalize for bitwise
 * determinism, next to the fused atomic one; page 5: w2 [E, H, I/2], scales
 * [E, H, I/32]).
 *   hq, hs          from moe_fc1_situ.
 *   expert_offsets, sorted_route, route_row   from moe_permute.
 *   topk_w          from moe_route (float [T, top_k]).
 *   w2, w2_s        uint8 [E_local, H, I/2], [E_local, H, I/32].
 *   mode            a moe_combine_t value (else MOE_ERR_ENUM).
 *   out             bf16 bits [T, H], row stride ld_out (>= H, multiple of 8):
 *                   out[t] = bf16_rne( sum over kept k of
 *                   topk_w[t,k] * y[route_row[t,k]] ) with float accumulation
 *                   (DETERMINISTIC: in k order, bitwise repeatable; ATOMIC: in
 *                   the order the atomic adds land); a token with no kept slot
 *                   gets zeros.
 *   workspace       the buffer moe_permute filled, of at least
 *                   moe_workspace_size(..., mode) bytes (DETERMINISTIC: holds
 *                   the per-route FC2 rows y [T*top_k, H] as fp16 of y / 2^e
 *                   with one exponent e per 64 columns, 2^-11 relative, below
 *                   the output's bf16 step; ATOMIC: the float [T, H] sums). */
moe_status_t moe_fc2_combine(const uint8_t* hq, const uint8_t* hs, int T, int H, int I,
                             int top_k, int E_local, const int32_t* expert_offsets,
                             const int32_t* sorted_route, const int32_t* route_row,
                             const float* topk_w, const uint8_t* w2, const uint8_t* w2_s,
                             int mode, uint16_t* out, int64_t ld_out, void* workspace,
                             size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Tiled weight layout (optional, one-time).  The calls above read the
 * checkpoint layout directly.  moe_prepack_w13 / moe_prepack_w2 reorder the
 * same bytes once, at load time, into a tiled layout whose blocks the FC
 * kernels read as whole contiguous pieces; moe_fc1_situ_tiled /
 * moe_fc2_combine_tiled then compute exactly what moe_fc1_situ /
 * moe_fc2_combine compute (this is the role of the weight and scale
 * transforms the pages apply after loading, page 5).
 *
 * Tiled layout, for a weight matrix of N rows and K columns per expert
 * (w13: N = 2I, K = H; w2: N = H, K = I): rows are grouped 512 at a time
 * (group cg) and K is cut into stages of 128.  Block (e, cg, s) holds
 *   data   32768 bytes: 16-byte chunk number (4w + i) * 64 + l is the logical
 *          16-byte chunk c = (l & 3) ^ ((l >> 3) & 3) of stage s of row
 *          r = 64w + 16i + l/4 (w < 8, i < 4, l < 64);
 *   scales 2048 bytes: dword r = the four scale bytes of row r for MX blocks
 *          4s .. 4s+3;
 * where group row r is global row: w13 — unit u = 8cg + r/64, b = (r/16) % 4,
 * row = (b < 2 ? 0 : I) + 32u + 16(b % 2) + r % 16 (gate rows of the unit,
 * then the matching up rows); w2 — 512cg + r.  Blocks are stored in
 * [e][cg][s] order; the tiled data and scale arrays have the sizes of the
 * checkpoint arrays.  Requires I % 256 == 0 (w13) and H % 512 == 0 (w2).
 * ------------------------------------------------------------------------- */

/* Reorder checkpoint w13 [E_local, 2I, H/2] + w13_s [E_local, 2I, H/32] into
 * w13t / w13t_s (same sizes, distinct buffers).  Asynchronous on `stream`. */
moe_status_t moe_prepack_w13(const uint8_t* w13, const uint8_t* w13_s, int E_local, int H, int I,
                             uint8_t* w13t, uint8_t* w13t_s, hipStream_t stream);

/* Row order of a w13 tensor (fixed values).  Page 1 ("Real checkpoint
 * contract") lists three: the Kimi-K3 checkpoint keeps [gate; up] halves
 * (rows [0, I) gate, [I, 2I) up), the CUTLASS runner expects [up; gate]
 * halves, and the GPT-OSS loader interleaves rows (row 2j gate j, row 2j+1 up
 * j; page 3's de-interleave takes rows 0::2 as gate, 1::2 as up). */
typedef enum moe_w13_layout {
  MOE_W13_GATE_UP = 0,
  MOE_W13_UP_GATE = 1,
  MOE_W13_INTERLEAVED = 2
} moe_w13_layout_t;

/* moe_prepack_w13 for a w13 / w13_s whose rows are in `layout` order (a
 * moe_w13_layout_t value; anything else is MOE_ERR_ENUM).  The tiled result
 * is the same bytes moe_prepack_w13 gives for the [gate; up] reordering of
 * the input, so moe_fc1_situ_tiled computes the same layer for every layout.
 * (The checkpoint-layout moe_fc1_situ reads [gate; up] only.) */
moe_status_t moe_prepack_w13_layout(const uint8_t* w13, const uint8_t* w13_s, int E_local, int H,
                                    int I, int layout, uint8_t* w13t, uint8_t* w13t_s,
                                    hipStream_t stream);

/* Reorder checkpoint w2 [E_local, H, I/2] + w2_s [E_local, H, I/32]. */
moe_status_t moe_prepack_w2(const uint8_t* w2, const uint8_t* w2_s, int E_local, int H, int I,
                            uint8_t* w2t, uint8_t* w2t_s, hipStream_t stream);

/* moe_fc1_situ on tiled w13 (from moe_prepack_w13); same results. */
moe_status_t moe_fc1_situ_tiled(const uint8_t* xq, const uint8_t* xs, int T, int H, int I,
                                int top_k, int E_local, const int32_t* expert_offsets,
                                const int32_t* sorted_route, const uint8_t* w13t,
                                const uint8_t* w13t_s, float situ_alpha, float situ_beta,
                                uint8_t* hq, uint8_t* hs, void* workspace, size_t ws_bytes,
                                hipStream_t stream);

/* moe_fc2_combine on tiled w2 (from moe_prepack_w2); same results. */
moe_status_t moe_fc2_combine_tiled(const uint8_t* hq, const uint8_t* hs, int T, int H, int I,
                                   int top_k, int E_local, const int32_t* expert_offsets,
                                   const int32_t* sorted_route, const int32_t* route_row,
                                   const float* topk_w, const uint8_t* w2t,
                                   const uint8_t* w2t_s, int mode, uint16_t* out,
                                   int64_t ld_out, void* workspace, size_t ws_bytes,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MI355MOE_H */
