// Kernel launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355moe {

hipError_t launch_route(const float* logits, int64_t ld, const float* bias, int T, int E, int K,
                        float scaling, int32_t* idx, float* w, hipStream_t stream);
hipError_t launch_quant(const uint16_t* x, int64_t ld, int T, int H, uint8_t* xq, uint8_t* xs,
                        hipStream_t stream);
// counts: int32 [perm_chunks(R)][E_local] scratch (used when R > kPermSingle).
hipError_t launch_permute(const int32_t* idx, int R, int offset, int E_local, int32_t* offs,
                          int32_t* sorted_route, int32_t* route_row, int32_t* tile_prefix,
                          int32_t* counts, hipStream_t stream);
// Route + quantise + group in one launch (front.hip), for batches that
// front_fusable accepts (T <= 16, E <= 1024, its LDS within 64 KB); the same
// bytes as launch_route, launch_quant and launch_permute.
bool front_fusable(int T, int E, int K, int E_local);
hipError_t launch_front(const float* logits, int64_t ld, const float* bias, int T, int E, int K,
                        float scaling, int32_t* topk_idx, float* topk_w, const uint16_t* x,
                        int64_t ld_x, int H, uint8_t* xq, uint8_t* xs, int offset, int E_local,
                        int32_t* offs, int32_t* sorted_route, int32_t* route_row,
                        int32_t* tile_prefix, hipStream_t stream);
// Quantise + group in one launch (front.hip), when the grouping is one
// workgroup (R <= kPermSingle); the same bytes as launch_quant and
// launch_permute.
bool quant_permute_fusable(int64_t R);
hipError_t launch_quant_permute(const uint16_t* x, int64_t ld_x, int T, int H, uint8_t* xq,
                                uint8_t* xs, const int32_t* idx, int R, int offset, int E_local,
                                int32_t* offs, int32_t* sorted_route, int32_t* route_row,
                                int32_t* tile_prefix, hipStream_t stream);
hipError_t launch_fc1(const uint8_t* xq, const uint8_t* xs, int T, int H, int I, int top_k,
                      int E_local, const int32_t* offs, const int32_t* sorted_route,
                      const uint8_t* w13, const uint8_t* w13_s, float alpha, float beta,
                      uint8_t* hq, uint8_t* hs, const int32_t* tile_prefix_all,
                      uint32_t* act_st, int32_t* sched, int n_cu, bool tiled,
                      hipStream_t stream);
// FC2 rows into y / ye (deterministic combine), or, with out_acc set, the
// atomic combine: each grouped row r adds topk_w[route] times its row into
// out_acc [T, H] (route = sorted_route[r]).
hipError_t launch_fc2(const uint8_t* hq, const uint8_t* hs, int T, int H, int I, int top_k,
                      int E_local, const int32_t* offs, const uint8_t* w2, const uint8_t* w2_s,
                      uint16_t* y, int8_t* ye, const int32_t* sorted_route,
                      const float* topk_w, float* out_acc, const int32_t* tile_prefix_all,
                      uint32_t* act_st, int32_t* sched, int n_cu, bool tiled,
                      hipStream_t stream);
struct FcParams;
// Prefill-shaped FC kernels (fc_prefill.hip): usable when K % 128 == 0, the
// weight rows split into whole 512-row groups and the operands fit 32-bit
// buffer offsets.  They read the 256-row tile prefix, and first restage the
// input's scale dwords into prm.act_st (stage-major, grouped-row order).
bool prefill_shape_ok(const FcParams& prm, bool fc1);
hipError_t launch_fc_prefill(bool fc1, bool tiled, FcParams prm, const int32_t* tile_prefix_all,
                             int n_cu, hipStream_t stream);
// One-time reordering of checkpoint-layout weights into the tiled layout
// (layout: w13 row order, 0 [gate; up], 1 [up; gate], 2 interleaved).
hipError_t launch_prepack(bool fc1, const uint8_t* w, const uint8_t* ws, int E_local, int N,
                          int K, int I, int layout, uint8_t* tw, uint8_t* tws,
                          hipStream_t stream);
hipError_t launch_combine(const uint16_t* y, const int8_t* ye, int H, const int32_t* route_row,
                          const float* topk_w, int T, int K, uint16_t* out, int64_t ld_out,
                          hipStream_t stream);
// Atomic combine: clear the float [T, H] sums before FC2; round them to bf16
// after it.
hipError_t launch_acc_clear(float* acc, int T, int H, hipStream_t stream);
hipError_t launch_acc_to_bf16(const float* acc, int T, int H, uint16_t* out, int64_t ld_out,
                              hipStream_t stream);

}  // namespace mi355moe
