// C ABI of the MoE layer: argument validation, device check, launches.
//
// Every entry validates its arguments with plain integer / pointer checks
// first (no HIP call), then checks once per device that it is a gfx950, then
// launches.  Nothing retries or falls back (page 1 keeps to fail-fast
// initialisation and forbids switching backends after a kernel failure).
#include <atomic>
#include <cstring>

#include "../../include/mi355moe.h"
#include "common.h"
#include "launch.h"

using namespace mi355moe;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per device: 0 = unknown, 1 = gfx950, 2 = other; and its compute-unit count.
// A cache of fixed device properties.
std::atomic<int> g_device_ok[256];
std::atomic<int> g_device_cus[256];

moe_status_t check_device(int* n_cu = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= 256) return MOE_ERR_UNSUPPORTED_DEVICE;
  int s = g_device_ok[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    g_device_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(s, std::memory_order_relaxed);
  }
  if (n_cu) *n_cu = g_device_cus[dev].load(std::memory_order_relaxed);
  return s == 1 ? MOE_OK : MOE_ERR_UNSUPPORTED_DEVICE;
}

moe_status_t finish(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool valid_hi(int H, int I) { return H >= 128 && I >= 128 && H % 128 == 0 && I % 128 == 0; }

bool valid_window(int top_k, int E_local) {
  return top_k >= 1 && top_k <= kMaxTopK && E_local >= 1 && E_local <= kMaxExperts;
}

// T * top_k routes and T * top_k * max(H, I) elements must fit the int32 /
// size_t arithmetic of the kernels.
bool valid_rows(int T, int top_k, int H, int I) {
  if (T < 0) return false;
  int64_t R = (int64_t)T * top_k;
  if (R > (int64_t)1 << 30) return false;
  int64_t wide = H > I ? H : I;
  return R * wide < ((int64_t)1 << 46);
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size or stride is out of range";
    case MOE_ERR_ALIGN: return "a pointer or stride is misaligned";
    case MOE_ERR_ENUM: return "an enum argument has no defined value";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case MOE_ERR_UNSUPPORTED_DEVICE: return "current device is not gfx950";
    case MOE_ERR_SCRATCH_LIMIT:
      return "sizes need more than the no-allocation entry point's static scratch";
    default: return "unknown status";
  }
}

size_t moe_workspace_size(int T, int top_k, int E_local, int H, int I, int mode) {
  if (!valid_hi(H, I) || !valid_window(top_k, E_local) || !valid_rows(T, top_k, H, I)) return 0;
  if (mode != MOE_COMBINE_DETERMINISTIC && mode != MOE_COMBINE_ATOMIC) return 0;
  return ws_layout(T, top_k, E_local, H, I, mode == MOE_COMBINE_ATOMIC).total;
}

moe_status_t moe_route(const float* logits, int64_t ld_logits, const float* bias, int T, int E,
                       int top_k, float routed_scaling, int32_t* topk_idx, float* topk_w,
                       hipStream_t stream) {
  if (T < 0 || E < 1 || E > kMaxExperts || top_k < 1 || top_k > kMaxTopK || top_k > E ||
      ld_logits < E || T > (1 << 30) / (top_k > 0 ? top_k : 1))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
      (bias && !aligned(bias, 4)))
    return MOE_ERR_ALIGN;
  moe_status_t s = check_device();
  if (s != MOE_OK) return s;
  return finish(launch_route(logits, ld_logits, bias, T, E, top_k, routed_scaling, topk_idx,
                             topk_w, stream));
}

moe_status_t moe_quant_mxfp8(const uint16_t* x, int64_t ld_x, int T, int H, uint8_t* xq,
                             uint8_t* xs, hipStream_t stream) {
  if (T < 0 || H < 32 || H % 32 != 0 || ld_x < H || (int64_t)T * H > ((int64_t)1 << 40))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !xq || !xs) return MOE_ERR_NULL;
  if (!aligned(x, 16) || ld_x % 8 != 0 || !aligned(xq, 16) || !aligned(xs, 4))
    return MOE_ERR_ALIGN;
  moe_status_t s = check_device();
  if (s != MOE_OK) return s;
  return finish(launch_quant(x, ld_x, T, H, xq, xs, stream));
}

moe_status_t moe_permute(const int32_t* topk_idx, int T, int top_k, int expert_offset,
                         int E_local, int32_t* expert_offsets, int32_t* sorted_route,
                         int32_t* route_row, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  if (T < 0 || !valid_window(top_k, E_local) || expert_offset < 0 ||
      (int64_t)T * top_k > ((int64_t)1 << 30))
    return MOE_ERR_SHAPE;
  if (!topk_idx && T > 0) return MOE_ERR_NULL;
  if (!expert_offsets || !workspace || (T > 0 && (!sorted_route || !route_row)))
    return MOE_ERR_NULL;
  if (!aligned(expert_offsets, 4) || !aligned(workspace, 256) ||
      (T > 0 && (!aligned(topk_idx, 4) || !aligned(sorted_route, 4) || !aligned(route_row, 4))))
    return MOE_ERR_ALIGN;
  // The schedule part of the workspace does not depend on H.
  if (ws_bytes < ws_layout(T, top_k, E_local, 0, 0).y) return MOE_ERR_WORKSPACE;
  moe_status_t s = check_device();
  if (s != MOE_OK) return s;
  WsLayout l = ws_layout(T, top_k, E_local, 0, 0);
  int32_t* prefix = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + l.tile_prefix);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + l.perm_counts);
  return finish(launch_permute(topk_idx, T * top_k, expert_offset, E_local, expert_offsets,
                               sorted_route, route_row, prefix, counts, stream));
}

moe_status_t moe_route_quant_permute(const float* logits, int64_t ld_logits, const float* bias,
                                     int T, int E, int top_k, float routed_scaling,
                                     const uint16_t* x, int64_t ld_x, int H, int expert_offset,
                                     int E_local, int32_t* topk_idx, float* topk_w, uint8_t* xq,
                                     uint8_t* xs, int32_t* expert_offsets, int32_t* sorted_route,
                                     int32_t* route_row, void* workspace, size_t ws_bytes,
                                     hipStream_t stream) {
  // The checks of moe_route, moe_quant_mxfp8 and moe_permute.
  if (T < 0 || E < 1 || E > kMaxExperts || top_k < 1 || top_k > kMaxTopK || top_k > E ||
      ld_logits < E || T > (1 << 30) / top_k)
    return MOE_ERR_SHAPE;
  if (H < 32 || H % 32 != 0 || ld_x < H || (int64_t)T * H > ((int64_t)1 << 40))
    return MOE_ERR_SHAPE;
  if (!valid_window(top_k, E_local) || expert_offset < 0) return MOE_ERR_SHAPE;
  if (!expert_offsets || !workspace) return MOE_ERR_NULL;
  if (T > 0 && (!logits || !topk_idx || !topk_w || !x || !xq || !xs || !sorted_route || !route_row))
    return MOE_ERR_NULL;
  if (!aligned(expert_offsets, 4) || !aligned(workspace, 256)) return MOE_ERR_ALIGN;
  if (T > 0 && (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
                (bias && !aligned(bias, 4)) || !aligned(x, 16) || ld_x % 8 != 0 ||
                !aligned(xq, 16) || !aligned(xs, 4) || !aligned(sorted_route, 4) ||
                !aligned(route_row, 4)))
    return MOE_ERR_ALIGN;
  if (ws_bytes < ws_layout(T, top_k, E_local, 0, 0).y) return MOE_ERR_WORKSPACE;
  moe_status_t s = check_device();
  if (s != MOE_OK) return s;
  WsLayout l = ws_layout(T, top_k, E_local, 0, 0);
  int32_t* prefix = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + l.tile_prefix);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + l.perm_counts);
  if (T > 0 && front_fusable(T, E, top_k, E_local))
    return finish(launch_front(logits, ld_logits, bias, T, E, top_k, routed_scaling, topk_idx,
                               topk_w, x, ld_x, H, xq, xs, expert_offset, E_local, expert_offsets,
                               sorted_route, route_row, prefix, stream));
  if (T > 0) {
    if (launch_route(logits, ld_logits, bias, T, E, top_k, routed_scaling, topk_idx, topk_w,
                     stream) != hipSuccess)
      return MOE_ERR_HIP;
    if (launch_quant(x, ld_x, T, H, xq, xs, stream) != hipSuccess) return MOE_ERR_HIP;
  }
  return finish(launch_permute(topk_idx, T * top_k, expert_offset, E_local, expert_offsets,
                               sorted_route, route_row, prefix, counts, stream));
}

moe_status_t moe_quant_permute(const uint16_t* x, int64_t ld_x, int T, int H,
                               const int32_t* topk_idx, int top_k, int expert_offset,
                               int E_local, uint8_t* xq, uint8_t* xs, int32_t* expert_offsets,
                               int32_t* sorted_route, int32_t* route_row, void* workspace,
                               size_t ws_bytes, hipStream_t stream) {
  // The checks of moe_quant_mxfp8 and moe_permute.
  if (T < 0 || H < 32 || H % 32 != 0 || ld_x < H || (int64_t)T * H > ((int64_t)1 << 40))
    return MOE_ERR_SHAPE;
  if (!valid_window(top_k, E_local) || expert_offset < 0 ||
      (int64_t)T * top_k > ((int64_t)1 << 30))
    return MOE_ERR_SHAPE;
  if (!expert_offsets || !workspace) return MOE_ERR_NULL;
  if (T > 0 && (!x || !xq || !xs || !topk_idx || !sorted_route || !route_row)) return MOE_ERR_NULL;
  if (!aligned(expert_offsets, 4) || !aligned(workspace, 256)) return MOE_ERR_ALIGN;
  if (T > 0 && (!aligned(x, 16) || ld_x % 8 != 0 || !aligned(xq, 16) || !aligned(xs, 4) ||
                !aligned(topk_idx, 4) || !aligned(sorted_route, 4) || !aligned(route_row, 4)))
    return MOE_ERR_ALIGN;
  if (ws_bytes < ws_layout(T, top_k, E_local, 0, 0).y) return MOE_ERR_WORKSPACE;
  moe_status_t s = check_device();
  if (s != MOE_OK) return s;
  WsLayout l = ws_layout(T, top_k, E_local, 0, 0);
  int32_t* prefix = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + l.tile_prefix);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + l.perm_counts);
  if (T > 0 && quant_permute_fusable(T * top_k))
    return finish(launch_quant_permute(x, ld_x, T, H, xq, xs, topk_idx, T * top_k, expert_offset,
                                       E_local, expert_offsets, sorted_route, route_row, prefix,
                                       stream));
  if (T > 0 && launch_quant(x, ld_x, T, H, xq, xs, stream) != hipSuccess) return MOE_ERR_HIP;
  return finish(launch_permute(topk_idx, T * top_k, expert_offset, E_local, expert_offsets,
                               sorted_route, route_row, prefix, counts, stream));
}

static moe_status_t fc1_impl(const uint8_t* xq, const uint8_t* xs, int T, int H, int I, int top_k,
                          int E_local, const int32_t* expert_offsets,
                          const int32_t* sorted_route, const uint8_t* w13,
                          const uint8_t* w13_s, float situ_alpha, float situ_beta, uint8_t* hq,
                          uint8_t* hs, void* workspace, size_t ws_bytes, hipStream_t stream,
                          bool tiled) {
  if (!valid_hi(H, I) || (tiled && I % 256 != 0) || !valid_window(top_k, E_local) || !valid_rows(T, top_k, H, I))
    return MOE_ERR_SHAPE;
  if (!(situ_alpha > 0.0f) || !(situ_beta > 0.0f)) return MOE_ERR_SHAPE;
  if (!expert_offsets || !w13 || !w13_s || !workspace) return MOE_ERR_NULL;
  if (T > 0 && (!xq || !xs || !sorted_route || !hq || !hs)) return MOE_ERR_NULL;
  if (!aligned(w13, 16) || !aligned(w13_s, 16) || !aligned(expert_offsets, 4) ||
      !aligned(workspace, 256))
    return MOE_ERR_ALIGN;
  if (T > 0 && (!aligned(xq, 16) || !aligned(xs, 16) || !aligned(sorted_route, 4) ||
                !aligned(hq, 16) || !aligned(hs, 4)))
    return MOE_ERR_ALIGN;
  WsLayout l = ws_layout(T, top_k, E_local, H, I);
  if (ws_bytes < l.y) return MOE_ERR_WORKSPACE;
  if (T == 0) return MOE_OK;
  int n_cu = 0;
  moe_status_t s = check_device(&n_cu);
  if (s != MOE_OK) return s;
  char* ws = static_cast<char*>(workspace);
  const int32_t* prefix = reinterpret_cast<const int32_t*>(ws + l.tile_prefix);
  uint32_t* act_st = reinterpret_cast<uint32_t*>(ws + l.act_st);
  int32_t* sched = reinterpret_cast<int32_t*>(ws + l.fc_sched);
  return finish(launch_fc1(xq, xs, T, H, I, top_k, E_local, expert_offsets, sorted_route, w13,
                           w13_s, situ_alpha, situ_beta, hq, hs, prefix, act_st, sched, n_cu,
                           tiled, stream));
}

moe_status_t moe_fc1_situ(const uint8_t* xq, const uint8_t* xs, int T, int H, int I, int top_k,
                          int E_local, const int32_t* expert_offsets,
                          const int32_t* sorted_route, const uint8_t* w13,
                          const uint8_t* w13_s, float situ_alpha, float situ_beta, uint8_t* hq,
                          uint8_t* hs, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return fc1_impl(xq, xs, T, H, I, top_k, E_local, expert_offsets, sorted_route, w13, w13_s,
                  situ_alpha, situ_beta, hq, hs, workspace, ws_bytes, stream, false);
}

moe_status_t moe_fc1_situ_tiled(const uint8_t* xq, const uint8_t* xs, int T, int H, int I,
                                int top_k, int E_local, const int32_t* expert_offsets,
                                const int32_t* sorted_route, const uint8_t* w13t,
                                const uint8_t* w13t_s, float situ_alpha, float situ_beta,
                                uint8_t* hq, uint8_t* hs, void* workspace, size_t ws_bytes,
                                hipStream_t stream) {
  return fc1_impl(xq, xs, T, H, I, top_k, E_local, expert_offsets, sorted_route, w13t, w13t_s,
                  situ_alpha, situ_beta, hq, hs, workspace, ws_bytes, stream, true);
}

static moe_status_t fc2_impl(const uint8_t* hq, const uint8_t* hs, int T, int H, int I,
                             int top_k, int E_local, const int32_t* expert_offsets,
                             const int32_t* sorted_route, const int32_t* route_row,
                             const float* topk_w, const uint8_t* w2, const uint8_t* w2_s, int mode,
                             uint16_t* out, int64_t ld_out, void* workspace, size_t ws_bytes,
                             hipStream_t stream, bool tiled) {
  if (!valid_hi(H, I) || !valid_window(top_k, E_local) || !valid_rows(T, top_k, H, I) ||
      ld_out < H || (tiled && H % 512 != 0))
    return MOE_ERR_SHAPE;
  if (mode != MOE_COMBINE_DETERMINISTIC && mode != MOE_COMBINE_ATOMIC) return MOE_ERR_ENUM;
  const bool atomic = mode == MOE_COMBINE_ATOMIC;
  if (!expert_offsets || !w2 || !w2_s || !workspace) return MOE_ERR_NULL;
  if (T > 0 && (!hq || !hs || !route_row || !topk_w || !out || (atomic && !sorted_route)))
    return MOE_ERR_NULL;
  if (!aligned(w2, 16) || !aligned(w2_s, 16) || !aligned(expert_offsets, 4) ||
      !aligned(workspace, 256))
    return MOE_ERR_ALIGN;
  if (T > 0 && (!aligned(hq, 16) || !aligned(hs, 16) || !aligned(route_row, 4) ||
                !aligned(topk_w, 4) || !aligned(out, 16) || ld_out % 8 != 0 ||
                (sorted_route && !aligned(sorted_route, 4))))
    return MOE_ERR_ALIGN;
  WsLayout l = ws_layout(T, top_k, E_local, H, I, atomic);
  if (ws_bytes < l.total) return MOE_ERR_WORKSPACE;
  if (T == 0) return MOE_OK;
  int n_cu = 0;
  moe_status_t s = check_device(&n_cu);
  if (s != MOE_OK) return s;
  char* ws = static_cast<char*>(workspace);
  const int32_t* prefix = reinterpret_cast<const int32_t*>(ws + l.tile_prefix);
  uint32_t* act_st = reinterpret_cast<uint32_t*>(ws + l.act_st);
  int32_t* sched = reinterpret_cast<int32_t*>(ws + l.fc_sched);
  if (atomic) {
    float* acc = reinterpret_cast<float*>(ws + l.y);
    if (launch_acc_clear(acc, T, H, stream) != hipSuccess) return MOE_ERR_HIP;
    if (launch_fc2(hq, hs, T, H, I, top_k, E_local, expert_offsets, w2, w2_s, nullptr, nullptr,
                   sorted_route, topk_w, acc, prefix, act_st, sched, n_cu, tiled,
                   stream) != hipSuccess)
      return MOE_ERR_HIP;
    return finish(launch_acc_to_bf16(acc, T, H, out, ld_out, stream));
  }
  uint16_t* y = reinterpret_cast<uint16_t*>(ws + l.y);
  int8_t* ye = reinterpret_cast<int8_t*>(ws + l.ye);
  if (launch_fc2(hq, hs, T, H, I, top_k, E_local, expert_offsets, w2, w2_s, y, ye, nullptr,
                 nullptr, nullptr, prefix, act_st, sched, n_cu, tiled, stream) != hipSuccess)
    return MOE_ERR_HIP;
  return finish(launch_combine(y, ye, H, route_row, topk_w, T, top_k, out, ld_out, stream));
}

moe_status_t moe_fc2_combine(const uint8_t* hq, const uint8_t* hs, int T, int H, int I,
                             int top_k, int E_local, const int32_t* expert_offsets,
                             const int32_t* sorted_route, const int32_t* route_row,
                             const float* topk_w, const uint8_t* w2, const uint8_t* w2_s,
                             int mode, uint16_t* out, int64_t ld_out, void* workspace,
                             size_t ws_bytes, hipStream_t stream) {
  return fc2_impl(hq, hs, T, H, I, top_k, E_local, expert_offsets, sorted_route, route_row,
                  topk_w, w2, w2_s, mode, out, ld_out, workspace, ws_bytes, stream, false);
}

moe_status_t moe_fc2_combine_tiled(const uint8_t* hq, const uint8_t* hs, int T, int H, int I,
                                   int top_k, int E_local, const int32_t* expert_offsets,
                                   const int32_t* sorted_route, const int32_t* route_row,
                                   const float* topk_w, const uint8_t* w2t,
                                   const uint8_t* w2t_s, int mode, uint16_t* out,
                                   int64_t ld_out, void* workspace, size_t ws_bytes,
                                   hipStream_t stream) {
  return fc2_impl(hq, hs, T, H, I, top_k, E_local, expert_offsets, sorted_route, route_row,
                  topk_w, w2t, w2t_s, mode, out, ld_out, workspace, ws_bytes, stream, true);
}

static moe_status_t prepack_impl(bool fc1, const uint8_t* w, const uint8_t* ws, int E_local,
                                 int H, int I, int layout, uint8_t* tw, uint8_t* tws,
                                 hipStream_t stream) {
  if (!valid_hi(H, I) || E_local < 1 || E_local > kMaxExperts) return MOE_ERR_SHAPE;
  if (layout < MOE_W13_GATE_UP || layout > MOE_W13_INTERLEAVED) return MOE_ERR_ENUM;
  if (fc1 ? (I % 256 != 0) : (H % 512 != 0)) return MOE_ERR_SHAPE;
  if (!w || !ws || !tw || !tws) return MOE_ERR_NULL;
  if (!aligned(w, 16) || !aligned(ws, 16) || !aligned(tw, 16) || !aligned(tws, 16))
    return MOE_ERR_ALIGN;
  moe_status_t s = check_device();
  if (s != MOE_OK) return s;
  const int N = fc1 ? 2 * I : H, K = fc1 ? H : I;
  return finish(launch_prepack(fc1, w, ws, E_local, N, K, I, layout, tw, tws, stream));
}

moe_status_t moe_prepack_w13(const uint8_t* w13, const uint8_t* w13_s, int E_local, int H, int I,
                             uint8_t* w13t, uint8_t* w13t_s, hipStream_t stream) {
  return prepack_impl(true, w13, w13_s, E_local, H, I, MOE_W13_GATE_UP, w13t, w13t_s, stream);
}

moe_status_t moe_prepack_w13_layout(const uint8_t* w13, const uint8_t* w13_s, int E_local, int H,
                                    int I, int layout, uint8_t* w13t, uint8_t* w13t_s,
                                    hipStream_t stream) {
  return prepack_impl(true, w13, w13_s, E_local, H, I, layout, w13t, w13t_s, stream);
}

moe_status_t moe_prepack_w2(const uint8_t* w2, const uint8_t* w2_s, int E_local, int H, int I,
                            uint8_t* w2t, uint8_t* w2t_s, hipStream_t stream) {
  return prepack_impl(false, w2, w2_s, E_local, H, I, MOE_W13_GATE_UP, w2t, w2t_s, stream);
}

}  // extern "C"
