// moe_permute_noalloc: the grouping call (moe_permute) for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The caller passes the inputs and the
// three grouping outputs; the tile schedule and the chunked histogram, which
// moe_permute keeps in the caller's workspace, live in a library-owned
// device array instead.
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy (kNoAllocScratchBytes, until the process ends).  Host
// code never passes the array's name to a kernel (in host code it is only a
// stand-in symbol, not a device address); it passes the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and cached per device.
//
// Every call on one GPU shares that GPU's array: calls that overlap on one
// GPU (two streams, two threads) race on it.  The grouping kernels write
// every word of the array they later read in the same call, so nothing needs
// clearing between calls.
#include <atomic>
#include <cstring>

#include "../../include/mi355moe.h"
#include "common.h"
#include "launch.h"

// 4 MiB: the schedule of 2^17 routes over 896 local experts (the chunked
// histogram takes 4 bytes per chunk and expert) needs under 1 MiB.
static constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

// Per device ordinal: the device address of its copy of `scratch`, looked up
// on the first call made with that device current (nullptr until then), and
// whether the device is a gfx950 (0 unknown, 1 yes, 2 no).
std::atomic<void*> g_scratch_ptr[256];
std::atomic<int> g_arch_ok[256];

moe_status_t scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= 256) return MOE_ERR_UNSUPPORTED_DEVICE;
  int ok = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (ok == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(ok, std::memory_order_relaxed);
  }
  if (ok != 1) return MOE_ERR_UNSUPPORTED_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

}  // namespace

using namespace mi355moe;

extern "C" moe_status_t moe_permute_noalloc(const int32_t* topk_idx, int T, int top_k,
                                            int expert_offset, int E_local,
                                            int32_t* expert_offsets, int32_t* sorted_route,
                                            int32_t* route_row, hipStream_t stream) {
  // The argument checks of moe_permute (no HIP call), then the scratch limit.
  if (T < 0 || top_k < 1 || top_k > kMaxTopK || E_local < 1 || E_local > kMaxExperts ||
      expert_offset < 0 || (int64_t)T * top_k > ((int64_t)1 << 30))
    return MOE_ERR_SHAPE;
  if (!topk_idx && T > 0) return MOE_ERR_NULL;
  if (!expert_offsets || (T > 0 && (!sorted_route || !route_row))) return MOE_ERR_NULL;
  if (!aligned4(expert_offsets) ||
      (T > 0 && (!aligned4(topk_idx) || !aligned4(sorted_route) || !aligned4(route_row))))
    return MOE_ERR_ALIGN;
  // The schedule part of moe_permute's workspace (it does not depend on H, I).
  const WsLayout l = ws_layout(T, top_k, E_local, 0, 0);
  if (l.y > kNoAllocScratchBytes) return MOE_ERR_SCRATCH_LIMIT;

  void* base = nullptr;
  const moe_status_t st = scratch_for_current_device(&base);
  if (st != MOE_OK) return st;
  int32_t* prefix = reinterpret_cast<int32_t*>(static_cast<char*>(base) + l.tile_prefix);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(base) + l.perm_counts);
  return launch_permute(topk_idx, T * top_k, expert_offset, E_local, expert_offsets,
                        sorted_route, route_row, prefix, counts, stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}
