"""ctypes binding of ``libmi355moe.so``: argument marshalling only.

Each function has the name of the C entry point it calls.  It checks dtype,
device, shape and contiguity of the torch tensors it is given (raising
``ValueError`` before anything reaches C), allocates outputs the caller did
not pass, and forwards raw device pointers plus the current HIP stream.  All
arithmetic of the layer runs in the library's HIP kernels; there is no other
path.  PyTorch serves only as the device-memory and stream provider.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmi355moe.so")

MOE_STATUS = {
    0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN", 4: "MOE_ERR_ENUM",
    5: "MOE_ERR_WORKSPACE", 6: "MOE_ERR_HIP", 7: "MOE_ERR_UNSUPPORTED_DEVICE",
    8: "MOE_ERR_SCRATCH_LIMIT",
}

# Entry points declared in include/mi355moe.h.
EXPORTS = (
    "moe_abi_version", "moe_strerror", "moe_workspace_size", "moe_route", "moe_quant_mxfp8",
    "moe_permute", "moe_fc1_situ", "moe_fc2_combine", "moe_prepack_w13", "moe_prepack_w2",
    "moe_fc1_situ_tiled", "moe_fc2_combine_tiled", "moe_route_quant_permute",
    "moe_prepack_w13_layout", "moe_permute_noalloc", "moe_quant_permute",
)

# moe_w13_layout_t values (row order of a w13 tensor)
W13_GATE_UP, W13_UP_GATE, W13_INTERLEAVED = 0, 1, 2
# moe_combine_t values (how moe_fc2_combine sums a token's top-k rows)
COMBINE_DETERMINISTIC, COMBINE_ATOMIC = 0, 1

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t


def load_library(path: str = _LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m mxfp8_mxfp4_experts_amd.build` "
            "(the MoE layer has no other implementation to fall back to)")
    lib = ctypes.CDLL(path)
    lib.moe_abi_version.restype = _I
    lib.moe_abi_version.argtypes = []
    lib.moe_strerror.restype = ctypes.c_char_p
    lib.moe_strerror.argtypes = [_I]
    lib.moe_workspace_size.restype = _SZ
    lib.moe_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I]
    lib.moe_route.restype = _I
    lib.moe_route.argtypes = [_P, _I64, _P, _I, _I, _I, _F, _P, _P, _P]
    lib.moe_quant_mxfp8.restype = _I
    lib.moe_quant_mxfp8.argtypes = [_P, _I64, _I, _I, _P, _P, _P]
    lib.moe_permute.restype = _I
    lib.moe_permute.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]
    lib.moe_permute_noalloc.restype = _I
    lib.moe_permute_noalloc.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P]
    lib.moe_quant_permute.restype = _I
    lib.moe_quant_permute.argtypes = [_P, _I64, _I, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                                      _SZ, _P]
    lib.moe_route_quant_permute.restype = _I
    lib.moe_route_quant_permute.argtypes = [_P, _I64, _P, _I, _I, _I, _F, _P, _I64, _I, _I, _I,
                                            _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.moe_fc1_situ.restype = _I
    lib.moe_fc1_situ.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _F, _F, _P, _P, _P,
                                 _SZ, _P]
    lib.moe_fc2_combine.restype = _I
    lib.moe_fc2_combine.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P,
                                    _I64, _P, _SZ, _P]
    lib.moe_fc1_situ_tiled.restype = _I
    lib.moe_fc1_situ_tiled.argtypes = lib.moe_fc1_situ.argtypes
    lib.moe_fc2_combine_tiled.restype = _I
    lib.moe_fc2_combine_tiled.argtypes = lib.moe_fc2_combine.argtypes
    for name in ("moe_prepack_w13", "moe_prepack_w2"):
        getattr(lib, name).restype = _I
        getattr(lib, name).argtypes = [_P, _P, _I, _I, _I, _P, _P, _P]
    lib.moe_prepack_w13_layout.restype = _I
    lib.moe_prepack_w13_layout.argtypes = [_P, _P, _I, _I, _I, _I, _P, _P, _P]
    return lib


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


class MoEError(RuntimeError):
    def __init__(self, name: str, status: int):
        msg = lib().moe_strerror(status).decode()
        super().__init__(f"{name} returned {MOE_STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(name: str, status: int):
    if status != 0:
        raise MoEError(name, status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape=None, contiguous=True, device=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _as_u16(x: torch.Tensor, name: str) -> torch.Tensor:
    if x.dtype == torch.bfloat16:
        return x.view(torch.uint16)   # same element size: any strides
    if x.dtype == torch.uint16:
        return x
    raise ValueError(f"{name} must be bfloat16 (or uint16 bf16 bits), got {x.dtype}")


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_workspace_size(T: int, top_k: int, E_local: int, H: int, I: int,
                       mode: int = COMBINE_DETERMINISTIC) -> int:
    n = lib().moe_workspace_size(T, top_k, E_local, H, I, int(mode))
    if n == 0:
        raise ValueError("invalid sizes or combine mode for moe_workspace_size")
    return n


def moe_route(logits: torch.Tensor, bias: Optional[torch.Tensor], top_k: int,
              routed_scaling: float = 1.0, topk_idx: Optional[torch.Tensor] = None,
              topk_w: Optional[torch.Tensor] = None):
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [T, E] with unit column stride")
    _need(logits, "logits", torch.float32, contiguous=False)
    T, E = logits.shape
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,), device=logits.device)
    if topk_idx is None:
        topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _need(topk_idx, "topk_idx", torch.int32, (T, top_k), device=logits.device)
    _need(topk_w, "topk_w", torch.float32, (T, top_k), device=logits.device)
    _check("moe_route", lib().moe_route(_ptr(logits), logits.stride(0), _ptr(bias), T, E, top_k,
                                        float(routed_scaling), _ptr(topk_idx), _ptr(topk_w),
                                        _stream()))
    return topk_idx, topk_w


def moe_quant_mxfp8(x: torch.Tensor, xq: Optional[torch.Tensor] = None,
                    xs: Optional[torch.Tensor] = None):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [T, H] with unit column stride")
    xb = x if x.dtype == torch.uint16 else (x.view(torch.uint16) if x.dtype == torch.bfloat16 else None)
    if xb is None:
        raise ValueError(f"x must be bfloat16 (or uint16 bf16 bits), got {x.dtype}")
    _need(xb, "x", torch.uint16, contiguous=False)
    T, H = x.shape
    if xq is None:
        xq = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    if xs is None:
        xs = torch.empty((T, H // 32), dtype=torch.uint8, device=x.device)
    _need(xq, "xq", torch.uint8, (T, H), device=x.device)
    _need(xs, "xs", torch.uint8, (T, H // 32), device=x.device)
    _check("moe_quant_mxfp8", lib().moe_quant_mxfp8(_ptr(xb), x.stride(0), T, H, _ptr(xq),
                                                    _ptr(xs), _stream()))
    return xq, xs


def moe_route_quant_permute(logits: torch.Tensor, bias: Optional[torch.Tensor], top_k: int,
                            routed_scaling: float, x: torch.Tensor, expert_offset: int,
                            E_local: int, workspace: torch.Tensor, topk_idx=None, topk_w=None,
                            xq=None, xs=None, expert_offsets=None, sorted_route=None,
                            route_row=None):
    """moe_route, moe_quant_mxfp8 and moe_permute as one call (same results)."""
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [T, E] with unit column stride")
    _need(logits, "logits", torch.float32, contiguous=False)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [T, H] with unit column stride")
    xb = x if x.dtype == torch.uint16 else (x.view(torch.uint16) if x.dtype == torch.bfloat16 else None)
    if xb is None:
        raise ValueError(f"x must be bfloat16 (or uint16 bf16 bits), got {x.dtype}")
    _need(xb, "x", torch.uint16, contiguous=False)
    T, E = logits.shape
    H = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x and logits must have the same number of rows")
    dev = logits.device
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,), device=dev)
    R = T * top_k
    topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev) if xq is None else xq
    xs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev) if xs is None else xs
    if expert_offsets is None:
        expert_offsets = torch.empty(E_local + 1, dtype=torch.int32, device=dev)
    sorted_route = torch.empty(R, dtype=torch.int32, device=dev) if sorted_route is None else sorted_route
    route_row = torch.empty(R, dtype=torch.int32, device=dev) if route_row is None else route_row
    _need(topk_idx, "topk_idx", torch.int32, (T, top_k), device=dev)
    _need(topk_w, "topk_w", torch.float32, (T, top_k), device=dev)
    _need(xq, "xq", torch.uint8, (T, H), device=dev)
    _need(xs, "xs", torch.uint8, (T, H // 32), device=dev)
    _need(expert_offsets, "expert_offsets", torch.int32, (E_local + 1,), device=dev)
    _need(sorted_route, "sorted_route", torch.int32, (R,), device=dev)
    _need(route_row, "route_row", torch.int32, (R,), device=dev)
    _need(workspace, "workspace", torch.uint8, device=dev)
    _check("moe_route_quant_permute", lib().moe_route_quant_permute(
        _ptr(logits), logits.stride(0), _ptr(bias), T, E, top_k, float(routed_scaling), _ptr(xb),
        x.stride(0), H, expert_offset, E_local, _ptr(topk_idx), _ptr(topk_w), _ptr(xq), _ptr(xs),
        _ptr(expert_offsets), _ptr(sorted_route), _ptr(route_row), _ptr(workspace),
        workspace.numel(), _stream()))
    return topk_idx, topk_w, xq, xs, expert_offsets, sorted_route, route_row


def moe_permute(topk_idx: torch.Tensor, expert_offset: int, E_local: int, workspace: torch.Tensor,
                expert_offsets=None, sorted_route=None, route_row=None):
    _need(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, top_k]")
    T, K = topk_idx.shape
    dev = topk_idx.device
    _need(workspace, "workspace", torch.uint8, device=dev)
    if expert_offsets is None:
        expert_offsets = torch.empty(E_local + 1, dtype=torch.int32, device=dev)
    if sorted_route is None:
        sorted_route = torch.empty(T * K, dtype=torch.int32, device=dev)
    if route_row is None:
        route_row = torch.empty(T * K, dtype=torch.int32, device=dev)
    _need(expert_offsets, "expert_offsets", torch.int32, (E_local + 1,), device=dev)
    _need(sorted_route, "sorted_route", torch.int32, (T * K,), device=dev)
    _need(route_row, "route_row", torch.int32, (T * K,), device=dev)
    _check("moe_permute", lib().moe_permute(_ptr(topk_idx), T, K, expert_offset, E_local,
                                            _ptr(expert_offsets), _ptr(sorted_route),
                                            _ptr(route_row), _ptr(workspace), workspace.numel(),
                                            _stream()))
    return expert_offsets, sorted_route, route_row


def moe_quant_permute(x: torch.Tensor, topk_idx: torch.Tensor, expert_offset: int, E_local: int,
                      workspace: torch.Tensor, xq=None, xs=None, expert_offsets=None,
                      sorted_route=None, route_row=None):
    """moe_quant_mxfp8 and moe_permute as one call (same results), for top-k
    ids computed elsewhere."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [T, H] with unit column stride")
    xb = x if x.dtype == torch.uint16 else (x.view(torch.uint16) if x.dtype == torch.bfloat16 else None)
    if xb is None:
        raise ValueError(f"x must be bfloat16 (or uint16 bf16 bits), got {x.dtype}")
    _need(xb, "x", torch.uint16, contiguous=False)
    _need(topk_idx, "topk_idx", torch.int32, device=x.device)
    if topk_idx.dim() != 2 or topk_idx.shape[0] != x.shape[0]:
        raise ValueError("topk_idx must be [T, top_k] with the rows of x")
    T, H = x.shape
    K = topk_idx.shape[1]
    dev = x.device
    _need(workspace, "workspace", torch.uint8, device=dev)
    if xq is None:
        xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
    if xs is None:
        xs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    if expert_offsets is None:
        expert_offsets = torch.empty(E_local + 1, dtype=torch.int32, device=dev)
    if sorted_route is None:
        sorted_route = torch.empty(T * K, dtype=torch.int32, device=dev)
    if route_row is None:
        route_row = torch.empty(T * K, dtype=torch.int32, device=dev)
    _need(xq, "xq", torch.uint8, (T, H), device=dev)
    _need(xs, "xs", torch.uint8, (T, H // 32), device=dev)
    _need(expert_offsets, "expert_offsets", torch.int32, (E_local + 1,), device=dev)
    _need(sorted_route, "sorted_route", torch.int32, (T * K,), device=dev)
    _need(route_row, "route_row", torch.int32, (T * K,), device=dev)
    _check("moe_quant_permute", lib().moe_quant_permute(
        _ptr(xb), x.stride(0), T, H, _ptr(topk_idx), K, expert_offset, E_local, _ptr(xq),
        _ptr(xs), _ptr(expert_offsets), _ptr(sorted_route), _ptr(route_row), _ptr(workspace),
        workspace.numel(), _stream()))
    return xq, xs, expert_offsets, sorted_route, route_row


def moe_permute_noalloc(topk_idx: torch.Tensor, expert_offset: int, E_local: int,
                        expert_offsets=None, sorted_route=None, route_row=None):
    """moe_permute without a workspace (the library's static scratch holds
    the schedule); same grouping outputs."""
    _need(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, top_k]")
    T, K = topk_idx.shape
    dev = topk_idx.device
    if expert_offsets is None:
        expert_offsets = torch.empty(E_local + 1, dtype=torch.int32, device=dev)
    if sorted_route is None:
        sorted_route = torch.empty(T * K, dtype=torch.int32, device=dev)
    if route_row is None:
        route_row = torch.empty(T * K, dtype=torch.int32, device=dev)
    _need(expert_offsets, "expert_offsets", torch.int32, (E_local + 1,), device=dev)
    _need(sorted_route, "sorted_route", torch.int32, (T * K,), device=dev)
    _need(route_row, "route_row", torch.int32, (T * K,), device=dev)
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(
        _ptr(topk_idx), T, K, expert_offset, E_local, _ptr(expert_offsets), _ptr(sorted_route),
        _ptr(route_row), _stream()))
    return expert_offsets, sorted_route, route_row


def moe_fc1_situ(xq, xs, top_k, expert_offsets, sorted_route, w13, w13_s, workspace,
                 situ_alpha: float = 4.0, situ_beta: float = 25.0, hq=None, hs=None,
                 tiled: bool = False):
    """``tiled``: w13 / w13_s come from ``moe_prepack_w13`` (calls
    moe_fc1_situ_tiled); they keep the checkpoint tensor shapes."""
    _need(xq, "xq", torch.uint8)
    T, H = xq.shape
    dev = xq.device
    _need(w13, "w13", torch.uint8, device=dev)
    if w13.dim() != 3 or w13.shape[2] != H // 2:
        raise ValueError("w13 must be [E_local, 2I, H/2]")
    E_local, twoI, _ = w13.shape
    I = twoI // 2
    _need(xs, "xs", torch.uint8, (T, H // 32), device=dev)
    _need(w13_s, "w13_s", torch.uint8, (E_local, twoI, H // 32), device=dev)
    _need(expert_offsets, "expert_offsets", torch.int32, (E_local + 1,), device=dev)
    _need(sorted_route, "sorted_route", torch.int32, (T * top_k,), device=dev)
    _need(workspace, "workspace", torch.uint8, device=dev)
    R = T * top_k
    if hq is None:
        hq = torch.empty((R, I), dtype=torch.uint8, device=dev)
    if hs is None:
        hs = torch.empty((R, I // 32), dtype=torch.uint8, device=dev)
    _need(hq, "hq", torch.uint8, (R, I), device=dev)
    _need(hs, "hs", torch.uint8, (R, I // 32), device=dev)
    name = "moe_fc1_situ_tiled" if tiled else "moe_fc1_situ"
    _check(name, getattr(lib(), name)(
        _ptr(xq), _ptr(xs), T, H, I, top_k, E_local, _ptr(expert_offsets), _ptr(sorted_route),
        _ptr(w13), _ptr(w13_s), float(situ_alpha), float(situ_beta), _ptr(hq), _ptr(hs),
        _ptr(workspace), workspace.numel(), _stream()))
    return hq, hs


def moe_fc2_combine(hq, hs, T, top_k, expert_offsets, sorted_route, route_row, topk_w, w2, w2_s,
                    workspace, out=None, tiled: bool = False, mode: int = COMBINE_DETERMINISTIC):
    """``tiled``: w2 / w2_s come from ``moe_prepack_w2`` (calls
    moe_fc2_combine_tiled).  ``mode``: COMBINE_DETERMINISTIC or
    COMBINE_ATOMIC (the workspace must be sized for it)."""
    _need(hq, "hq", torch.uint8)
    R, I = hq.shape
    dev = hq.device
    _need(w2, "w2", torch.uint8, device=dev)
    if w2.dim() != 3 or w2.shape[2] != I // 2:
        raise ValueError("w2 must be [E_local, H, I/2]")
    E_local, H, _ = w2.shape
    if R != T * top_k:
        raise ValueError("hq must have T * top_k rows")
    _need(hs, "hs", torch.uint8, (R, I // 32), device=dev)
    _need(w2_s, "w2_s", torch.uint8, (E_local, H, I // 32), device=dev)
    _need(expert_offsets, "expert_offsets", torch.int32, (E_local + 1,), device=dev)
    _need(sorted_route, "sorted_route", torch.int32, (R,), device=dev)
    _need(route_row, "route_row", torch.int32, (R,), device=dev)
    _need(topk_w, "topk_w", torch.float32, (T, top_k), device=dev)
    _need(workspace, "workspace", torch.uint8, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if out.dim() != 2 or out.shape[0] != T or out.shape[1] != H or out.stride(1) != 1:
        raise ValueError("out must be [T, H] with unit column stride")
    ob = _as_u16(out, "out")
    _need(ob, "out", torch.uint16, contiguous=False, device=dev)
    name = "moe_fc2_combine_tiled" if tiled else "moe_fc2_combine"
    _check(name, getattr(lib(), name)(
        _ptr(hq), _ptr(hs), T, H, I, top_k, E_local, _ptr(expert_offsets), _ptr(sorted_route),
        _ptr(route_row), _ptr(topk_w), _ptr(w2), _ptr(w2_s), int(mode), _ptr(ob), out.stride(0),
        _ptr(workspace), workspace.numel(), _stream()))
    return out


def _weight_pair(name, w, w_s):
    """A checkpoint weight [E, N, K/2] and its scales [E, N, K/32]: shapes and
    dtypes checked here, since the kernels read every byte they imply."""
    _need(w, name + " weights", torch.uint8)
    if w.dim() != 3 or w.shape[2] % 16 != 0:
        raise ValueError(f"{name} weights must be [E, N, K/2] with K a multiple of 32")
    E, N, half_k = w.shape
    _need(w_s, name + " scales", torch.uint8, (E, N, 2 * half_k // 32), device=w.device)
    return E, N, 2 * half_k


def _prepack(name, w, w_s, H, I):
    tw = torch.empty_like(w)
    tws = torch.empty_like(w_s)
    _check(name, getattr(lib(), name)(_ptr(w), _ptr(w_s), w.shape[0], H, I, _ptr(tw), _ptr(tws),
                                      _stream()))
    return tw, tws


def moe_prepack_w13(w13, w13_s):
    """Checkpoint w13 [E, 2I, H/2] + scales [E, 2I, H/32] -> tiled copies
    (same shapes)."""
    E, twoI, H = _weight_pair("moe_prepack_w13", w13, w13_s)
    return _prepack("moe_prepack_w13", w13, w13_s, H, twoI // 2)


def moe_prepack_w13_layout(w13, w13_s, layout: int):
    """w13 [E, 2I, H/2] + scales [E, 2I, H/32] whose rows are in ``layout``
    order (W13_GATE_UP, W13_UP_GATE or W13_INTERLEAVED) -> tiled copies."""
    E, twoI, H = _weight_pair("moe_prepack_w13_layout", w13, w13_s)
    tw, tws = torch.empty_like(w13), torch.empty_like(w13_s)
    _check("moe_prepack_w13_layout", lib().moe_prepack_w13_layout(
        _ptr(w13), _ptr(w13_s), E, H, twoI // 2, int(layout), _ptr(tw), _ptr(tws), _stream()))
    return tw, tws


def moe_prepack_w2(w2, w2_s):
    """Checkpoint w2 [E, H, I/2] + scales [E, H, I/32] -> tiled copies (same
    shapes)."""
    E, H, I = _weight_pair("moe_prepack_w2", w2, w2_s)
    return _prepack("moe_prepack_w2", w2, w2_s, H, I)
