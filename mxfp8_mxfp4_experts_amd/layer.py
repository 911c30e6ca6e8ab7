"""``MoELayer``: the five C calls of the expert layer, in order, on one stream.

Buffers (routing outputs, MXFP8 activations, grouping, FC1 output and the
workspace) are allocated once for ``max_tokens`` and reused, so a call
allocates nothing but its output (or nothing when ``out`` is given).

With ``tiled=True`` (the default where the shapes allow it: I % 256 == 0 and
H % 512 == 0) the weights are reordered once into the library's tiled layout
at construction and the tiled FC entry points are used; results are the same.

``combine`` picks how FC2 sums each token's top-k rows: "deterministic" (the
default; rows summed in slot order by a second kernel, bitwise repeatable) or
"atomic" (added into float sums in the FC2 epilogue).

``w13_layout`` names the row order of the given w13 / w13_s (W13_GATE_UP, the
checkpoint's [gate; up] halves, by default; W13_UP_GATE or W13_INTERLEAVED
are reordered by the tiled prepack, so they need the tiled layout).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _binding as B


class MoELayer:
    def __init__(self, w13, w13_s, w2, w2_s, *, top_k: int, E: int, expert_offset: int = 0,
                 routed_scaling: float = 1.0, situ_alpha: float = 4.0, situ_beta: float = 25.0,
                 max_tokens: int = 1, tiled: Optional[bool] = None,
                 combine: str = "deterministic", w13_layout: int = B.W13_GATE_UP):
        for name, t in (("w13", w13), ("w13_s", w13_s), ("w2", w2), ("w2_s", w2_s)):
            B._need(t, name, torch.uint8)
        if w13.dim() != 3 or w2.dim() != 3:
            raise ValueError("w13 must be [E_local, 2I, H/2] and w2 [E_local, H, I/2]")
        self.E_local, twoI, half_h = w13.shape
        self.H, self.I = 2 * half_h, twoI // 2
        E_local, H, I = self.E_local, self.H, self.I
        for name, t, shape in (("w13_s", w13_s, (E_local, 2 * I, H // 32)),
                               ("w2", w2, (E_local, H, I // 2)),
                               ("w2_s", w2_s, (E_local, H, I // 32))):
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
        if combine not in ("deterministic", "atomic"):
            raise ValueError('combine must be "deterministic" or "atomic"')
        self.combine_mode = B.COMBINE_ATOMIC if combine == "atomic" else B.COMBINE_DETERMINISTIC
        if tiled is None:
            tiled = self.I % 256 == 0 and self.H % 512 == 0
        self.tiled = tiled
        if w13_layout != B.W13_GATE_UP and not tiled:
            raise ValueError("a w13 row order other than [gate; up] needs the tiled layout")
        if tiled:
            w13, w13_s = B.moe_prepack_w13_layout(w13, w13_s, w13_layout)
            w2, w2_s = B.moe_prepack_w2(w2, w2_s)
        self.w13, self.w13_s, self.w2, self.w2_s = w13, w13_s, w2, w2_s
        self.top_k, self.E, self.expert_offset = top_k, E, expert_offset
        self.routed_scaling, self.alpha, self.beta = routed_scaling, situ_alpha, situ_beta
        self.device = w13.device
        self._alloc(max_tokens)

    def with_combine(self, combine: str) -> "MoELayer":
        """A layer sharing these (already prepacked) weights whose FC2 sums
        with the other combine mode; it has buffers of its own."""
        if combine not in ("deterministic", "atomic"):
            raise ValueError('combine must be "deterministic" or "atomic"')
        other = object.__new__(MoELayer)
        other.__dict__.update(self.__dict__)
        other.combine_mode = B.COMBINE_ATOMIC if combine == "atomic" else B.COMBINE_DETERMINISTIC
        other._alloc(self.max_tokens)
        return other

    def _alloc(self, T: int):
        dev, K, H, I = self.device, self.top_k, self.H, self.I
        R = T * K
        self.max_tokens = T
        self.topk_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
        self.xs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        self.expert_offsets = torch.empty(self.E_local + 1, dtype=torch.int32, device=dev)
        self.sorted_route = torch.empty(R, dtype=torch.int32, device=dev)
        self.route_row = torch.empty(R, dtype=torch.int32, device=dev)
        self.hq = torch.empty((R, I), dtype=torch.uint8, device=dev)
        self.hs = torch.empty((R, I // 32), dtype=torch.uint8, device=dev)
        n = B.moe_workspace_size(T, K, self.E_local, H, I, self.combine_mode)
        self.workspace = torch.empty(n, dtype=torch.uint8, device=dev)

    def __call__(self, x: torch.Tensor, logits: torch.Tensor, bias: Optional[torch.Tensor],
                 out: Optional[torch.Tensor] = None, topk_idx: Optional[torch.Tensor] = None,
                 topk_w: Optional[torch.Tensor] = None) -> torch.Tensor:
        """x bf16 [T, H]; logits float [T, E]; bias float [E] or None.

        ``topk_idx``/``topk_w`` (int32 / float [T, top_k]) replace the routing
        step when given (e.g. masked -1 slots)."""
        T = x.shape[0]
        if T > self.max_tokens:
            self._alloc(T)
        K = self.top_k
        R = T * K
        idx, w = self.topk_idx[:T], self.topk_w[:T]
        xq, xs = self.xq[:T], self.xs[:T]
        if topk_idx is None:
            # routing, quantisation and grouping as one call
            B.moe_route_quant_permute(logits, bias, K, self.routed_scaling, x, self.expert_offset,
                                      self.E_local, self.workspace, idx, w, xq, xs,
                                      self.expert_offsets, self.sorted_route[:R],
                                      self.route_row[:R])
        else:
            idx, w = topk_idx, topk_w
            # quantisation and grouping as one call
            B.moe_quant_permute(x, idx, self.expert_offset, self.E_local, self.workspace, xq, xs,
                                self.expert_offsets, self.sorted_route[:R], self.route_row[:R])
        B.moe_fc1_situ(xq, xs, K, self.expert_offsets, self.sorted_route[:R], self.w13,
                       self.w13_s, self.workspace, self.alpha, self.beta, self.hq[:R],
                       self.hs[:R], tiled=self.tiled)
        return B.moe_fc2_combine(self.hq[:R], self.hs[:R], T, K, self.expert_offsets,
                                 self.sorted_route[:R], self.route_row[:R], w, self.w2, self.w2_s,
                                 self.workspace, out, tiled=self.tiled, mode=self.combine_mode)
