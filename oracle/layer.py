"""The MoE expert layer step by step, in float64.

Test infrastructure only (see ``oracle/__init__``).

Page tags used below: page 1 = the SM120 FlashInfer MXFP4 experiment log for
Kimi-K3 (sections "Serving call chain", "Key sources" table, "Real checkpoint
contract", "Phase 2 correctness harness", "NaN/Inf decision record"); page 5 =
the Kimi-K3 MoE path notes for SM100 (module construction, weight/scale
layouts, pre-dispatch quantisation).
"""
from __future__ import annotations

import numpy as np

from .codecs import (
    bf16_to_f64,
    mxfp4_dequantize,
    mxfp8_dequantize,
    mxfp8_quantize,
)


# --------------------------------------------------------------------------
# a1: routing
# --------------------------------------------------------------------------
def route(logits, bias, top_k: int, routed_scaling: float = 1.0):
    """Sigmoid scores, correction bias used only to pick experts, top-k,
    weights renormalised from the unbiased scores.

    Page 1, "Serving call chain" (sigmoid + correction bias + top-k 16 +
    renormalise) and "Key sources" table, routing row (the bias only selects;
    the weights gather the bias-free sigmoid scores and are normalised);
    page 5 (routed_scaling_factor passed to the expert module).

    Readings where the pages are silent: the sigmoid is evaluated in float64
    and rounded once to float32; the selection key is one float32 addition
    ``s + bias``; plain top-k (one expert group); equal keys rank the lower
    expert index first; output slots ordered by key descending; weights are
    ``s_k / sum_j s_j`` in float64 times ``routed_scaling``, rounded to
    float32.  Returns (ids int32 [T,K], weights float32 [T,K]).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    s = (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, dtype=np.float32)
    key = s + b[None, :]                       # float32 + float32, one rounding
    assert key.dtype == np.float32
    # Stable sort of -key: equal keys keep ascending expert order.
    order = np.argsort(-key, axis=1, kind="stable")[:, :top_k]
    ids = order.astype(np.int32)
    sel = np.take_along_axis(s, order, axis=1).astype(np.float64)
    total = np.zeros(T, np.float64)
    for k in range(top_k):                     # plain left-to-right sum
        total += sel[:, k]
    w = (sel / total[:, None]) * float(routed_scaling)
    return ids, w.astype(np.float32)


# --------------------------------------------------------------------------
# a2: MXFP8 activation quantisation
# --------------------------------------------------------------------------
def quant_x(x_bf16_bits):
    """bf16 activations -> E4M3 codes + one E8M0 scale per 32 along H.

    Page 5, pre-dispatch step (bf16, absmax per 32 elements, UE8M0 scale,
    E4M3 payload); page 1 "NaN/Inf decision record" (saturating finite
    conversion, no 0xFF scale).  Returns (xq uint8 [T,H], xs uint8 [T,H/32]).
    """
    return mxfp8_quantize(bf16_to_f64(x_bf16_bits))


# --------------------------------------------------------------------------
# a3: grouping of routes by local expert
# --------------------------------------------------------------------------
def permute(topk_idx, expert_offset: int, E_local: int):
    """Keep routes whose global id lies in the local window, group them by
    local expert, stably in flattened (token, slot) order.

    Page 1, "TP/EP expert mapping" (each rank holds a contiguous block of
    whole experts; global ids are mapped to the local window) and the
    coverage matrix of "Phase 2 correctness harness" (masked -1 slots, empty
    experts).  Returns (expert_offsets int32 [E_local+1], sorted_route int32
    [n_kept] of flattened route indices, route_row int32 [T*K] giving each
    route's row in the grouped order or -1 when dropped).
    """
    idx = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    local = idx - expert_offset
    keep = (idx >= 0) & (local >= 0) & (local < E_local)
    counts = np.zeros(E_local, np.int64)
    for e in local[keep]:
        counts[e] += 1
    offsets = np.zeros(E_local + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    sorted_route = np.empty(int(offsets[-1]), np.int64)
    route_row = np.full(idx.shape[0], -1, np.int64)
    for r in range(idx.shape[0]):              # ascending route index = stable
        if keep[r]:
            e = local[r]
            sorted_route[cursor[e]] = r
            route_row[r] = cursor[e]
            cursor[e] += 1
    return offsets.astype(np.int32), sorted_route.astype(np.int32), route_row.astype(np.int32)


# --------------------------------------------------------------------------
# a5: SiTU
# --------------------------------------------------------------------------
def situ(g, u, alpha: float = 4.0, beta: float = 25.0):
    """SiTU gate of page 1, "Real checkpoint contract":
    gate' = alpha * tanh(gate / alpha) * sigmoid(gate) (sigmoid of the raw
    gate), up' = beta * tanh(up / beta), out = gate' * up', with alpha = 4
    and beta = 25 (the config's gate beta / linear beta)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    return (alpha * np.tanh(g / alpha) * sig) * (beta * np.tanh(u / beta))


# --------------------------------------------------------------------------
# a4 + a5 + a6: FC1, SiTU, requantisation
# --------------------------------------------------------------------------
def fc1_situ_requant(xq, xs, expert_offsets, sorted_route, top_k, w13, w13_s,
                     alpha=4.0, beta=25.0, return_acc=False, return_pre=False,
                     return_absum=False):
    """Per local expert: gather its routed rows of the MXFP8 activations,
    multiply by the dequantised MXFP4 w13 (exact in float64), split the
    result into the gate half (columns < I) and the up half (columns >= I),
    apply SiTU, and requantise to MXFP8 per 32 intermediate columns.

    Page 1, "Serving call chain" (grouped GEMM1 -> gated activation) and
    "Real checkpoint contract" (w1 and w3 loaded into the two contiguous
    halves of w13: [gate; up]); page 5 (w13 [E, 2I, H/2] with scales
    [E, 2I, H/32]).  The requantisation follows the same MXFP8 rule as the
    activations (the FC2 activation scale slot); the SiTU output is not
    rounded before it.  Rows are in grouped order.
    Returns (hq uint8 [n_kept, I], hs uint8 [n_kept, I/32]) and, with
    ``return_acc``, the float64 FC1 accumulators [n_kept, 2I]; with
    ``return_pre``, the float64 SiTU output before requantisation; with
    ``return_absum``, the sums of |products| behind each accumulator,
    |A| @ |W|^T [n_kept, 2I] (report only: the scale of an accumulation
    error, used to judge a requantised byte that differs).
    """
    w13 = np.asarray(w13)
    E_local, twoI, _ = w13.shape
    I = twoI // 2
    n_kept = int(expert_offsets[-1])
    a_all = np.empty((n_kept, I), np.float64)
    acc_all = np.empty((n_kept, twoI), np.float64) if return_acc else None
    abs_all = np.empty((n_kept, twoI), np.float64) if return_absum else None
    for e in range(E_local):
        r0, r1 = int(expert_offsets[e]), int(expert_offsets[e + 1])
        if r1 == r0:
            continue
        tokens = np.asarray(sorted_route[r0:r1]) // top_k
        A = mxfp8_dequantize(xq[tokens], xs[tokens])
        W = mxfp4_dequantize(w13[e], w13_s[e])
        acc = A @ W.T
        if return_acc:
            acc_all[r0:r1] = acc
        if return_absum:
            abs_all[r0:r1] = np.abs(A) @ np.abs(W).T
        a_all[r0:r1] = situ(acc[:, :I], acc[:, I:], alpha, beta)
    hq, hs = mxfp8_quantize(a_all) if n_kept else (np.zeros((0, I), np.uint8), np.zeros((0, I // 32), np.uint8))
    extra = (([acc_all] if return_acc else []) + ([a_all] if return_pre else [])
             + ([abs_all] if return_absum else []))
    return (hq, hs, *extra) if extra else (hq, hs)


# --------------------------------------------------------------------------
# a7: FC2
# --------------------------------------------------------------------------
def fc2(hq, hs, expert_offsets, w2, w2_s):
    """Per local expert: dequantised MXFP8 rows times dequantised MXFP4 w2
    (page 5: w2 [E, H, I/2] with scales [E, H, I/32]); exact in float64.
    Returns y float64 [n_kept, H] in grouped order."""
    w2 = np.asarray(w2)
    E_local, H, _ = w2.shape
    n_kept = int(expert_offsets[-1])
    y = np.zeros((n_kept, H), np.float64)
    for e in range(E_local):
        r0, r1 = int(expert_offsets[e]), int(expert_offsets[e + 1])
        if r1 == r0:
            continue
        A = mxfp8_dequantize(hq[r0:r1], hs[r0:r1])
        W = mxfp4_dequantize(w2[e], w2_s[e])
        y[r0:r1] = A @ W.T
    return y


# --------------------------------------------------------------------------
# a8: combine
# --------------------------------------------------------------------------
def combine(y, route_row, topk_w, T: int, top_k: int):
    """out[t] = sum over kept slots k (in k order) of w[t,k] * y[row(t,k)].

    Page 1, "Serving call chain" (finalize after GEMM2) and "Phase 2
    correctness harness" (non-fused finalize for determinism).  Dropped
    slots (masked -1 or another GPU's experts) add nothing; a token with no
    kept slot gives zeros.  Unrounded float64 [T, H]."""
    H = y.shape[1] if y.ndim == 2 else 0
    out = np.zeros((T, H), np.float64)
    rr = np.asarray(route_row).reshape(T, top_k)
    w = np.asarray(topk_w, dtype=np.float32).reshape(T, top_k).astype(np.float64)
    for k in range(top_k):
        m = rr[:, k] >= 0
        out[m] += w[m, k][:, None] * y[rr[m, k]]
    return out


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def oracle_layer(x_bf16, logits, bias, w13, w13_s, w2, w2_s, *, top_k,
                 expert_offset=0, routed_scaling=1.0, alpha=4.0, beta=25.0,
                 topk_idx=None, topk_w=None, report=False):
    """All steps a1..a8; returns a dict of every intermediate.

    ``topk_idx``/``topk_w`` may be given to bypass routing (masked-slot
    cases); weights are indexed by local expert.  With ``report`` the dict
    also holds the FC1 accumulators ``acc`` and their sums of |products|
    ``absum`` (report only)."""
    x_bf16 = np.asarray(x_bf16)
    T = x_bf16.shape[0]
    w13 = np.asarray(w13)
    E_local = w13.shape[0]
    if topk_idx is None:
        topk_idx, topk_w = route(logits, bias, top_k, routed_scaling)
    xq, xs = quant_x(x_bf16)
    offs, sroute, rrow = permute(topk_idx, expert_offset, E_local)
    fc1 = fc1_situ_requant(xq, xs, offs, sroute, top_k, w13, w13_s, alpha, beta,
                           return_acc=report, return_pre=True, return_absum=report)
    hq, hs = fc1[0], fc1[1]
    a = fc1[3] if report else fc1[2]
    y = fc2(hq, hs, offs, w2, w2_s)
    out = combine(y, rrow, topk_w, T, top_k)
    res = dict(topk_idx=topk_idx, topk_w=topk_w, xq=xq, xs=xs, expert_offsets=offs,
               sorted_route=sroute, route_row=rrow, hq=hq, hs=hs, a=a, y=y, out=out)
    if report:
        res.update(acc=fc1[2], absum=fc1[4])
    return res


def oracle_tokens(tokens, x_bf16, topk_idx, topk_w, weight_fn, *, top_k, expert_offset,
                  E_local, alpha=4.0, beta=25.0):
    """Layer output for a subset of tokens only, one route at a time.

    Used on full-size workloads where the whole oracle would take too long:
    each sampled token's kept routes are evaluated independently (routing
    and quantisation are per token, FC1/FC2 per route), so the result equals
    the corresponding rows of ``oracle_layer``.  ``weight_fn(e_local)``
    returns (w13[e], w13_s[e], w2[e], w2_s[e]) as numpy arrays.
    Returns dict(out [n,H] float64, h {(j, k): (hq, hs, SiTU output before
    requantisation, FC1 accumulators, their sums of |products|)} for sampled
    token j and slot k; the last two are report only).
    """
    tokens = list(tokens)
    xq, xs = quant_x(np.asarray(x_bf16)[tokens])
    need = {}
    for j, t in enumerate(tokens):
        for k in range(top_k):
            g = int(topk_idx[t, k])
            e = g - expert_offset
            if g >= 0 and 0 <= e < E_local:
                need.setdefault(e, []).append((j, k))
    H = xq.shape[1]
    out = np.zeros((len(tokens), H), np.float64)
    ys = {}
    hqs = {}
    for e in sorted(need):
        w13e, w13se, w2e, w2se = weight_fn(e)
        rows = [j for j, _ in need[e]]
        A = mxfp8_dequantize(xq[rows], xs[rows])
        W = mxfp4_dequantize(w13e, w13se)
        acc = A @ W.T
        absum = np.abs(A) @ np.abs(W).T
        I = W.shape[0] // 2
        a = situ(acc[:, :I], acc[:, I:], alpha, beta)
        hq, hs = mxfp8_quantize(a)
        W2 = mxfp4_dequantize(w2e, w2se)
        y = mxfp8_dequantize(hq, hs) @ W2.T
        for i, (j, k) in enumerate(need[e]):
            ys[(j, k)] = y[i]
            hqs[(j, k)] = (hq[i], hs[i], a[i], acc[i], absum[i])
    for j, t in enumerate(tokens):
        for k in range(top_k):
            if (j, k) in ys:
                out[j] += float(np.float32(topk_w[t, k])) * ys[(j, k)]
    return dict(out=out, h=hqs)

