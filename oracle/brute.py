"""Brute-force restatement of the layer for tiny shapes (checks the oracle).

Test infrastructure only (see ``oracle/__init__``).

Everything here works one token and one route at a time with Python scalars
and explicit loops: a full sort of all experts per token, per-element
dequantisation with ``math.ldexp``, dense dot products, and the combine
summed slot by slot.  It shares only the element codecs with
``oracle.layer`` (those are pinned on their own), so a mistake in the
grouping, gathering, gate/up split, SiTU wiring, requantisation or combine of
``oracle.layer`` shows up as a mismatch.
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import e2m1_decode, e4m3_decode, e4m3_encode, mx_exponent


def _bf16(bits: int) -> float:
    return float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0])


def _sig(v: float) -> float:
    if v < -745.0:
        return 0.0
    return 1.0 / (1.0 + math.exp(-v))


def _quant_row(vals):
    """MXFP8-encode one row (list of floats) group by group."""
    codes, scales = [], []
    for g0 in range(0, len(vals), 32):
        grp = vals[g0:g0 + 32]
        amax = max(abs(v) for v in grp)
        e = int(mx_exponent(np.array([amax]), 448.0)[0])
        scales.append(e + 127)
        for v in grp:
            codes.append(int(e4m3_encode(np.array([math.ldexp(v, -e)]))[0]))
    return codes, scales


_E4M3 = [float(v) for v in e4m3_decode(np.arange(256))]
_E2M1 = [float(v) for v in e2m1_decode(np.arange(16))]


def _deq8(codes, scales):
    return [_E4M3[c] * math.ldexp(1.0, scales[j // 32] - 127) for j, c in enumerate(codes)]


def _deq4_row(packed_row, scale_row):
    out = []
    for byte in packed_row:
        for nib in (int(byte) & 0xF, int(byte) >> 4):   # element 2j low, 2j+1 high
            k = len(out)
            out.append(_E2M1[nib] * math.ldexp(1.0, int(scale_row[k // 32]) - 127))
    return out


def brute_force_layer(x_bf16, logits, bias, w13, w13_s, w2, w2_s, *, top_k,
                      expert_offset=0, routed_scaling=1.0, alpha=4.0, beta=25.0,
                      topk_idx=None, topk_w=None):
    """Returns dict(topk_idx, topk_w, out [T,H] float64, h {(t,k): (codes, scales)})."""
    x_bf16 = np.asarray(x_bf16)
    T, H = x_bf16.shape
    E_local = np.asarray(w13).shape[0]
    I = np.asarray(w13).shape[1] // 2
    if topk_idx is None:
        E = np.asarray(logits).shape[1]
        ids = np.zeros((T, top_k), np.int32)
        ws = np.zeros((T, top_k), np.float32)
        for t in range(T):
            scores = []
            for e in range(E):
                s = float(np.float32(_sig(float(logits[t, e]))))
                b = 0.0 if bias is None else float(bias[e])
                key = float(np.float32(np.float32(s) + np.float32(b)))
                scores.append((key, e, s))
            # Sort by key descending, then index ascending.
            scores.sort(key=lambda z: (-z[0], z[1]))
            top = scores[:top_k]
            tot = 0.0
            for z in top:
                tot += z[2]
            for k, z in enumerate(top):
                ids[t, k] = z[1]
                ws[t, k] = np.float32(z[2] / tot * routed_scaling)
        topk_idx, topk_w = ids, ws
    out = np.zeros((T, H), np.float64)
    hs_all = {}
    cache = {}

    def _row(key, packed, scale):
        if key not in cache:
            cache[key] = _deq4_row(packed, scale)
        return cache[key]

    for t in range(T):
        xrow = [_bf16(b) for b in x_bf16[t]]
        xc, xsc = _quant_row(xrow)
        a = _deq8(xc, xsc)
        for k in range(top_k):
            g = int(topk_idx[t, k])
            e = g - expert_offset
            if g < 0 or not (0 <= e < E_local):
                continue
            gate = []
            up = []
            for n in range(2 * I):
                w = _row(("w13", e, n), w13[e][n], w13_s[e][n])
                acc = 0.0
                for i in range(H):
                    acc += a[i] * w[i]
                (gate if n < I else up).append(acc)
            act = []
            for n in range(I):
                gv, uv = gate[n], up[n]
                act.append(alpha * math.tanh(gv / alpha) * _sig(gv) * beta * math.tanh(uv / beta))
            hc, hsc = _quant_row(act)
            hs_all[(t, k)] = (hc, hsc)
            h = _deq8(hc, hsc)
            for o in range(H):
                w = _row(("w2", e, o), w2[e][o], w2_s[e][o])
                y = 0.0
                for i in range(I):
                    y += h[i] * w[i]
                out[t, o] += float(topk_w[t, k]) * y
    return dict(topk_idx=topk_idx, topk_w=topk_w, out=out, h=hs_all)
