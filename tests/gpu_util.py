"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle.codecs import f64_to_bf16_value

_WEIGHT_CACHE = {}


def full_size_weights(E=896, H=7168, I=3584):
    """The 896-expert weight set shared by the full-size workloads, drawn on
    the GPU once per process."""
    import synth

    key = (E, H, I)
    if key not in _WEIGHT_CACHE:
        _WEIGHT_CACHE.clear()
        torch.cuda.empty_cache()
        cfg = synth.custom_config("weights", 0, T=1, H=H, I=I, E=E, K=1, E_local=E)
        _WEIGHT_CACHE[key] = synth.make_expert_weights(cfg, device="cuda")
        torch.cuda.synchronize()
    return _WEIGHT_CACHE[key]


def to_np(t):
    return t.detach().cpu().numpy()


def run_steps(layer, x, logits, bias, topk_idx=None, topk_w=None):
    """Run the layer through the binding; return every intermediate as numpy."""
    out = layer(x, logits, bias, topk_idx=topk_idx, topk_w=topk_w)
    torch.cuda.synchronize()
    T = x.shape[0]
    R = T * layer.top_k
    res = dict(
        out_bits=to_np(out.view(torch.uint16)),
        xq=to_np(layer.xq[:T]), xs=to_np(layer.xs[:T]),
        expert_offsets=to_np(layer.expert_offsets), sorted_route=to_np(layer.sorted_route[:R]),
        route_row=to_np(layer.route_row[:R]), hq=to_np(layer.hq[:R]), hs=to_np(layer.hs[:R]),
    )
    if topk_idx is None:
        res["topk_idx"] = to_np(layer.topk_idx[:T])
        res["topk_w"] = to_np(layer.topk_w[:T])
    res["out"] = (res["out_bits"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return res


def output_stats(out, ref):
    """max|out-ref| / RMS(ref), cosine, and the bf16 format floor, in float64."""
    ref = np.asarray(ref, np.float64)
    out = np.asarray(out, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = float(np.abs(out - ref).max()) if ref.size else 0.0
    denom = float(np.linalg.norm(out) * np.linalg.norm(ref))
    cos = float(np.dot(out.ravel(), ref.ravel()) / denom) if denom > 0 else 1.0
    floor = float(np.abs(f64_to_bf16_value(ref) - ref).max()) / rms if rms > 0 else 0.0
    return dict(max_err_over_rms=err / rms if rms > 0 else err, cosine=cos, bf16_floor=floor,
                rms=rms)


def assert_output_close(out, ref, tag=""):
    st = output_stats(out, ref)
    print(f"[{tag}] max|err|/RMS={st['max_err_over_rms']:.4g} cosine={st['cosine']:.8f} "
          f"bf16 floor={st['bf16_floor']:.4g}", flush=True)
    assert np.all(np.isfinite(out))
    assert st["max_err_over_rms"] <= 2e-2, st
    assert st["cosine"] >= 0.9995, st
    return st


E4M3_POS = None


def _e4m3_grid():
    global E4M3_POS
    if E4M3_POS is None:
        from oracle.codecs import E4M3_TABLE
        E4M3_POS = E4M3_TABLE[:0x7F].copy()
    return E4M3_POS


def check_requant(hq_g, hs_g, a_ref, hq_ref, hs_ref, tag="", max_frac=1e-3, mid_tol=0.05):
    """The GPU requantises float32 accumulators, the oracle exact float64 ones,
    so a byte may differ where the exact value sits next to an E4M3 rounding
    point.  Each differing element must be the E4M3 rounding of some value
    within ``mid_tol`` of the exact one (in units of the scaled element, whose
    range is [0, 448]; the float32 error of the GPU's SiTU output is about
    1e-4 there): |v - y| <= |rne(y) - y| + 2 * mid_tol.  A differing scale
    must keep the group's absmax within (224, 448] up to 1e-3.  Returns the
    differing dequantised amounts, float64 [rows, I]."""
    from oracle.codecs import e4m3_decode, e4m3_encode, mxfp8_dequantize

    hq_g, hs_g = np.asarray(hq_g), np.asarray(hs_g)
    rows, I = hq_g.shape
    frac_q = byte_mismatch(hq_g, hq_ref)
    frac_s = byte_mismatch(hs_g, hs_ref)
    print(f"[{tag}] hq mismatch {frac_q:.3g}, hs mismatch {frac_s:.3g}", flush=True)
    assert frac_q <= max_frac and frac_s <= max_frac, (frac_q, frac_s)
    a = np.asarray(a_ref, np.float64).reshape(rows, I // 32, 32)
    amax = np.abs(a).max(-1)
    eg = hs_g.astype(np.int64) - 127
    bad_s = hs_g != hs_ref
    if bad_s.any():
        r = amax[bad_s] * np.ldexp(1.0, -eg[bad_s])
        assert np.all((r > 224 * (1 - 1e-3)) & (r <= 448 * (1 + 1e-3))), "scale flip not at a boundary"
    diff = (hq_g != hq_ref).reshape(rows, I // 32, 32) | bad_s[..., None]
    if diff.any():
        y = (a * np.ldexp(1.0, -eg)[..., None])[diff]        # exact value at the GPU's scale
        cg = hq_g.reshape(rows, I // 32, 32)[diff]
        rne = e4m3_encode(y)
        other = cg != rne                                     # not the correctly rounded code
        if other.any():
            # The GPU rounds a value y' with |y' - y| <= mid_tol to its nearest
            # grid point v, so |v - y| <= |rne(y) - y| + 2 * mid_tol.
            yo = y[other]
            vg = e4m3_decode(cg[other])
            vr = e4m3_decode(rne[other])
            yc = np.clip(yo, -448.0, 448.0)
            excess = np.abs(vg - yc) - np.abs(vr - yc)
            worst = int(np.argmax(excess))
            assert excess[worst] <= 2 * mid_tol, (
                f"requantised byte {cg[other][worst]:#04x} for exact scaled value "
                f"{yo[worst]!r} (nearest code {rne[other][worst]:#04x}) is "
                f"{excess[worst]:.4g} farther than the nearest")
    return mxfp8_dequantize(hq_g, hs_g) - mxfp8_dequantize(hq_ref, hs_ref)


def flip_allowance(delta, tokens, K, route_row, topk_w, expert_of_row, w2_deq, H):
    """Largest change of the given output rows that the differing FC2 inputs
    can cause: sum over kept slots of |w| * |W2_e| @ |delta(row)|, where
    ``delta(row)`` is the dequantised difference of that grouped row (or None)
    and ``w2_deq(e)`` returns dequantised W2 [H, I]."""
    cache = {}
    out = np.zeros((len(tokens), H))
    for j, t in enumerate(tokens):
        for k in range(K):
            row = int(route_row[t * K + k])
            d = delta(row) if row >= 0 else None
            if d is None or not np.any(d):
                continue
            e = int(expert_of_row(row))
            if e not in cache:
                cache[e] = np.abs(w2_deq(e))
            out[j] += abs(float(np.float32(topk_w[t, k]))) * (cache[e] @ np.abs(d))
    return out


def assert_output_with_allowance(out, ref, allowance, tag=""):
    st = output_stats(out, ref)
    allow = 0.0 if allowance is None else allowance
    excess = np.abs(np.asarray(out, np.float64) - ref) - np.asarray(allow)
    worst = float(excess.max()) / st["rms"] if st["rms"] > 0 else float(excess.max())
    print(f"[{tag}] max|err|/RMS={st['max_err_over_rms']:.4g} (beyond the requant-flip bound "
          f"{worst:.4g}) cosine={st['cosine']:.8f} bf16 floor={st['bf16_floor']:.4g}", flush=True)
    assert np.all(np.isfinite(out))
    assert worst <= 2e-2, st
    assert st["cosine"] >= 0.9995, st
    return st


def byte_mismatch(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    return float(np.mean(a != b)) if a.size else 0.0
