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


# Bound on the block-scaled MFMA's accumulation error: one 16x16x128 MFMA
# step adds at most ACC_EPS times the sum of |products| of its 128-K slice
# (tests/test_gpu_numerics.py measures at most 8.9e-6, about 2^-16.8, for a
# single step with the layer's value distributions; 2^-15 leaves a factor of
# 3.4), so by the triangle inequality a dot product over K is off by at most
# ACC_EPS times its whole sum of |products| (measured at K = 7168: 3.6e-7).
ACC_EPS = 2.0 ** -15


def situ_f32_error(g, u, alpha=4.0, beta=25.0):
    """Bound on the kernel's float32 SiTU error at exact inputs g, u (checked
    on the device by tests/test_gpu_numerics.py): (32 + 2|g|) 2^-24 relative
    (float32 roundings and the exponent's), plus 2^-22 of each tanh factor's
    scale (alpha, beta) times the other factor, where 1 - e^(-2y) cancels."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        sg = 1.0 / (1.0 + np.exp(-g))
        gate = alpha * np.tanh(g / alpha) * sg
        up = beta * np.tanh(u / beta)
        rel = (32.0 + 2.0 * np.abs(g)) * 2.0 ** -24 * np.abs(gate * up)
        cancel = 2.0 ** -22 * (alpha * sg * np.abs(up) + beta * np.abs(gate))
    return rel + cancel + 1e-36


def situ_error_bound(g, u, absum_g, absum_u, alpha=4.0, beta=25.0):
    """Largest |SiTU_gpu - SiTU(g, u)| when the GPU's accumulators carry at
    most ACC_EPS * absum of error and its float32 SiTU is within
    situ_f32_error (both checked in tests/test_gpu_numerics.py): first-order
    terms with a 25% margin plus the second-order ones."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        tg, tu = np.tanh(g / alpha), np.tanh(u / beta)
        sg = 1.0 / (1.0 + np.exp(-g))
        gate, up = alpha * tg * sg, beta * tu
        dgate = (1.0 - tg * tg) * sg + alpha * tg * sg * (1.0 - sg)
        dup = 1.0 - tu * tu
        dg, du = ACC_EPS * np.asarray(absum_g), ACC_EPS * np.asarray(absum_u)
        first = np.abs(dgate * up) * dg + np.abs(gate * dup) * du
        second = 0.5 * (np.abs(up) * dg * dg + 0.1 * np.abs(gate) * du * du) + np.abs(dgate * dup) * dg * du
        bound = 1.25 * first + second + situ_f32_error(g, u, alpha, beta)
    return np.where(np.isfinite(bound), bound, np.inf)


def check_requant(hq_g, hs_g, hq_ref, hs_ref, a_ref, acc_ref, absum_ref, tag="", max_frac=5e-3,
                  alpha=4.0, beta=25.0):
    """The GPU requantises float32 accumulators, the oracle exact float64 ones,
    so a byte may differ where the exact value sits next to an E4M3 rounding
    point or a scale boundary.  Every byte is held to what the GPU's measured
    error allows: with da = situ_error_bound(...) for each element,
      * the GPU's scale exponent lies between the rule's exponents for the
        group absmax minus and plus max(da) over the group;
      * the GPU's element code lies between the nearest-even codes of
        (a - da) / 2^e and (a + da) / 2^e at the GPU's exponent e.
    At most ``max_frac`` of the bytes of the rows may differ.  Returns the
    differing dequantised amounts, float64 [rows, I]."""
    from oracle.codecs import e4m3_decode, e4m3_encode, mx_exponent, mxfp8_dequantize

    hq_g, hs_g = np.asarray(hq_g), np.asarray(hs_g)
    rows, I = hq_g.shape
    frac_q = byte_mismatch(hq_g, hq_ref)
    frac_s = byte_mismatch(hs_g, hs_ref)
    print(f"[{tag}] hq mismatch {frac_q:.3g}, hs mismatch {frac_s:.3g}", flush=True)
    assert frac_q <= max_frac and frac_s <= max_frac, (frac_q, frac_s)
    a = np.asarray(a_ref, np.float64).reshape(rows, I)
    acc = np.asarray(acc_ref, np.float64).reshape(rows, 2 * I)
    absum = np.asarray(absum_ref, np.float64).reshape(rows, 2 * I)
    da = situ_error_bound(acc[:, :I], acc[:, I:], absum[:, :I], absum[:, I:], alpha, beta)
    ag = np.where(np.isnan(a), 0.0, np.abs(a)).reshape(rows, I // 32, 32)
    dag = da.reshape(rows, I // 32, 32).max(-1)
    amax = ag.max(-1)
    eg = hs_g.astype(np.int64) - 127
    e_lo = mx_exponent(np.maximum(amax - dag, 0.0), 448.0)
    e_hi = mx_exponent(amax + dag, 448.0)
    bad_s = (eg < e_lo) | (eg > e_hi)
    assert not bad_s.any(), f"[{tag}] scale byte outside what the error bound allows"
    diff = (hq_g != np.asarray(hq_ref)).reshape(rows, I // 32, 32) | (hs_g != hs_ref)[..., None]
    if diff.any():
        scale = np.ldexp(1.0, -eg)[..., None]
        a3 = a.reshape(rows, I // 32, 32)
        d3 = da.reshape(rows, I // 32, 32)
        lo = e4m3_decode(e4m3_encode(((a3 - d3) * scale)[diff]))
        hi = e4m3_decode(e4m3_encode(((a3 + d3) * scale)[diff]))
        vg = e4m3_decode(hq_g.reshape(rows, I // 32, 32)[diff])
        ok = (vg >= lo) & (vg <= hi) | ~np.isfinite(a3[diff])
        if not ok.all():
            i = int(np.argmin(ok))
            raise AssertionError(
                f"[{tag}] requantised value {vg[i]!r} outside [{lo[i]!r}, {hi[i]!r}] "
                f"(exact scaled {(a3 * scale)[diff][i]!r})")
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


def assert_output_with_allowance(out, ref, allowance, tag="", raw=True):
    """The output bar, max|out - ref| <= 2e-2 RMS(ref) and cosine >= 0.9995.

    ``raw``: on the raw error (the named workloads).  Otherwise (small test
    shapes, H <= 1024, where an output sums few terms and one E4M3 step of a
    single FC2 input can move it by more than 2% of its RMS) on the error
    beyond ``allowance``, the largest change the differing requantised bytes
    can cause; check_requant has already held each of those bytes to the
    measured hardware error.  Both figures are printed."""
    st = output_stats(out, ref)
    allow = 0.0 if allowance is None else allowance
    excess = np.abs(np.asarray(out, np.float64) - ref) - np.asarray(allow)
    beyond = float(excess.max()) / st["rms"] if st["rms"] > 0 else float(excess.max())
    print(f"[{tag}] max|err|/RMS={st['max_err_over_rms']:.4g} (beyond the requant-flip bound "
          f"{beyond:.4g}) cosine={st['cosine']:.8f} bf16 floor={st['bf16_floor']:.4g}", flush=True)
    assert np.all(np.isfinite(out))
    assert (st["max_err_over_rms"] if raw else beyond) <= 2e-2, st
    assert st["cosine"] >= 0.9995, st
    return st


def byte_mismatch(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    return float(np.mean(a != b)) if a.size else 0.0
