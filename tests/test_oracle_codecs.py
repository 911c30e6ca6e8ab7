"""Pins of the oracle's element codecs (CPU only).

Each check compares the oracle with something other than itself: the OCP MX
closed forms, torch's own float8 conversions (an independent implementation),
exhaustive nearest-value search, or exact rational arithmetic.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kimi_k3_facts.json")


def _all_bf16_f64():
    bits = np.arange(65536, dtype=np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def test_e4m3_closed_form_extremes():
    # OCP E4M3 ("fn"): largest finite 448 at 0x7E, smallest normal 2^-6 at
    # 0x08, smallest subnormal 2^-9 at 0x01, S.1111.111 is NaN, no infinity.
    t = C.E4M3_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    fin = t[:0x7F]
    assert np.all(np.diff(fin) > 0) and np.isfinite(t).sum() == 254


def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = C.e4m3_decode(np.arange(256))
    same = (ref == ours) | (np.isnan(ref) & np.isnan(ours))
    assert same.all()


def test_e4m3_encode_matches_torch_rne_on_every_bf16():
    # torch converts float32 -> float8_e4m3fn with round-to-nearest-even and
    # no saturation (values >= 464 become NaN), so compare below 464.
    v = _all_bf16_f64()
    fin = np.isfinite(v) & (np.abs(v) < 464.0)
    ours = C.e4m3_encode(v[fin])
    ref = torch.from_numpy(v[fin].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates_and_keeps_sign_of_zero():
    v = np.array([464.0, 1e30, np.inf, -500.0, -np.inf, -1e-30, -0.0, 0.0, np.nan])
    assert list(C.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x80, 0x00, 0x00]


def test_e4m3_encode_is_nearest_with_even_ties_bruteforce():
    # Independent brute force: distance to all 127 magnitudes; ties -> even code.
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(-450, 450, 20000),
        rng.uniform(-2 ** -5, 2 ** -5, 20000),
        # exact midpoints between neighbouring codes
        (C.E4M3_TABLE[1:0x7E] + C.E4M3_TABLE[2:0x7F]) / 2,
    ])
    mags = C.E4M3_TABLE[:0x7F]
    for x in v:
        d = np.abs(mags - abs(x))
        best = np.flatnonzero(d == d.min())
        code = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        code |= 0x80 if np.signbit(x) else 0
        assert C.e4m3_encode(np.array([x]))[0] == code, x


def test_e8m0_matches_torch_and_pages():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = C.e8m0_decode(np.arange(256))
    assert np.array_equal(ref[:255], ours[:255]) and np.isnan(ours[255]) and np.isnan(ref[255])
    facts = json.load(open(GOLDEN))["e8m0"]
    assert np.isfinite(C.e8m0_decode(facts["max_finite_byte"]))
    assert np.isnan(C.e8m0_decode(facts["nan_byte"]))


def test_e2m1_from_bit_fields():
    # E2M1: 2 exponent bits (bias 1), 1 mantissa bit, subnormal m * 0.5.
    for c in range(16):
        s, ex, m = c >> 3, (c >> 1) & 3, c & 1
        mag = 0.5 * m if ex == 0 else 2.0 ** (ex - 1) * (1 + 0.5 * m)
        val = -mag if s else mag
        assert C.e2m1_decode(np.array([c]))[0] == val
    assert C.E2M1_MAGS.max() == 6.0


def test_mx_exponent_exact_against_rationals():
    # e = min{e : amax <= 448 * 2^e}: check with exact Fractions on every
    # positive finite bf16 amax.
    v = _all_bf16_f64()
    amax = v[(v > 0) & np.isfinite(v)]
    e = C.mx_exponent(amax, 448.0)
    for a, ee in zip(amax[::7], e[::7]):
        fa = Fraction(float(a))
        lim = lambda k: Fraction(448) * (Fraction(2) ** int(k))
        if ee > -127:
            assert fa <= lim(ee) and fa > lim(ee - 1)
        else:
            assert fa <= lim(-127)
    assert C.mx_exponent(np.array([0.0]), 448.0)[0] == -127
    assert C.mx_exponent(np.array([np.inf]), 448.0)[0] == 127
    # the rule is monotone and never clips
    assert np.all(np.diff(e) >= 0)


def test_mxfp8_group_invariants():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    codes, sc = C.mxfp8_quantize(v)
    assert codes.shape == v.shape and sc.shape == (64, 8)
    assert not np.any(sc == 0xFF)
    assert not np.any((codes & 0x7F) == 0x7F)
    deq = C.mxfp8_dequantize(codes, sc)
    g = np.abs(v).reshape(64, 8, 32)
    scale = C.e8m0_decode(sc)
    # absmax lands in (224, 448] after scaling: no clipping, top code used.
    r = g.max(-1) / scale
    assert np.all(r <= 448) and np.all(r > 224)
    # error <= half a step of the element grid (relative 2^-4 for normals,
    # absolute 2^-10 * scale for subnormals).
    err = np.abs(deq - v).reshape(64, 8, 32)
    bound = np.maximum(np.abs(v).reshape(64, 8, 32) * 2.0 ** -4, 2.0 ** -10 * scale[..., None])
    assert np.all(err <= bound)


def test_mxfp4_nibble_order_and_scale_rows():
    # element 2j in the low nibble, 2j+1 in the high nibble; scale [row, k/32]
    packed = np.zeros((2, 32), np.uint8)
    packed[0, 0] = 0x72          # k=0 -> code 2 (1.0), k=1 -> code 7 (6.0)
    packed[1, 17] = 0x0B         # k=34 -> code 0xB (-1.5)
    sc = np.full((2, 2), 127, np.uint8)
    sc[1, 1] = 130               # second group of row 1 scaled by 8
    v = C.mxfp4_dequantize(packed, sc)
    assert v[0, 0] == 1.0 and v[0, 1] == 6.0 and v[1, 34] == -12.0
    assert np.count_nonzero(v) == 3


def test_checkpoint_shapes_match_layout():
    # The [rows, K/2] packed and [rows, K/32] scale forms reproduce the shapes
    # printed for the real checkpoint (H = 3584 routed latent, I = 3072).
    f = json.load(open(GOLDEN))["checkpoint_expert_tensors"]
    H, I = f["routed_latent_H"], f["intermediate_I"]
    assert f["w1.weight_packed"] == [I, H // 2] and f["w1.weight_scale"] == [I, H // 32]
    assert f["w2.weight_packed"] == [H, I // 2] and f["w2.weight_scale"] == [H, I // 32]
    facts = json.load(open(GOLDEN))["x_sf_view"]
    assert facts["bytes_per_int32"] * facts["elements_per_scale"] == 128


def test_f64_to_bf16_value_matches_torch_on_float32_inputs():
    """The report-only bf16 rounding agrees with torch's own float32 ->
    bfloat16 conversion (round to nearest, ties to even) on float32 values:
    random magnitudes across the exponent range, exact bf16 midpoints (ties),
    their float32 neighbours, subnormals, the largest finite values."""
    import torch

    from oracle.codecs import f64_to_bf16_value

    rng = np.random.default_rng(3)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-130, 120, 20000))).astype(np.float32)
    grid = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    grid = grid[np.isfinite(grid)]
    mid = (grid.view(np.uint32) + np.uint32(0x8000)).view(np.float32)     # exact ties
    mid = mid[np.isfinite(mid)]
    near = np.concatenate([np.nextafter(mid, np.float32(np.inf)),
                           np.nextafter(mid, np.float32(-np.inf))])
    x = np.concatenate([v, mid, near, np.float32([3.3e38, -3.3e38, 1e-45, -1e-45, 0.0, -0.0])])
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = f64_to_bf16_value(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_f64_to_bf16_value_is_a_nearest_bf16_of_float64_inputs():
    """On float64 values that are not float32 values, the result is a bf16
    value no farther from the input than either bf16 neighbour of it, in
    exact rational arithmetic (the float64 -> float32 -> bf16 double rounding
    can only pick the other of two equally near values on an exact tie)."""
    from fractions import Fraction

    from oracle.codecs import f64_to_bf16_value

    rng = np.random.default_rng(4)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))
    got = f64_to_bf16_value(v)
    bits = got.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)                       # a bf16 value
    up = (bits + 0x10000).view(np.float32).astype(np.float64)
    dn = (bits - 0x10000).view(np.float32).astype(np.float64)
    for x, r, a, b in zip(v, got, up, dn):
        d = abs(Fraction(float(r)) - Fraction(float(x)))
        assert d <= abs(Fraction(float(a)) - Fraction(float(x)))
        assert d <= abs(Fraction(float(b)) - Fraction(float(x)))
