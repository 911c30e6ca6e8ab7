"""Element codecs of the MX formats, written from their definitions.

Test infrastructure only (see ``oracle/__init__``).

* E4M3 (OCP 8-bit float, "fn" variant): sign, 4 exponent bits (bias 7),
  3 mantissa bits; subnormals m * 2**-9; largest finite 448; no infinities;
  S.1111.111 is NaN.  Page 5 ("forward" notes) quantises activations to
  "fp8 e4m3"; page 1 ("NaN/Inf decision record") fixes the conversion to
  saturate to a finite value.
* E2M1 (4-bit float): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the
  sign.  Page 1 ("real checkpoint contract") stores two per byte.
* E8M0 (unsigned power-of-two scale): byte b is 2**(b-127) for b in
  0x00..0xFE, 0xFF is NaN (page 1, "NaN/Inf decision record").

The scale exponent of a 32-element group follows the reading taken where the
pages only say "absmax -> UE8M0 scale": the smallest power of two that keeps
the group's absmax within the element format's largest finite value, so no
element clips (page 5 pre-dispatch notes; page 1 "saturating finite").
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
GROUP = 32


def _e4m3_table() -> np.ndarray:
    v = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        ex = (c >> 3) & 0xF
        m = c & 7
        if ex == 0xF and m == 7:
            v[c] = np.nan
        elif ex == 0:
            v[c] = s * m * 2.0 ** -9
        else:
            v[c] = s * (1.0 + m / 8.0) * 2.0 ** (ex - 7)
    return v


E4M3_TABLE = _e4m3_table()
# Non-negative finite magnitudes in code order 0x00..0x7E (strictly increasing).
_E4M3_POS = E4M3_TABLE[:0x7F].copy()

E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_TABLE = np.concatenate([E2M1_MAGS, -E2M1_MAGS])


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_decode(codes) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e8m0_decode(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code to each float64 ``y`` (ties to the even code).

    Magnitudes beyond 448 saturate to 448; the sign of zero is kept (a
    negative value that rounds to zero gives 0x80); NaN gives 0x00.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    finite_a = np.where(np.isnan(a), 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_E4M3_POS, finite_a, side="left")     # first magnitude >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = finite_a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - finite_a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(finite_a == _E4M3_POS[hi], hi, code).astype(np.uint8)
    code |= (np.signbit(y) & ~np.isnan(y)).astype(np.uint8) << 7
    return code


def mx_exponent(amax, elem_max: float) -> np.ndarray:
    """Smallest integer e with amax <= elem_max * 2**e, clamped to [-127, 127].

    amax == 0 gives -127; an infinite amax gives 127."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where((amax > 0) & np.isfinite(amax), amax, 1.0)
    _, q = np.frexp(safe)                       # safe = m * 2**q, m in [0.5, 1)
    e = q.astype(np.int64) - 1 - int(np.floor(np.log2(elem_max)))
    # Settle e exactly with power-of-two comparisons (all exact in float64).
    for _ in range(3):
        e = np.where(safe > elem_max * np.ldexp(1.0, e), e + 1, e)
    for _ in range(3):
        e = np.where(safe <= elem_max * np.ldexp(1.0, e - 1), e - 1, e)
    e = np.where(amax == 0, -127, e)
    e = np.where(np.isinf(amax), 127, e)
    return np.clip(e, -127, 127)


def mxfp8_quantize(v):
    """MXFP8 (E4M3 elements, E8M0 scale per 32 along the last axis).

    ``v``: float64 ``[rows, K]`` with K a multiple of 32.
    Returns (codes uint8 [rows, K], scale bytes uint8 [rows, K/32]).
    NaN elements are ignored by the absmax and encode as 0x00."""
    v = np.asarray(v, dtype=np.float64)
    rows, K = v.shape
    g = v.reshape(rows, K // GROUP, GROUP)
    a = np.abs(g)
    amax = np.max(np.where(np.isnan(a), 0.0, a), axis=-1)
    e = mx_exponent(amax, E4M3_MAX)
    y = g * np.ldexp(1.0, -e)[..., None]
    codes = e4m3_encode(y).reshape(rows, K)
    return codes, (e + 127).astype(np.uint8)


def mxfp8_dequantize(codes, scales) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    v = e4m3_decode(codes).reshape(rows, K // GROUP, GROUP)
    return (v * e8m0_decode(scales)[..., None]).reshape(rows, K)


def mxfp4_dequantize(packed, scales) -> np.ndarray:
    """Packed E2M1 ``[rows, K/2]`` (element 2j in the low nibble of byte j,
    element 2j+1 in the high nibble) with E8M0 scales ``[rows, K/32]``."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    K = 2 * half
    v = np.empty((rows, K), np.float64)
    v[:, 0::2] = E2M1_TABLE[packed & 0xF]
    v[:, 1::2] = E2M1_TABLE[packed >> 4]
    v = v.reshape(rows, K // GROUP, GROUP) * e8m0_decode(scales)[..., None]
    return v.reshape(rows, K)


def bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_value(v) -> np.ndarray:
    """Nearest bf16 value (ties to even), returned as float64 (report only)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)   # RNE to f32 first
    b = f.view(np.uint32).astype(np.uint64)
    # Round the f32 to 8 significant bits; double rounding through f32 can only
    # matter on exact bf16 midpoints of the f64 value, which reporting ignores.
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.view(np.float32).astype(np.float64)
