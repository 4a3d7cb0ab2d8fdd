"""fp8 quantise-dequantise emulation (test infrastructure).

The "additions" page's feature table lists dynamic per-tensor fp8 with the
e4m3 and e5m2 formats; the "overview" page (section 4) describes quantise /
dequantise around each scaled matmul. The formats are the OCP 8-bit floats:

  e4m3: 4 exponent bits (bias 7), 3 mantissa bits, no infinity, largest
        finite 448, smallest normal 2^-6, subnormal step 2^-9.
  e5m2: 5 exponent bits (bias 15), 2 mantissa bits, largest finite 57344,
        smallest normal 2^-14, subnormal step 2^-16.

Per-tensor dynamic scaling: s = fmax / amax(X) in fp32 (s = 1 when amax is
0 or not finite). The pages do not say in which precision X * s is formed;
the reading here is fp32 (the precision the scale itself is held in), so
the code of an element is RNE(clamp(fp32(fp32(x) * s), -fmax, fmax)) with
round-to-nearest-even and saturation, and the dequantised value is
code / s. Everything after the fp32 product is exact in float64.
"""
from __future__ import annotations

import numpy as np

FORMATS = {
    # name: (mantissa bits, smallest normal exponent, largest finite)
    "e4m3": (3, -6, 448.0),
    "e5m2": (2, -14, 57344.0),
}
_BIAS = {"e4m3": 7, "e5m2": 15}


def round_fp8(x, fmt):
    """Nearest representable value of ``fmt`` (ties to even), saturating at
    +-fmax. Returns float64."""
    m, emin, fmax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, E = np.frexp(a)                  # a = f * 2^E, f in [0.5, 1)
    e = np.maximum(E - 1, emin)         # exponent of the binade (subnormals: emin)
    q = np.ldexp(1.0, (e - m).astype(np.int64))   # spacing of representable values
    r = np.rint(a / q) * q
    r = np.minimum(r, fmax)
    r = np.where(a == 0, 0.0, r)
    return np.copysign(r, x)


def encode(v, fmt):
    """Byte code (uint8) of values that ``fmt`` represents exactly: sign bit,
    biased exponent (0 for subnormals and zero), mantissa."""
    m, emin, _ = FORMATS[fmt]
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, E = np.frexp(a)
    e = np.maximum(E - 1, emin)
    normal = (a >= 2.0 ** emin)
    frac = np.where(normal, a / np.ldexp(1.0, e.astype(np.int64)) - 1.0,
                    a / 2.0 ** emin)                  # mantissa fraction in [0, 1)
    mant = np.rint(frac * (1 << m)).astype(np.int64)
    assert np.all(np.abs(frac * (1 << m) - mant) == 0), "value not representable"
    bexp = np.where(normal, e + _BIAS[fmt], 0).astype(np.int64)
    sign = np.signbit(v).astype(np.int64)
    return ((sign << 7) | (bexp << m) | mant).astype(np.uint8)


def decode(codes, fmt):
    """Values of byte codes (float64); NaN / infinity codes are not used."""
    m, emin, _ = FORMATS[fmt]
    c = np.asarray(codes).astype(np.int64)
    bexp = (c >> m) & ((1 << (7 - m)) - 1)
    mant = c & ((1 << m) - 1)
    mag = np.where(bexp == 0, mant / (1 << m) * 2.0 ** emin,
                   (1.0 + mant / (1 << m)) * np.ldexp(1.0, (bexp - _BIAS[fmt]).astype(np.int64)))
    return np.where(c & 0x80, -mag, mag)


def round_bf16(x):
    """Nearest bfloat16 value (8 significant bits, ties to even) of float32
    values, returned as float32: add half of the dropped 16 bits (plus the
    kept bit for ties) and truncate. Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def scale_for(x, fmt):
    """Per-tensor scale fmax / amax, in float32 as a device would hold it."""
    fmax = FORMATS[fmt][2]
    amax = float(np.max(np.abs(x))) if np.size(x) else 0.0
    if amax == 0.0 or not np.isfinite(amax):
        return np.float32(1.0)
    return np.float32(np.float32(fmax) / np.float32(amax))


def scaled(x, s, fmt):
    """fp32(fp32(x) * s), clamped to +-fmax (exact in the result's float64)."""
    fmax = FORMATS[fmt][2]
    xs = np.asarray(x).astype(np.float32) * np.float32(s)
    return np.clip(xs.astype(np.float64), -fmax, fmax)


def quantize(x, fmt):
    """(byte codes, scale) of x under its dynamic per-tensor scale."""
    s = scale_for(x, fmt)
    return encode(round_fp8(scaled(x, s, fmt), fmt), fmt), s


def qdq(x, fmt):
    """Quantise with the dynamic per-tensor scale and dequantise."""
    s = scale_for(x, fmt)
    return (round_fp8(scaled(x, s, fmt), fmt) / float(s)).astype(np.asarray(x).dtype)
