"""fp8 quantise-dequantise emulation (test infrastructure).

The "additions" page's feature table lists dynamic per-tensor fp8 with the
e4m3 and e5m2 formats; the "overview" page (section 4) describes quantise /
dequantise around each scaled matmul. The formats are the OCP 8-bit floats:

  e4m3: 4 exponent bits (bias 7), 3 mantissa bits, no infinity, largest
        finite 448, smallest normal 2^-6, subnormal step 2^-9.
  e5m2: 5 exponent bits (bias 15), 2 mantissa bits, largest finite 57344,
        smallest normal 2^-14, subnormal step 2^-16.

Per-tensor dynamic scaling: s = fmax / amax(X) (s = 1 when amax = 0);
Q(X) = round(clamp(X * s, -fmax, fmax)) / s, with round-to-nearest-even and
saturation. Values are computed in float64.
"""
from __future__ import annotations

import numpy as np

FORMATS = {
    # name: (mantissa bits, smallest normal exponent, largest finite)
    "e4m3": (3, -6, 448.0),
    "e5m2": (2, -14, 57344.0),
}


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


def scale_for(x, fmt):
    """Per-tensor scale fmax / amax, in float32 as a device would hold it."""
    fmax = FORMATS[fmt][2]
    amax = float(np.max(np.abs(x))) if np.size(x) else 0.0
    if amax == 0.0 or not np.isfinite(amax):
        return np.float32(1.0)
    return np.float32(fmax / np.float32(amax))


def qdq(x, fmt):
    """Quantise with the dynamic per-tensor scale and dequantise."""
    s = float(scale_for(x, fmt))
    fmax = FORMATS[fmt][2]
    xs = np.clip(np.asarray(x, dtype=np.float64) * s, -fmax, fmax)
    return (round_fp8(xs, fmt) / s).astype(np.asarray(x).dtype)
