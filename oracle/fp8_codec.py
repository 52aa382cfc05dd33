"""OCP 8-bit float codecs (E4M3FN and E5M2) written from the format definitions.

TEST INFRASTRUCTURE ONLY (imported by tests; never by the GPU path).

The FP8 configuration quantises linear-layer operands per tensor: scale
s = fmax / amax (s = 1 when amax = 0), code = round-to-nearest-even of x*s
with saturation to +-fmax.  The pages only say "FP8 matrix products" (the
d24 speedrun on the "supa beginna nanochat" page and the alpha-nanochat-d24
model card); the format choice (OCP e4m3 forward, e5m2 gradients) and the
current per-tensor amax scaling are this project's reading.

E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
        S.1111.111 is NaN, largest finite 448, smallest subnormal 2**-9.
E5M2:   1 sign, 5 exponent bits (bias 15), 2 mantissa bits, IEEE-like
        (exponent 31 = inf/NaN), largest finite 57344, smallest subnormal 2**-16.
"""
from __future__ import annotations

import numpy as np

FORMATS = {
    "e4m3": dict(ebits=4, mbits=3, bias=7, fmax=448.0),
    "e5m2": dict(ebits=5, mbits=2, bias=15, fmax=57344.0),
}


def decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    """uint8 codes -> fp64 values (NaN for NaN codes, +-inf for e5m2 infs)."""
    f = FORMATS[fmt]
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> f["mbits"]) & ((1 << f["ebits"]) - 1)
    m = c & ((1 << f["mbits"]) - 1)
    scale_m = float(1 << f["mbits"])
    normal = (1.0 + m / scale_m) * np.exp2(e.astype(np.float64) - f["bias"])
    sub = (m / scale_m) * 2.0 ** (1 - f["bias"])
    v = np.where(e == 0, sub, normal)
    emax = (1 << f["ebits"]) - 1
    if fmt == "e4m3":
        v = np.where((e == emax) & (m == 7), np.nan, v)
    else:
        v = np.where((e == emax) & (m == 0), np.inf, v)
        v = np.where((e == emax) & (m != 0), np.nan, v)
    return sign * v


def finite_table(fmt: str):
    """All finite non-negative values with their codes, ascending by value."""
    codes = np.arange(0, 128, dtype=np.int64)
    vals = decode(codes, fmt)
    ok = np.isfinite(vals)
    return codes[ok], vals[ok]


def encode(x: np.ndarray, fmt: str) -> np.ndarray:
    """Values -> codes: saturate to +-fmax, then round to nearest, ties to the
    code with an even mantissa (RNE).  The sign of zero is kept."""
    f = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    codes, vals = finite_table(fmt)
    a = np.minimum(np.abs(x), f["fmax"])
    hi = np.searchsorted(vals, a, side="left")          # vals[hi] >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = np.abs(a - vals[lo])
    dhi = np.abs(vals[hi] - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((codes[hi] & 1) == 0))
    c = np.where(pick_hi, codes[hi], codes[lo])
    neg = np.signbit(x)
    return (c | np.where(neg, 0x80, 0)).astype(np.uint8)


SCALE_CAP = 2.0 ** 64


def quantize_tensor(x: np.ndarray, fmt: str, dtype=np.float64):
    """Current per-tensor scaling: returns (codes, scale) with x ~ decode/scale.

    scale = fmax / amax (1 when amax = 0, at most 2**64), and each code is the
    RNE-with-saturation encoding of x * scale.  ``dtype`` is the precision in
    which the scale and the products x * scale are rounded before encoding
    (float64 by default; float32 reproduces a quantiser that works in fp32,
    where the rounded product decides the code)."""
    x = np.asarray(x, dtype=dtype)
    amax = dtype(np.max(np.abs(x))) if x.size else dtype(0.0)
    fmax = dtype(FORMATS[fmt]["fmax"])
    scale = min(fmax / amax, dtype(SCALE_CAP)) if amax > 0 else dtype(1.0)
    scale = dtype(scale)
    y = (x * scale).astype(dtype)
    return encode(y.astype(np.float64), fmt), float(scale)
