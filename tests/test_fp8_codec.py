"""Pins for the oracle's OCP fp8 codecs: exhaustive and brute force."""
import numpy as np
import pytest

from oracle import fp8_codec as F


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_every_finite_code_round_trips(fmt):
    codes = np.arange(256, dtype=np.uint8)
    vals = F.decode(codes, fmt)
    fin = np.isfinite(vals)
    back = F.encode(vals[fin], fmt)
    np.testing.assert_array_equal(back, codes[fin])


def test_format_constants():
    assert F.decode(np.array([0x7E]), "e4m3")[0] == 448.0
    assert np.isnan(F.decode(np.array([0x7F]), "e4m3")[0])
    assert F.decode(np.array([0x01]), "e4m3")[0] == 2.0 ** -9
    assert F.decode(np.array([0x7B]), "e5m2")[0] == 57344.0
    assert np.isinf(F.decode(np.array([0x7C]), "e5m2")[0])
    assert F.decode(np.array([0x01]), "e5m2")[0] == 2.0 ** -16
    assert F.decode(np.array([0x38]), "e4m3")[0] == 1.0
    assert F.decode(np.array([0x3C]), "e5m2")[0] == 1.0


def brute_encode(x, fmt):
    """Nearest of all finite codes (with x's sign), ties to even mantissa."""
    fmax = F.FORMATS[fmt]["fmax"]
    a = min(abs(x), fmax)
    best = None
    for c in range(128):
        v = F.decode(np.array([c]), fmt)[0]
        if not np.isfinite(v):
            continue
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    return best[1] | (0x80 if np.signbit(x) else 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_encode_equals_brute_force(fmt):
    rng = np.random.default_rng(7)
    fmax = F.FORMATS[fmt]["fmax"]
    x = np.concatenate([
        rng.standard_normal(300) * fmax / 8,
        rng.standard_normal(100) * 2.0 ** -8,
        np.array([fmax * 1.2, -fmax * 3, 0.0, -0.0]),
    ])
    # exact midpoints between neighbouring codes exercise the tie rule
    codes, vals = F.finite_table(fmt)
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids[::7], -mids[3::11]])
    got = F.encode(x, fmt)
    want = np.array([brute_encode(v, fmt) for v in x], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_quantize_tensor_scale():
    x = np.array([0.5, -2.0, 1.0])
    c, s = F.quantize_tensor(x, "e4m3")
    assert s == 448.0 / 2.0
    assert F.decode(c, "e4m3")[1] == -448.0
    c0, s0 = F.quantize_tensor(np.zeros(4), "e4m3")
    assert s0 == 1.0 and np.all(c0 == 0)
