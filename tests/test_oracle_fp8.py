"""Pins of the oracle's FP8 map storage (OCP E4M3 codes with a per-row fp32
scale).  The values follow from the format's definition: the largest finite
value 448 = 1.75 * 2^8, the smallest normal 2^-6, the smallest subnormal
2^-9, 1.0 = S.0111.000; codes of one sign are ordered like their values."""
import numpy as np

from oracle import kvx_oracle as O


def test_e4m3_value_table():
    v = O.e4m3_values()
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x30] == 0.5
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254
    assert np.all(np.diff(v[:127]) > 0)                  # codes ordered like values
    assert np.array_equal(v[128:255], -v[:127])
    # every step is a power of two times 1/8 of the binade (2^-9 for the subnormals)
    steps = np.diff(v[:127])
    assert np.all(steps[:7] == 2.0 ** -9) and steps[-1] == 32.0


def test_e4m3_encode_round_trip_ties_and_saturation():
    v = O.e4m3_values()
    codes = np.array([c for c in range(256) if np.isfinite(v[c])])
    assert np.array_equal(O.e4m3_encode(v[codes]), codes.astype(np.uint8))
    lo, hi = v[:126], v[1:127]
    mid = (lo + hi) / 2
    got = O.e4m3_encode(mid)
    even = np.where(np.arange(126) % 2 == 0, np.arange(126), np.arange(1, 127))
    assert np.array_equal(got, even.astype(np.uint8))    # ties to the even code
    eps = (hi - lo) * 1e-6
    assert np.array_equal(O.e4m3_encode(mid - eps), np.arange(126, dtype=np.uint8))
    assert np.array_equal(O.e4m3_encode(mid + eps), np.arange(1, 127, dtype=np.uint8))
    assert list(O.e4m3_encode([449.0, 464.0, 500.0, 1e9, -1e9, -0.0])) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80]
    assert list(O.e4m3_encode([2.0 ** -10, 2.0 ** -10 * 1.01, 2.0 ** -11])) == [0x00, 0x01, 0x00]


def test_quantize_rows():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((6, 300)).astype(np.float32)
    w[1] = 0.0
    w[2, 17] = 1e4                                         # one outlier
    w[3] *= np.float32(1e-30)                              # tiny row
    q, s = O.quantize_fp8(w)
    assert s.dtype == np.float32 and s[1] == 1.0 and np.all(q[1] == 0)
    for r in (0, 2, 3, 4, 5):
        assert s[r] == np.float32(np.max(np.abs(w[r])) / np.float32(448.0))
        assert np.any((q[r] & 0x7F) == 0x7E)               # the row's largest magnitude maps to 448
    d = O.fp8_dequant(q, s)
    # nearest code: error at most half a step, a step being at most 2^-3 of the value's binade
    err = np.abs(d - w.astype(np.float64))
    bound = np.maximum(np.abs(w.astype(np.float64)) * 2.0 ** -4, s[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
