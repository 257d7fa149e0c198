"""Pins of the oracle's number formats against things that are not the oracle.

bf16 rounding and e4m3 coding are checked against torch's CPU casts (library
routines), exhaustively where the domain is small; e4m3 decode against the
format's closed-form table; the f32 quotient of the static quant against a
float64 division rounded once.
"""
import numpy as np
import pytest
import torch

from oracle import bf16_from_f64, bf16_to_f64, e4m3_decode, e4m3_encode, quantize_static


def _torch_bf16_bits(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _torch_e4m3(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_bf16_round_matches_torch_on_random_f32_patterns():
    r = np.random.default_rng(7)
    bits = r.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    # ties: f32 values exactly halfway between two bf16 values, both parities
    ties = ((r.integers(0, 2**16, 20000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[~np.isnan(ties)]
    for arr in (f, ties):
        got = bf16_from_f64(arr.astype(np.float64))
        want = _torch_bf16_bits(arr)
        assert got.size == arr.size and np.array_equal(got, want)


def test_bf16_round_trip_all_patterns():
    v = bf16_to_f64(ALL_BF16)
    fin = ~np.isnan(v)
    assert fin.sum() == 65536 - 2 * 127
    assert np.array_equal(bf16_from_f64(v[fin]), ALL_BF16[fin])


def test_e4m3_decode_table():
    c = np.arange(256, dtype=np.uint8)
    v = e4m3_decode(c)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2
    # closed-form anchors of OCP E4M3FN
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x38] == 1.0 and v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    # against torch's decode of every finite code
    fin = ~np.isnan(v)
    tv = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(v[fin], tv[fin])


def test_e4m3_round_trip_all_finite_codes():
    c = np.arange(256, dtype=np.uint8)
    fin = (c & 0x7F) != 0x7F
    assert fin.sum() == 254
    back = e4m3_encode(e4m3_decode(c[fin]).astype(np.float32))
    assert np.array_equal(back, c[fin])


def test_e4m3_monotone():
    x = np.sort(np.random.default_rng(3).uniform(-600, 600, 200000)).astype(np.float32)
    v = e4m3_decode(e4m3_encode(x))
    assert np.all(np.diff(v) >= 0)


@pytest.mark.parametrize("scale", [1.0, np.float32(4.0 / 448.0), 0.37, 3.0e-3, 17.25])
def test_e4m3_exhaustive_vs_torch_over_bf16_inputs(scale):
    x = bf16_to_f64(ALL_BF16).astype(np.float32)
    q = (x / np.float32(scale)).astype(np.float32)
    ok = ~np.isnan(q)
    got = e4m3_encode(q[ok])
    want = _torch_e4m3(q[ok])
    assert got.size == int(ok.sum()) and np.array_equal(got, want)


def test_e4m3_reading_points():
    cases = {1.0625: 0x38, 1.1875: 0x3A, 432.0: 0x7E, 2.0 ** -10: 0x00, -2.0 ** -10: 0x80,
             -0.0: 0x80, 465.0: 0x7E, -1e30: 0xFE, np.inf: 0x7E, -np.inf: 0xFE,
             3 * 2.0 ** -10: 0x02, 2.0 ** -6 - 2.0 ** -10: 0x08}
    for v, c in cases.items():
        assert int(e4m3_encode(np.float32(v))) == c, v
    assert int(e4m3_encode(np.float32(np.nan))) == 0x7F
    assert int(e4m3_encode(-np.float32(np.nan))) == 0xFF


def test_quantize_static_uses_correctly_rounded_f32_quotient():
    s = np.float32(4.0 / 448.0)
    assert s.view(np.uint32) == 0x3C124925
    x = bf16_to_f64(ALL_BF16)
    ok = np.isfinite(x)
    # a float64 quotient of two float32 values rounded once to float32 is the
    # correctly rounded float32 quotient
    q64 = (x[ok] / np.float64(s)).astype(np.float32)
    want = e4m3_encode(q64)
    got = quantize_static(ALL_BF16[ok], np.array([s]))
    assert np.array_equal(got, want)
    # the reciprocal of s is 111.99999 in float32, so a hard-coded 112 would be wrong
    assert np.float32(1.0) / s != np.float32(112.0)
