"""Pins of the oracle's storage formats.

bfloat16 is checked against torch's round-to-nearest-even cast (a library
routine) and the bit layout 1+8+7; e4m3fn decoding against torch's
float8_e4m3fn conversion for all 256 codes, and encoding against a brute-force
nearest search over every finite code with ties to the even mantissa (NumKong
for Python page, "Scalar Types" and "Buffer-First Casting").
"""

import numpy as np
import torch

from oracle import formats


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        rng.standard_normal(1000)]).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(formats.bf16_round(x), want)


def test_bf16_ties_subnormals_overflow():
    r = formats.bf16_round
    assert r(1.0 + 2.0 ** -8) == 1.0                        # tie -> even mantissa
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6        # tie -> even (up)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7  # above the tie
    assert r(2.0 ** -133) == 2.0 ** -133                    # smallest subnormal
    assert r(1.4 * 2.0 ** -134) == 2.0 ** -133              # rounds up to it
    assert r(0.5 * 2.0 ** -133) == 0.0                      # tie with zero -> 0
    assert r(formats.BF16_MAX) == formats.BF16_MAX
    assert np.isinf(r(2.0 ** 128))
    assert np.isinf(r(formats.BF16_MAX + 2.0 ** 119))       # at the overflow tie
    assert r(-3.0) == -3.0 and np.signbit(r(-0.0))
    assert np.isnan(r(np.nan))


def test_bf16_bits_roundtrip_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = formats.bf16_value(bits)
    torch_vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(torch_vals)
    np.testing.assert_array_equal(vals[finite], torch_vals[finite])
    np.testing.assert_array_equal(np.isnan(vals), np.isnan(torch_vals))
    ok = ~np.isnan(vals)
    np.testing.assert_array_equal(formats.bf16_bits(vals[ok]), bits[ok])


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    vals = formats.e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(vals), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(vals[ok], ref[ok])
    # format facts: max 448, smallest normal 2**-6, smallest subnormal 2**-9, NaN S.1111.111
    assert vals[0x7E] == 448.0 and vals[0x08] == 2.0 ** -6 and vals[0x01] == 2.0 ** -9
    assert vals[0x38] == 1.0 and np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert np.sum(np.isnan(vals)) == 2 and not np.any(np.isinf(vals))


def _brute_e4m3(x):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = formats.e4m3_value(codes)
    out = np.empty(len(x), dtype=np.uint8)
    for i, xi in enumerate(x):
        t = min(max(xi, -448.0), 448.0)                  # saturating
        d = np.abs(vals - t)
        best = np.nonzero(d == d.min())[0]
        cand = codes[best]
        # ties: the even mantissa; among +-0 keep the input's sign
        even = [c for c in cand if (c & 1) == 0] or list(cand)
        if len(even) > 1:
            even = [c for c in even if bool(c & 0x80) == bool(np.signbit(xi))]
        out[i] = even[0]
    return out


def test_e4m3_encode_is_nearest_code_ties_even():
    codes = np.arange(256, dtype=np.uint8)
    vals = np.sort(formats.e4m3_value(codes)[~np.isnan(formats.e4m3_value(codes))])
    vals = np.unique(vals)
    mids = (vals[:-1] + vals[1:]) / 2.0                    # exact ties
    rng = np.random.default_rng(1)
    x = np.concatenate([mids, vals, rng.uniform(-470, 470, 3000),
                        rng.standard_normal(3000) * 2.0 ** rng.integers(-12, 4, 3000),
                        [0.0, -0.0, 447.9, 460.0, 463.9, 464.0, 500.0, -1e6, 2.0 ** -10, 3 * 2.0 ** -11]])
    np.testing.assert_array_equal(formats.e4m3_code(x), _brute_e4m3(x))


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(50000) * 100).clip(-448, 448).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(formats.e4m3_code(x), ref)


def test_fp8_quantize_rows():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128))
    codes, scale = formats.fp8_quantize(x)
    assert np.all(scale == np.abs(x).max(axis=1).astype(np.float32).astype(np.float64) / 448.0
                  ) or np.all(np.abs(scale * 448.0 / np.abs(x).max(axis=1) - 1) < 2.0 ** -23)
    # the absmax element lands on +-448 exactly
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(formats.e4m3_value(codes[np.arange(64), am])) == 448.0)
    # dequantised error within half a code step (relative 2**-4) plus subnormal spacing
    deq = formats.e4m3_value(codes) * scale[:, None]
    assert np.all(np.abs(deq - x) <= np.abs(x) * 2.0 ** -4 + scale[:, None] * 2.0 ** -10)
    z, zs = formats.fp8_quantize(np.zeros((2, 8)))
    assert np.all(z == 0) and np.all(zs == 0)
