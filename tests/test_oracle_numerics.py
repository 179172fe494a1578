"""Pins of the oracle's storage codecs (CPU).

The E4M3 decode and encode are checked against (a) hand-derived values from
the OCP E4M3 layout (tests/golden/e4m3_*.txt), (b) torch's independent
``float8_e4m3fn`` conversion over every code and every bf16 input, and the bf16
rounding against torch's ``bfloat16`` conversion.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import numerics as nx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def test_e4m3_decode_golden_table():
    table = nx.e4m3_value_table()
    n = 0
    for code_s, val_s in _rows("e4m3_codes.txt"):
        code, val = int(code_s, 16), float(val_s)
        got = table[code]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val, (hex(code), got, val)
            assert math.copysign(1.0, got) == math.copysign(1.0, val), hex(code)
        n += 1
    assert n >= 25


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = nx.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]


def test_e4m3_decode_scale_applies_in_fp64():
    codes = np.array([0x38, 0x7E, 0x01], dtype=np.uint8)
    s = np.float32(0.3)
    got = nx.e4m3_decode(codes, float(s))
    assert np.array_equal(got, np.array([1.0, 448.0, 2.0**-9]) * np.float64(s))


def test_e4m3_encode_golden_edges():
    n = 0
    for row in _rows("e4m3_encode_edges.txt"):
        x, s, code = float(row[0]), float(row[1]), int(row[2], 16)
        got = int(nx.e4m3_encode(np.array([x], dtype=np.float32), s)[0])
        assert got == code, (row, hex(got))
        n += 1
    assert n >= 25


def _all_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    return bits.view(np.float32)


def test_e4m3_encode_exhaustive_bf16_vs_torch():
    x = _all_bf16_as_f32()
    got = nx.e4m3_encode(x, 1.0)
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    a = np.abs(x)
    in_range = np.isfinite(x) & (a < 464.0)  # torch does not saturate past the tie
    assert np.array_equal(got[in_range], ref[in_range])
    big = np.isfinite(x) & (a >= 464.0) | np.isinf(x)
    assert np.all(got[big & ~np.signbit(x)] == 0x7E)
    assert np.all(got[big & np.signbit(x)] == 0xFE)
    assert np.all(got[np.isnan(x)] == 0x7F)


def test_e4m3_encode_is_nearest_value():
    """Brute force: the code's value is a nearest representable to |y|."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(4000) * rng.choice([1e-3, 0.1, 10.0, 200.0], 4000)).astype(np.float32)
    codes = nx.e4m3_encode(x, 1.0)
    vals = nx.e4m3_decode(codes)
    finite = nx.e4m3_value_table()[:0x7F]
    for xi, vi in zip(x.astype(np.float64), vals):
        if abs(xi) >= 448:
            assert abs(vi) == 448
            continue
        best = np.min(np.abs(finite - abs(xi)))
        assert abs(abs(vi) - abs(xi)) == best
        assert (vi == 0) or (math.copysign(1, vi) == math.copysign(1, xi))


def test_e4m3_encode_divides_in_fp32_before_rounding():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(5000).astype(np.float32)
    s = np.float32(0.0123)
    y = (x / s).astype(np.float32)
    assert np.array_equal(nx.e4m3_encode(x, float(s)), nx.e4m3_encode(y, 1.0))
    # powers of two divide exactly
    assert np.array_equal(nx.e4m3_encode(x, 0.25), nx.e4m3_encode(x * np.float32(4.0), 1.0))


def test_bf16_decode_exact_and_round_trip():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(10000).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(nx.bf16_bits_to_f64(bits), ref)


def test_f32_to_bf16_matches_torch_rne():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40, -1e-40], np.float32),
        # exact ties: low 16 bits = 0x8000 with both parities of the kept part
        np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32).view(np.float32),
    ])
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nx.f32_to_bf16_bits(x), ref)
    nan = nx.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert (int(nan[0]) & 0x7F80) == 0x7F80 and (int(nan[0]) & 0x7F) != 0


def test_bf16_ties_go_to_even():
    # 1 + 2^-8 sits halfway between bf16 1.0 (0x3F80) and 1 + 2^-7 (0x3F81)
    x = np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8], dtype=np.float32)
    got = nx.f32_to_bf16_bits(x)
    assert list(got) == [0x3F80, 0x3F82]


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_encode_storage_identity_copies_bits(src):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(64).astype(np.float32)
    v = x if src == "f32" else nx.f32_to_bf16_bits(x)
    out = nx.encode_storage(v, src, src)
    assert out.dtype == v.dtype and np.array_equal(out.view(np.uint8), v.view(np.uint8))
