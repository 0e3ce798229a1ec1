"""Pins of the oracle's number formats (CPU only).

E4M3 decode and encode are checked exhaustively against the format's field
definition, against an exact rational rounding written from the IEEE rule
(tests/exact.py), and against PyTorch's CPU float8_e4m3fn cast.  BF16 is
checked against the exact rounding and PyTorch's bfloat16 cast.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs
from tests import exact


def test_e4m3_decode_landmarks():
    d = codecs.e4m3_decode
    assert d(0x00) == 0.0 and not np.signbit(d(0x00))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    assert d(0x01) == 2.0 ** -9            # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert d(0x08) == 2.0 ** -6            # smallest normal
    assert d(0x38) == 1.0
    assert d(0x7E) == 448.0                # largest finite, the 448 of amax/448
    assert d(0xFE) == -448.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert np.isfinite(codecs.E4M3_TABLE).sum() == 254


def test_e4m3_decode_is_monotone_and_symmetric():
    pos = codecs.E4M3_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(codecs.E4M3_TABLE[0x80:0xFF], -pos)


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.e4m3_decode(np.arange(256))
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(ours), fin)
    assert np.array_equal(ours[fin], ref[fin])


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(codecs.e4m3_encode_rne(codecs.e4m3_decode(codes)), codes)


def _midpoints():
    v = codecs.E4M3_TABLE[:0x7F]
    return v[:-1], v[1:], (v[:-1] + v[1:]) / 2


def test_e4m3_midpoints_round_to_even_code():
    lo, hi, mid = _midpoints()
    got = codecs.e4m3_encode_rne(mid)
    lo_c = codecs.e4m3_encode_rne(lo)
    hi_c = codecs.e4m3_encode_rne(hi)
    want = np.where(lo_c % 2 == 0, lo_c, hi_c)
    assert np.array_equal(got, want)
    # and just off the midpoint it goes to the nearer neighbour
    eps = np.spacing(mid)
    assert np.array_equal(codecs.e4m3_encode_rne(mid - 4 * eps), lo_c)
    assert np.array_equal(codecs.e4m3_encode_rne(mid + 4 * eps), hi_c)
    assert np.array_equal(codecs.e4m3_encode_rne(-mid), want | 0x80)


def test_e4m3_saturation_nan_and_signed_zero():
    enc = codecs.e4m3_encode_rne
    assert list(enc([448.0, 449.0, 463.9, 464.0, 1e6, np.inf])) == [0x7E] * 6
    assert list(enc([-449.0, -1e6])) == [0xFE, 0xFE]
    assert enc(np.nan) == 0x7F
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(2.0 ** -11) == 0x00          # below half the smallest subnormal
    assert enc(-(2.0 ** -11)) == 0x80


def test_e4m3_encode_matches_exact_rational_rounding():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.uniform(-470, 470, 3000),
        rng.standard_normal(3000) * 2.0 ** rng.integers(-12, 9, 3000),
        _midpoints()[2], -_midpoints()[2],
    ])
    got = codecs.e4m3_encode_rne(vals)
    for v, c in zip(vals, got):
        r = exact.to_e4m3_value(Fraction(float(v)))
        assert c == exact.e4m3_code_of_value(r, negative_zero=v < 0), (v, c)


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(2)
    _, _, mid = _midpoints()
    eps = np.spacing(mid)
    vals = np.concatenate([
        mid, mid - eps, mid + eps, -mid,
        mid * (1 - 2.0 ** -23), mid * (1 + 2.0 ** -23),
        rng.uniform(-464, 464, 1_000_000),
        rng.standard_normal(200_000) * 2.0 ** -8,
    ])
    # PyTorch casts float64 to FP8 through float32, so compare on values that
    # float32 holds exactly (no double rounding on either side).
    vals = vals.astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codecs.e4m3_encode_rne(vals.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_matches_exact_rounding_and_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # halfway cases: low 16 bits exactly 0x8000, with both parities of bit 16
    half = ((rng.integers(0, 2 ** 16, 2000, dtype=np.uint64) << 16) | 0x8000).astype(np.uint32)
    hx = half.view(np.float32)
    x = np.concatenate([x, hx[np.isfinite(hx)], np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8])])
    got = codecs.bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    for v in x[:300]:
        r = exact.to_bf16_value(Fraction(float(v)))
        back = codecs.bf16_to_f32(codecs.bf16_rne(np.float32(v)))
        if isinstance(r, float):               # overflow to infinity
            assert np.isinf(back)
        else:
            assert Fraction(float(back)) == r
    assert codecs.bf16_rne(np.float32(1 + 2 ** -8)) == 0x3F80      # tie -> even
    assert codecs.bf16_rne(np.float32(1 + 3 * 2 ** -8)) == 0x3F82  # tie -> even


def test_bf16_to_f32_is_exact_embedding():
    b = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    f = codecs.bf16_to_f32(b)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(f[fin], ref[fin])


@pytest.mark.parametrize("v", [0.1, 1 / 3, 447.9, 1e-3, 2.0 ** -10 * 3])
def test_f32_rounding_is_ieee(v):
    assert Fraction(float(codecs.f32(v))) == exact.to_f32_value(Fraction(v))
