"""Pins of the oracle's MXFP4 weight path against things other than itself.

The MXFP4 format (E2M1 codes, UE8M0 scales per 32 K elements) is the SM100
kernel's weight format ("MegaMoE SM90 Implementation Design (Final)" §2.1 and
§15.2).  The pins:

* E2M1: the defining properties of the format (largest magnitude 6, smallest
  positive 0.5, eight sign-symmetric magnitudes, strictly increasing codes, at
  most two significant bits), and every value is an E4M3 value.
* UE8M0: PyTorch's own ``float8_e8m0fnu`` decode, all 256 codes.
* The MX GEMMs reduce exactly to the pinned FP8 GEMMs when the scaled weight
  values are E4M3 values (block exponents 2^-3 .. 2^3) and the FP8 weight
  scales are 1: same sums, same result bits.
* The whole layer with MXFP4 weights equals the FP8 layer on the equivalent
  FP8 weights, bit for bit.
* Exactness of the block dots with widely spread block exponents: exact
  rational brute force.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from fp8_mixture_experts_amd import synthetic as S
from oracle import codecs as C
from oracle import moe


def test_e2m1_format_properties():
    v = C.E2M1_TABLE
    assert v.shape == (16,)
    pos = v[:8]
    assert pos[0] == 0 and not np.signbit(pos[0])
    assert np.all(np.diff(pos) > 0)                     # codes ordered by magnitude
    assert pos.max() == 6.0 and pos[1] == 0.5           # largest / smallest positive
    assert np.array_equal(v[8:], -pos) and np.all(np.signbit(v[8:]))
    for x in pos[1:]:                                   # at most two significant bits
        m, _ = np.frexp(x)                              # x = m * 2^e, m in [0.5, 1)
        assert (m * 4) == int(m * 4)
    # every E2M1 value is an E4M3 value (so it converts exactly to E4M3 / F16)
    assert set(v.tolist()) <= set(C.E4M3_TABLE[np.isfinite(C.E4M3_TABLE)].tolist())


def test_unpack_low_nibble_first():
    p = np.array([[0x21, 0xF7]], np.uint8)
    assert C.unpack_e2m1(p).tolist() == [[1, 2, 7, 15]]


def test_ue8m0_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    got = C.ue8m0_decode(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    # float32 has no 2^-127: torch gives it as the float32 subnormal, as does float64 rounded
    assert np.array_equal(got[:255].astype(np.float32), ref[:255])


def _e4m3_equivalent(packed, e8):
    """E4M3 codes of the decoded MXFP4 values (exact when representable)."""
    vals = C.mxfp4_decode(packed, e8)
    codes = C.e4m3_encode_rne(vals)
    assert np.array_equal(C.e4m3_decode(codes), vals)      # representable: exact
    return codes


def _rand_mx(rng, rows, K, lo=124, hi=130):
    packed = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    e8 = rng.integers(lo, hi + 1, (rows, K // 32), dtype=np.uint8)
    return packed, e8


def test_l1_mx_reduces_to_fp8():
    rng = np.random.default_rng(1)
    m, N, H = 5, 128, 384
    a = rng.integers(0, 256, (m, H), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x10
    a_sf = rng.uniform(0.5, 2, (m, H // 128)).astype(np.float32)
    packed, e8 = _rand_mx(rng, N, H)
    got = moe.l1_gemm_mx(a, a_sf, packed, e8)
    want = moe.l1_gemm(a, a_sf, _e4m3_equivalent(packed, e8), np.ones((N // 128, H // 128)))
    assert np.array_equal(got, want)


def test_l2_mx_reduces_to_fp8():
    rng = np.random.default_rng(2)
    m, H, I = 4, 128, 256
    a = rng.integers(0, 256, (m, I), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x22
    s = rng.uniform(0.01, 1, (m, I // 64))
    packed, e8 = _rand_mx(rng, H, I)
    got = moe.l2_gemm_mx(a, s, packed, e8)
    want = moe.l2_gemm(a, s, _e4m3_equivalent(packed, e8), np.ones((1, I // 128)))
    assert np.array_equal(got, want)


def test_l1_mx_exact_with_spread_exponents():
    # block exponents 2^-12 .. 2^12 inside one 128-wide K block: still exact
    rng = np.random.default_rng(3)
    m, N, H = 2, 3, 128
    a = rng.integers(0, 256, (m, H), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x31
    a_sf = np.ones((m, 1), np.float32)
    packed, _ = _rand_mx(rng, N, H)
    e8 = np.array([[115, 139, 127, 120]] * N, np.uint8)
    got = moe.l1_gemm_mx(a, a_sf, packed, e8)
    codes = C.unpack_e2m1(packed)

    def frac_e4m3(c):
        s, e, mm = c >> 7, (c >> 3) & 15, c & 7
        v = Fraction(mm, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(mm, 8)) * Fraction(2) ** (e - 7)
        return -v if s else v

    def frac_e2m1(c):
        s, e, mm = c >> 3, (c >> 1) & 3, c & 1
        v = Fraction(mm, 2) if e == 0 else (1 + Fraction(mm, 2)) * Fraction(2) ** (e - 1)
        return -v if s else v

    for r in range(m):
        for n in range(N):
            tot = sum(frac_e4m3(int(a[r, c])) * frac_e2m1(int(codes[n, c])) *
                      Fraction(2) ** (int(e8[n, c // 32]) - 127) for c in range(H))
            assert got[r, n] == float(tot) and Fraction(got[r, n]) == tot


@pytest.mark.parametrize("fmt_pair", [("tiny_mxfp4", "tiny")])
def test_layer_mx_equals_fp8_on_equivalent_weights(fmt_pair):
    mx_name, _ = fmt_pair
    inp = S.make_inputs(mx_name)
    E = inp["w1_fp4"].shape[0]
    # re-encode the MXFP4 weights' values as FP8 codes with unit block scales;
    # the generated block exponents are within 2^-9 .. 2^-5, so rescale each
    # expert's values by a power of two into E4M3's range and undo it in the
    # FP8 weight scales (exact)
    w1 = C.mxfp4_decode(inp["w1_fp4"], inp["w1_e8"])
    w2 = C.mxfp4_decode(inp["w2_fp4"], inp["w2_e8"])
    sh = 8.0
    fp8 = dict(inp)
    for key in ("w1_fp4", "w1_e8", "w2_fp4", "w2_e8"):
        del fp8[key]
    fp8["w1"] = C.e4m3_encode_rne(w1 * 2.0 ** sh)
    fp8["w2"] = C.e4m3_encode_rne(w2 * 2.0 ** sh)
    assert np.array_equal(C.e4m3_decode(fp8["w1"]), w1 * 2.0 ** sh)
    assert np.array_equal(C.e4m3_decode(fp8["w2"]), w2 * 2.0 ** sh)
    N, H = w1.shape[1:]
    I = w2.shape[2]
    fp8["w1_sf"] = np.full((E, N // 128, H // 128), 2.0 ** -sh, np.float32)
    fp8["w2_sf"] = np.full((E, H // 128, I // 128), 2.0 ** -sh, np.float32)
    a = moe.forward(inp)
    b = moe.forward(fp8)
    for key in ("l2_acts", "l2_acts_sf", "comb", "y"):
        assert np.array_equal(a[key], b[key]), key


def test_generator_mxfp4_round_trip():
    # the input generator's E2M1 rounding: every decoded weight is the nearest
    # E2M1 multiple of its block scale (ties to even), saturating at 6
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((8, 64)) * 0.02).astype(np.float32)
    w[0, :4] = [0.0, -0.0, 1e-3, -1e-3]
    packed, e8 = S._quantize_mxfp4(w)
    dec = C.mxfp4_decode(packed, e8)
    scale = np.repeat(C.ue8m0_decode(e8), 32, axis=1)
    q = w.astype(np.float64) / scale
    grid = np.concatenate([-C.E2M1_TABLE[:8][::-1], C.E2M1_TABLE[:8]])
    best = np.abs(q[..., None] - grid).min(axis=-1)
    err = np.abs(dec / scale - np.clip(q, -6, 6))
    assert np.all(err <= best + 1e-12)
    amax = np.abs(w.reshape(8, 2, 32)).max(-1)
    assert np.all(np.abs(dec).reshape(8, 2, 32).max(-1) <= 6 * C.ue8m0_decode(e8))
    assert np.all(amax < 8 * C.ue8m0_decode(e8))       # X = floor(log2 amax) - 2
