"""Number formats of the layer, written out from their definitions (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The layer stores activations and weights as FP8 E4M3 with float32 scale
factors, and emits BF16 ("SM90 design" §1.1 decision 7, §5.3, §10.1 step 5,
§11.1).  The E4M3 variant is the OCP "fn" one that PyTorch quantises to, since
the design asks the scale-factor path to agree with PyTorch's standard FP8
quantisation (§1.1 decision 7): sign | 4 exponent bits (bias 7) | 3 mantissa
bits, no infinities, S.1111.111 is NaN, largest finite magnitude 448
(the divisor in ``sf = amax / 448`` of §10.1 step 5).
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def _e4m3_value(code: int) -> float:
    """Value of one E4M3 code by the format's definition."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (-6)          # subnormal: 0.mmm x 2^(1-7)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)  # normal: 1.mmm x 2^(e-7)
    return -mag if s else mag


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_rne(values) -> np.ndarray:
    """float64 values -> uint8 E4M3 codes, round to nearest, ties to even.

    Finite magnitudes above 448 saturate to 448 (everything in (448, 464]
    already rounds there; the layer never produces more than 448 times
    (1 + 2^-23), because every value is divided by amax/448 of its own group).
    NaN encodes as 0x7F.  The sign of zero is kept.
    """
    v = np.asarray(values, dtype=np.float64)
    nan = np.isnan(v)
    neg = np.signbit(v)
    a = np.where(nan, 0.0, np.abs(v))
    a = np.minimum(a, E4M3_MAX)
    # Spacing of representable values around a: 2^(e-3) inside binade
    # [2^e, 2^(e+1)) for e >= -6, and the subnormal spacing 2^-9 below 2^-6.
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    quantum = np.ldexp(1.0, e - 3)
    n = np.rint(a / quantum)                 # exact scaling; rint is half-to-even
    r = n * quantum                          # representable (may be 2^(e+1))
    # Representable value -> code.
    _, rex = np.frexp(r)
    re = rex - 1
    sub = r < 2.0 ** (-6)
    mant_sub = np.rint(r / 2.0 ** (-9)).astype(np.int64)
    re_c = np.maximum(re, -6)
    mant_norm = np.rint((r / np.ldexp(1.0, re_c) - 1.0) * 8.0).astype(np.int64)
    code = np.where(sub, mant_sub, ((re_c + 7) << 3) | mant_norm)
    code = np.where(neg, code | 0x80, code)
    code = np.where(nan, E4M3_NAN, code)
    return code.astype(np.uint8)


def bf16_rne(values_f32) -> np.ndarray:
    """float32 values -> uint16 BF16 bit patterns, round to nearest, ties to even.

    BF16 keeps the upper 16 bits of a float32.  Adding 0x7FFF plus the lowest
    kept bit to the 32-bit pattern and truncating rounds the discarded half:
    below half rounds down, above rounds up, exactly half rounds to the even
    kept pattern (a carry into the exponent is the correct next binade, and
    past the largest finite value it gives infinity).  NaN stays a quiet NaN.
    """
    x = np.asarray(values_f32, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, (((u >> 16) & 0x8000) | 0x7FC0).astype(np.uint16), r)
    return r


def bf16_to_f32(bits) -> np.ndarray:
    """uint16 BF16 bit patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32(x) -> np.ndarray:
    """Round float64 values to float32 (IEEE round to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------
# MXFP4 weights ("SM90 design" §2.1 and §15.2: the SM100 kernel's weights are
# FP4 E2M1 with UE8M0 scale factors, one per 32 K elements).  The formats are
# those of the OCP microscaling (MX) specification: E2M1 is sign | 2 exponent
# bits (bias 1) | 1 mantissa bit, no infinities or NaN, largest magnitude 6;
# UE8M0 is an unsigned 8-bit power-of-two exponent with bias 127, 0xFF = NaN.
# Two E2M1 codes share a byte, the first (even K) in the low nibble.
# --------------------------------------------------------------------------

MX_BLOCK = 32


def _e2m1_value(code: int) -> float:
    """Value of one E2M1 code by the format's definition."""
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = m * 0.5                           # subnormal: 0.m x 2^(1-1)
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)  # normal: 1.m x 2^(e-1)
    return -mag if s else mag


E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """4-bit E2M1 codes (one per array element) -> float64 values (exact)."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def unpack_e2m1(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes: element 2i from the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def ue8m0_decode(e) -> np.ndarray:
    """UE8M0 exponent bytes -> float64 2^(e - 127); 0xFF is NaN."""
    e = np.asarray(e, dtype=np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 0xFF, np.nan, v)


def mxfp4_decode(packed, scales) -> np.ndarray:
    """MXFP4 rows -> float64 values.

    ``packed`` [..., K/2] E2M1 pairs, ``scales`` [..., K/32] UE8M0.  Element c
    is e2m1(code c) * 2^(scales[c // 32] - 127), exact in float64 for every
    code and scale.
    """
    v = e2m1_decode(unpack_e2m1(packed))
    s = np.repeat(ue8m0_decode(scales), MX_BLOCK, axis=-1)
    return v * s
