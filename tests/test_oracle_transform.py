"""Pins of the oracle's W1 transform (oracle/transform.py).

The interleave is checked against the page's own statement of it as block
copies ("SM90 design" §15.1); the scale handling against what rounding at a
ratio must give: a pure permutation when both source scales are equal, exact
halving at ratio 1/2 above the subnormals, and at most half an E4M3 step of
error otherwise.
"""

import numpy as np

from oracle import codecs, transform


def _blocks_as_listed(w):
    """The page's loop: for i in steps of 8, stored rows 2i..2i+8 <- gate
    rows i..i+8 and 2i+8..2i+16 <- up rows N/2+i..N/2+i+8."""
    E, N, H = w.shape
    half = N // 2
    out = np.empty_like(w)
    for i in range(0, half, 8):
        out[:, 2 * i:2 * i + 8] = w[:, i:i + 8]
        out[:, 2 * i + 8:2 * i + 16] = w[:, half + i:half + i + 8]
    return out


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, 0x3C, c).astype(np.uint8)     # no NaN


def test_interleave_matches_the_listed_block_copies():
    rng = np.random.default_rng(1)
    w = _codes(rng, (2, 512, 256))
    sf = np.ones((2, 4, 2), np.float32)
    out, out_sf = transform.transform_w1(w, sf)
    assert np.array_equal(out, _blocks_as_listed(w))
    assert np.array_equal(out_sf, sf)


def test_equal_source_scales_move_codes_unchanged():
    rng = np.random.default_rng(2)
    E, I, H = 3, 256, 384
    w = rng.integers(0, 256, (E, 2 * I, H), dtype=np.uint8)    # NaN and -0 codes included
    s = rng.uniform(0.01, 2.0, (E, I // 128, H // 128)).astype(np.float32)
    sf = np.concatenate([s, s], axis=1)                         # gate block b == up block b
    out, out_sf = transform.transform_w1(w, sf)
    ref = _blocks_as_listed(w)
    nan = (ref & 0x7F) == 0x7F
    assert np.array_equal(out[~nan], ref[~nan])
    assert np.all(out[nan] == 0x7F)                            # NaN keeps its code, sign dropped
    nb = 2 * I // 128
    for n in range(nb):
        assert np.array_equal(out_sf[:, n], s[:, n // 2])


def test_ratio_one_half_halves_values_exactly():
    rng = np.random.default_rng(3)
    E, I, H = 1, 128, 128
    w = _codes(rng, (E, 2 * I, H))
    mag = np.abs(codecs.e4m3_decode(w))
    w = np.where(mag >= 2.0 ** -5, w, 0x38).astype(np.uint8)   # halving stays normal
    sf = np.array([[[0.5]], [[1.0]]], np.float32).reshape(1, 2, 1)   # gate 0.5, up 1.0
    out, out_sf = transform.transform_w1(w, sf)
    assert np.all(out_sf == 1.0)
    ref = _blocks_as_listed(w)
    before = codecs.e4m3_decode(ref) * np.where(_row_is_gate(2 * I), 0.5, 1.0)[None, :, None]
    after = codecs.e4m3_decode(out) * 1.0
    assert np.array_equal(after, before)


def _row_is_gate(n):
    return (np.arange(n) % 16) < 8


def test_rerounding_error_is_at_most_half_a_step():
    rng = np.random.default_rng(4)
    E, I, H = 2, 256, 256
    w = _codes(rng, (E, 2 * I, H))
    sf = rng.uniform(0.001, 1.0, (E, 2 * I // 128, H // 128)).astype(np.float32)
    out, out_sf = transform.transform_w1(w, sf)
    src = transform.interleave_rows(2 * I)
    blk = src // 128
    v_in = codecs.e4m3_decode(w[:, src, :]) * np.repeat(sf[:, blk, :], 128, axis=2)
    s_out = np.repeat(np.repeat(out_sf, 128, axis=1), 128, axis=2)
    v_out = codecs.e4m3_decode(out) * s_out
    # half a step: 2^-4 relative in the normal range, 2^-10 absolute (x s) below it
    bound = np.maximum(np.abs(v_in) * 2.0 ** -4, 2.0 ** -10 * s_out)
    assert np.all(np.abs(v_out - v_in) <= bound * (1 + 1e-12))
    # the rows whose source scale is the block's scale keep their codes
    same = np.repeat(sf[:, blk, :], 128, axis=2) == s_out
    assert np.array_equal(out[same], w[:, src, :][same])
    assert same.any() and (~same).any()


def test_zero_scale_blocks_give_zero_codes():
    rng = np.random.default_rng(5)
    w = _codes(rng, (1, 256, 128))
    sf = np.zeros((1, 2, 1), np.float32)
    out, out_sf = transform.transform_w1(w, sf)
    assert np.all(out == 0) and np.all(out_sf == 0)
