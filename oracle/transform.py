"""Weight transform of the expert layer (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The layer takes W1 with its gate and up rows interleaved with granularity 8
("SM90 design" §15.1): stored row 16g + r is gate row 8g + r for r < 8 and up
row 8g + r - 8 for r >= 8.  Its scales are one float32 per 128x128 block of
the stored tensor (§15.2; reading: the blocks are blocks of the interleaved
tensor).  A model's W1 usually comes the plain way, all I gate rows then all I
up rows, each quantised per 128x128 block of that tensor.  Interleaving moves
64 gate rows of source block n // 2 and 64 up rows of source block
I/128 + n // 2 into stored block n, so the stored block needs one scale for
rows that had two: it takes the larger one, s' = max(s_gate, s_up), and the
rows whose source scale s is smaller are re-rounded:
code' = e4m3_rne(q(code) * (s / s')), the ratio and the product in float64.
A block whose two source scales are both 0 gets scale 0 and codes 0x00.
W2 and its scales need no transform (§15.1).
"""

import numpy as np

from .codecs import e4m3_decode, e4m3_encode_rne

BLOCK = 128
GRANULE = 8


def interleave_rows(two_i):
    """Source row (in the plain [gate; up] order) of every stored row."""
    i = two_i // 2
    r = np.arange(two_i)
    g, o = r // (2 * GRANULE), r % (2 * GRANULE)
    return np.where(o < GRANULE, GRANULE * g + o, i + GRANULE * g + o - GRANULE)


def transform_w1(w1, w1_sf):
    """Plain W1 [E, 2I, H] codes and scales [E, 2I/128, H/128] -> the
    interleaved layout with per-stored-block scales."""
    w1 = np.asarray(w1, np.uint8)
    sf = np.asarray(w1_sf, np.float32)
    E, N, H = w1.shape
    src = interleave_rows(N)
    src_blk = src // BLOCK                                  # source scale block of each stored row
    out = np.empty_like(w1)
    out_sf = np.empty_like(sf)
    nb = N // BLOCK
    for n in range(nb):
        rows = np.arange(n * BLOCK, (n + 1) * BLOCK)
        blocks = np.unique(src_blk[rows])
        s_new = sf[:, blocks, :].max(axis=1)                # [E, H/128]
        out_sf[:, n, :] = s_new
        for r in rows:
            s_src = sf[:, src_blk[r], :].astype(np.float64)     # [E, H/128]
            s_dst = s_new.astype(np.float64)
            with np.errstate(invalid="ignore", divide="ignore"):
                ratio = np.where(s_dst > 0, s_src / np.where(s_dst > 0, s_dst, 1.0), 0.0)
            ratio = np.repeat(ratio, BLOCK, axis=1)             # per column
            v = e4m3_decode(w1[:, src[r], :]) * ratio
            codes = e4m3_encode_rne(v)
            codes = np.where(np.repeat(s_dst, BLOCK, axis=1) > 0, codes, 0).astype(np.uint8)
            out[:, r, :] = codes
    return out, out_sf
