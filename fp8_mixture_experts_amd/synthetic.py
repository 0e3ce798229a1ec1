"""Seeded synthetic inputs for the expert layer (shared by tests and bench).

This module builds inputs only.  It holds none of the layer's arithmetic:
inputs are quantised to FP8 E4M3 with PyTorch's own CPU cast
(``torch.float8_e4m3fn``), never with the oracle's encoder or a GPU kernel.

Workloads (names are what they are; sizes as stated):

=========  =====  =====  =====  ===  ==  =========================================
name       T      H      I      E    k   routing
=========  =====  =====  =====  ===  ==  =========================================
tiny       64     512    256    8    2   uniform
decode     128    7168   2048   32   8   uniform
mid        576    7168   2048   32   8   Zipf(0.8) over a random expert order
prefill    8192   7168   2048   32   8   Zipf(1.2), 2 experts get no tokens,
                                         0.1% of x channels scaled by 50
wide       4096   4096   1536   64   2   uniform
=========  =====  =====  =====  ===  ==  =========================================

Recipe:
* x: float32 N(0,1) [T, H] (prefill: round(0.001*H) channels drawn without
  replacement are multiplied by 50), rounded to BF16, then quantised per token
  per 128 channels: sf = float32(amax / 448), codes = e4m3(x / sf).
* W1 [E, 2I, H] (stored gate/up interleaved) and W2 [E, H, I]: float32
  N(0, 0.02^2), quantised per 128x128 block of the stored tensor by the same
  rule.  decode, mid and prefill share one weight set.
* MXFP4 workloads (``*_mxfp4``) quantise the same float32 weights per row and
  32 K elements instead: shared exponent X = floor(log2(amax)) - 2 (the OCP
  MX rule for E2M1, whose largest exponent is 2), codes = E2M1 of w / 2^X
  rounded to nearest, ties to even, saturating at 6, two codes per byte (the
  first in the low nibble), scale byte X + 127.  PyTorch has no CPU cast to
  FP4, so that rounding is written out below; it builds inputs only.
* Routing: per token, k distinct experts by Gumbel-top-k on log expert weights
  (successive sampling without replacement).  Uniform: equal weights.  Zipf(s):
  a seeded permutation pi of the active experts, expert pi(r) weighted
  (r+1)^-s; experts with weight 0 are never drawn.  topk_idx keeps draw order.
* topk_weights: softmax (float64) of k float32 N(0,1) logits, stored float32.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    hidden: int
    intermediate: int
    experts: int
    topk: int
    routing: str = "uniform"          # "uniform" | "zipf"
    zipf_s: float = 0.0
    zero_experts: int = 0
    outlier_frac: float = 0.0
    outlier_scale: float = 50.0
    seed: int = 0                     # x / routing / logits streams
    weight_seed: int = 0              # weight stream (shared between workloads)
    weight_std: float = 0.02
    weight_format: str = "fp8"        # "fp8" | "mxfp4"


WORKLOADS = {
    "tiny": Workload("tiny", 64, 512, 256, 8, 2, seed=20261202, weight_seed=20261000),
    "decode": Workload("decode", 128, 7168, 2048, 32, 8, seed=20261203, weight_seed=20261100),
    "mid": Workload("mid", 576, 7168, 2048, 32, 8, routing="zipf", zipf_s=0.8,
                    seed=20261204, weight_seed=20261100),
    "prefill": Workload("prefill", 8192, 7168, 2048, 32, 8, routing="zipf", zipf_s=1.2,
                        zero_experts=2, outlier_frac=0.001, seed=20261205,
                        weight_seed=20261100),
    "wide": Workload("wide", 4096, 4096, 1536, 64, 2, seed=20261206, weight_seed=20261300),
}
for _n in ("tiny", "decode", "mid", "prefill"):
    WORKLOADS[_n + "_mxfp4"] = dataclasses.replace(WORKLOADS[_n], name=_n + "_mxfp4",
                                                   weight_format="mxfp4")


def custom(name="custom", **kw) -> Workload:
    """A small workload of any shape, for tests."""
    base = dict(tokens=16, hidden=256, intermediate=128, experts=4, topk=2,
                seed=7, weight_seed=8)
    base.update(kw)
    return Workload(name, **base)


# ---------------------------------------------------------------------------

def _quantize_blocks(v: torch.Tensor, rows: int, cols: int):
    """float32 [..., R, C] -> (uint8 codes, float32 scales [..., R/rows, C/cols])."""
    *lead, R, C = v.shape
    b = v.reshape(*lead, R // rows, rows, C // cols, cols)
    amax = b.abs().amax(dim=(-3, -1), keepdim=True)
    sf = amax / FP8_MAX
    q = torch.where(sf > 0, b / torch.where(sf > 0, sf, torch.ones_like(sf)),
                    torch.zeros_like(b))
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, R, C)
    return codes.numpy(), sf.reshape(*lead, R // rows, C // cols).numpy().astype(np.float32)


# E2M1 magnitudes by code 0..7 and the midpoints between neighbours
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MID = (_E2M1_MAG[1:] + _E2M1_MAG[:-1]) / 2


def _quantize_mxfp4(v: np.ndarray):
    """float32 [R, C] -> (E2M1 pairs uint8 [R, C/2], UE8M0 uint8 [R, C/32])."""
    R, C = v.shape
    b = v.astype(np.float64).reshape(R, C // 32, 32)
    amax = np.abs(b).max(axis=-1)
    with np.errstate(divide="ignore"):
        x = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    x = np.clip(x, -127, 127).astype(np.int64)
    q = b / np.ldexp(1.0, x)[..., None]
    a = np.abs(q)
    lo = np.searchsorted(_E2M1_MID, a, side="left")
    tie = (lo < len(_E2M1_MID)) & (a == _E2M1_MID[np.minimum(lo, len(_E2M1_MID) - 1)])
    code = np.where(tie & (lo % 2 == 1), lo + 1, lo).astype(np.uint8)   # ties to even
    code |= np.where(np.signbit(q), 8, 0).astype(np.uint8)
    code = code.reshape(R, C)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, (x + 127).astype(np.uint8)


def _gen_normal(seed_seq, shape, std):
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _weights_one_expert(args):
    s1, s2, N, H, I, std, fmt = args
    w1 = _gen_normal(s1, (N, H), std)
    w2 = _gen_normal(s2, (H, I), std)
    if fmt == "mxfp4":
        return _quantize_mxfp4(w1) + _quantize_mxfp4(w2)
    c1, f1 = _quantize_blocks(torch.from_numpy(w1), 128, 128)
    c2, f2 = _quantize_blocks(torch.from_numpy(w2), 128, 128)
    return c1, f1, c2, f2


_WEIGHT_CACHE: dict = {}


def make_weights(wl: Workload, threads: int | None = None):
    """Quantised expert weights of a workload (cached per process)."""
    key = (wl.weight_seed, wl.experts, wl.hidden, wl.intermediate, wl.weight_std,
           wl.weight_format)
    if key in _WEIGHT_CACHE:
        return _WEIGHT_CACHE[key]
    E, H, I = wl.experts, wl.hidden, wl.intermediate
    N = 2 * I
    mx = wl.weight_format == "mxfp4"
    if not mx and wl.weight_format != "fp8":
        raise ValueError(wl.weight_format)
    kids = np.random.SeedSequence(wl.weight_seed).spawn(2 * E)
    if mx:
        shapes = [(N, H // 2), (N, H // 32), (H, I // 2), (H, I // 32)]
        dtypes = [np.uint8] * 4
        names = ["w1_fp4", "w1_e8", "w2_fp4", "w2_e8"]
    else:
        shapes = [(N, H), (N // 128, H // 128), (H, I), (H // 128, I // 128)]
        dtypes = [np.uint8, np.float32, np.uint8, np.float32]
        names = ["w1", "w1_sf", "w2", "w2_sf"]
    arrs = [np.empty((E,) + sh, dt) for sh, dt in zip(shapes, dtypes)]
    jobs = [(kids[2 * e], kids[2 * e + 1], N, H, I, wl.weight_std, wl.weight_format)
            for e in range(E)]
    if threads is None:
        threads = min(16, max(1, len(_affinity())))
    with ThreadPoolExecutor(threads) as ex:
        for e, parts in enumerate(ex.map(_weights_one_expert, jobs)):
            for arr, part in zip(arrs, parts):
                arr[e] = part
    out = dict(zip(names, arrs))
    _WEIGHT_CACHE[key] = out
    return out


def _affinity():
    try:
        import os
        return os.sched_getaffinity(0)
    except Exception:  # pragma: no cover
        return {0}


def make_routing(wl: Workload, rng: np.random.Generator):
    E, T, k = wl.experts, wl.tokens, wl.topk
    weight = np.ones(E, np.float64)
    if wl.routing == "zipf":
        zero = rng.choice(E, wl.zero_experts, replace=False) if wl.zero_experts else np.array([], int)
        live = np.setdiff1d(np.arange(E), zero)
        order = rng.permutation(live)
        weight = np.zeros(E, np.float64)
        weight[order] = np.arange(1, len(order) + 1, dtype=np.float64) ** (-wl.zipf_s)
    elif wl.routing != "uniform":
        raise ValueError(wl.routing)
    with np.errstate(divide="ignore"):
        logw = np.log(weight)
    keys = logw[None, :] + rng.gumbel(size=(T, E))
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return idx.astype(np.int32)


def make_activations(wl: Workload, rng: np.random.Generator):
    T, H = wl.tokens, wl.hidden
    x = rng.standard_normal((T, H), dtype=np.float32)
    if wl.outlier_frac > 0:
        n = int(round(wl.outlier_frac * H))
        ch = rng.choice(H, n, replace=False)
        x[:, ch] *= np.float32(wl.outlier_scale)
    xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32)
    codes, sf = _quantize_blocks(xb, 1, 128)
    return codes, sf


def make_inputs(wl: Workload | str, tokens: int | None = None):
    """All inputs of one forward call as numpy arrays (host memory)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if tokens is not None:
        wl = dataclasses.replace(wl, tokens=tokens)
    sx, sr, sl = np.random.SeedSequence(wl.seed).spawn(3)
    x, x_sf = make_activations(wl, np.random.Generator(np.random.PCG64(sx)))
    topk_idx = make_routing(wl, np.random.Generator(np.random.PCG64(sr)))
    logits = np.random.Generator(np.random.PCG64(sl)).standard_normal(
        (wl.tokens, wl.topk), dtype=np.float32).astype(np.float64)
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    topk_weights = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    inp = dict(x=x, x_sf=x_sf, topk_idx=topk_idx, topk_weights=topk_weights)
    inp.update(make_weights(wl))
    inp["workload"] = wl
    return inp
