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


def _gen_normal(seed_seq, shape, std):
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _weights_one_expert(args):
    s1, s2, N, H, I, std = args
    w1 = torch.from_numpy(_gen_normal(s1, (N, H), std))
    w2 = torch.from_numpy(_gen_normal(s2, (H, I), std))
    c1, f1 = _quantize_blocks(w1, 128, 128)
    c2, f2 = _quantize_blocks(w2, 128, 128)
    return c1, f1, c2, f2


_WEIGHT_CACHE: dict = {}


def make_weights(wl: Workload, threads: int | None = None):
    """Quantised expert weights of a workload (cached per process)."""
    key = (wl.weight_seed, wl.experts, wl.hidden, wl.intermediate, wl.weight_std)
    if key in _WEIGHT_CACHE:
        return _WEIGHT_CACHE[key]
    E, H, I = wl.experts, wl.hidden, wl.intermediate
    N = 2 * I
    kids = np.random.SeedSequence(wl.weight_seed).spawn(2 * E)
    w1 = np.empty((E, N, H), np.uint8)
    w1_sf = np.empty((E, N // 128, H // 128), np.float32)
    w2 = np.empty((E, H, I), np.uint8)
    w2_sf = np.empty((E, H // 128, I // 128), np.float32)
    jobs = [(kids[2 * e], kids[2 * e + 1], N, H, I, wl.weight_std) for e in range(E)]
    if threads is None:
        threads = min(16, max(1, len(_affinity())))
    with ThreadPoolExecutor(threads) as ex:
        for e, (c1, f1, c2, f2) in enumerate(ex.map(_weights_one_expert, jobs)):
            w1[e], w1_sf[e], w2[e], w2_sf[e] = c1, f1, c2, f2
    out = dict(w1=w1, w1_sf=w1_sf, w2=w2, w2_sf=w2_sf)
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
