"""GPU parity at the full sizes of the benchmark workloads, in the launch
configuration the benchmark times (the default plan, no pool copy).

decode, mid and wide (and mid with MXFP4 weights) are compared in full: the
whole dispatch (counts, offsets, slot map, source rows) bit-exactly, the
re-quantised activations and their scales of every valid pool row, the BF16
partial of every active route and every row of y, against the oracle's full
forward.  The prefill batches (65,536 routes) are compared on the whole
dispatch and on every route of a set of at least 192 tokens chosen to land
in the first and last pool block of every XCD's range of pool blocks, in the
first and last (partly filled) pool block of every expert, at the cuts of
the N-major tile groups, plus seeded random tokens; the oracle computes those
tokens one by one.  With the pool kept (keep_pool = 1) the pool copies are
bit-exact and y is identical to the run without them.  The split phases (L1
and L2 tiles as two concurrent kernels) are compared with the oracle on the
full decode batch.
"""

import numpy as np
import pytest

from fp8_mixture_experts_amd import binding as B
from fp8_mixture_experts_amd import synthetic as S
from oracle import moe
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

FULL = ["decode", "mid", "wide", "mid_mxfp4"]
SAMPLED = ["prefill", "prefill_mxfp4"]

# MI355X: 8 XCDs; the expert kernel gives each a contiguous range of pool blocks
N_XCD = 8


def _check_dispatch(v, d, label):
    assert np.array_equal(v["counts"], d["counts"]), label
    assert np.array_equal(v["offsets"], d["offsets"]), label
    assert np.array_equal(v["slot_map"], d["slot_map"]), label
    assert np.array_equal(v["src"], d["src"]), label


def _compare_full(inp, ref, run, label):
    T = inp["x"].shape[0]
    v = run.views(T)
    _check_dispatch(v, ref, label)
    valid = ref["src"] >= 0
    same = G.check_codes(v["l2_acts"][valid], ref["l2_acts"][valid], label)
    G.check_sf(v["l2_sf"][:, valid], ref["l2_acts_sf"][:, valid], label)
    act = ref["active"].reshape(-1)
    perr = G.rel_frobenius(v["comb"][act], ref["comb"][act])
    assert perr <= 2e-3, f"{label}: partials rel frobenius {perr:.3g}"
    yerr = G.check_y(run.y(), ref["y"], label)
    print(f"[{label}] {int(valid.sum())} routes: codes identical {same:.6f}, "
          f"partials {perr:.2e}, y {yerr:.2e}", flush=True)


@pytest.mark.parametrize("name", FULL)
def test_full_size_all_routes(name):
    inp = S.make_inputs(name)
    T, H = inp["x"].shape
    E, _, _, k = G.layer_dims(inp)
    print(f"[{name}] T={T} H={H} E={E} k={k}: oracle forward", flush=True)
    ref = moe.forward(inp)
    run = G.Runner(inp)
    try:
        print(f"[{name}] GPU forward", flush=True)
        assert run.forward() == 0
        _compare_full(inp, ref, run, name)
    finally:
        run.close()


def test_split_phases_full_decode_match_oracle():
    inp = S.make_inputs("decode")
    ref = moe.forward(inp)
    for kw in (dict(split_l2_cus=8), dict(split_l2_cus=16), dict(split_l2_xcds=3)):
        print(f"[decode {kw}] GPU forward", flush=True)
        run = G.Runner(inp, **kw)
        try:
            assert run.forward() == 0
            _compare_full(inp, ref, run, f"decode {kw}")
        finally:
            run.close()


def boundary_tokens(d, topk_idx, block_m, n_major, n_xcd, extra, seed):
    """Tokens whose routes land on the pool rows where the expert kernel's
    tiles change hands: the first and last valid row of the first and last
    pool block of every XCD range, the first row of every expert and its last
    (in a partly filled pool block), the first row of every N-major tile
    group, plus `extra` seeded random tokens."""
    counts, offsets, src = d["counts"], d["offsets"], d["src"]
    k = topk_idx.shape[1]
    E = counts.shape[0]
    blocks = []                      # (expert, first row, valid rows) per pool block
    for e in range(E):
        for m in range((int(counts[e]) + block_m - 1) // block_m):
            r0 = int(offsets[e]) + m * block_m
            blocks.append((e, r0, min(block_m, int(counts[e]) - m * block_m)))
    M = len(blocks)
    chosen = set()

    def take(pb, first=True, last=True):
        _, r0, n = blocks[pb]
        for r, want in ((r0, first), (r0 + n - 1, last)):
            if want:
                chosen.add(int(src[r]) // k)

    starts = {}
    for pb, (e, _, _) in enumerate(blocks):
        starts.setdefault(e, pb)
    for x in range(n_xcd):
        lo, hi = M * x // n_xcd, M * (x + 1) // n_xcd
        if hi > lo:
            take(lo)
            take(hi - 1)
            if n_major:
                G_ = 2 if block_m == 64 else 4
                for pb in range(lo, hi):
                    e = blocks[pb][0]
                    r0 = max(starts[e], lo)
                    if (pb - r0) % G_ == 0:
                        take(pb, last=False)
    for e, pb in starts.items():
        take(pb, last=False)
        take(pb + (int(counts[e]) + block_m - 1) // block_m - 1, first=False)
    rng = np.random.default_rng(seed)
    T = topk_idx.shape[0]
    pool = np.setdiff1d(np.arange(T), np.array(sorted(chosen)))
    chosen.update(rng.choice(pool, min(extra, pool.size), replace=False).tolist())
    return sorted(chosen)


@pytest.mark.parametrize("name", SAMPLED)
def test_prefill_boundary_tokens(name):
    inp = S.make_inputs(name)
    T, H = inp["x"].shape
    E, _, I, k = G.layer_dims(inp)
    run = G.Runner(inp)
    try:
        plan = B.mega_moe_plan(run.layer.cfg, T)
        print(f"[{name}] T={T} block_m {plan.block_m} n_major {plan.l2_n_major}: GPU forward",
              flush=True)
        assert run.forward() == 0
        v = run.views(T)
        d = moe.dispatch(inp["topk_idx"], E)
        _check_dispatch(v, d, name)
        toks = boundary_tokens(d, inp["topk_idx"], plan.block_m, plan.l2_n_major, N_XCD,
                               extra=32, seed=1234)
        assert len(toks) >= 192, len(toks)
        print(f"[{name}] oracle on {len(toks)} tokens", flush=True)
        ref = moe.forward_tokens(inp, toks)
        got_codes, want_codes, got_sf, want_sf, got_p, want_p = [], [], [], [], [], []
        for t in toks:
            for j, r in ref[t]["routes"].items():
                s = d["slot_map"][t, j]
                got_codes.append(v["l2_acts"][s])
                want_codes.append(r["l2_acts"])
                got_sf.append(v["l2_sf"][:, s])
                want_sf.append(r["l2_acts_sf"])
                got_p.append(v["comb"][t * k + j])
                want_p.append(r["part"])
        same = G.check_codes(np.array(got_codes), np.array(want_codes), name)
        G.check_sf(np.array(got_sf), np.array(want_sf), name)
        perr = G.rel_frobenius(np.array(got_p), np.array(want_p))
        assert perr <= 2e-3, f"{name}: partials rel frobenius {perr:.3g}"
        y = run.y()
        yerr = G.check_y(y[toks], np.array([ref[t]["y"] for t in toks]), name)
        print(f"[{name}] {len(got_codes)} routes of {len(toks)} tokens: codes identical "
              f"{same:.6f}, partials {perr:.2e}, y {yerr:.2e}", flush=True)
    finally:
        run.close()


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_pool_copy_full_size(name):
    """keep_pool = 1: the pool copies equal the routed rows bit for bit, and y
    is identical to the default run's."""
    inp = S.make_inputs(name)
    T = inp["x"].shape[0]
    E, _, _, k = G.layer_dims(inp)
    d = moe.dispatch(inp["topk_idx"], E)
    ys = []
    for keep in (0, 1):
        print(f"[{name}] keep_pool {keep}: GPU forward", flush=True)
        run = G.Runner(inp, keep_pool=keep)
        try:
            assert run.forward() == 0
            ys.append(run.y().copy())
            if keep:
                v = run.views(T)
                _check_dispatch(v, d, name)
                rows = np.nonzero(d["src"] >= 0)[0]
                tok = d["src"][rows] // k
                assert np.array_equal(v["l1_acts"][rows], inp["x"][tok])
                assert np.array_equal(v["l1_sf"][:, rows], inp["x_sf"][tok].T)
                assert np.array_equal(v["l1_w"][rows],
                                      inp["topk_weights"].reshape(-1)[d["src"][rows]])
        finally:
            run.close()
    assert np.array_equal(ys[0], ys[1])
