"""GPU parity at the full sizes of the benchmark workloads, in the launch
configuration the benchmark times (the default plan), with FP8 weights and,
for mid and prefill, MXFP4 weights.

At these sizes the whole dispatch (counts, offsets, slot map, source rows) and
the pool copies are checked bit-exactly against the oracle's dispatch, and a
sample of tokens (first, last and seeded random ones) is checked against the
oracle's per-token computation: their routes' re-quantised activations, scales
and BF16 partials, and their rows of y.
"""

import numpy as np
import pytest

from fp8_mixture_experts_amd import synthetic as S
from oracle import codecs, moe
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

WORKLOADS = ["decode", "mid", "wide", "prefill", "mid_mxfp4", "prefill_mxfp4"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_full_size_workload(name):
    inp = S.make_inputs(name)
    T, H = inp["x"].shape
    E, _, _, k = G.layer_dims(inp)
    print(f"[{name}] T={T} H={H} E={E} k={k}", flush=True)
    run = G.Runner(inp, keep_pool=1)
    try:
        assert run.forward() == 0
        v = run.views(T, full=False)
        d = moe.dispatch(inp["topk_idx"], E)
        assert np.array_equal(v["counts"], d["counts"])
        assert np.array_equal(v["offsets"], d["offsets"])
        assert np.array_equal(v["slot_map"], d["slot_map"])
        assert np.array_equal(v["src"], d["src"])
        full = run.views(T, full=True)
        rows = np.nonzero(d["src"] >= 0)[0]
        tok = d["src"][rows] // k
        assert np.array_equal(full["l1_acts"][rows], inp["x"][tok])
        assert np.array_equal(full["l1_sf"][:, rows], inp["x_sf"][tok].T)
        assert np.array_equal(full["l1_w"][rows], inp["topk_weights"].reshape(-1)[d["src"][rows]])
        y = run.y()
        assert np.all(np.isfinite(codecs.bf16_to_f32(y)))
        rng = np.random.default_rng(1234)
        sample = sorted({0, T - 1, *rng.choice(T, 6, replace=False).tolist()})
        ref = moe.forward_tokens(inp, sample)
        got_codes, want_codes, got_sf, want_sf = [], [], [], []
        for t in sample:
            for j, r in ref[t]["routes"].items():
                s = d["slot_map"][t, j]
                got_codes.append(full["l2_acts"][s])
                want_codes.append(r["l2_acts"])
                got_sf.append(full["l2_sf"][:, s])
                want_sf.append(r["l2_acts_sf"])
                comb = full["comb"][t * k + j]
                assert G.rel_frobenius(comb, r["part"]) <= 2e-3, (t, j)
        G.check_codes(np.array(got_codes), np.array(want_codes), name)
        G.check_sf(np.array(got_sf), np.array(want_sf), name)
        err = G.check_y(y[sample], np.array([ref[t]["y"] for t in sample]), name)
        print(f"[{name}] sampled y rel frobenius {err:.2e}", flush=True)
    finally:
        run.close()
