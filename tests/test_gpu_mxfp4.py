"""GPU parity of the layer with MXFP4 weights (E2M1 codes with UE8M0 scales per
32 K elements, the SM100 kernel's weight format of the "MegaMoE SM90
Implementation Design (Final)" page, §2.1 and §15.2), through
``mega_moe_forward_mxfp4``, against the float64 oracle's MXFP4 path.

The same acceptance rules as the FP8 weights apply (tests/gpu_util.py):
dispatch and pool copies bit-exact, re-quantised activations by the code rule,
partials and y by relative Frobenius error.  Small shapes run at every tile
height, with ragged tails, several pool blocks per expert and a single expert;
the 128-token decode batch runs at full size over all routes.  A block scale
outside the exact range of the L1 path must raise its device error bit.
"""

import dataclasses

import numpy as np
import pytest

from fp8_mixture_experts_amd import binding as B
from fp8_mixture_experts_amd import synthetic as S
from oracle import moe
from tests import gpu_util as G
from tests.test_gpu_layer import EDGE, SMALL, _compare_all

pytestmark = pytest.mark.gpu

MX_SMALL = {name: dataclasses.replace(wl, name=name + "_mxfp4", weight_format="mxfp4")
            for name, wl in SMALL.items()}

_cache = {}


def _case(name):
    if name not in _cache:
        inp = S.make_inputs(MX_SMALL[name])
        _cache[name] = (inp, moe.forward(inp))
    return _cache[name]


@pytest.mark.parametrize("name", list(MX_SMALL))
@pytest.mark.parametrize("block_m", [0, 32, 64, 128])
def test_mxfp4_layer_matches_oracle(name, block_m):
    inp, ref = _case(name)
    print(f"[{name} mxfp4] block_m {block_m}", flush=True)
    run = G.Runner(inp, block_m=block_m)
    try:
        assert run.forward() == 0
        err = _compare_all(inp, ref, run, f"{name} mxfp4 block_m {block_m}")
        print(f"{name} mxfp4 block_m {block_m}: y rel frobenius {err:.2e}")
    finally:
        run.close()


def test_mxfp4_ignores_wide_tile_setting():
    # the MXFP4 path always runs 128-column tiles; a 256-column config must
    # give the same bits as the default
    inp, ref = _case("many_blocks")
    outs = []
    for bn in (0, 256):
        run = G.Runner(inp, block_m=128, block_n=bn)
        try:
            assert run.forward() == 0
            _compare_all(inp, ref, run, f"many_blocks mxfp4 block_n {bn}")
            outs.append(run.y().copy())
        finally:
            run.close()
    assert np.array_equal(outs[0], outs[1])


def test_mxfp4_decode_full_size_all_routes():
    inp = S.make_inputs("decode_mxfp4")
    print("[decode_mxfp4] full size", flush=True)
    ref = moe.forward(inp)
    run = G.Runner(inp)
    try:
        assert run.forward() == 0
        err = _compare_all(inp, ref, run, "decode_mxfp4")
        print(f"decode_mxfp4: y rel frobenius {err:.2e}")
    finally:
        run.close()


def test_mxfp4_scale_outside_exact_range_is_reported():
    inp, _ = _case("ragged")
    for e8, flagged in ((103, True), (104, False), (140, False), (141, True)):
        bad = dict(inp)
        bad["w1_e8"] = inp["w1_e8"].copy()
        bad["w1_e8"][0, 5, 1] = e8
        run = G.Runner(bad)
        try:
            status = run.forward()
            assert bool(status & B.MEGA_MOE_DEVERR_SCALE_RANGE) == flagged, (e8, status)
            assert status & ~B.MEGA_MOE_DEVERR_SCALE_RANGE == 0, (e8, status)
        finally:
            run.close()


def test_mxfp4_and_fp8_calls_share_a_handle():
    # one handle serves both weight formats, in any order
    mx_inp, mx_ref = _case("skewed")
    fp8_inp = S.make_inputs(SMALL["skewed"])
    fp8_ref = moe.forward(fp8_inp)
    run = G.Runner(mx_inp)
    dev8 = G.to_device(fp8_inp)
    try:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
        for _ in range(2):
            assert run.forward() == 0
            G.check_y(run.y(), mx_ref["y"], "skewed mxfp4")
            B.mega_moe_forward(run.layer.handle, fp8_inp["x"].shape[0], dev8["x"], dev8["x_sf"],
                               dev8["topk_idx"], dev8["topk_weights"], dev8["w1"], dev8["w1_sf"],
                               dev8["w2"], dev8["w2_sf"], dev8["y"], stream)
            assert run.layer.status() == 0
            G.check_y(run.y(dev8), fp8_ref["y"], "skewed fp8")
    finally:
        run.close()


@pytest.mark.parametrize("name", list(EDGE))
def test_mxfp4_edge_shapes_match_oracle(name):
    # the largest hidden / intermediate (64 scale blocks of a weight row
    # block), top-k equal to the expert count, one expert with many pool
    # blocks and a single token, with MXFP4 weights, at the planned, 64- and
    # 128-row tiles
    wl = dataclasses.replace(EDGE[name], name=name + "_mxfp4", weight_format="mxfp4")
    inp = S.make_inputs(wl)
    ref = moe.forward(inp)
    for bm in (0, 64, 128):
        print(f"[{name} mxfp4] block_m {bm}", flush=True)
        run = G.Runner(inp, block_m=bm)
        try:
            assert run.forward() == 0
            _compare_all(inp, ref, run, f"{name} mxfp4 block_m {bm}")
        finally:
            run.close()
