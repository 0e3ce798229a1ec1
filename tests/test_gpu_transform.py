"""GPU parity of the W1 transform (mega_moe_transform_w1) with the oracle's.

Integer/byte work: codes and scales must match bit for bit, over every E4M3
code (NaN, both zeros, subnormals) and scale pairs that are equal, at ratio
1/2, at random ratios and both zero.  Then the layer runs on transformed
weights and is compared with the oracle on the same weights.
"""

import numpy as np
import pytest
import torch

from fp8_mixture_experts_amd import binding as B
from fp8_mixture_experts_amd import synthetic as S
from oracle import moe, transform
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _plain(rng, E, I, H):
    w = rng.integers(0, 256, (E, 2 * I, H), dtype=np.uint8)
    nb, kb = 2 * I // 128, H // 128
    sf = rng.uniform(1e-4, 1.0, (E, nb, kb)).astype(np.float32)
    # some stored blocks with equal source scales, some at ratio 1/2, one pair of zeros
    sf[0, nb // 2] = sf[0, 0]
    sf[-1, 0, 0] = 2.0 * sf[-1, nb // 2, 0]
    sf[-1, 0, -1] = 0.0
    sf[-1, nb // 2, -1] = 0.0
    return w, sf


def _run(w, sf):
    E, N, H = w.shape
    d_w = torch.from_numpy(w).cuda()
    d_sf = torch.from_numpy(sf).cuda()
    out = torch.empty_like(d_w)
    out_sf = torch.empty_like(d_sf)
    B.mega_moe_transform_w1(E, H, N // 2, d_w.data_ptr(), d_sf.data_ptr(), out.data_ptr(),
                            out_sf.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return out.cpu().numpy(), out_sf.cpu().numpy()


@pytest.mark.parametrize("shape", [(3, 256, 384), (2, 128, 7168), (1, 2048, 256)])
def test_transform_matches_oracle_bit_exactly(shape):
    E, I, H = shape
    rng = np.random.default_rng(E * 1000 + I + H)
    w, sf = _plain(rng, E, I, H)
    got, got_sf = _run(w, sf)
    want, want_sf = transform.transform_w1(w, sf)
    assert np.array_equal(got_sf, want_sf)
    diff = np.nonzero(got != want)
    assert len(diff[0]) == 0, (len(diff[0]), got[diff][:8], want[diff][:8])


def test_layer_on_transformed_weights_matches_oracle():
    inp = S.make_inputs(S.custom("ragged", tokens=37, hidden=384, intermediate=256, experts=5,
                                 topk=3, seed=3, weight_seed=4))
    E, N, H = inp["w1"].shape
    rng = np.random.default_rng(77)
    w, sf = _plain(rng, E, N // 2, H)
    # keep the weights' magnitude near the generator's: codes of N(0, 1) x small scales
    w = np.where((w & 0x7F) >= 0x7E, 0x38, w).astype(np.uint8)     # no NaN, no +-448
    sf = (sf * 0.02 / 448.0 * 8.0).astype(np.float32)
    got, got_sf = _run(w, sf)
    inp["w1"], inp["w1_sf"] = got, got_sf
    ref = moe.forward(inp)
    run = G.Runner(inp)
    try:
        assert run.forward() == 0
        T = inp["x"].shape[0]
        v = run.views(T, full=False)
        valid = ref["src"] >= 0
        G.check_codes(v["l2_acts"][valid], ref["l2_acts"][valid], "transformed")
        G.check_y(run.y(), ref["y"], "transformed")
    finally:
        run.close()
