"""The allocation-free forward (mega_moe_forward_noalloc) against the handle
forward (mega_moe_forward), both through the C ABI.

Both launch the same kernels in the same order, so on two calls in a row, the
second with fewer tokens (a ragged batch), y must agree bit for bit.  Device
error bits are reported per call through the caller's word (an invalid
expert id sets one, the next clean call reports none), and a call whose
workspace would not fit the library's scratch array is refused before any
work is issued.
"""

import numpy as np
import pytest
import torch

from fp8_mixture_experts_amd import binding as B
from fp8_mixture_experts_amd import synthetic as S
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _args(dev):
    return (dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], dev["w1"], dev["w1_sf"],
            dev["w2"], dev["w2_sf"])


def _handle_forward(dims, max_tokens, n, dev, stream):
    E, H, I, k = dims
    layer = B.MegaMoE(E, H, I, k, max_tokens)
    try:
        y = torch.empty((n, H), dtype=torch.int16, device="cuda:0")
        B.mega_moe_forward(layer.handle, n, *_args(dev), y, stream)
        assert layer.status() == 0
        return y.cpu().numpy().view(np.uint16)
    finally:
        layer.close()


def test_noalloc_matches_handle_forward_on_two_calls():
    inp = S.make_inputs("decode")
    dims = G.layer_dims(inp)
    E, H, I, k = dims
    T = inp["x"].shape[0]
    dev = G.to_device(inp)
    stream = torch.cuda.current_stream().cuda_stream
    cfg = B.make_config(E, H, I, k, T)
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for n in (T, 45):
        print(f"[noalloc] {n} tokens", flush=True)
        want = _handle_forward(dims, T, n, dev, stream)
        y = torch.full((n, H), -1, dtype=torch.int16, device="cuda:0")
        B.mega_moe_forward_noalloc(cfg, n, *_args(dev), y, err, stream)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        got = y.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), f"{n} tokens: y differs from the handle forward"


def test_noalloc_reports_each_calls_errors():
    inp = S.make_inputs("tiny")
    E, H, I, k = G.layer_dims(inp)
    T = inp["x"].shape[0]
    dev = G.to_device(inp)
    stream = torch.cuda.current_stream().cuda_stream
    cfg = B.make_config(E, H, I, k, T)
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    y = torch.empty((T, H), dtype=torch.int16, device="cuda:0")
    bad = dict(dev)
    bad["topk_idx"] = dev["topk_idx"].clone()
    bad["topk_idx"][3, 1] = E                       # an invalid expert: route skipped, bit set
    B.mega_moe_forward_noalloc(cfg, T, *_args(bad), y, err, stream)
    torch.cuda.synchronize()
    assert int(err.item()) == B.MEGA_MOE_DEVERR_BAD_EXPERT
    err.zero_()
    B.mega_moe_forward_noalloc(cfg, T, *_args(dev), y, err, stream)
    torch.cuda.synchronize()
    assert int(err.item()) == 0                    # no bit carried over from the call before
    want = _handle_forward((E, H, I, k), T, T, dev, stream)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), want)


def test_noalloc_refuses_what_does_not_fit():
    inp = S.make_inputs("decode")
    E, H, I, k = G.layer_dims(inp)
    dev = G.to_device(inp)
    y = torch.empty((8, H), dtype=torch.int16, device="cuda:0")
    big = B.make_config(E, H, I, k, 8192)
    stream = torch.cuda.current_stream().cuda_stream
    with pytest.raises(B.MegaMoEError) as ei:
        B.mega_moe_forward_noalloc(big, 8192, *_args(dev), y, None, stream)
    assert ei.value.code == B.MEGA_MOE_ERR_INVALID_ARG
    assert "scratch" in B.mega_moe_last_error()
    kept = B.make_config(E, H, I, k, 128, keep_pool=1)
    with pytest.raises(B.MegaMoEError) as ei:
        B.mega_moe_forward_noalloc(kept, 128, *_args(dev), y, None, stream)
    assert ei.value.code == B.MEGA_MOE_ERR_INVALID_ARG
