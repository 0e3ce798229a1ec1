"""A forward call captured in a HIP graph replays to the eager result.

``mega_moe_forward`` allocates nothing, never synchronises and issues no
memory sets (every counter and queue head it uses is reset by its own dispatch
kernel), so a serving loop can capture it once and replay it.  The graph is
replayed several times with eager forwards and synchronisations in between,
the output cleared before each replay, and every replay must equal the eager
result bit for bit.
"""

import numpy as np
import pytest
import torch

from fp8_mixture_experts_amd import synthetic as S
from tests import gpu_util as G
from tests.test_gpu_layer import SMALL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,fmt", [("ragged", "fp8"), ("many_blocks", "fp8"),
                                      ("skewed", "mxfp4")])
def test_captured_forward_replays_to_the_eager_result(name, fmt):
    wl = SMALL[name]
    if fmt == "mxfp4":
        import dataclasses
        wl = dataclasses.replace(wl, name=name + "_mxfp4", weight_format="mxfp4")
    inp = S.make_inputs(wl)
    print(f"[{name} {fmt}] capture", flush=True)
    run = G.Runner(inp)
    try:
        assert run.forward() == 0
        want = run.y().copy()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run.forward(sync=False)                   # warm-up on the capture side stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            run.forward(sync=False)
        torch.cuda.synchronize()
        for i in range(3):
            run.clear_y()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(run.y(), want), f"replay {i}"
            assert run.forward() == 0                   # eager work between replays
            assert np.array_equal(run.y(), want)
        assert run.layer.status() == 0
    finally:
        run.close()
