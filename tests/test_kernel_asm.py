"""Checks on the compiled expert kernel (gfx950 assembly, built here with hipcc).

* No instance spills to scratch, and each fits the 256 registers per lane that
  two workgroups per CU leave every wave.
* Every L2 write-back (``buffer_wbl2``, the release before a pool block is
  marked readable from other XCDs) and every L2 invalidation (``buffer_inv``,
  the acquire of a workgroup reading another XCD's block) is followed by a
  full wait before the next atomic or barrier: without it the mark can become
  visible, or the other waves can load, before the cache operation is done.
* No full drain of the direct global->LDS loads (``s_waitcnt vmcnt(0)``) sits
  in the matrix code.  The K loop keeps S - 1 steps of loads in flight and
  waits only for the oldest; a drain there serialises the pipeline without
  changing any result, so only this check catches it.  The compiler inserts
  one when a stage is read through a type it cannot tell apart from the data
  the direct loads write (a float or struct-typed read of LDS), which is why
  every read of a stage goes through an integer vector type.
"""

import os
import re
import subprocess
import tempfile

import pytest

from fp8_mixture_experts_amd import build as BLD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "fp8_mixture_experts_amd", "csrc", "expert_ffn.hip")


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(BLD.HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "ef.s")
        cmd = [BLD.HIPCC, "-x", "hip", *BLD.COMMON, *BLD.DEVICE_ONLY, "--offload-device-only",
               "-S", SRC, "-o", out]
        cmd = [c for c in cmd if c != "-fPIC"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    lines = text.split("\n")
    starts = [(i, l.split(":")[0]) for i, l in enumerate(lines)
              if l.startswith("_ZN8mega_moe14moe_expert_ffn")]
    assert starts, "no expert kernel instances found"
    bodies = {}
    for n, (i, name) in enumerate(starts):
        j = starts[n + 1][0] if n + 1 < len(starts) else len(lines)
        bodies[name] = lines[i:j]
    # kernel metadata: one YAML list entry per kernel, fields in any order
    meta = {}
    section = text[text.index("amdhsa.kernels:"):]
    for chunk in section.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", chunk)
        if not name or "moe_expert_ffn" not in name.group(1):
            continue
        get = lambda k, c=chunk: int(re.search(r"\." + k + r":\s+(\d+)", c).group(1))
        meta[name.group(1)] = dict(vgpr=get("vgpr_count"), scratch=get("private_segment_fixed_size"))
    return bodies, meta


def test_every_instance_fits_without_spills(kernels):
    _, meta = kernels
    assert len(meta) >= 8
    for name, m in meta.items():
        assert m["scratch"] == 0, (name, m)
        assert m["vgpr"] <= 256, (name, m)


def test_no_load_drain_in_the_matrix_code(kernels):
    bodies, _ = kernels
    for name, body in bodies.items():
        for k, line in enumerate(body):
            if "s_waitcnt" in line and "vmcnt(0)" in line:
                window = body[k + 1:k + 60]
                assert not any("v_mfma" in x for x in window), (
                    f"{name}: full load drain before matrix code at line {k}")


def test_cache_writeback_and_invalidate_are_waited_for(kernels):
    bodies, _ = kernels
    seen = 0
    for name, body in bodies.items():
        code = [x.strip() for x in body if x.startswith("\t") and not x.strip().startswith(";")]
        for k, line in enumerate(code):
            if line.startswith(("buffer_wbl2", "buffer_inv")):
                seen += 1
                nxt = [x for x in code[k + 1:k + 40]
                       if x.startswith(("s_waitcnt", "global_atomic", "buffer_atomic", "s_barrier"))]
                assert nxt and nxt[0].startswith("s_waitcnt") and "vmcnt(0)" in nxt[0], (
                    f"{name}: {line} not followed by a full wait: {nxt[:3]}")
    assert seen >= 8
