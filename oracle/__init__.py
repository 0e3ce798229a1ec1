"""CPU oracle for the fused FP8 mixture-of-experts expert layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing); the two
meet only at the seeded synthetic inputs, which are data.

The oracle is a plain, slow, float64 restatement of the layer that the page
"MegaMoE SM90 Implementation Design (Final)" describes (cited below as
"SM90 design", with its section numbers), completed where that page is silent
by the page "PR357 Green-Context Split MegaMoE code review" (cited as
"PR357 review"):

* ``codecs``  OCP FP8 E4M3 decode/encode (round-to-nearest-even, saturating),
  BF16 round-to-nearest-even, and the MXFP4 weight format (E2M1 codes with
  UE8M0 scales per 32 K elements) of the page's SM100 variant.
* ``moe``     dispatch (counts, 128-aligned offsets, stable slot map, source
  metadata, pool copies), the L1 block-scaled GEMM, SwiGLU times the top-k
  weight, per-64 amax re-quantisation, the L2 block-scaled GEMM with per-64
  activation scales, the BF16 partial cast and the FP32 top-k combine; the
  two GEMMs also for MXFP4 weights.

Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself (exhaustive codec properties, a library cast, exact rational brute
force, closed forms and metamorphic relations).  Parity unpinned: which of two
adjacent FP8 codes (or BF16 values) is produced when the exact intermediate lies
within float32 noise of a rounding midpoint; the GPU comparison tolerates one
code step there.
"""

from . import codecs, moe  # noqa: F401
