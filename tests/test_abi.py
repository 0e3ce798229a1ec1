"""C-ABI library checks that need no GPU: it loads, exports every entry point
its header declares, validates configurations, and plans calls by the tiers of
"MegaMoE SM90 Implementation Design (Final)" 12.2 and 13.1 (golden file)."""

import math
import os
import re

import pytest

from fp8_mixture_experts_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return B.load()


def _declared():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", f)).read()
            names |= set(re.findall(r"^\s*(?:int|int32_t|int64_t|const char\*)\s+(mega_moe_\w+)\s*\(",
                                    txt, flags=re.M))
    return names


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"mega_moe_create", "mega_moe_forward", "mega_moe_destroy"} <= names
    assert names == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_token_alignment_is_largest_block_m(lib):
    assert B.mega_moe_token_alignment() == 128


def _cfg(**kw):
    base = dict(num_experts=32, hidden=7168, intermediate=2048, num_topk=8, max_tokens=128)
    base.update(kw)
    return B.make_config(**base)


def test_plan_matches_golden_tiers():
    rows = [l.split() for l in open(os.path.join(ROOT, "tests/golden/block_m_tiers.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) >= 10
    for t, k, e, exp, bm, nm, bn in rows:
        cfg = _cfg(num_experts=int(e), num_topk=int(k), max_tokens=max(int(t), 1))
        p = B.mega_moe_plan(cfg, int(t))
        assert math.isclose(p.expected_tokens_per_expert, float(exp), rel_tol=1e-6)
        assert (p.block_m, p.l2_n_major, p.block_n) == (int(bm), int(nm), int(bn)), (t, k, e)
        assert p.l1_n_blocks == 2 * 2048 // p.block_n and p.l2_n_blocks == 7168 // p.block_n


@pytest.mark.parametrize("kw", [dict(activation_clamp=10.0), dict(activation_clamp=0.25),
                                dict(fast_math=1), dict(fast_math=1, activation_clamp=3.0)])
def test_activation_options_are_accepted(kw):
    assert B.mega_moe_workspace_bytes(_cfg(**kw)) > 0
    B.mega_moe_plan(_cfg(**kw), 128)


def test_plan_keeps_128_columns_where_256_do_not_fit():
    # 64-row tiles go 256 wide only when H splits into 256-column tiles (2I
    # always does: I is a multiple of 128)
    assert B.mega_moe_plan(_cfg(hidden=7296), 128).block_n == 128       # H = 57 x 128
    assert B.mega_moe_plan(_cfg(intermediate=2176), 128).block_n == 256  # 2I = 17 x 256
    assert B.mega_moe_plan(_cfg(), 128).block_n == 256
    assert B.mega_moe_plan(_cfg(), 4096).block_n == 128                  # 128-row tiles


def test_plan_overrides():
    p = B.mega_moe_plan(_cfg(block_m=32, l2_n_major=1), 8192)
    assert p.block_m == 32 and p.l2_n_major == 1
    p = B.mega_moe_plan(_cfg(block_m=128, l2_n_major=0), 1)
    assert p.block_m == 128 and p.l2_n_major == 0
    p = B.mega_moe_plan(_cfg(block_m=64, block_n=256), 128)
    assert p.block_n == 256 and p.l1_n_blocks == 16 and p.l2_n_blocks == 28
    p = B.mega_moe_plan(_cfg(block_m=128, block_n=128), 8192)
    assert p.block_n == 128 and p.l1_n_blocks == 32 and p.l2_n_blocks == 56


@pytest.mark.parametrize("kw", [dict(hidden=100), dict(intermediate=192), dict(num_topk=0),
                                dict(num_experts=0), dict(num_experts=5000), dict(max_tokens=-1),
                                dict(block_m=48), dict(l2_n_major=2), dict(block_n=192),
                                dict(block_m=32, block_n=256),
                                dict(hidden=7296, block_n=256), dict(activation_clamp=0.0),
                                dict(activation_clamp=-1.0), dict(activation_clamp=math.nan),
                                dict(fast_math=2), dict(split_l2_cus=-1), dict(split_l2_cus=32),
                                dict(split_l2_xcds=-1), dict(split_l2_xcds=16),
                                dict(split_l2_cus=4, split_l2_xcds=2)])
def test_invalid_configs_are_rejected(kw):
    assert B.mega_moe_workspace_bytes(_cfg(**kw)) == -1
    with pytest.raises(B.MegaMoEError) as ei:
        B.mega_moe_plan(_cfg(**kw), 1)
    assert ei.value.code == B.MEGA_MOE_ERR_INVALID_ARG
    assert B.mega_moe_last_error()


@pytest.mark.parametrize("kw", [dict(hidden=8320), dict(intermediate=8320)])
def test_unbuilt_options_are_unsupported(kw):
    with pytest.raises(B.MegaMoEError) as ei:
        B.mega_moe_plan(_cfg(**kw), 1)
    assert ei.value.code == B.MEGA_MOE_ERR_UNSUPPORTED


def test_workspace_bytes_cover_the_layer_buffers():
    R = 8192 * 8
    P = (R + 127 * 32 + 127) // 128 * 128
    # re-quantised acts + BF16 partials dominate, with the pool-ordered
    # activation scales; the pool copy of the rows only with keep_pool
    n = B.mega_moe_workspace_bytes(_cfg(max_tokens=8192))
    assert n >= P * 2048 + R * 7168 * 2 + P * (7168 // 128) * 4
    assert n < 1.1 * (P * 2048 + R * 7168 * 2) + (64 << 20)
    kept = B.mega_moe_workspace_bytes(_cfg(max_tokens=8192, keep_pool=1))
    assert kept - n >= P * 7168 + P * 4
    assert kept - n < P * 7168 + P * 4 + 1024
    assert B.mega_moe_workspace_bytes(_cfg(max_tokens=0)) > 0


@pytest.mark.parametrize("n_xcd,cus,seen", [(8, 256, 0), (8, 256, 0xFF), (1, 32, 0), (1, 32, 0x8),
                                            (2, 64, 0x6), (4, 128, 0xF0)])
def test_xcd_layout_accepted(n_xcd, cus, seen):
    # one work queue per XCD: any ids that fall into distinct queues id % n
    assert B.mega_moe_check_xcd_layout(n_xcd, cus, seen) == 0


@pytest.mark.parametrize("n_xcd,cus,seen", [
    (0, 256, 0), (17, 272, 0), (8, 260, 0), (3, 256, 0),    # count unknown or CUs uneven
    (8, 256, 0x7F),                                           # an XCD reports no workgroup
    (2, 64, 0x5),                                             # ids 0 and 2 share queue 0
    (1, 32, 0x3),                                             # two XCDs behind one count
])
def test_xcd_layout_refused(n_xcd, cus, seen):
    # a layout where an L2 tile could run on another XCD than the L1 tiles it
    # reads would need cache write-backs the kernel does not do: refused
    with pytest.raises(B.MegaMoEError) as ei:
        B.mega_moe_check_xcd_layout(n_xcd, cus, seen)
    assert ei.value.code == B.MEGA_MOE_ERR_UNSUPPORTED
    assert "XCD" in B.mega_moe_last_error()


def test_forward_rejects_bad_calls_without_touching_the_gpu():
    # NULL handle and out-of-range token counts fail synchronously
    with pytest.raises(B.MegaMoEError) as ei:
        B.mega_moe_forward(None, 4, *([0] * 9), None)
    assert ei.value.code == B.MEGA_MOE_ERR_INVALID_ARG
    with pytest.raises(B.MegaMoEError) as ei:
        B.mega_moe_forward_mxfp4(None, 4, *([0] * 9), None)
    assert ei.value.code == B.MEGA_MOE_ERR_INVALID_ARG


def test_create_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(B.MegaMoEError) as ei:
        B.mega_moe_create(_cfg())
    assert ei.value.code in (B.MEGA_MOE_ERR_HIP, B.MEGA_MOE_ERR_UNSUPPORTED)


def test_transform_rejects_bad_arguments():
    """Argument errors return before any HIP call, so no GPU is needed."""
    with pytest.raises(B.MegaMoEError) as ei:
        B.mega_moe_transform_w1(1, 100, 128, 16, 16, 16, 16, 0)
    assert ei.value.code == B.MEGA_MOE_ERR_INVALID_ARG
    with pytest.raises(B.MegaMoEError) as ei:                    # in and out overlap
        B.mega_moe_transform_w1(1, 128, 128, 1 << 20, 1 << 12, (1 << 20) + 256, 1 << 13, 0)
    assert ei.value.code == B.MEGA_MOE_ERR_INVALID_ARG


def _layouts():
    # expert pool-block counts: empty, single blocks, runs longer than a
    # group, zero-block experts, and one huge expert
    rng = __import__("numpy").random.default_rng(5)
    yield [0]
    yield [1]
    yield [3, 0, 1, 9, 2, 0, 0, 5]
    yield list(rng.integers(0, 4, 32))
    yield list(rng.integers(0, 12, 64))
    yield [63] + list(rng.integers(1, 20, 29))


@pytest.mark.parametrize("bm,nm,bn", [(32, 0, 128), (32, 1, 128), (64, 0, 128), (64, 1, 256),
                                      (128, 0, 256), (128, 1, 128)])
@pytest.mark.parametrize("n_xcd", [1, 3, 8])
def test_tile_order_visits_every_tile_once(bm, nm, bn, n_xcd):
    # every (pool block, N block) of each phase exactly once; each XCD stays
    # within its contiguous range of pool blocks; N-major groups are runs of
    # one expert's blocks inside a range, at most G long, and take each N
    # block over their blocks before the next N block
    plan = B.mega_moe_plan(_cfg(block_m=bm, l2_n_major=nm, block_n=bn), 4096)
    assert (plan.block_m, plan.l2_n_major, plan.block_n) == (bm, nm, bn)
    G = (2 if bm == 64 else 4) if nm else 1
    for counts in _layouts():
        starts = [0]
        for c in counts:
            starts.append(starts[-1] + int(c))
        M = starts[-1]
        expert = [e for e, c in enumerate(counts) for _ in range(int(c))]
        for phase, nbs in ((1, plan.l1_n_blocks), (2, plan.l2_n_blocks)):
            pb, nb = B.mega_moe_tile_order(plan, starts, n_xcd, phase)
            pairs = list(zip(pb, nb))
            assert sorted(pairs) == [(p, n) for p in range(M) for n in range(nbs)]
            want = []
            for x in range(n_xcd):
                lo, hi = M * x // n_xcd, M * (x + 1) // n_xcd
                p = lo
                while p < hi:
                    q = p
                    while q < hi and q - p < G and expert[q] == expert[p]:
                        q += 1
                    want += [(r, n) for n in range(nbs) for r in range(p, q)]
                    p = q
            assert pairs == want


def test_tile_order_rejects_bad_arguments():
    plan = B.mega_moe_plan(_cfg(), 128)
    for starts, n_xcd, phase in (([0, 4], 0, 1), ([0, 4], 17, 1), ([0, 4], 8, 3),
                                 ([1, 4], 8, 1), ([0, 4, 2], 8, 1)):
        with pytest.raises(B.MegaMoEError) as ei:
            B.mega_moe_tile_order(plan, starts, n_xcd, phase)
        assert ei.value.code == B.MEGA_MOE_ERR_INVALID_ARG
    plan.block_m = 48
    with pytest.raises(B.MegaMoEError):
        B.mega_moe_tile_order(plan, [0, 4], 8, 1)


def test_noalloc_forward_refusals_need_no_gpu():
    # every check of the allocation-free forward runs before it touches a
    # device: the pointers below are aligned stand-ins that are never used
    fake = 1 << 20
    tensors = [fake] * 9
    big = _cfg(max_tokens=8192)
    with pytest.raises(B.MegaMoEError) as ei:
        B.mega_moe_forward_noalloc(big, 8192, *tensors, None, None)
    assert ei.value.code == B.MEGA_MOE_ERR_INVALID_ARG
    assert "scratch" in B.mega_moe_last_error()
    for cfg, n in ((_cfg(max_tokens=128, keep_pool=1), 128),
                   (_cfg(max_tokens=128, split_l2_cus=4), 128),
                   (_cfg(max_tokens=128, split_l2_xcds=2), 128),
                   (_cfg(max_tokens=128), 129)):
        with pytest.raises(B.MegaMoEError) as ei:
            B.mega_moe_forward_noalloc(cfg, n, *tensors, None, None)
        assert ei.value.code == B.MEGA_MOE_ERR_INVALID_ARG
    with pytest.raises(B.MegaMoEError):
        B.mega_moe_forward_noalloc(_cfg(max_tokens=128), 128, *([0] * 9), None, None)
    assert B.mega_moe_forward_noalloc(_cfg(max_tokens=128), 0, *([0] * 9), None, None) == 0
