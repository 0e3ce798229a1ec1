"""Thin Python binding of the C ABI in include/mega_moe.h (ctypes).

Argument marshalling only: every step of the layer runs in the HIP library.
Functions keep the C names; tensors are passed as device pointers
(``tensor.data_ptr()``) and the stream as ``torch.cuda.current_stream()``'s
handle.  PyTorch is used only for device memory and streams.  Loading fails
loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmega_moe.so")

MEGA_MOE_OK = 0
MEGA_MOE_ERR_INVALID_ARG = -1
MEGA_MOE_ERR_UNSUPPORTED = -2
MEGA_MOE_ERR_HIP = -3
MEGA_MOE_ERR_OUT_OF_MEMORY = -4
MEGA_MOE_ERR_DEVICE = -5
MEGA_MOE_DEVERR_BAD_EXPERT = 0x1
MEGA_MOE_DEVERR_WAIT_TIMEOUT = 0x2
MEGA_MOE_DEVERR_SCALE_RANGE = 0x4

EXPORTS = ["mega_moe_create", "mega_moe_forward", "mega_moe_forward_mxfp4", "mega_moe_destroy",
           "mega_moe_get_status",
           "mega_moe_last_error", "mega_moe_workspace_bytes", "mega_moe_token_alignment",
           "mega_moe_plan", "mega_moe_tile_order", "mega_moe_get_views", "mega_moe_set_recv_stats",
           "mega_moe_transform_w1", "mega_moe_profile_begin",
           "mega_moe_profile_end", "mega_moe_check_xcd_layout", "mega_moe_forward_noalloc"]


class mega_moe_config(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("num_topk", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("activation_clamp", ctypes.c_float),
                ("fast_math", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("l2_n_major", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("split_l2_cus", ctypes.c_int32), ("keep_pool", ctypes.c_int32),
                ("split_l2_xcds", ctypes.c_int32)]


class mega_moe_plan_info(ctypes.Structure):
    _fields_ = [("expected_tokens_per_expert", ctypes.c_float), ("block_m", ctypes.c_int32),
                ("l2_n_major", ctypes.c_int32), ("l1_n_blocks", ctypes.c_int32),
                ("l2_n_blocks", ctypes.c_int32), ("block_n", ctypes.c_int32)]


class mega_moe_views(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("slot_map", ctypes.c_void_p), ("src", ctypes.c_void_p),
                ("l1_acts", ctypes.c_void_p), ("l1_acts_sf", ctypes.c_void_p),
                ("l1_topk_weights", ctypes.c_void_p), ("l2_acts", ctypes.c_void_p),
                ("l2_acts_sf", ctypes.c_void_p), ("combine_buf", ctypes.c_void_p),
                ("pool_rows_capacity", ctypes.c_int64), ("last_num_tokens", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m "
                           "fp8_mixture_experts_amd.build or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.mega_moe_create.argtypes = [ctypes.POINTER(mega_moe_config), ctypes.POINTER(vp)]
    lib.mega_moe_create.restype = ctypes.c_int
    lib.mega_moe_forward.argtypes = [vp, i32] + [vp] * 9 + [vp]
    lib.mega_moe_forward.restype = ctypes.c_int
    lib.mega_moe_forward_mxfp4.argtypes = [vp, i32] + [vp] * 9 + [vp]
    lib.mega_moe_forward_mxfp4.restype = ctypes.c_int
    lib.mega_moe_destroy.argtypes = [vp]
    lib.mega_moe_destroy.restype = ctypes.c_int
    lib.mega_moe_get_status.argtypes = [vp, vp]
    lib.mega_moe_get_status.restype = ctypes.c_int
    lib.mega_moe_last_error.argtypes = []
    lib.mega_moe_last_error.restype = ctypes.c_char_p
    lib.mega_moe_workspace_bytes.argtypes = [ctypes.POINTER(mega_moe_config)]
    lib.mega_moe_workspace_bytes.restype = i64
    lib.mega_moe_token_alignment.argtypes = []
    lib.mega_moe_token_alignment.restype = i32
    lib.mega_moe_plan.argtypes = [ctypes.POINTER(mega_moe_config), i32,
                                  ctypes.POINTER(mega_moe_plan_info)]
    lib.mega_moe_plan.restype = ctypes.c_int
    lib.mega_moe_tile_order.argtypes = [ctypes.POINTER(mega_moe_plan_info), i32, ctypes.POINTER(i32),
                                        i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.mega_moe_tile_order.restype = ctypes.c_int
    lib.mega_moe_get_views.argtypes = [vp, ctypes.POINTER(mega_moe_views)]
    lib.mega_moe_get_views.restype = ctypes.c_int
    lib.mega_moe_transform_w1.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.mega_moe_transform_w1.restype = ctypes.c_int
    lib.mega_moe_set_recv_stats.argtypes = [vp, vp]
    lib.mega_moe_set_recv_stats.restype = ctypes.c_int
    lib.mega_moe_profile_begin.argtypes = [vp, i32]
    lib.mega_moe_profile_begin.restype = ctypes.c_int
    lib.mega_moe_profile_end.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32,
                                         ctypes.POINTER(i32)]
    lib.mega_moe_profile_end.restype = ctypes.c_int
    lib.mega_moe_check_xcd_layout.argtypes = [i32, i32, ctypes.c_uint32]
    lib.mega_moe_check_xcd_layout.restype = ctypes.c_int
    lib.mega_moe_forward_noalloc.argtypes = [ctypes.POINTER(mega_moe_config), i32] + [vp] * 10 + [vp]
    lib.mega_moe_forward_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


class MegaMoEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mega_moe error {code}: {msg}")
        self.code = code


def _check(rc: int) -> int:
    if rc < 0:
        raise MegaMoEError(rc, load().mega_moe_last_error().decode())
    return rc


def make_config(num_experts, hidden, intermediate, num_topk, max_tokens, block_m=0,
                l2_n_major=-1, activation_clamp=math.inf, fast_math=0,
                block_n=0, split_l2_cus=0, keep_pool=0, split_l2_xcds=0) -> mega_moe_config:
    return mega_moe_config(num_experts, hidden, intermediate, num_topk, max_tokens,
                           activation_clamp, fast_math, block_m, l2_n_major, block_n,
                           split_l2_cus, keep_pool, split_l2_xcds)


# ---- the C entry points, one Python function each ---------------------------

def mega_moe_create(cfg: mega_moe_config) -> int:
    h = ctypes.c_void_p()
    _check(load().mega_moe_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h.value


def mega_moe_forward(handle, num_tokens, x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf,
                     y, stream) -> int:
    """All tensor arguments are device pointers (int) or tensors with data_ptr()."""
    ptr = lambda t: t if isinstance(t, int) else t.data_ptr()   # noqa: E731
    return _check(load().mega_moe_forward(
        handle, num_tokens, ptr(x), ptr(x_sf), ptr(topk_idx), ptr(topk_weights), ptr(w1),
        ptr(w1_sf), ptr(w2), ptr(w2_sf), ptr(y), stream))


def mega_moe_forward_mxfp4(handle, num_tokens, x, x_sf, topk_idx, topk_weights, w1, w1_scale,
                           w2, w2_scale, y, stream) -> int:
    """MXFP4 weights (E2M1 pairs + UE8M0 per 32 K); pointers as mega_moe_forward."""
    ptr = lambda t: t if isinstance(t, int) else t.data_ptr()   # noqa: E731
    return _check(load().mega_moe_forward_mxfp4(
        handle, num_tokens, ptr(x), ptr(x_sf), ptr(topk_idx), ptr(topk_weights), ptr(w1),
        ptr(w1_scale), ptr(w2), ptr(w2_scale), ptr(y), stream))


def mega_moe_forward_noalloc(cfg: mega_moe_config, num_tokens, x, x_sf, topk_idx, topk_weights,
                             w1, w1_sf, w2, w2_sf, y, dev_errors, stream) -> int:
    """The allocation-free forward (no handle).  Tensor arguments are device
    pointers (int) or tensors with data_ptr(); dev_errors may be None."""
    ptr = lambda t: t if t is None or isinstance(t, int) else t.data_ptr()   # noqa: E731
    return _check(load().mega_moe_forward_noalloc(
        ctypes.byref(cfg), num_tokens, ptr(x), ptr(x_sf), ptr(topk_idx), ptr(topk_weights),
        ptr(w1), ptr(w1_sf), ptr(w2), ptr(w2_sf), ptr(y), ptr(dev_errors), stream))


def mega_moe_destroy(handle) -> int:
    return _check(load().mega_moe_destroy(handle))


def mega_moe_get_status(handle, stream) -> int:
    return _check(load().mega_moe_get_status(handle, stream))


def mega_moe_last_error() -> str:
    return load().mega_moe_last_error().decode()


def mega_moe_check_xcd_layout(num_xcds: int, num_cus: int, seen_ids: int = 0) -> int:
    return _check(load().mega_moe_check_xcd_layout(num_xcds, num_cus, seen_ids))


def mega_moe_workspace_bytes(cfg: mega_moe_config) -> int:
    return load().mega_moe_workspace_bytes(ctypes.byref(cfg))


def mega_moe_token_alignment() -> int:
    return load().mega_moe_token_alignment()


def mega_moe_plan(cfg: mega_moe_config, num_tokens: int) -> mega_moe_plan_info:
    out = mega_moe_plan_info()
    _check(load().mega_moe_plan(ctypes.byref(cfg), num_tokens, ctypes.byref(out)))
    return out


def mega_moe_tile_order(plan: mega_moe_plan_info, block_start, n_xcd: int, phase: int):
    """The expert kernel's tile order for pool blocks laid out by block_start
    (each expert's first pool block, then the total): (pool block, N block)
    lists over all XCD ranges, each XCD's tiles in queue order (phase 1 L1,
    phase 2 L2)."""
    E = len(block_start) - 1
    starts = (ctypes.c_int32 * (E + 1))(*block_start)
    nbs = plan.l1_n_blocks if phase == 1 else plan.l2_n_blocks
    n = max(block_start[-1] * nbs, 0) if E >= 0 else 0
    pb = (ctypes.c_int32 * max(n, 1))()
    nb = (ctypes.c_int32 * max(n, 1))()
    _check(load().mega_moe_tile_order(ctypes.byref(plan), E, starts, n_xcd, phase, pb, nb))
    return list(pb[:n]), list(nb[:n])


def mega_moe_get_views(handle) -> mega_moe_views:
    out = mega_moe_views()
    _check(load().mega_moe_get_views(handle, ctypes.byref(out)))
    return out


def mega_moe_transform_w1(num_experts, hidden, intermediate, w1_plain, w1_sf_plain, w1_out,
                          w1_sf_out, stream) -> int:
    """Device pointers (ints); see include/mega_moe.h."""
    return _check(load().mega_moe_transform_w1(num_experts, hidden, intermediate, w1_plain,
                                               w1_sf_plain, w1_out, w1_sf_out, stream))


def mega_moe_set_recv_stats(handle, stats) -> int:
    """stats: device pointer of int32 [E] (or None to turn the statistics off)."""
    return _check(load().mega_moe_set_recv_stats(handle, stats))


def mega_moe_profile_begin(handle, max_calls: int) -> int:
    return _check(load().mega_moe_profile_begin(handle, max_calls))


def mega_moe_profile_end(handle, capacity: int):
    """Returns a list of (dispatch_ms, expert_ms, combine_ms) per timed call."""
    buf = (ctypes.c_float * (3 * max(capacity, 1)))()
    n = ctypes.c_int32()
    _check(load().mega_moe_profile_end(handle, buf, capacity, ctypes.byref(n)))
    return [(buf[3 * i], buf[3 * i + 1], buf[3 * i + 2]) for i in range(n.value)]


# ---- convenience wrapper (still marshalling only) ---------------------------

class MegaMoE:
    """Owns one handle; ``forward`` takes device tensors and writes ``y``."""

    def __init__(self, num_experts, hidden, intermediate, num_topk, max_tokens, **kw):
        self.cfg = make_config(num_experts, hidden, intermediate, num_topk, max_tokens, **kw)
        self.handle = mega_moe_create(self.cfg)

    def forward(self, x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf, y, stream=None):
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        return mega_moe_forward(self.handle, x.shape[0], x, x_sf, topk_idx, topk_weights, w1,
                                w1_sf, w2, w2_sf, y, stream)

    def forward_mxfp4(self, x, x_sf, topk_idx, topk_weights, w1, w1_scale, w2, w2_scale, y,
                      stream=None):
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        return mega_moe_forward_mxfp4(self.handle, x.shape[0], x, x_sf, topk_idx, topk_weights,
                                      w1, w1_scale, w2, w2_scale, y, stream)

    def status(self, stream=None) -> int:
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        return mega_moe_get_status(self.handle, stream)

    def views(self) -> mega_moe_views:
        return mega_moe_get_views(self.handle)

    def close(self):
        if self.handle:
            mega_moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
