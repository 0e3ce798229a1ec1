"""The expert layer, step by step, in float64 on the CPU (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Notation: T tokens, H hidden, I expert intermediate, E local experts, k top-k.
A "route" is one (token t, slot j) pair, flat index f = t*k + j.

Readings taken where the pages leave a step open (each is listed, with its
reason, in the design notes of the repository):

* Scale factors are applied per 128-wide K block of the L1 GEMM and per 64-wide
  K half of the L2 GEMM, on the raw block dot products ("SM90 design" §5.3 and
  §5.4); the weight scale layout is (E, N/128, K/128) float32 (§15.2).
* L1 weight rows are stored gate/up interleaved with granularity 8 (§15.1):
  stored rows 16g..16g+7 are the gate rows of outputs 8g..8g+7 and rows
  16g+8..16g+15 the up rows of the same outputs.  The 128x128 weight scale
  blocks are blocks of the stored (interleaved) tensor.
* The top-k weight multiplies the SwiGLU output before the amax (§10.1 steps
  2-4), so the combine is an unweighted sum.
* One float32 scale ``amax / 448`` per row per 64 intermediate columns (§5.4,
  §10.1 step 5); an all-zero group gets scale 0 and codes 0.
* The L2 result is cast to BF16 before it is scattered (§11.1) and the combine
  sums the BF16 partials of the active slots in float32, in slot order, and
  casts the sum to BF16 (§11.2; "PR357 review" §6.3).
* A slot is active when 0 <= topk_idx < E; others are skipped everywhere.
* The optional activation clamp (a finite float32 ``clamp``) clamps the gate
  and the up value to [-clamp, clamp] before SiLU (§10.1 step 3); +inf is no
  clamp, the default.
* Pool segments of each expert start at multiples of 128 and routes keep
  ascending flat order inside their expert's segment.
"""

import math

import numpy as np

from .codecs import (E4M3_MAX, bf16_rne, bf16_to_f32, e4m3_decode,
                     e4m3_encode_rne, f32, mxfp4_decode)

POOL_ALIGN = 128     # pool segment alignment = largest BLOCK_M ("SM90 design" §13.1)
K_BLOCK = 128        # K granularity of activation and weight scales (§1.1, §15.2)
L2_SF_GROUP = 64     # per-64 re-quantisation group (§5.4)
GATE_UP_GRANULE = 8  # gate/up interleave granularity (§15.1)


# --------------------------------------------------------------------------
# Dispatch ("SM90 design" §3.3 phase 1, §9.2)
# --------------------------------------------------------------------------

def dispatch(topk_idx, num_experts):
    """Per-expert counts, pool offsets, slot map and source metadata.

    Returns dict with
      counts   int64 [E]      routes per expert
      offsets  int64 [E+1]    offsets[e+1] = offsets[e] + align_up(counts[e], 128)
      slot_map int64 [T, k]   pool row of route (t, j), -1 if inactive
      src      int64 [P]      flat route index held by each pool row, -1 = padding
      active   bool  [T, k]
    """
    topk_idx = np.asarray(topk_idx)
    T, k = topk_idx.shape
    flat = topk_idx.reshape(-1).astype(np.int64)
    active = (flat >= 0) & (flat < num_experts)
    counts = np.bincount(flat[active], minlength=num_experts).astype(np.int64)
    padded = (counts + POOL_ALIGN - 1) // POOL_ALIGN * POOL_ALIGN
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    slot_map = np.full(T * k, -1, dtype=np.int64)
    fill = offsets[:-1].copy()
    for f in range(T * k):               # ascending flat route order
        if active[f]:
            e = flat[f]
            slot_map[f] = fill[e]
            fill[e] += 1
    src = np.full(int(offsets[-1]), -1, dtype=np.int64)
    routes = np.nonzero(active)[0]
    src[slot_map[routes]] = routes
    return dict(counts=counts, offsets=offsets, slot_map=slot_map.reshape(T, k),
                src=src, active=active.reshape(T, k))


def gather_pool(x, x_sf, topk_weights, disp):
    """Copies of each routed token's FP8 row, its scales and its top-k weight.

    ``l1_acts`` [P, H] uint8, ``l1_acts_sf`` [H/128, P] float32 (pool-row
    minor, "SM90 design" §9.2), ``l1_w`` [P] float32.  Padding rows are zero.
    """
    T, H = x.shape
    k = disp["slot_map"].shape[1]
    P = disp["src"].shape[0]
    l1_acts = np.zeros((P, H), dtype=np.uint8)
    l1_acts_sf = np.zeros((H // K_BLOCK, P), dtype=np.float32)
    l1_w = np.zeros(P, dtype=np.float32)
    routes = np.nonzero(disp["src"] >= 0)[0]
    f = disp["src"][routes]
    t = f // k
    l1_acts[routes] = x[t]
    l1_acts_sf[:, routes] = x_sf[t].T
    l1_w[routes] = np.asarray(topk_weights, dtype=np.float32).reshape(-1)[f]
    return dict(l1_acts=l1_acts, l1_acts_sf=l1_acts_sf, l1_w=l1_w)


# --------------------------------------------------------------------------
# L1 GEMM + SwiGLU + re-quantisation ("SM90 design" §5.1-5.3, §10.1)
# --------------------------------------------------------------------------

def l1_gemm(a_codes, a_sf, w1_codes, w1_sf):
    """acc[r, n] = sum_kb a_sf[r, kb] * w1_sf[n // 128, kb] * D_kb[r, n].

    D_kb is the raw dot of the decoded codes over K block kb.  Every E4M3 value
    is an integer multiple of 2^-9 below 2^9, so D_kb is a sum of multiples of
    2^-18 below 2^49 in magnitude: exact in float64 whatever the summation
    order.  a_codes [m, H], a_sf [m, H/128], w1_codes [N, H], w1_sf [N/128, H/128].
    """
    A = e4m3_decode(a_codes)
    B = e4m3_decode(w1_codes)
    m, H = A.shape
    N = B.shape[0]
    acc = np.zeros((m, N), dtype=np.float64)
    sw_cols = np.repeat(np.asarray(w1_sf, np.float64), K_BLOCK, axis=0)  # [N, H/128]
    a_sf = np.asarray(a_sf, np.float64)
    for kb in range(H // K_BLOCK):
        ks = slice(kb * K_BLOCK, (kb + 1) * K_BLOCK)
        D = A[:, ks] @ B[:, ks].T
        acc += (a_sf[:, kb][:, None] * sw_cols[:, kb][None, :]) * D
    return acc


def swiglu_weighted(acc, topk_w, clamp=math.inf):
    """h[r, i] = silu(gate) * up * topk_w[r] on the interleaved L1 output.

    Output i takes its gate from stored column 16*(i//8) + i%8 and its up from
    16*(i//8) + 8 + i%8 ("SM90 design" §15.1); silu(g) = g / (1 + exp(-g))
    (§10.1 step 3).  With a finite ``clamp`` the gate and the up value are
    each first clamped to [-clamp, clamp] (§10.1 step 3, the activation clamp
    option); +inf means no clamp.
    """
    m, N = acc.shape
    I = N // 2
    i = np.arange(I)
    gate_col = 2 * GATE_UP_GRANULE * (i // GATE_UP_GRANULE) + i % GATE_UP_GRANULE
    up_col = gate_col + GATE_UP_GRANULE
    g = acc[:, gate_col]
    u = acc[:, up_col]
    if math.isfinite(clamp):
        c = float(clamp)
        g = np.clip(g, -c, c)
        u = np.clip(u, -c, c)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    return silu * u * np.asarray(topk_w, np.float64)[:, None]


def quantize_per64(h):
    """Per-row, per-64-column amax -> float32 scale amax/448 -> E4M3 codes.

    ("SM90 design" §10.1 steps 4-6.)  Returns codes [m, I] uint8 and scales
    [m, I/64] float32.  The division is done in float64 by the float32 scale.
    """
    m, I = h.shape
    g = h.reshape(m, I // L2_SF_GROUP, L2_SF_GROUP)
    amax = np.abs(g).max(axis=-1)
    sf = f32(amax / E4M3_MAX)
    sf64 = sf.astype(np.float64)[..., None]
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.where(sf64 > 0, g / np.where(sf64 > 0, sf64, 1.0), 0.0)
    return e4m3_encode_rne(q).reshape(m, I), sf


# --------------------------------------------------------------------------
# L2 GEMM + BF16 cast ("SM90 design" §5.4, §11.1)
# --------------------------------------------------------------------------

def l2_gemm(a_codes, a_sf64, w2_codes, w2_sf):
    """acc[r, n] = sum_kb w2_sf[n//128, kb] * (s0 * D0 + s1 * D1), float64.

    D0, D1 are the exact raw dots over the two 64-wide halves of K block kb and
    s0 = a_sf64[r, 2kb], s1 = a_sf64[r, 2kb+1] their per-64 activation scales.
    a_codes [m, I], a_sf64 [m, I/64], w2_codes [H, I], w2_sf [H/128, I/128].
    """
    A = e4m3_decode(a_codes)
    B = e4m3_decode(w2_codes)
    m, I = A.shape
    H = B.shape[0]
    acc = np.zeros((m, H), dtype=np.float64)
    sw_cols = np.repeat(np.asarray(w2_sf, np.float64), K_BLOCK, axis=0)  # [H, I/128]
    s = np.asarray(a_sf64, np.float64)
    for kb in range(I // K_BLOCK):
        halves = []
        for hh in range(2):
            c0 = kb * K_BLOCK + hh * L2_SF_GROUP
            ks = slice(c0, c0 + L2_SF_GROUP)
            D = A[:, ks] @ B[:, ks].T
            halves.append(s[:, 2 * kb + hh][:, None] * D)
        acc += sw_cols[:, kb][None, :] * (halves[0] + halves[1])
    return acc


def l1_gemm_mx(a_codes, a_sf, w1_packed, w1_e8):
    """L1 with MXFP4 weights: acc[r, n] = sum_kb a_sf[r, kb] * D_kb[r, n].

    D_kb is the dot over K block kb of the decoded activations and the decoded
    weights, each weight already carrying the UE8M0 scale of its 32-wide block
    (the SM100 format, "SM90 design" §2.1, §15.2); the activations keep their
    float32 per-128 scales.  A product of an E4M3 and a scaled E2M1 value is a
    multiple of 2^(s-10) below 2^(s+12) for block exponent s, so the 128
    products of D_kb lie on one grid of 2^(s_min-10) below 2^(s_max+19): D_kb
    is exact in float64 whatever the summation order whenever the four block
    exponents of a 128-wide K block differ by at most 24.  a_codes [m, H],
    a_sf [m, H/128], w1_packed [N, H/2] E2M1 pairs, w1_e8 [N, H/32] UE8M0.
    """
    A = e4m3_decode(a_codes)
    B = mxfp4_decode(w1_packed, w1_e8)
    m, H = A.shape
    acc = np.zeros((m, B.shape[0]), dtype=np.float64)
    a_sf = np.asarray(a_sf, np.float64)
    for kb in range(H // K_BLOCK):
        ks = slice(kb * K_BLOCK, (kb + 1) * K_BLOCK)
        acc += a_sf[:, kb][:, None] * (A[:, ks] @ B[:, ks].T)
    return acc


def l2_gemm_mx(a_codes, a_sf64, w2_packed, w2_e8):
    """L2 with MXFP4 weights: acc[r, n] = sum_kb (s0 * D0 + s1 * D1).

    D0, D1 are the dots over the two 64-wide halves of K block kb of the
    decoded activations and the decoded, block-scaled weights (exact in
    float64 when the two block exponents of a half differ by at most 25, by
    the argument of ``l1_gemm_mx``); s0, s1 the per-64 activation scales.
    There is no separate weight scale.  a_codes [m, I], a_sf64 [m, I/64],
    w2_packed [H, I/2], w2_e8 [H, I/32].
    """
    A = e4m3_decode(a_codes)
    B = mxfp4_decode(w2_packed, w2_e8)
    m, I = A.shape
    acc = np.zeros((m, B.shape[0]), dtype=np.float64)
    s = np.asarray(a_sf64, np.float64)
    for kb in range(I // K_BLOCK):
        halves = []
        for hh in range(2):
            c0 = kb * K_BLOCK + hh * L2_SF_GROUP
            ks = slice(c0, c0 + L2_SF_GROUP)
            halves.append(s[:, 2 * kb + hh][:, None] * (A[:, ks] @ B[:, ks].T))
        acc += halves[0] + halves[1]
    return acc


def expert_rows(a_codes, a_sf, topk_w, w1_codes, w1_sf, w2_codes, w2_sf, clamp=math.inf):
    """The whole per-route expert computation for some rows of one expert.

    Rows are independent, so this serves the full layer (all rows of an
    expert) and sampled checks (any subset) alike.  Returns
    ``l2_acts`` [m, I] uint8, ``l2_acts_sf`` [m, I/64] float32 and
    ``part`` [m, H] uint16 BF16.
    """
    acc1 = l1_gemm(a_codes, a_sf, w1_codes, w1_sf)
    return _rows_after_l1(acc1, topk_w, clamp,
                          lambda codes, sf: l2_gemm(codes, sf, w2_codes, w2_sf))


def expert_rows_mx(a_codes, a_sf, topk_w, w1_packed, w1_e8, w2_packed, w2_e8, clamp=math.inf):
    """``expert_rows`` with MXFP4 weights (same outputs)."""
    acc1 = l1_gemm_mx(a_codes, a_sf, w1_packed, w1_e8)
    return _rows_after_l1(acc1, topk_w, clamp,
                          lambda codes, sf: l2_gemm_mx(codes, sf, w2_packed, w2_e8))


def _rows_after_l1(acc1, topk_w, clamp, l2):
    h = swiglu_weighted(acc1, topk_w, clamp)
    codes, sf = quantize_per64(h)
    acc2 = l2(codes, sf.astype(np.float64))
    part = bf16_rne(f32(acc2))
    return dict(l2_acts=codes, l2_acts_sf=sf, part=part)


def _expert_fn(inp, clamp):
    """(rows of expert e) -> expert_rows result, for either weight format.

    MXFP4 inputs carry ``w1_fp4``, ``w1_e8``, ``w2_fp4``, ``w2_e8``; FP8 inputs
    ``w1``, ``w1_sf``, ``w2``, ``w2_sf``.
    """
    if "w1_fp4" in inp:
        return lambda e, a, a_sf, w: expert_rows_mx(a, a_sf, w, inp["w1_fp4"][e], inp["w1_e8"][e],
                                                    inp["w2_fp4"][e], inp["w2_e8"][e], clamp)
    return lambda e, a, a_sf, w: expert_rows(a, a_sf, w, inp["w1"][e], inp["w1_sf"][e],
                                             inp["w2"][e], inp["w2_sf"][e], clamp)


def _num_experts(inp):
    return (inp["w1_fp4"] if "w1_fp4" in inp else inp["w1"]).shape[0]


# --------------------------------------------------------------------------
# Combine ("SM90 design" §11.2; "PR357 review" §6.3)
# --------------------------------------------------------------------------

def combine(part_by_route, active):
    """y[t] = bf16(sum over active j, ascending, of float32(part[t*k+j])).

    ``part_by_route`` [T*k, H] uint16 (rows of inactive routes are ignored),
    ``active`` [T, k] bool.  Float32 running sum from +0.
    """
    T, k = active.shape
    H = part_by_route.shape[1]
    acc = np.zeros((T, H), dtype=np.float32)
    p = part_by_route.reshape(T, k, H)
    for j in range(k):
        m = active[:, j]
        acc[m] = acc[m] + bf16_to_f32(p[m, j])
    return bf16_rne(acc)


# --------------------------------------------------------------------------
# The whole layer
# --------------------------------------------------------------------------

def forward(inp, clamp=math.inf):
    """Full layer on one GPU's share: all routes local.

    ``inp`` holds x [T,H] uint8, x_sf [T,H/128] f32, topk_idx [T,k] int32,
    topk_weights [T,k] f32 and either FP8 weights w1 [E,2I,H] uint8, w1_sf
    [E,2I/128,H/128] f32, w2 [E,H,I] uint8, w2_sf [E,H/128,I/128] f32 or
    MXFP4 weights w1_fp4 [E,2I,H/2], w1_e8 [E,2I,H/32], w2_fp4 [E,H,I/2],
    w2_e8 [E,H,I/32] (uint8).  Returns every intermediate the layer defines
    plus ``y`` [T,H] uint16 BF16.
    """
    x, x_sf = inp["x"], inp["x_sf"]
    topk_idx, topk_w = inp["topk_idx"], inp["topk_weights"]
    T, H = x.shape
    E = _num_experts(inp)
    I = (inp["w2_fp4"].shape[2] * 2) if "w2_fp4" in inp else inp["w2"].shape[2]
    k = topk_idx.shape[1]
    rows_of = _expert_fn(inp, clamp)
    disp = dispatch(topk_idx, E)
    pool = gather_pool(x, x_sf, topk_w, disp)
    P = disp["src"].shape[0]
    l2_acts = np.zeros((P, I), dtype=np.uint8)
    l2_acts_sf = np.zeros((I // L2_SF_GROUP, P), dtype=np.float32)
    comb = np.zeros((T * k, H), dtype=np.uint16)
    for e in range(E):
        c = int(disp["counts"][e])
        if c == 0:
            continue
        rows = np.arange(disp["offsets"][e], disp["offsets"][e] + c)
        out = rows_of(e, pool["l1_acts"][rows], pool["l1_acts_sf"][:, rows].T, pool["l1_w"][rows])
        l2_acts[rows] = out["l2_acts"]
        l2_acts_sf[:, rows] = out["l2_acts_sf"].T
        comb[disp["src"][rows]] = out["part"]
    y = combine(comb, disp["active"])
    res = dict(disp)
    res.update(pool)
    res.update(l2_acts=l2_acts, l2_acts_sf=l2_acts_sf, comb=comb, y=y)
    return res


def forward_tokens(inp, tokens, clamp=math.inf):
    """``y`` rows of the given tokens only, plus their per-route results.

    Each token's output depends only on its own routes, so a sample of tokens
    can be checked at any size.  Returns dict token -> {"y": [H] uint16,
    "routes": {j: expert_rows result for that single route}}.
    """
    x, x_sf = inp["x"], inp["x_sf"]
    topk_idx, topk_w = inp["topk_idx"], inp["topk_weights"]
    E = _num_experts(inp)
    k = topk_idx.shape[1]
    H = x.shape[1]
    rows_of = _expert_fn(inp, clamp)
    work = {}
    for t in tokens:
        for j in range(k):
            e = int(topk_idx[t, j])
            if 0 <= e < E:
                work.setdefault(e, []).append((int(t), j))
    per_route = {}
    for e, lst in work.items():
        ts = np.array([t for t, _ in lst])
        js = np.array([j for _, j in lst])
        out = rows_of(e, x[ts], x_sf[ts], topk_w[ts, js])
        for n, (t, j) in enumerate(lst):
            per_route[(t, j)] = {key: val[n] for key, val in out.items()}
    result = {}
    for t in tokens:
        t = int(t)
        act = np.array([[0 <= int(topk_idx[t, j]) < E for j in range(k)]])
        part = np.zeros((k, H), dtype=np.uint16)
        for j in range(k):
            if act[0, j]:
                part[j] = per_route[(t, j)]["part"]
        y = combine(part, act)[0]
        result[t] = dict(y=y, routes={j: per_route[(t, j)] for j in range(k) if act[0, j]})
    return result
