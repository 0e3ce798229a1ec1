"""Pins of the oracle's layer arithmetic (CPU only).

The oracle follows "MegaMoE SM90 Implementation Design (Final)": the L1 GEMM
with per-128 block scales (§5.3), SwiGLU times the top-k weight and per-64 FP8
re-quantisation (§10.1), the gate/up interleave (§15.1), the L2 GEMM with
per-64 activation scales (§5.4), the BF16 partial cast (§11.1) and the FP32
combine (§11.2).  Each is tied here to something other than the oracle:

* an exact-rational brute force of the whole layer (integers, Fractions and
  60-digit Decimal exp), bit-exact on a tiny case;
* exactness of the raw block dots, the library matmul with unit scales, and a
  dequantise-then-matmul second form;
* a closed form for SwiGLU and the re-quantisation (one-hot weights);
* the interleave against a de-interleaved gate/up computation;
* metamorphic relations (power-of-two scalings, token permutation, expert
  relabelling, k = 1), and the summation order of the combine.
"""

import decimal
import math
from fractions import Fraction

import numpy as np
import pytest

from fp8_mixture_experts_amd import synthetic as S
from oracle import codecs, moe
from tests import exact

decimal.getcontext().prec = 60


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    c = np.where((c & 0x7F) == 0x7F, 0x38, c)      # no NaN codes
    return c.astype(np.uint8)


# --------------------------------------------------------------------------
# Exact brute force of the whole layer
# --------------------------------------------------------------------------

def _dec(fr: Fraction) -> decimal.Decimal:
    return decimal.Decimal(fr.numerator) / decimal.Decimal(fr.denominator)


def brute_layer(inp, clamp=None):
    x, x_sf = inp["x"], inp["x_sf"]
    idx, tw = inp["topk_idx"], inp["topk_weights"]
    w1, w1_sf, w2, w2_sf = inp["w1"], inp["w1_sf"], inp["w2"], inp["w2_sf"]
    T, H = x.shape
    E, N, _ = w1.shape
    I = N // 2
    k = idx.shape[1]
    xi = [[exact.e4m3_int9(int(c)) for c in row] for row in x]
    routes = {}
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if not 0 <= e < E:
                continue
            w1i = [[exact.e4m3_int9(int(c)) for c in row] for row in w1[e]]
            acc = []
            for n in range(N):
                s = Fraction(0)
                for kb in range(H // 128):
                    d = sum(xi[t][c] * w1i[n][c] for c in range(kb * 128, kb * 128 + 128))
                    s += Fraction(float(x_sf[t, kb])) * Fraction(float(w1_sf[e, n // 128, kb])) \
                        * Fraction(d, 2 ** 18)
                acc.append(s)
            h = []
            for i in range(I):
                g = acc[16 * (i // 8) + i % 8]
                u = acc[16 * (i // 8) + 8 + i % 8]
                if clamp is not None:
                    c = Fraction(clamp)
                    g = max(-c, min(c, g))
                    u = max(-c, min(c, u))
                gd = _dec(g)
                silu = gd / (1 + (-gd).exp())
                h.append(Fraction(silu * _dec(u) * _dec(Fraction(float(tw[t, j])))))
            codes, sfs = [], []
            for grp in range(I // 64):
                hs = h[64 * grp: 64 * grp + 64]
                amax = max(abs(v) for v in hs)
                sf = exact.to_f32_value(amax / 448)
                sfs.append(sf)
                for v in hs:
                    # a zero scale (amax = 0, or amax / 448 below the smallest
                    # float32) gives the code +0 for every value of the group
                    q = v / sf if sf != 0 else Fraction(0)
                    codes.append(exact.e4m3_code_of_value(exact.to_e4m3_value(q),
                                                          negative_zero=(v < 0 and sf != 0)))
            ci = [exact.e4m3_int9(c) for c in codes]
            w2i = [[exact.e4m3_int9(int(c)) for c in row] for row in w2[e]]
            part = []
            for n in range(H):
                s = Fraction(0)
                for kb in range(I // 128):
                    halves = Fraction(0)
                    for hh in range(2):
                        c0 = kb * 128 + 64 * hh
                        d = sum(ci[c] * w2i[n][c] for c in range(c0, c0 + 64))
                        halves += sfs[2 * kb + hh] * Fraction(d, 2 ** 18)
                    s += Fraction(float(w2_sf[e, n // 128, kb])) * halves
                part.append(exact.to_bf16_value(exact.to_f32_value(s)))
            routes[(t, j)] = dict(codes=codes, sf=sfs, part=part)
    y = []
    for t in range(T):
        row = []
        for n in range(H):
            acc = Fraction(0)
            for j in range(k):
                if (t, j) in routes:
                    acc = exact.to_f32_value(acc + routes[(t, j)]["part"][n])
            row.append(exact.to_bf16_value(acc))
        y.append(row)
    return routes, y


@pytest.mark.slow
def test_layer_matches_exact_brute_force():
    wl = S.custom(tokens=4, hidden=128, intermediate=128, experts=2, topk=2, seed=11,
                  weight_seed=12, weight_std=0.05)
    inp = S.make_inputs(wl)
    inp["topk_idx"][3, 1] = -1                     # one inactive slot
    out = moe.forward(inp)
    routes, y = brute_layer(inp)
    for (t, j), r in routes.items():
        s = out["slot_map"][t, j]
        assert list(out["l2_acts"][s]) == r["codes"]
        assert [Fraction(float(v)) for v in out["l2_acts_sf"][:, s]] == r["sf"]
        got = codecs.bf16_to_f32(out["comb"][t * 2 + j])
        assert [Fraction(float(v)) for v in got] == r["part"]
    yf = codecs.bf16_to_f32(out["y"])
    for t in range(4):
        assert [Fraction(float(v)) for v in yf[t]] == y[t]


@pytest.mark.slow
def test_layer_with_activation_clamp_matches_exact_brute_force():
    """The clamp (0.25, below most |gate| and |up| of these inputs) in the
    float64 oracle against the exact layer with the clamp applied in rationals."""
    wl = S.custom(tokens=3, hidden=128, intermediate=128, experts=2, topk=2, seed=21,
                  weight_seed=22, weight_std=0.05)
    inp = S.make_inputs(wl)
    clamp = 0.25
    acc = moe.l1_gemm(inp["x"][:1], inp["x_sf"][:1], inp["w1"][int(inp["topk_idx"][0, 0])],
                      inp["w1_sf"][int(inp["topk_idx"][0, 0])])
    assert np.mean(np.abs(acc) > clamp) > 0.3          # the clamp really bites
    out = moe.forward(inp, clamp=clamp)
    routes, y = brute_layer(inp, clamp=clamp)
    for (t, j), r in routes.items():
        s = out["slot_map"][t, j]
        assert list(out["l2_acts"][s]) == r["codes"]
        assert [Fraction(float(v)) for v in out["l2_acts_sf"][:, s]] == r["sf"]
    yf = codecs.bf16_to_f32(out["y"])
    for t in range(3):
        assert [Fraction(float(v)) for v in yf[t]] == y[t]


@pytest.mark.slow
def test_layer_with_subnormal_topk_weights_matches_exact_brute_force():
    """Top-k weights in float32's subnormal range (an underflowed softmax):
    1e-40 gives scales amax / 448 that are themselves subnormal, 1e-45 (the
    smallest subnormal) scales that round to zero.  The float64 oracle must
    still agree bit for bit with the exact layer."""
    wl = S.custom(tokens=3, hidden=128, intermediate=128, experts=2, topk=2, seed=31,
                  weight_seed=32, weight_std=0.05)
    inp = S.make_inputs(wl)
    inp["topk_weights"][0, 1] = np.float32(1e-40)
    inp["topk_weights"][2, 0] = np.float32(1e-45)
    out = moe.forward(inp)
    routes, y = brute_layer(inp)
    s01 = out["l2_acts_sf"][:, out["slot_map"][0, 1]]
    assert np.all((s01 > 0) & (s01 < np.float32(2.0 ** -126)))     # subnormal scales
    assert np.all(out["l2_acts_sf"][:, out["slot_map"][2, 0]] == 0)  # scales round to zero
    for (t, j), r in routes.items():
        s = out["slot_map"][t, j]
        assert list(out["l2_acts"][s]) == r["codes"], (t, j)
        assert [Fraction(float(v)) for v in out["l2_acts_sf"][:, s]] == r["sf"], (t, j)
    yf = codecs.bf16_to_f32(out["y"])
    for t in range(3):
        assert [Fraction(float(v)) for v in yf[t]] == y[t]


def test_clamp_at_or_above_every_value_changes_nothing():
    rng = np.random.default_rng(31)
    acc = rng.normal(0, 3, (5, 256))
    w = rng.uniform(0.1, 1, 5)
    ref = moe.swiglu_weighted(acc, w)
    assert np.array_equal(moe.swiglu_weighted(acc, w, clamp=float(np.abs(acc).max())), ref)
    assert np.array_equal(moe.swiglu_weighted(acc, w, clamp=1e30), ref)


def test_saturated_clamp_gives_four_values():
    """Every gate and up beyond +-c: h / w takes only +-c*s(c) and +-c*s(-c),
    with the logistic s computed here through tanh."""
    rng = np.random.default_rng(32)
    c = 1.5
    acc = rng.choice([-1, 1], (4, 256)) * rng.uniform(2.0, 9.0, (4, 256))
    w = rng.uniform(0.1, 1, 4)
    h = moe.swiglu_weighted(acc, w, clamp=c) / w[:, None]
    sig = lambda v: 0.5 * (1.0 + math.tanh(v / 2.0))
    pos, neg = c * sig(c), -c * sig(-c)       # silu(c), silu(-c)
    want = {round(v, 12) for v in (pos * c, -pos * c, neg * c, -neg * c)}
    assert {round(v, 12) for v in h.ravel()} <= want
    # gate > c and up > c gives silu(c) * c
    sel = (acc[:, 0:8] > 0) & (acc[:, 8:16] > 0)
    assert np.allclose(h[:, 0:8][sel], pos * c, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# GEMM exactness and second forms
# --------------------------------------------------------------------------

def test_raw_block_dot_is_exact():
    rng = np.random.default_rng(5)
    a = _rand_codes(rng, (3, 128))
    w = _rand_codes(rng, (128, 128))
    acc = moe.l1_gemm(a, np.ones((3, 1), np.float32), w, np.ones((1, 1), np.float32))
    for r in range(3):
        for n in range(0, 128, 17):
            want = sum(exact.e4m3_value_of_code(int(a[r, c])) *
                       exact.e4m3_value_of_code(int(w[n, c])) for c in range(128))
            assert Fraction(acc[r, n]) == want


def test_unit_scales_reduce_to_library_matmul():
    rng = np.random.default_rng(6)
    a = _rand_codes(rng, (5, 512))
    w1 = _rand_codes(rng, (256, 512))
    acc = moe.l1_gemm(a, np.ones((5, 4), np.float32), w1, np.ones((2, 4), np.float32))
    assert np.array_equal(acc, codecs.e4m3_decode(a) @ codecs.e4m3_decode(w1).T)
    w2 = _rand_codes(rng, (256, 512))
    acc2 = moe.l2_gemm(a, np.ones((5, 8)), w2, np.ones((2, 4), np.float32))
    assert np.array_equal(acc2, codecs.e4m3_decode(a) @ codecs.e4m3_decode(w2).T)


def test_scaled_gemms_match_dequantise_then_matmul():
    rng = np.random.default_rng(7)
    m, H, N, I = 6, 384, 256, 256
    a = _rand_codes(rng, (m, H))
    asf = rng.uniform(0.01, 2, (m, H // 128)).astype(np.float32)
    w = _rand_codes(rng, (N, H))
    wsf = rng.uniform(0.01, 2, (N // 128, H // 128)).astype(np.float32)
    deq_a = codecs.e4m3_decode(a) * np.repeat(asf.astype(np.float64), 128, axis=1)
    deq_w = codecs.e4m3_decode(w) * np.repeat(np.repeat(wsf.astype(np.float64), 128, 0), 128, 1)
    ref = deq_a @ deq_w.T
    got = moe.l1_gemm(a, asf, w, wsf)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    # L2 form: per-64 activation scales
    a2 = _rand_codes(rng, (m, I))
    s64 = rng.uniform(0.01, 2, (m, I // 64))
    w2 = _rand_codes(rng, (N, I))
    w2sf = rng.uniform(0.01, 2, (N // 128, I // 128)).astype(np.float32)
    deq_a2 = codecs.e4m3_decode(a2) * np.repeat(s64, 64, axis=1)
    deq_w2 = codecs.e4m3_decode(w2) * np.repeat(np.repeat(w2sf.astype(np.float64), 128, 0), 128, 1)
    ref2 = deq_a2 @ deq_w2.T
    got2 = moe.l2_gemm(a2, s64, w2, w2sf)
    assert np.max(np.abs(got2 - ref2)) <= 1e-12 * np.max(np.abs(ref2))


# --------------------------------------------------------------------------
# Interleave, SwiGLU and re-quantisation
# --------------------------------------------------------------------------

def _interleave_rows(gate, up):
    """Stored row r holds gate row 8*(r//16) + r%16 when r%16 < 8, else the up
    row 8*(r//16) + r%16 - 8 (granularity-8 interleave, SM90 design §15.1)."""
    I = gate.shape[0]
    r = np.arange(2 * I)
    src = 8 * (r // 16) + (r % 16) % 8
    is_up = (r % 16) >= 8
    return np.where(is_up[:, None], up[src], gate[src])


def test_interleaved_swiglu_equals_deinterleaved_formula():
    rng = np.random.default_rng(8)
    I, H, m = 128, 256, 4
    gate = _rand_codes(rng, (I, H))
    up = _rand_codes(rng, (I, H))
    a = _rand_codes(rng, (m, H))
    w = rng.uniform(0.1, 1, m)
    acc = moe.l1_gemm(a, np.ones((m, 2), np.float32), _interleave_rows(gate, up),
                      np.ones((2, 2), np.float32))
    h = moe.swiglu_weighted(acc, w)
    A = codecs.e4m3_decode(a)
    G = A @ codecs.e4m3_decode(gate).T
    U = A @ codecs.e4m3_decode(up).T
    with np.errstate(over="ignore"):
        ref = G / (1 + np.exp(-G)) * U * w[:, None]
    assert np.array_equal(h, ref)


def test_swiglu_quant_closed_form_with_one_hot_weights():
    """W1 gate and up rows of output i both pick channel c_i with code 1.0 and
    unit scales, so h_i = silu(v) * v * w with v = q(x[c_i]) * x_sf."""
    rng = np.random.default_rng(9)
    H, I = 256, 128
    x = _rand_codes(rng, (1, H))
    x[0, :] = np.where(np.abs(codecs.e4m3_decode(x[0])) > 8, 0x3C, x[0])  # keep |v| modest
    xsf = np.array([[0.75, 1.5]], np.float32)
    ch = rng.permutation(H)[:I]
    gate = np.zeros((I, H), np.uint8)
    gate[np.arange(I), ch] = 0x38                  # code of 1.0
    w1 = _interleave_rows(gate, gate)
    w = np.float32(0.3)
    out = moe.expert_rows(x, xsf, np.array([w]), w1, np.ones((2, 2), np.float32),
                          np.zeros((H, I), np.uint8), np.ones((2, 1), np.float32))
    hs = []
    for i in range(I):
        v = exact.e4m3_value_of_code(int(x[0, ch[i]])) * Fraction(float(xsf[0, ch[i] // 128]))
        vd = _dec(v)
        hs.append(Fraction(vd / (1 + (-vd).exp()) * vd * _dec(Fraction(float(w)))))
    for grp in range(I // 64):
        g = hs[64 * grp: 64 * grp + 64]
        sf = exact.to_f32_value(max(abs(v) for v in g) / 448)
        assert Fraction(float(out["l2_acts_sf"][0, grp])) == sf
        want = [exact.e4m3_code_of_value(exact.to_e4m3_value(v / sf), v < 0) for v in g]
        assert list(out["l2_acts"][0, 64 * grp: 64 * grp + 64]) == want
    assert np.all(out["part"] == 0)                # W2 = 0 -> zero partials


def test_quantize_all_zero_group():
    h = np.zeros((2, 128))
    h[1, 64:] = np.linspace(-1, 1, 64)
    codes, sf = moe.quantize_per64(h)
    assert sf[0, 0] == 0 and sf[0, 1] == 0 and sf[1, 0] == 0
    assert np.all(codes[0] == 0) and np.all(codes[1, :64] == 0)
    assert sf[1, 1] == np.float32(1 / 448)
    assert codes[1, 64] == 0xFE and codes[1, 127] == 0x7E    # +/-amax -> +/-448


# --------------------------------------------------------------------------
# Metamorphic relations on the whole layer
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def small():
    wl = S.custom(tokens=24, hidden=256, intermediate=256, experts=4, topk=3, seed=21,
                  weight_seed=22)
    inp = S.make_inputs(wl)
    return inp, moe.forward(inp)


def test_topk_weight_power_of_two_scales_only_sf(small):
    inp, base = small
    for m in (3, -2):
        inp2 = dict(inp, topk_weights=(inp["topk_weights"] * np.float32(2.0 ** m)))
        out = moe.forward(inp2)
        assert np.array_equal(out["l2_acts"], base["l2_acts"])
        assert np.array_equal(out["l2_acts_sf"], base["l2_acts_sf"] * np.float32(2.0 ** m))
        assert np.array_equal(codecs.bf16_to_f32(out["y"]),
                              codecs.bf16_to_f32(base["y"]) * np.float32(2.0 ** m))


def test_w2_scale_power_of_two_scales_output(small):
    inp, base = small
    inp2 = dict(inp, w2_sf=inp["w2_sf"] * np.float32(4.0))
    out = moe.forward(inp2)
    assert np.array_equal(out["l2_acts"], base["l2_acts"])
    assert np.array_equal(codecs.bf16_to_f32(out["comb"]), codecs.bf16_to_f32(base["comb"]) * 4)
    assert np.array_equal(codecs.bf16_to_f32(out["y"]), codecs.bf16_to_f32(base["y"]) * 4)


def test_token_permutation_permutes_output(small):
    inp, base = small
    perm = np.random.default_rng(1).permutation(24)
    inp2 = dict(inp, x=inp["x"][perm], x_sf=inp["x_sf"][perm],
                topk_idx=inp["topk_idx"][perm], topk_weights=inp["topk_weights"][perm])
    out = moe.forward(inp2)
    assert np.array_equal(out["y"], base["y"][perm])


def test_expert_relabelling_leaves_output(small):
    inp, base = small
    pi = np.array([2, 0, 3, 1])
    inv = np.argsort(pi)
    inp2 = dict(inp, topk_idx=pi[inp["topk_idx"]].astype(np.int32),
                w1=inp["w1"][inv], w1_sf=inp["w1_sf"][inv],
                w2=inp["w2"][inv], w2_sf=inp["w2_sf"][inv])
    out = moe.forward(inp2)
    assert np.array_equal(out["y"], base["y"])


def test_single_slot_output_is_the_partial(small):
    inp, _ = small
    inp2 = dict(inp, topk_idx=inp["topk_idx"][:, :1].copy(),
                topk_weights=np.ones((24, 1), np.float32))
    out = moe.forward(inp2)
    assert np.array_equal(out["y"], out["comb"])


def test_sampled_tokens_match_full_forward(small):
    inp, base = small
    got = moe.forward_tokens(inp, [0, 5, 23])
    for t, r in got.items():
        assert np.array_equal(r["y"], base["y"][t])
        for j, rr in r["routes"].items():
            s = base["slot_map"][t, j]
            assert np.array_equal(rr["l2_acts"], base["l2_acts"][s])
            assert np.array_equal(rr["part"], base["comb"][t * 3 + j])


def test_combine_sums_in_ascending_slot_order():
    # float32 running sum of [1, 2^-8, 2^-24, 2^-24] stays 1 + 2^-8 (each
    # 2^-24 is a tie that rounds to even), whose BF16 tie rounds to 1.0; the
    # reverse order accumulates 2^-23 first and gives 1 + 2^-7.
    vals = np.float32([1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24])
    part = codecs.bf16_rne(vals)[None, :, None].repeat(1, 2).reshape(4, 1)
    assert np.array_equal(codecs.bf16_to_f32(part[:, 0]), vals)
    y = moe.combine(part, np.ones((1, 4), bool))
    assert y[0, 0] == 0x3F80
    y_rev = moe.combine(part[::-1].copy(), np.ones((1, 4), bool))
    assert y_rev[0, 0] == 0x3F81
    # inactive slots are skipped; a token with none gets +0
    y0 = moe.combine(part, np.zeros((1, 4), bool))
    assert y0[0, 0] == 0
