"""Pins of the CPU oracle to facts fixed outside it (CPU only).

Each test checks the oracle against something it cannot agree with by
construction: values worked by hand from the pages' equations, exact rational
arithmetic on tiny layers, special cases that reduce to a textbook routine,
invariants of the definition, and the fp32 error bound the guard band claims.
"""

import itertools
import json
import math
import os
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from synth import pack_nibbles, quantize_q4g32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _layer(**kw):
    base = dict(gated=False, w_gate=None, s_gate=None, s_up=None, s_down=None,
                p1=None, p2=None, b_p=None, tau=0.5, act_dtype="f32")
    base.update(kw)
    base.setdefault("d_ffn", np.asarray(base["w_up"]).shape[0])
    return SimpleNamespace(**base)


# ----------------------------------------------------------------------------
# Hand-worked fixtures
# ----------------------------------------------------------------------------

def test_golden_tiny_ffn():
    fx = json.load(open(os.path.join(GOLDEN, "tiny_ffn.json")))
    x_all = np.array(fx["x"], dtype=np.float64)
    for case in fx["cases"]:
        layer = _layer(gated=case["gated"],
                       w_gate=np.array(fx["w_gate"], float) if case["gated"] else None,
                       w_up=np.array(fx["w_up"], float), w_down_t=np.array(fx["w_down_t"], float),
                       b=np.array(fx["b"], float), p1=np.array(fx["p1"], float),
                       p2=np.array(fx["p2"], float), b_p=np.array(fx["b_p"], float),
                       tau=case["tau"])
        x = x_all[case["tokens"]]
        out = oracle.forward(layer, x, case["mode"])
        assert out["idx"].tolist() == case["idx"], case
        assert out["count"] == len(case["idx"])
        assert np.array_equal(out["y64"], np.array(case["y"], dtype=np.float64)), case
        if "z" in case:
            assert np.array_equal(out["z"], np.array(case["z"], dtype=np.float64)), case


def test_golden_int4_decode():
    fx = json.load(open(os.path.join(GOLDEN, "int4_decode.json")))
    q = np.array(fx["bytes"], dtype=np.uint8)
    s = np.array(fx["scales"], dtype=np.float16)
    v = oracle.dequant_q4g32(q, s)
    assert v.shape == (1, 64)
    assert v[0, :6].tolist() == fx["values_head"]
    assert v[0, 32:34].tolist() == fx["values_group1_head"]
    assert v[0, 62:64].tolist() == fx["values_tail"]
    assert np.count_nonzero(v) == 8   # 5 in group 0, 3 in group 1


# ----------------------------------------------------------------------------
# Special cases that reduce to textbook routines (catch transposed operands,
# swapped gate/up, and scatter/gather confusion)
# ----------------------------------------------------------------------------

def _perm_matrix(perm, cols):
    m = np.zeros((len(perm), cols))
    m[np.arange(len(perm)), perm] = 1.0
    return m


@pytest.mark.parametrize("mode", ["exact", "dense"])
def test_selection_up_identity_down(mode):
    rng = np.random.default_rng(5)
    d, n = 12, 9
    sel = rng.permutation(d)[:n]                 # neuron i reads input column sel[i]
    x = rng.standard_normal((3, d))
    layer = _layer(w_up=_perm_matrix(sel, d), w_down_t=np.eye(n, d), b=np.zeros(n))
    y = oracle.forward(layer, x, mode)["y64"]
    expect = np.zeros((3, d))
    expect[:, :n] = np.maximum(x[:, sel], 0.0)   # y_c = relu(x[sel[c]]) for c < n
    assert np.array_equal(y, expect)


def test_identity_up_selection_down():
    rng = np.random.default_rng(6)
    d = n = 10
    perm = rng.permutation(d)
    x = rng.standard_normal((2, d))
    layer = _layer(w_up=np.eye(n, d), w_down_t=_perm_matrix(perm, d), b=np.zeros(n))
    y = oracle.forward(layer, x, "dense")["y64"]
    expect = np.zeros((2, d))
    expect[:, perm] = np.maximum(x, 0.0)         # neuron i writes output column perm[i]
    assert np.array_equal(y, expect)


def test_gated_elementwise_product():
    rng = np.random.default_rng(7)
    d = n = 8
    perm = rng.permutation(d)
    x = rng.standard_normal((4, d))
    bias = rng.standard_normal(n)
    layer = _layer(gated=True, w_gate=np.eye(n, d), w_up=_perm_matrix(perm, d),
                   w_down_t=np.eye(n, d), b=bias)
    y = oracle.forward(layer, x, "dense")["y64"]
    assert np.allclose(y, np.maximum(x + bias, 0.0) * x[:, perm], rtol=0, atol=1e-15)


def test_predictor_selection_case():
    rng = np.random.default_rng(8)
    d, r, n = 9, 6, 5
    s1 = rng.permutation(d)[:r]
    s2 = rng.permutation(r)[:n]
    x = rng.standard_normal((2, d))
    b_p = rng.standard_normal(n)
    z = oracle.predictor_logits(x, _perm_matrix(s1, d), _perm_matrix(s2, r), b_p)
    assert np.array_equal(z, np.maximum(x[:, s1], 0.0)[:, s2] + b_p)


def test_threshold_logit_and_strictness():
    assert oracle.threshold_logit(0.5) == 0.0
    assert math.isclose(oracle.threshold_logit(0.75), math.log(3.0), rel_tol=0, abs_tol=1e-15)
    assert math.isclose(oracle.threshold_logit(0.25), -math.log(3.0), rel_tol=0, abs_tol=1e-15)
    z = np.array([[0.0, -0.0, 1e-300, -1e-300, 5.0]])
    assert oracle.predicted_mask(z, 0.5).tolist() == [[False, False, True, False, True]]
    # sigmoid(z) > tau agrees with the logit test wherever sigmoid is well away from tau
    zz = np.linspace(-8, 8, 161)
    for tau in (0.2, 0.5, 0.9):
        sig = 1.0 / (1.0 + np.exp(-zz))
        far = np.abs(sig - tau) > 1e-9
        assert np.array_equal(oracle.predicted_mask(zz, tau)[far], (sig > tau)[far])


# ----------------------------------------------------------------------------
# Exact rational brute force on tiny layers
# ----------------------------------------------------------------------------

def _dyadic(rng, shape, lo=-8, hi=8, denom=4):
    return rng.integers(lo, hi + 1, size=shape) / denom


def _brute_force(x, wg, wu, wd, b, p1, p2, bp, gated, mode, tau_logit_is_zero=True):
    """Pure-Python Fraction arithmetic straight from the equations."""
    F = Fraction
    n, d = len(wu), len(wu[0])
    r = len(p1)
    ys, masks = [], []
    a_all = []
    for t in range(len(x)):
        xt = [F(v) for v in x[t]]
        g, u = [], []
        for i in range(n):
            gi = sum(xt[k] * F(wg[i][k] if gated else wu[i][k]) for k in range(d)) + F(b[i])
            ui = sum(xt[k] * F(wu[i][k]) for k in range(d)) if gated else F(1)
            g.append(gi)
            u.append(ui)
        a_all.append([max(g[i], F(0)) * u[i] for i in range(n)])
        if mode == "predicted":
            h = [max(sum(xt[k] * F(p1[j][k]) for k in range(d)), F(0)) for j in range(r)]
            z = [sum(h[j] * F(p2[i][j]) for j in range(r)) + F(bp[i]) for i in range(n)]
            masks.append([z[i] > 0 for i in range(n)])
        elif mode == "exact":
            masks.append([g[i] > 0 for i in range(n)])
        else:
            masks.append([True] * n)
    union = [any(m[i] for m in masks) for i in range(n)]
    idx = [i for i in range(n) if union[i]]
    for t in range(len(x)):
        ys.append([sum((a_all[t][i] * F(wd[i][c]) for i in idx), F(0)) for c in range(d)])
    return idx, ys


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("mode", ["predicted", "exact", "dense"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rational_brute_force(gated, mode, seed):
    rng = np.random.default_rng(100 + seed)
    d, n, r, B = 6, 7, 4, 3
    wg = _dyadic(rng, (n, d)) if gated else None
    wu, wd = _dyadic(rng, (n, d)), _dyadic(rng, (n, d))
    b, x = _dyadic(rng, n), _dyadic(rng, (B, d))
    p1, p2, bp = _dyadic(rng, (r, d)), _dyadic(rng, (n, r)), _dyadic(rng, n)
    layer = _layer(gated=gated, w_gate=wg, w_up=wu, w_down_t=wd, b=b, p1=p1, p2=p2, b_p=bp)
    out = oracle.forward(layer, x, mode)
    idx, ys = _brute_force(x.tolist(), None if wg is None else wg.tolist(), wu.tolist(), wd.tolist(),
                           b.tolist(), p1.tolist(), p2.tolist(), bp.tolist(), gated, mode)
    assert out["idx"].tolist() == idx
    assert [[Fraction(v) for v in row] for row in out["y64"]] == ys


# ----------------------------------------------------------------------------
# Invariants of the definition
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("gated", [False, True])
def test_neuron_additivity_all_masks(gated):
    """y(M) = sum_{i in M} y({i}) for every subset M of an 8-neuron layer."""
    rng = np.random.default_rng(11)
    d, n = 5, 8
    layer = _layer(gated=gated, w_gate=_dyadic(rng, (n, d)) if gated else None,
                   w_up=_dyadic(rng, (n, d)), w_down_t=_dyadic(rng, (n, d)), b=_dyadic(rng, n))
    x = _dyadic(rng, (2, d))
    single = [oracle.forward_masked(layer, x, [i])["y64"] for i in range(n)]
    for k in range(n + 1):
        for subset in itertools.combinations(range(n), k):
            y = oracle.forward_masked(layer, x, list(subset))["y64"]
            expect = sum((single[i] for i in subset), np.zeros_like(y))
            assert np.array_equal(y, expect)


def test_zero_mask_gives_positive_zero():
    rng = np.random.default_rng(12)
    layer = _layer(w_up=rng.standard_normal((6, 4)), w_down_t=rng.standard_normal((6, 4)),
                   b=rng.standard_normal(6), act_dtype="f16")
    out = oracle.forward_masked(layer, rng.standard_normal((2, 4)), [])
    assert np.all(out["y"] == 0) and not np.signbit(out["y"]).any()


@pytest.mark.parametrize("gated", [False, True])
def test_exact_relu_support_equals_dense(gated):
    rng = np.random.default_rng(13)
    d, n = 64, 200
    layer = _layer(gated=gated, w_gate=rng.standard_normal((n, d)) if gated else None,
                   w_up=rng.standard_normal((n, d)), w_down_t=rng.standard_normal((n, d)),
                   b=rng.standard_normal(n))
    x = rng.standard_normal((3, d))
    ex = oracle.forward(layer, x, "exact")
    de = oracle.forward(layer, x, "dense")
    assert 0 < ex["count"] < n
    assert np.allclose(ex["y64"], de["y64"], rtol=1e-13, atol=1e-13)
    # neurons outside the support have exactly zero activation
    outside = np.setdiff1d(np.arange(n), ex["idx"])
    assert np.all(ex["a"][:, outside] == 0)


def test_permutation_equivariance():
    rng = np.random.default_rng(14)
    d, n = 16, 40
    wg, wu, wd = (rng.standard_normal((n, d)) for _ in range(3))
    b = rng.standard_normal(n)
    x = rng.standard_normal((2, d))
    perm = rng.permutation(n)
    l1 = _layer(gated=True, w_gate=wg, w_up=wu, w_down_t=wd, b=b)
    l2 = _layer(gated=True, w_gate=wg[perm], w_up=wu[perm], w_down_t=wd[perm], b=b[perm])
    o1, o2 = oracle.forward(l1, x, "exact"), oracle.forward(l2, x, "exact")
    assert o1["count"] == o2["count"]
    assert np.array_equal(np.sort(perm[o2["idx"]]), o1["idx"])
    assert np.allclose(o1["y64"], o2["y64"], rtol=1e-13, atol=1e-13)


def test_batch_union_is_set_union():
    rng = np.random.default_rng(15)
    m = rng.random((5, 300)) < 0.1
    idx, count = oracle.compact(oracle.union_mask(m))
    expect = sorted(set().union(*[set(np.flatnonzero(row).tolist()) for row in m]))
    assert idx.tolist() == expect and count == len(expect)
    assert idx.dtype == np.int32


def test_compact_matches_loop():
    rng = np.random.default_rng(16)
    for n in (0, 1, 63, 64, 65, 1000):
        for dens in (0.0, 0.05, 0.5, 1.0):
            m = rng.random(n) < dens
            idx, count = oracle.compact(m)
            assert idx.tolist() == [i for i in range(n) if m[i]]
            assert count == int(sum(bool(v) for v in m))


# ----------------------------------------------------------------------------
# int4 decoding
# ----------------------------------------------------------------------------

def test_int4_roundtrip_with_encoder():
    rng = np.random.default_rng(17)
    q = rng.integers(-8, 8, size=(5, 128))
    packed = pack_nibbles(q)
    assert packed.shape == (5, 64) and packed.dtype == np.uint8
    dec = oracle.dequant_q4g32(packed, np.ones((5, 4), dtype=np.float16))
    assert np.array_equal(dec, q.astype(np.float64))


def test_int4_quantizer_error_bound():
    rng = np.random.default_rng(18)
    w = (rng.standard_normal((7, 256)) / 16).astype(np.float32)
    packed, s = quantize_q4g32(w)
    dec = oracle.dequant_q4g32(packed, s)
    step = np.repeat(s.astype(np.float64), 32, axis=1)
    # |w - q s| <= s/2 plus the fp16 rounding of s times |q| <= 8
    assert np.all(np.abs(dec - w) <= step * (0.5 + 8 * 2.0 ** -11) + 1e-12)


# ----------------------------------------------------------------------------
# The guard band bounds real fp32 evaluations
# ----------------------------------------------------------------------------

def _f32_sequential(x, w, b):
    acc = np.zeros((x.shape[0], w.shape[0]), dtype=np.float32)
    x32, w32 = x.astype(np.float32), w.astype(np.float32)
    for k in range(x.shape[1]):
        acc = acc + x32[:, k:k + 1] * w32[:, k][None, :]
    return acc + b.astype(np.float32)


def test_guard_band_bounds_fp32_exact():
    rng = np.random.default_rng(19)
    d, n = 512, 300
    w = (rng.standard_normal((n, d)) / math.sqrt(d)).astype(np.float16)
    b = rng.standard_normal(n).astype(np.float32)
    x = rng.standard_normal((4, d)).astype(np.float16)
    g64 = x.astype(np.float64) @ w.astype(np.float64).T + b
    band = oracle.guard_band_exact(x, w, b)
    for g32 in (_f32_sequential(x, w, b),
                x.astype(np.float32) @ w.astype(np.float32).T + b):
        assert np.all(np.abs(g32.astype(np.float64) - g64) <= band / oracle.GUARD_SAFETY)


def test_guard_band_bounds_fp32_predictor():
    rng = np.random.default_rng(20)
    d, r, n = 256, 64, 400
    p1 = (rng.standard_normal((r, d)) / math.sqrt(d)).astype(np.float16)
    p2 = (rng.standard_normal((n, r)) / math.sqrt(r)).astype(np.float16)
    b_p = rng.standard_normal(n).astype(np.float32)
    x = rng.standard_normal((3, d)).astype(np.float16)
    z64 = oracle.predictor_logits(x, p1, p2, b_p)
    h32 = np.maximum(_f32_sequential(x, p1, np.zeros(r)), 0).astype(np.float32)
    z32 = _f32_sequential(h32, p2, b_p)
    band = oracle.guard_band_predictor(x, p1, p2, b_p)
    assert np.all(np.abs(z32.astype(np.float64) - z64) <= band / oracle.GUARD_SAFETY)


def test_certain_union():
    v = np.array([[1.0, -1.0, 0.1, -0.1], [-1.0, -1.0, -0.1, -0.05]])
    band = np.full_like(v, 0.2)
    on, off = oracle.certain_union(v, band)
    assert on.tolist() == [True, False, False, False]
    assert off.tolist() == [False, True, False, False]


def test_round_to_act_is_round_half_even():
    # 2049 lies halfway between the fp16 neighbours 2048 and 2050; ties go to even (2048)
    y = oracle.round_to_act(np.array([2049.0, 2051.0, 1.0 + 2.0 ** -11]), "f16")
    assert y.tolist() == [2048.0, 2052.0, 1.0]


# ----------------------------------------------------------------------------
# forward_masked: the sparse operator on a given list, pinned on its own
# ----------------------------------------------------------------------------

def test_forward_masked_golden_lists():
    """Each hand-worked case's list through forward_masked gives the hand-worked y."""
    fx = json.load(open(os.path.join(GOLDEN, "tiny_ffn.json")))
    x_all = np.array(fx["x"], dtype=np.float64)
    for case in fx["cases"]:
        layer = _layer(gated=case["gated"],
                       w_gate=np.array(fx["w_gate"], float) if case["gated"] else None,
                       w_up=np.array(fx["w_up"], float), w_down_t=np.array(fx["w_down_t"], float),
                       b=np.array(fx["b"], float), tau=case["tau"])
        out = oracle.forward_masked(layer, x_all[case["tokens"]], case["idx"])
        assert np.array_equal(out["y64"], np.array(case["y"], dtype=np.float64)), case


def _nibble_values(packed_row):
    """Signed int4 values of one packed row, decoded from the format statement in the test."""
    vals = []
    for byte in packed_row:
        for nib in (int(byte) & 0xF, int(byte) >> 4):      # low nibble first: the even element
            vals.append(nib - 16 if nib >= 8 else nib)
    return vals


def _brute_masked(x, wg, wu, wd, b, gated, idx):
    """y_t = sum over the listed neurons of ReLU(g) u W_downT, in Fraction arithmetic."""
    F = Fraction
    ys = []
    for xt in x:
        xt = [F(v) for v in xt]
        y = [F(0)] * len(wd[0])
        for i in idx:
            pre = wg[i] if gated else wu[i]
            g = sum(xt[k] * pre[k] for k in range(len(xt))) + F(b[i])
            u = sum(xt[k] * wu[i][k] for k in range(len(xt))) if gated else F(1)
            a = max(g, F(0)) * u
            y = [y[c] + a * wd[i][c] for c in range(len(y))]
        ys.append(y)
    return ys


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_forward_masked_rational_subsets(gated, seed):
    rng = np.random.default_rng(300 + seed)
    d, n, B = 6, 9, 2
    wg = _dyadic(rng, (n, d)) if gated else None
    wu, wd, b, x = _dyadic(rng, (n, d)), _dyadic(rng, (n, d)), _dyadic(rng, n), _dyadic(rng, (B, d))
    layer = _layer(gated=gated, w_gate=wg, w_up=wu, w_down_t=wd, b=b)
    F = Fraction
    fr = (lambda m: [[F(v) for v in row] for row in m.tolist()])
    for k in (0, 1, 3, n):
        for _ in range(3):
            idx = sorted(rng.choice(n, size=k, replace=False).tolist())
            got = oracle.forward_masked(layer, x, idx)["y64"]
            ref = _brute_masked(x.tolist(), None if wg is None else fr(wg), fr(wu), fr(wd), b.tolist(), gated, idx)
            assert [[F(v) for v in row] for row in got] == ref, idx


@pytest.mark.parametrize("gated", [False, True])
def test_forward_masked_int4_distinct_scales(gated):
    """int4 rows with different scales per matrix and per group: a swap of the gate and up rows,
    of their scales, or a bias on u instead of g changes y."""
    rng = np.random.default_rng(310 + int(gated))
    d, n, B = 64, 6, 2
    mats, scales = [], []
    for m in range(3):
        q = rng.integers(-8, 8, size=(n, d))
        s = (np.float16(2.0) ** rng.integers(-3, 2, size=(n, d // 32))).astype(np.float16) * np.float16(1 + m)
        mats.append(pack_nibbles(q))
        scales.append(s)
    b = _dyadic(rng, n)
    x = _dyadic(rng, (B, d))
    layer = _layer(gated=gated, w_gate=mats[0] if gated else None, s_gate=scales[0] if gated else None,
                   w_up=mats[1], s_up=scales[1], w_down_t=mats[2], s_down=scales[2], b=b, d_ffn=n)
    F = Fraction

    def rows(m):
        out = []
        for i in range(n):
            vals = _nibble_values(mats[m][i])
            out.append([F(v) * F(float(scales[m][i][k // 32])) for k, v in enumerate(vals)])
        return out

    wg, wu, wd = rows(0) if gated else None, rows(1), rows(2)
    for idx in ([0], [1, 4], list(range(n))):
        got = oracle.forward_masked(layer, x, idx)["y64"]
        ref = _brute_masked(x.tolist(), wg, wu, wd, b.tolist(), gated, idx)
        assert [[F(v) for v in row] for row in got] == ref, idx
    # and it agrees with forward() on forward()'s own list
    for mode in ("exact", "dense"):
        full = oracle.forward(layer, x, mode)
        assert np.array_equal(oracle.forward_masked(layer, x, full["idx"])["y64"], full["y64"])


def test_forward_masked_matches_forward_on_its_list():
    rng = np.random.default_rng(320)
    d, n, r = 32, 40, 8
    for gated in (False, True):
        layer = _layer(gated=gated, w_gate=_dyadic(rng, (n, d)) if gated else None, w_up=_dyadic(rng, (n, d)),
                       w_down_t=_dyadic(rng, (n, d)), b=_dyadic(rng, n), p1=_dyadic(rng, (r, d)),
                       p2=_dyadic(rng, (n, r)), b_p=_dyadic(rng, n))
        x = _dyadic(rng, (3, d))
        for mode in ("predicted", "exact", "dense"):
            full = oracle.forward(layer, x, mode)
            assert np.array_equal(oracle.forward_masked(layer, x, full["idx"])["y64"], full["y64"]), (gated, mode)


# ----------------------------------------------------------------------------
# The probabilistic bands bound real fp32 evaluations in several orders, and are
# tighter than the rigorous ones
# ----------------------------------------------------------------------------

def _f32_orders(x, w, b, rng):
    """fp32 evaluations of x w^T + b: sequential, reversed, a random order, and BLAS's own."""
    k = x.shape[1]
    out = [_f32_sequential(x, w, b), _f32_sequential(x[:, ::-1], w[:, ::-1], b)]
    perm = rng.permutation(k)
    out.append(_f32_sequential(x[:, perm], w[:, perm], b))
    out.append(x.astype(np.float32) @ w.astype(np.float32).T + b.astype(np.float32))
    return out


def test_prob_band_bounds_fp32_exact():
    rng = np.random.default_rng(21)
    d, n = 2048, 200
    w = (rng.standard_normal((n, d)) / math.sqrt(d)).astype(np.float16)
    b = rng.standard_normal(n).astype(np.float32)
    x = rng.standard_normal((3, d)).astype(np.float16)
    g64 = x.astype(np.float64) @ w.astype(np.float64).T + b
    band = oracle.prob_band_exact(x, w, b)
    assert np.all(band <= oracle.guard_band_exact(x, w, b) / oracle.GUARD_SAFETY)
    worst = 0.0
    for g32 in _f32_orders(x, w, b, rng):
        err = np.abs(g32.astype(np.float64) - g64)
        assert np.all(err <= band)
        worst = max(worst, float((err / band).max()))
    assert worst > 1e-4   # the errors are real, not zero: the check has something to bound


def test_prob_band_bounds_fp32_predictor():
    rng = np.random.default_rng(22)
    d, r, n = 1024, 128, 300
    p1 = (rng.standard_normal((r, d)) / math.sqrt(d)).astype(np.float16)
    p2 = (rng.standard_normal((n, r)) / math.sqrt(r)).astype(np.float16)
    b_p = rng.standard_normal(n).astype(np.float32)
    x = rng.standard_normal((2, d)).astype(np.float16)
    z64 = oracle.predictor_logits(x, p1, p2, b_p)
    band = oracle.prob_band_predictor(x, p1, p2, b_p)
    assert np.all(band <= oracle.guard_band_predictor(x, p1, p2, b_p) / oracle.GUARD_SAFETY)
    zero = np.zeros(r, dtype=np.float32)
    for h32 in _f32_orders(x, p1, zero, rng):
        h32 = np.maximum(h32, 0).astype(np.float32)
        for z32 in _f32_orders(h32, p2, b_p, rng):
            assert np.all(np.abs(z32.astype(np.float64) - z64) <= band)



# ----------------------------------------------------------------------------
# Hot set (predicted mode with always-computed neurons)
# ----------------------------------------------------------------------------

def test_hot_set_golden():
    """The hand-worked layer of tests/golden/tiny_ffn.json, token 0, tau = 0.5: the predictor alone
    selects {0}; a hot set {1} adds neuron 1, whose g = -1 < 0 contributes 0, so y is unchanged; a
    hot set {2} adds neuron 2 (a = ReLU(1) * 3 = 3, down row [0, 1, 0, -1]): y = [-3, 3, 0, -9]."""
    fx = json.load(open(os.path.join(GOLDEN, "tiny_ffn.json")))
    layer = _layer(gated=True, w_gate=np.array(fx["w_gate"], float), w_up=np.array(fx["w_up"], float),
                   w_down_t=np.array(fx["w_down_t"], float), b=np.array(fx["b"], float),
                   p1=np.array(fx["p1"], float), p2=np.array(fx["p2"], float), b_p=np.array(fx["b_p"], float))
    x = np.array(fx["x"], float)[[0]]
    for hot, idx, y in ((None, [0], [-3, 0, 0, -6]), ([0], [0], [-3, 0, 0, -6]), ([1], [0, 1], [-3, 0, 0, -6]),
                        ([2], [0, 2], [-3, 3, 0, -9]), ([0, 1, 2], [0, 1, 2], [-3, 3, 0, -9])):
        out = oracle.forward(layer, x, "predicted", hot=hot)
        assert out["idx"].tolist() == idx and out["y64"].tolist() == [y], hot


@pytest.mark.parametrize("gated", [False, True])
def test_hot_set_limits_and_brute_force(gated):
    """An empty hot set is the predicted mode; every neuron hot is the dense mode; in between the
    list is the hot set joined with the predictor's choice, checked in Fraction arithmetic on a
    dyadic layer (as an id list and as a boolean mask)."""
    rng = np.random.default_rng(400 + int(gated))
    d, n, r, B = 6, 9, 4, 2
    wg = _dyadic(rng, (n, d)) if gated else None
    wu, wd, b, x = _dyadic(rng, (n, d)), _dyadic(rng, (n, d)), _dyadic(rng, n), _dyadic(rng, (B, d))
    p1, p2, bp = _dyadic(rng, (r, d)), _dyadic(rng, (n, r)), _dyadic(rng, n)
    layer = _layer(gated=gated, w_gate=wg, w_up=wu, w_down_t=wd, b=b, p1=p1, p2=p2, b_p=bp)
    pred = oracle.forward(layer, x, "predicted")
    assert np.array_equal(oracle.forward(layer, x, "predicted", hot=[])["y64"], pred["y64"])
    dense = oracle.forward(layer, x, "dense")
    full = oracle.forward(layer, x, "predicted", hot=np.ones(n, dtype=bool))
    assert full["idx"].tolist() == list(range(n)) and np.array_equal(full["y64"], dense["y64"])
    F = Fraction
    fr = (lambda m: [[F(v) for v in row] for row in m.tolist()])
    for hot in ([3], [0, 5, 8], [1, 2, 4, 6, 7]):
        out = oracle.forward(layer, x, "predicted", hot=hot)
        as_mask = np.zeros(n, dtype=bool)
        as_mask[hot] = True
        assert np.array_equal(oracle.forward(layer, x, "predicted", hot=as_mask)["idx"], out["idx"])
        expect = sorted(set(hot) | set(pred["idx"].tolist()))
        assert out["idx"].tolist() == expect
        ref = _brute_masked(x.tolist(), None if wg is None else fr(wg), fr(wu), fr(wd), b.tolist(), gated, expect)
        assert [[F(v) for v in row] for row in out["y64"]] == ref
