"""The seeded generators reproduce the pages' statistics (CPU only)."""

import numpy as np
import pytest
from scipy.stats import norm

import oracle
from synth import CONFIGS, config_by_name, make_layer, make_tokens, make_lattice_layer, make_lattice_tokens
from synth.configs import LayerConfig
from synth.layers import (firing_probs, firing_probs_by_rank, normal_matrix, top_share,
                          zipf_exponent, predictor_bias)


def _small_cfg(**kw):
    base = dict(name="small", cfg_id=50, workload="small", d_model=256, d_ffn=512, rank=64, gated=True,
                w_dtype="f16", p_dtype="f16", act_dtype="f16", n_layers=2, tokens=4000,
                density=0.10, zipf_s=1.1)
    base.update(kw)
    return LayerConfig(**base)


def test_configs_shapes():
    toy, l7, o30, f40, l70 = CONFIGS
    assert (toy.d_model, toy.d_ffn, toy.rank, toy.gated, toy.w_dtype) == (512, 2048, 64, False, "f32")
    assert (l7.d_model, l7.d_ffn, l7.rank, l7.gated, l7.n_layers) == (4096, 11008, 1024, True, 32)
    assert (o30.d_model, o30.d_ffn, o30.gated, o30.n_layers) == (7168, 28672, False, 48)
    assert (f40.d_model, f40.d_ffn, f40.w_dtype, f40.n_layers) == (8192, 32768, "q4g32", 60)
    assert (l70.d_model, l70.d_ffn, l70.gated, l70.batches, l70.n_layers) == (8192, 28672, True, (1, 4, 16), 80)
    assert config_by_name("llama7b") is l7


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_firing_probs_mean_cap_and_order(cfg):
    p = firing_probs_by_rank(cfg.d_ffn, cfg.density, zipf_exponent(cfg))
    assert abs(p.mean() - cfg.density) < 1e-9
    assert p.max() <= 0.99 + 1e-15 and p.min() > 0
    assert np.all(np.diff(p) <= 0)


def test_opt30b_locality_26_percent_carry_80_percent():
    cfg = config_by_name("opt30b")
    s = zipf_exponent(cfg)
    p = firing_probs_by_rank(cfg.d_ffn, cfg.density, s)
    assert abs(top_share(p, 0.26) - 0.80) < 1e-6
    assert 1.05 < s < 1.15


def test_firing_probs_permuted_per_layer():
    cfg = config_by_name("toy")
    p0, p0b, p1 = firing_probs(cfg, 0), firing_probs(cfg, 0), firing_probs(cfg, 1)
    assert np.array_equal(p0, p0b)
    assert not np.array_equal(p0, p1)
    assert np.array_equal(np.sort(p0), np.sort(p1))


def test_blocked_matrix_regenerates_any_row_range():
    full = normal_matrix(0, (7, 0, 1), 3000, 16, 0.5)
    part = normal_matrix(0, (7, 0, 1), 3000, 16, 0.5, row_start=1000, row_stop=2100)
    assert np.array_equal(full[1000:2100], part)


def test_layer_determinism_and_dtypes():
    cfg = config_by_name("toy")
    a, b = make_layer(cfg, 0), make_layer(cfg, 0)
    for name in ("w_up", "w_down_t", "b", "p1", "p2", "b_p"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    assert a.w_up.dtype == np.float32 and a.w_up.shape == (2048, 512)
    assert a.p1.shape == (64, 512) and a.p2.shape == (2048, 64)
    assert a.b.dtype == np.float32 and a.b_p.dtype == np.float32
    x = make_tokens(cfg, 0, 10)
    assert x.shape == (10, 512) and x.dtype == np.float32
    assert np.array_equal(x[3:7], make_tokens(cfg, 0, 4, start=3))


def test_weight_scale_is_one_over_d():
    cfg = _small_cfg(d_model=1024)
    layer = make_layer(cfg, 0, with_predictor=False)
    var = layer.w_up.astype(np.float64).var()
    assert abs(var * 1024 - 1.0) < 0.01


def test_bias_places_firing_rate_closed_form():
    """g_i ~ N(b_i, |w_i|^2) for x ~ N(0, I): the empirical rate of g_i > 0 matches p_i."""
    cfg = _small_cfg()
    layer = make_layer(cfg, 0, with_predictor=False)
    x = make_tokens(cfg, 0, 4000)
    g, _ = oracle.pre_activations(x, oracle.dense_weights(layer.w_gate), oracle.dense_weights(layer.w_up),
                                  layer.b, True)
    rate = (g > 0).mean(axis=0)
    p = layer.p
    # each per-neuron rate is Binomial(T, p_i)/T: aggregate z-scores must look standard normal
    zs = (rate - p) / np.sqrt(p * (1 - p) / x.shape[0])
    assert abs(zs.mean()) < 0.15 and 0.8 < zs.std() < 1.2
    assert abs(rate.mean() - cfg.density) < 0.005


def test_predictor_bias_places_predicted_density():
    cfg = config_by_name("toy")
    layer = make_layer(cfg, 0)
    x = make_tokens(cfg, 0, 1000)
    z = oracle.predictor_logits(x, layer.p1, layer.p2, layer.b_p)
    dens = oracle.predicted_mask(z, 0.5).mean()
    assert abs(dens - cfg.density) < 0.03, dens


def test_predictor_bias_formula_on_independent_units():
    """With orthogonal P1 rows the hidden units are independent; the mean logit then matches."""
    rng = np.random.default_rng(3)
    d, r, n = 64, 64, 50
    p1 = np.eye(r, d) * 2.0
    p2 = rng.standard_normal((n, r)) / 8
    p = np.full(n, 0.5)
    b_p = predictor_bias(p1, p2, p)
    x = rng.standard_normal((20000, d))
    z = oracle.predictor_logits(x, p1, p2, b_p)
    # at p = 0.5 the bias cancels the mean: E z = 0
    assert np.all(np.abs(z.mean(axis=0)) < 0.06)


def test_int4_layer_scales_and_range():
    cfg = _small_cfg(w_dtype="q4g32", gated=False, d_model=256, d_ffn=128)
    layer = make_layer(cfg, 0, with_predictor=False)
    assert layer.w_up.dtype == np.uint8 and layer.w_up.shape == (128, 128)
    assert layer.s_up.dtype == np.float16 and layer.s_up.shape == (128, 8)
    w = oracle.dequant_q4g32(layer.w_up, layer.s_up)
    q = w / np.repeat(layer.s_up.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(q) <= 8) and np.all(q == np.rint(q))
    # the per-group maximum uses the top code (|q| == 7) almost everywhere
    assert (np.abs(q).reshape(128, 8, 32).max(axis=2) == 7).mean() > 0.95


@pytest.mark.parametrize("w_dtype", ["f16", "f32", "q4g32"])
def test_lattice_layer_is_exact(w_dtype):
    layer = make_lattice_layer(d=256, n=300, r=64, gated=True, w_dtype=w_dtype)
    x = make_lattice_tokens(256, 3)
    assert set(np.unique(x.astype(np.float64))) <= {-1.0, 0.0, 1.0}
    out = oracle.forward(layer, x, "predicted")
    assert np.all(out["z"] == np.rint(out["z"]))
    assert np.any(out["z"] == 0)          # ties at the threshold are present
    assert 0 < out["count"] < 300
    # every value is a multiple of 1/8 below 2^21: exact in fp32 under any summation order
    y8 = out["y64"] * 8
    assert np.all(y8 == np.rint(y8)) and np.all(np.abs(y8) < 2 ** 24)


def test_hot_set_and_words():
    """The host side of the hot set: the neurons that fired on at least the given share of the
    calibration tokens, packed as the library's bit set (bit b of word w = neuron 32 w + b)."""
    from activation_sparse_decode_relu_amd.hotset import hot_set, hot_words
    counts = np.array([3, 10, 10, 0, 9, 10, 1, 10, 10, 10, 10, 10, 10, 2] + [0] * 20 + [10])
    mask = hot_set(counts, 10, 0.99)
    assert np.flatnonzero(mask).tolist() == [1, 2, 5, 7, 8, 9, 10, 11, 12, 34]
    assert np.flatnonzero(hot_set(counts, 10, 0.9)).tolist() == [1, 2, 4, 5, 7, 8, 9, 10, 11, 12, 34]
    words = hot_words(mask)
    assert words.dtype == np.uint32 and words.size == 2
    assert words[0] == (1 << 1) | (1 << 2) | (1 << 5) | (1 << 7) | (0b111111 << 7) and words[1] == 1 << 2
    back = [32 * w + b for w in range(2) for b in range(32) if (int(words[w]) >> b) & 1]
    assert back == np.flatnonzero(mask).tolist()
