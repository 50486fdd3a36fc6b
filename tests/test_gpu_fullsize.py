"""GPU parity at the workloads' full sizes, on sampled layers and tokens.

Each workload's layer is generated at its real shape (LLaMA-7B, OPT-30B,
Falcon-40B int4, Llama2-70B; batch 1, and 4 and 16 for the 70B shape), run
through the C ABI in the same launch configuration the benchmark times, and
compared with the oracle: the index list must be the GPU's own decisions
(bit-exact), must agree with the oracle wherever the oracle's decision lies
outside the fp32 guard band, and y must lie within rel-L2 1e-3 of the oracle
evaluated on the GPU's index list.
"""

import numpy as np
import pytest

import oracle
from synth import config_by_name, make_layer, make_tokens

from gpu_util import announce, check_decisions, check_idx_valid, rel_l2_rows, run_forward, run_predict

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_CACHE = {}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    for h, _ in _CACHE.values():
        h.close()
    _CACHE.clear()
    torch.cuda.empty_cache()


def _layer(name, layer_idx, max_batch=1, predictor=True):
    key = (name, layer_idx, max_batch, predictor)
    if key not in _CACHE:
        for k in list(_CACHE):                 # keep one full-size layer resident at a time
            _CACHE.pop(k)[0].close()
        import activation_sparse_decode_relu_amd as pi
        cfg = config_by_name(name)
        layer = make_layer(cfg, layer_idx, with_predictor=predictor)
        _CACHE[key] = (pi.upload_layer(layer, "cuda", max_batch=max_batch), layer)
    return _CACHE[key]


def _check_predicted(name, layer_idx, B, start):
    cfg = config_by_name(name)
    announce(f"full-size {name} layer {layer_idx} predicted B={B} tokens [{start}, {start + B})")
    h, layer = _layer(name, layer_idx, max_batch=max(cfg.batches))
    x = make_tokens(cfg, layer_idx, B, start=start)
    idx, count, y = run_forward(h, x, "predicted")
    check_idx_valid(idx, count, layer.d_ffn)
    pidx, pcount, z = run_predict(h, x)
    assert np.array_equal(pidx, idx), "predict and forward disagree on the index list"
    thr = np.float32(oracle.threshold_logit(layer.tau))
    own = np.flatnonzero((z > thr).any(axis=0))
    assert np.array_equal(idx, own), "index list is not the GPU's own decisions"
    zo = oracle.predictor_logits(x, layer.p1, layer.p2, layer.b_p)
    band = oracle.guard_band_predictor(x, layer.p1, layer.p2, layer.b_p)
    # every GPU logit lies within the rigorous fp32 error bound of the exact logit ...
    assert np.all(np.abs(z.astype(np.float64) - zo) <= band / oracle.GUARD_SAFETY), "logit outside the fp32 bound"
    # ... so every decision outside the (doubled) band agrees with the oracle
    check_decisions(idx, layer.d_ffn, zo, band, oracle.threshold_logit(layer.tau))
    ref = oracle.forward_masked(layer, x, idx)["y64"]
    err = rel_l2_rows(y, ref)
    assert err.max() <= 1e-3, err
    # the density the generator places is about the workload's target
    assert 0.3 * cfg.density * layer.d_ffn < count < 3.0 * cfg.density * layer.d_ffn * B


def _check_exact(name, layer_idx, start):
    cfg = config_by_name(name)
    announce(f"full-size {name} layer {layer_idx} exact B=1 token {start}")
    h, layer = _layer(name, layer_idx, max_batch=max(cfg.batches))
    x = make_tokens(cfg, layer_idx, 1, start=start)
    idx, count, y = run_forward(h, x, "exact")
    check_idx_valid(idx, count, layer.d_ffn)
    pre = oracle.dense_weights(layer.w_gate, layer.s_gate) if layer.gated else oracle.dense_weights(layer.w_up,
                                                                                                      layer.s_up)
    g = x.astype(np.float64) @ pre.T + layer.b
    band = oracle.guard_band_exact(x, pre, layer.b)
    del pre
    check_decisions(idx, layer.d_ffn, g, band, 0.0)
    ref = oracle.forward_masked(layer, x, idx)["y64"]
    assert rel_l2_rows(y, ref).max() <= 1e-3


@pytest.mark.parametrize("layer_idx", [0, 31])
def test_llama7b_predicted(layer_idx):
    for t in (0, 100, 255):
        _check_predicted("llama7b", layer_idx, 1, t)


def test_llama7b_exact():
    for t in (3, 200):
        _check_exact("llama7b", 16, t)


def test_llama7b_dense():
    announce("full-size llama7b layer 5 dense B=1")
    h, layer = _layer("llama7b", 5)
    x = make_tokens(config_by_name("llama7b"), 5, 1, start=7)
    idx, count, y = run_forward(h, x, "dense")
    assert count == layer.d_ffn and np.array_equal(idx, np.arange(layer.d_ffn))
    ref = oracle.forward_masked(layer, x, idx)["y64"]
    assert rel_l2_rows(y, ref).max() <= 1e-3


def test_opt30b_predicted():
    for t in (0, 128):
        _check_predicted("opt30b", 47, 1, t)


def test_opt30b_exact():
    _check_exact("opt30b", 47, 9)


def test_falcon40b_int4_predicted():
    for t in (0, 77):
        _check_predicted("falcon40b", 0, 1, t)


def test_falcon40b_int4_exact():
    _check_exact("falcon40b", 59, 5)


@pytest.mark.parametrize("B", [1, 4, 16])
def test_llama70b_batches(B):
    _check_predicted("llama70b", 0, B, 16 * B)
