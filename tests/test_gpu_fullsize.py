"""GPU parity at the workloads' full sizes, on sampled layers and tokens.

Each workload's layers 0, L/2 and L-1 are generated at their real shape (LLaMA-7B, OPT-30B,
Falcon-40B int4, Llama2-70B at batch 1, 4 and 16), run through the C ABI in the launch
configuration the benchmark times, and compared with the oracle on 16 seeded tokens per layer
and mode:

* the index list must be the GPU's own decisions, bit-exact (checked through the logits);
* every GPU logit (or, in exact mode, decision value) must lie within the rigorous fp32 error
  bound of the exact value, and within the much tighter probabilistic bound;
* the list must agree with the oracle for every neuron outside twice the probabilistic band;
  the per-token decisions inside it (either decision is correct there) are counted, reported
  and capped at 1 %, and the batch-union decisions they leave open are reported;
* y must lie within rel-L2 1e-3 of the oracle evaluated on the GPU's index list.
"""

import numpy as np
import pytest

import oracle
from synth import config_by_name, make_layer, make_tokens

from gpu_util import announce, check_decisions, check_idx_valid, rel_l2_rows, run_forward, run_predict

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOKENS = 16            # sampled tokens per (layer, mode)
IN_BAND_CAP = 0.01     # most decisions allowed inside the doubled probabilistic band


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def _sampled_layers(name):
    L = config_by_name(name).n_layers
    return sorted({0, L // 2, L - 1})


def _upload(name, layer_idx):
    import activation_sparse_decode_relu_amd as pi
    cfg = config_by_name(name)
    layer = make_layer(cfg, layer_idx)
    return pi.upload_layer(layer, "cuda", max_batch=max(cfg.batches)), layer


class InBand:
    """Counts the per-token decisions inside the doubled probabilistic band (capped), and the
    batch-union decisions left open by them (reported: with B tokens a neuron's union is open
    when any token is in the band and none is certainly on)."""

    def __init__(self, what):
        self.what, self.inside, self.total, self.union_open, self.union_total = what, 0, 0, 0, 0

    def add(self, values, band, threshold, union_open):
        v = np.atleast_2d(values)
        self.inside += int(np.count_nonzero(np.abs(v - threshold) <= np.atleast_2d(band)))
        self.total += v.size
        self.union_open += union_open
        self.union_total += v.shape[1]

    def close(self):
        frac = self.inside / max(1, self.total)
        announce(f"  {self.what}: {self.inside} of {self.total} token decisions inside the band ({100 * frac:.3f} %); "
                 f"{self.union_open} of {self.union_total} union decisions open")
        assert frac <= IN_BAND_CAP, f"{self.what}: {frac:.4%} of decisions inside the band"


def _check_predicted(h, layer, cfg, B, n_batches, start0):
    counter = InBand(f"{cfg.name} layer {layer.index} predicted B={B}")
    thr = oracle.threshold_logit(layer.tau)
    for k in range(n_batches):
        start = start0 + k * B
        x = make_tokens(cfg, layer.index, B, start=start)
        idx, count, y = run_forward(h, x, "predicted")
        check_idx_valid(idx, count, layer.d_ffn)
        pidx, pcount, z = run_predict(h, x)
        assert pcount == count and np.array_equal(pidx, idx), "predict and forward disagree on the index list"
        own = np.flatnonzero((z > np.float32(thr)).any(axis=0))
        assert np.array_equal(idx, own), "index list is not the GPU's own decisions"
        zo = oracle.predictor_logits(x, layer.p1, layer.p2, layer.b_p)
        err = np.abs(z.astype(np.float64) - zo)
        rig = oracle.guard_band_predictor(x, layer.p1, layer.p2, layer.b_p) / oracle.GUARD_SAFETY
        prob = oracle.prob_band_predictor(x, layer.p1, layer.p2, layer.b_p)
        assert np.all(err <= rig), "logit outside the rigorous fp32 bound"
        assert np.all(err <= prob), f"logit outside the probabilistic bound (worst {np.max(err / prob):.3g} of it)"
        band = oracle.GUARD_SAFETY * prob
        counter.add(zo, band, thr, check_decisions(idx, layer.d_ffn, zo, band, thr))
        ref = oracle.forward_masked(layer, x, idx)["y64"]
        err_y = rel_l2_rows(y, ref)
        assert err_y.max() <= 1e-3, err_y
        # the generator's density is about the workload's target
        assert 0.3 * cfg.density * layer.d_ffn < count < 3.0 * cfg.density * layer.d_ffn * B
    counter.close()


def _pre_matrix(layer):
    return oracle.dense_weights(layer.w_gate, layer.s_gate) if layer.gated else oracle.dense_weights(
        layer.w_up, layer.s_up)


def _check_exact(h, layer, cfg, B, n_batches, start0, pre):
    counter = InBand(f"{cfg.name} layer {layer.index} exact B={B}")
    for k in range(n_batches):
        x = make_tokens(cfg, layer.index, B, start=start0 + k * B)
        idx, count, y = run_forward(h, x, "exact")
        check_idx_valid(idx, count, layer.d_ffn)
        g = x.astype(np.float64) @ pre.T + layer.b
        prob = oracle.prob_band_exact(x, pre, layer.b)
        band = oracle.GUARD_SAFETY * prob
        counter.add(g, band, 0.0, check_decisions(idx, layer.d_ffn, g, band, 0.0))
        ref = oracle.forward_masked(layer, x, idx)["y64"]
        assert rel_l2_rows(y, ref).max() <= 1e-3
    counter.close()


def _check_dense(h, layer, cfg, tokens, start0):
    x = make_tokens(cfg, layer.index, tokens, start=start0)
    all_idx = np.arange(layer.d_ffn)
    ref = oracle.forward_masked(layer, x, all_idx)["y64"]
    for t in range(tokens):
        idx, count, y = run_forward(h, x[t:t + 1], "dense")
        assert count == layer.d_ffn and np.array_equal(idx, all_idx)
        assert rel_l2_rows(y, ref[t:t + 1]).max() <= 1e-3


def _run_config(name, layer_idx, exact_batches=(1,), dense_tokens=2):
    cfg = config_by_name(name)
    announce(f"full-size {name} layer {layer_idx}: generating")
    h, layer = _upload(name, layer_idx)
    try:
        for B in cfg.batches:
            announce(f"full-size {name} layer {layer_idx} predicted B={B}")
            _check_predicted(h, layer, cfg, B, max(1, TOKENS // B), start0=0)
        pre = _pre_matrix(layer)
        for B in exact_batches:
            announce(f"full-size {name} layer {layer_idx} exact B={B}")
            _check_exact(h, layer, cfg, B, max(1, TOKENS // B), start0=TOKENS, pre=pre)
        del pre
        if dense_tokens:
            announce(f"full-size {name} layer {layer_idx} dense B=1")
            _check_dense(h, layer, cfg, dense_tokens, start0=2 * TOKENS)
    finally:
        h.close()
        torch.cuda.empty_cache()


@pytest.mark.parametrize("layer_idx", _sampled_layers("llama7b"))
def test_llama7b(layer_idx):
    _run_config("llama7b", layer_idx)


@pytest.mark.parametrize("layer_idx", _sampled_layers("opt30b"))
def test_opt30b(layer_idx):
    _run_config("opt30b", layer_idx)


@pytest.mark.parametrize("layer_idx", _sampled_layers("falcon40b"))
def test_falcon40b_int4(layer_idx):
    _run_config("falcon40b", layer_idx)


@pytest.mark.parametrize("layer_idx", _sampled_layers("llama70b"))
def test_llama70b(layer_idx):
    _run_config("llama70b", layer_idx, exact_batches=(1, 16))
