"""GPU parity of batches past 16 tokens (17 to 64; fp16 weights and activations, d a multiple of
128) on the matrix cores: the exact and dense modes in two or four 16-token tiles, each weight
fragment applied to every tile.  A PREDICTED call runs as EXACT_RELU there, without the
predictor.

Integer-lattice layers make every sum exact, so lists and y must match the oracle bit for bit,
and a 64-token call must equal four 16-token calls bit for bit (a token's y does not depend on
its batch mates in exact mode).  Random full-size layers (LLaMA-7B and Llama2-70B at 64 tokens,
OPT-30B non-gated at 32) check the decisions outside the guard band and y within rel-L2 1e-3 of
the oracle on the GPU's own list, in exact and dense modes.
"""

import numpy as np
import pytest

import oracle
from synth import config_by_name, firing_probs, make_lattice_layer, make_lattice_tokens, make_layer, make_tokens

from gpu_util import announce, check_decisions, check_idx_valid, rel_l2_rows, run_forward, run_masked, run_predict

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_decode_relu_amd  # noqa: F401  (fails loudly if the library is missing)


def _pi():
    import activation_sparse_decode_relu_amd as pi
    return pi


def _bitwise(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


# d = 640: one full 512-column down slice and a ragged one; n = 1000: 15 full 64-neuron groups
# and a ragged one; B = 17 and 33 leave ragged token tiles, 32 and 64 fill them.
@pytest.mark.parametrize("gated", [True, False], ids=["gated", "nongated"])
@pytest.mark.parametrize("mode", ["exact", "dense"])
@pytest.mark.parametrize("B", [17, 32, 33, 64])
def test_lattice_bit_exact_large_batch(gated, mode, B):
    d, n, r = 640, 1000, 128
    announce(f"large batch lattice gated={gated} mode={mode} B={B} d={d} n={n}")
    layer = make_lattice_layer(d, n, r, gated, seed=71 + B)
    x = make_lattice_tokens(d, B, seed=81 + B)
    ref = oracle.forward(layer, x, mode)
    h = _pi().upload_layer(layer, "cuda", max_batch=64)
    idx, count, y = run_forward(h, x, mode)
    check_idx_valid(idx, count, n)
    assert count == ref["count"] and np.array_equal(idx, ref["idx"])
    assert _bitwise(y, ref["y"]), "y differs bitwise from the oracle"
    h.close()


def test_lattice_large_batch_equals_16_token_calls():
    d, n, r = 1024, 3001, 128
    announce(f"large batch lattice: 64 tokens against four calls of 16, d={d} n={n}")
    layer = make_lattice_layer(d, n, r, True, seed=91)
    x = make_lattice_tokens(d, 64, seed=92)
    h = _pi().upload_layer(layer, "cuda", max_batch=64)
    _, _, y64 = run_forward(h, x, "exact")
    for q in range(4):
        xs = x[16 * q:16 * (q + 1)]
        _, _, y16 = run_forward(h, xs, "exact")
        assert _bitwise(y64[16 * q:16 * (q + 1)], y16), f"tokens {16 * q}..{16 * q + 15}"
        assert _bitwise(y16, oracle.forward(layer, xs, "exact")["y"])
    h.close()


def test_predicted_runs_as_exact_past_16_tokens():
    pi = _pi()
    d, n, r = 640, 1000, 128
    announce("large batch: PREDICTED past 16 tokens runs as EXACT_RELU; predict and lists refuse")
    layer = make_lattice_layer(d, n, r, True, seed=101)
    h = pi.upload_layer(layer, "cuda", max_batch=64)
    x = make_lattice_tokens(d, 40, seed=102)
    ref = oracle.forward(layer, x, "exact")
    idx, count, y = run_forward(h, x, "predicted")
    assert count == ref["count"] and np.array_equal(idx, ref["idx"]) and _bitwise(y, ref["y"])
    assert h.launch_plan(40, "predicted") == ("group", "down", "finish")
    assert h.launch_plan(64, "dense") == ("group", "down", "finish")
    assert h.launch_plan(16, "predicted") == ("pred_hidden", "group", "down", "finish")
    # up to 16 tokens the same handle still runs the predictor
    x16 = x[:16]
    ref16 = oracle.forward(layer, x16, "predicted")
    idx16, _, y16 = run_forward(h, x16, "predicted")
    assert np.array_equal(idx16, ref16["idx"]) and _bitwise(y16, ref16["y"])
    with pytest.raises(pi.PiError) as e:
        run_predict(h, x)
    assert e.value.status == 4
    with pytest.raises(pi.PiError) as e:
        run_masked(h, x, [0, 5])
    assert e.value.status == 4
    h.close()


@pytest.mark.parametrize("name,B", [("llama7b", 64), ("opt30b", 32), ("llama70b", 64)])
def test_random_full_size_layer_large_batch(name, B):
    cfg = config_by_name(name)
    announce(f"large batch: random {name} layer 0 at {B} tokens, exact and dense")
    layer = make_layer(cfg, 0)
    h = _pi().upload_layer(layer, "cuda", max_batch=64)
    try:
        x = make_tokens(cfg, 0, B, start=96)
        idx, count, y = run_forward(h, x, "exact")
        check_idx_valid(idx, count, layer.d_ffn)
        pre = oracle.dense_weights(layer.w_gate, layer.s_gate) if layer.gated else oracle.dense_weights(layer.w_up,
                                                                                                        layer.s_up)
        g = x.astype(np.float64) @ pre.T + layer.b
        band = oracle.GUARD_SAFETY * oracle.prob_band_exact(x, pre, layer.b)
        del pre
        inside = int(np.count_nonzero(np.abs(g) <= band))
        announce(f"  {inside} of {g.size} token decisions inside the band ({100 * inside / g.size:.3f} %)")
        assert inside <= 0.01 * g.size
        check_decisions(idx, layer.d_ffn, g, band, 0.0)
        # the union of B exact supports covers about sum_i 1 - (1 - p_i)^B of the layer
        u = float(np.mean(1.0 - (1.0 - firing_probs(cfg, 0)) ** B))
        assert abs(count / layer.d_ffn - u) < 0.05, (count / layer.d_ffn, u)
        ref = oracle.forward_masked(layer, x, idx)["y64"]
        assert rel_l2_rows(y, ref).max() <= 1e-3
        _, dcount, yd = run_forward(h, x, "dense")
        assert dcount == layer.d_ffn
        assert rel_l2_rows(yd, oracle.forward_masked(layer, x, np.arange(layer.d_ffn))["y64"]).max() <= 1e-3
    finally:
        h.close()
        torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [20, 40])
def test_large_activation_step_keeps_fp32(B):
    """An |a| of 2^15 or more cannot be split into two fp16 parts.  The batched down projection's
    32-neuron step holding it stays on the fp32 MFMA, the other steps split.  y stays bit-exact on
    a lattice layer whose one neuron has a of about 40000 on every token."""
    d, n, r = 512, 1000, 128
    announce(f"large batch: a step with |a| >= 2^15 keeps fp32, B={B}")
    layer = make_lattice_layer(d, n, r, False, seed=111)
    big = 37                                  # in the second 32-neuron step of the first chunk
    layer.b = np.array(layer.b, copy=True)
    layer.b[big] = 40000.0                    # a = ReLU(u + b) with u a small integer
    w = np.array(layer.w_down_t, copy=True)
    w[big] = 0
    w[big, 3], w[big, 300] = 1, -1            # y columns 3 and 300 carry about +-40000
    layer.w_down_t = w
    x = make_lattice_tokens(d, B, seed=112)
    h = _pi().upload_layer(layer, "cuda", max_batch=64)
    for mode in ("dense", "exact"):
        ref = oracle.forward(layer, x, mode)
        assert np.all(np.abs(ref["a"][:, big]) >= 32768), "the case does not hold a large activation"
        idx, count, y = run_forward(h, x, mode)
        check_idx_valid(idx, count, n)
        assert count == ref["count"] and np.array_equal(idx, ref["idx"])
        assert _bitwise(y, ref["y"]), f"{mode}: y differs bitwise from the oracle"
        assert np.all(np.abs(y[:, 3].astype(np.float64)) > 30000)
    h.close()
