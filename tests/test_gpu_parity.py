"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Sizes span several tiles and a ragged tail; exact cases use integer-lattice
layers, on which every sum is exact, so indices and outputs must match bit for
bit.  Random layers compare indices outside the fp32 guard band and y within
rel-L2 1e-5 (fp32) / 1e-3 (fp16) of the oracle evaluated on the GPU's own
index list.
"""

import numpy as np
import pytest

import oracle
from synth import config_by_name, make_layer, make_lattice_layer, make_lattice_tokens, make_tokens

from gpu_util import (announce, check_decisions, check_idx_valid, dev_tensor, rel_l2_rows, run_forward,
                      run_masked, run_predict, tol_for)

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


LATTICE_DTYPES = [("f16", "f16", "f16"), ("f32", "f32", "f32"), ("q4g32", "f16", "f16"), ("f16", "f32", "f32")]


@pytest.mark.parametrize("dtypes", LATTICE_DTYPES, ids=lambda t: "-".join(t))
@pytest.mark.parametrize("gated", [True, False], ids=["gated", "nongated"])
@pytest.mark.parametrize("mode", ["predicted", "exact", "dense"])
@pytest.mark.parametrize("B", [1, 3, 16])
def test_lattice_bit_exact(dtypes, gated, mode, B):
    w_dt, p_dt, a_dt = dtypes
    d, n, r = 576, 1000, 128        # 1000 = 15 full mask words + a ragged one; d = 1 full + 1 partial tile
    announce(f"lattice {dtypes} gated={gated} mode={mode} B={B} d={d} n={n} r={r}")
    layer = make_lattice_layer(d, n, r, gated, w_dtype=w_dt, p_dtype=p_dt, act_dtype=a_dt, seed=7)
    x = make_lattice_tokens(d, B, act_dtype=a_dt, seed=11 + B)
    ref = oracle.forward(layer, x, mode)
    h = _pi().upload_layer(layer, "cuda", max_batch=16)
    idx, count, y = run_forward(h, x, mode)
    check_idx_valid(idx, count, n)
    assert count == ref["count"]
    assert np.array_equal(idx, ref["idx"])
    assert np.array_equal(y.view(np.uint8), ref["y"].view(np.uint8)), "y differs bitwise from the oracle"
    if mode == "predicted":
        pidx, pcount, z = run_predict(h, x)
        assert np.array_equal(pidx, ref["idx"])
        assert np.array_equal(z.astype(np.float64), ref["z"])
    h.close()


@pytest.mark.parametrize("mode", ["predicted", "exact", "dense"])
def test_toy_config_tokens(mode):
    """All 1000 seeded tokens of the toy workload, one call each."""
    cfg = config_by_name("toy")
    announce(f"toy layer 0 mode={mode} all {cfg.tokens} tokens B=1")
    layer = make_layer(cfg, 0)
    x = make_tokens(cfg, 0, cfg.tokens)
    h = _pi().upload_layer(layer, "cuda", max_batch=16)
    thr = oracle.threshold_logit(layer.tau)
    if mode == "predicted":
        zo_all = oracle.predictor_logits(x, layer.p1, layer.p2, layer.b_p)
        band_all = oracle.GUARD_SAFETY * oracle.prob_band_predictor(x, layer.p1, layer.p2, layer.b_p)
        rig_all = oracle.guard_band_predictor(x, layer.p1, layer.p2, layer.b_p) / oracle.GUARD_SAFETY
    elif mode == "exact":
        zo_all, _ = oracle.pre_activations(x, None, layer.w_up, layer.b, False)
        band_all = oracle.GUARD_SAFETY * oracle.prob_band_exact(x, layer.w_up, layer.b)
    ambiguous = 0
    for t in range(x.shape[0]):
        xt = x[t:t + 1]
        idx, count, y = run_forward(h, xt, mode)
        check_idx_valid(idx, count, layer.d_ffn)
        if mode == "predicted":
            pidx, _, z = run_predict(h, xt)
            assert np.array_equal(pidx, idx)
            assert np.array_equal(idx, np.flatnonzero(z[0] > np.float32(thr)))   # own decisions, bit-exact
            err = np.abs(z[0].astype(np.float64) - zo_all[t])
            assert np.all(err <= rig_all[t]) and np.all(err <= band_all[t] / oracle.GUARD_SAFETY), t
            ambiguous += check_decisions(idx, layer.d_ffn, zo_all[t:t + 1], band_all[t:t + 1], thr)
        elif mode == "exact":
            ambiguous += check_decisions(idx, layer.d_ffn, zo_all[t:t + 1], band_all[t:t + 1], 0.0)
        else:
            assert np.array_equal(idx, np.arange(layer.d_ffn))
        ref = oracle.forward_masked(layer, xt, idx)["y64"]
        assert rel_l2_rows(y, ref).max() <= tol_for(layer.act_dtype), t
    # decisions inside the doubled probabilistic band are accepted either way; keep them rare
    announce(f"  toy {mode}: {ambiguous} of {x.shape[0] * layer.d_ffn} decisions inside the band")
    assert ambiguous <= 0.01 * x.shape[0] * layer.d_ffn, ambiguous
    h.close()


@pytest.mark.parametrize("B", [2, 4, 16])
@pytest.mark.parametrize("mode", ["predicted", "exact"])
def test_toy_config_batch_union(B, mode):
    cfg = config_by_name("toy")
    announce(f"toy layer 0 mode={mode} union batch B={B}")
    layer = make_layer(cfg, 0)
    x = make_tokens(cfg, 0, B, start=100)
    h = _pi().upload_layer(layer, "cuda", max_batch=16)
    idx, count, y = run_forward(h, x, mode)
    check_idx_valid(idx, count, layer.d_ffn)
    thr = oracle.threshold_logit(layer.tau)
    if mode == "predicted":
        vals = oracle.predictor_logits(x, layer.p1, layer.p2, layer.b_p)
        band = oracle.GUARD_SAFETY * oracle.prob_band_predictor(x, layer.p1, layer.p2, layer.b_p)
    else:
        vals, _ = oracle.pre_activations(x, None, layer.w_up, layer.b, False)
        band, thr = oracle.GUARD_SAFETY * oracle.prob_band_exact(x, layer.w_up, layer.b), 0.0
    check_decisions(idx, layer.d_ffn, vals, band, thr)
    # the batch's list is the union of the per-token lists (set algebra, bit-exact)
    if mode == "predicted":
        union = set()
        for t in range(B):
            union |= set(run_predict(h, x[t:t + 1])[0].tolist())
        assert idx.tolist() == sorted(union)
    ref = oracle.forward_masked(layer, x, idx)["y64"]
    assert rel_l2_rows(y, ref).max() <= 1e-5
    if mode == "exact":
        # a token's exact-mode output does not depend on its batch mates
        for t in range(B):
            _, _, yt = run_forward(h, x[t:t + 1], mode)
            assert rel_l2_rows(y[t:t + 1], yt).max() <= 1e-5
    h.close()


def test_forward_masked_edges():
    cfg = config_by_name("toy")
    announce("forward_masked edge lists: empty, single, full, random")
    layer = make_layer(cfg, 0)
    x = make_tokens(cfg, 0, 3)
    h = _pi().upload_layer(layer, "cuda", max_batch=4)
    y0 = run_masked(h, x, [])
    assert np.all(y0 == 0) and not np.signbit(y0).any(), "an empty list must write +0.0"
    for sel in ([0], [layer.d_ffn - 1], list(range(layer.d_ffn)),
                sorted(np.random.default_rng(1).choice(layer.d_ffn, 300, replace=False).tolist())):
        y = run_masked(h, x, sel)
        ref = oracle.forward_masked(layer, x, sel)["y64"]
        assert rel_l2_rows(y, ref).max() <= 1e-5
    _, _, yd = run_forward(h, x, "dense")
    yf = run_masked(h, x, list(range(layer.d_ffn)))
    assert rel_l2_rows(yf, yd).max() <= 1e-6
    h.close()


def test_exact_equals_dense():
    cfg = config_by_name("toy")
    announce("exact-ReLU sparse vs dense")
    layer = make_layer(cfg, 0)
    x = make_tokens(cfg, 0, 4, start=200)
    h = _pi().upload_layer(layer, "cuda", max_batch=4)
    for t in range(4):
        _, _, ye = run_forward(h, x[t:t + 1], "exact")
        _, _, yd = run_forward(h, x[t:t + 1], "dense")
        assert rel_l2_rows(ye, yd).max() <= 1e-5
    h.close()


def test_run_to_run_bitwise_determinism():
    cfg = config_by_name("toy")
    announce("determinism: repeated calls")
    layer = make_layer(cfg, 0)
    x = make_tokens(cfg, 0, 4, start=300)
    h = _pi().upload_layer(layer, "cuda", max_batch=4)
    for mode in ("predicted", "exact", "dense"):
        a = run_forward(h, x, mode)
        b = run_forward(h, x, mode)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[2].view(np.uint8), b[2].view(np.uint8))
    h.close()


@pytest.mark.parametrize("d,n,r,gated,B", [(64, 1, 64, True, 1), (64, 65, 64, False, 16), (128, 63, 64, True, 5),
                                           (640, 129, 64, False, 2)])
def test_small_and_ragged_shapes(d, n, r, gated, B):
    announce(f"small shape d={d} n={n} r={r} gated={gated} B={B}")
    layer = make_lattice_layer(d, n, r, gated, seed=3, w_nonzero=0.5, down_nonzero=0.25)
    x = make_lattice_tokens(d, B, seed=5)
    h = _pi().upload_layer(layer, "cuda", max_batch=16)
    for mode in ("predicted", "exact", "dense"):
        ref = oracle.forward(layer, x, mode)
        idx, count, y = run_forward(h, x, mode)
        assert count == ref["count"] and np.array_equal(idx, ref["idx"]), mode
        assert np.array_equal(y.view(np.uint8), ref["y"].view(np.uint8)), mode
    h.close()


def test_shared_workspace_across_layers():
    """Two layers bound to one workspace, called in turn on one stream."""
    cfg = config_by_name("toy")
    announce("two layers sharing one workspace")
    pi = _pi()
    l0, l1 = make_layer(cfg, 0), make_layer(cfg, 0)
    l1.b = (l1.b + 0.5).astype(np.float32)     # a different layer
    h0 = pi.upload_layer(l0, "cuda", max_batch=1)
    h1 = pi.upload_layer(l1, "cuda", max_batch=1, workspace=h0.workspace)
    x = make_tokens(cfg, 0, 2, start=400)
    for t in range(2):
        for lay, h in ((l0, h0), (l1, h1), (l0, h0)):
            idx, _, y = run_forward(h, x[t:t + 1], "exact")
            ref = oracle.forward_masked(lay, x[t:t + 1], idx)["y64"]
            assert rel_l2_rows(y, ref).max() <= 1e-5
    h1.close()
    h0.close()


def test_graph_replay_matches_eager():
    cfg = config_by_name("toy")
    announce("hipGraph capture and replay of forward")
    layer = make_layer(cfg, 0)
    x = make_tokens(cfg, 0, 1, start=500)
    pi = _pi()
    h = pi.upload_layer(layer, "cuda", max_batch=1)
    xt = dev_tensor(x)
    y = torch.empty_like(xt)
    idx = torch.empty(layer.d_ffn, dtype=torch.int32, device="cuda")
    count = torch.empty(1, dtype=torch.int32, device="cuda")
    h.forward(xt, y, "predicted", idx, count)
    torch.cuda.synchronize()
    y_eager, idx_eager = y.clone(), idx[:int(count.item())].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        h.forward(xt, y, "predicted", idx, count)   # warm-up on the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            h.forward(xt, y, "predicted", idx, count)
    torch.cuda.synchronize()
    for rep in range(4):
        y.fill_(float("nan"))
        count.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep}"
        assert torch.equal(idx[:int(count.item())], idx_eager), f"replay {rep}"
        h.forward(xt, y, "exact")   # eager work between replays
        torch.cuda.synchronize()
    h.close()


def test_invalid_arguments_enqueue_nothing():
    pi = _pi()
    cfg = config_by_name("toy")
    announce("argument validation")
    layer = make_layer(cfg, 0)
    h = pi.upload_layer(layer, "cuda", max_batch=2)
    x = dev_tensor(make_tokens(cfg, 0, 3))
    y = torch.empty_like(x)
    with pytest.raises(pi.PiError) as e:
        h.forward(x, y, "predicted")          # batch 3 > max_batch 2
    assert e.value.status == 1
    with pytest.raises(pi.PiError):
        h.forward(x[:1], y[:1], 7)            # unknown mode
    with pytest.raises(pi.PiError):
        h.forward(x[:1], None, "dense")           # y is NULL
    h.close()


@pytest.mark.parametrize("mode", ["predicted", "exact", "dense"])
@pytest.mark.parametrize("B", [1, 4])
def test_lattice_large_group_shape(mode, B):
    """A layer wide enough for 128-neuron groups of 8 waves, with a ragged last group."""
    d, n, r = 256, 16500, 64
    announce(f"lattice large-group shape d={d} n={n} mode={mode} B={B}")
    layer = make_lattice_layer(d, n, r, True, seed=21)
    x = make_lattice_tokens(d, B, seed=22)
    ref = oracle.forward(layer, x, mode)
    h = _pi().upload_layer(layer, "cuda", max_batch=4)
    idx, count, y = run_forward(h, x, mode)
    assert count == ref["count"] and np.array_equal(idx, ref["idx"])
    assert np.array_equal(y.view(np.uint8), ref["y"].view(np.uint8))
    sel = ref["idx"][::3]
    ym = run_masked(h, x, sel)
    assert np.array_equal(ym.view(np.uint8), oracle.forward_masked(layer, x, sel)["y"].view(np.uint8))
    h.close()
