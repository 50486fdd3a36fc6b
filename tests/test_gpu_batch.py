"""GPU parity of the batched matrix-core path (2 to 16 tokens, fp16 weights,
activations and predictor, d and r multiples of 128) against the CPU oracle.

Integer-lattice layers make every MFMA sum exact, so the mask, the index list and
y must match the oracle bit for bit.  Random layers check decisions outside the
fp32 guard band, y within rel-L2 1e-3 of the oracle on the GPU's own list, and
that batch-1 calls (the vector path) agree with the batched path.
"""

import numpy as np
import pytest

import oracle
from synth import make_lattice_layer, make_lattice_tokens, make_layer, make_tokens
from synth.configs import LayerConfig

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


# d = 640: one full 512-column slice and one slice with a single active wave;
# n = 1000: 15 full 64-neuron groups and a ragged one; r = 128 and 256.
@pytest.mark.parametrize("r", [128, 256])
@pytest.mark.parametrize("gated", [True, False], ids=["gated", "nongated"])
@pytest.mark.parametrize("mode", ["predicted", "exact", "dense"])
@pytest.mark.parametrize("B", [2, 5, 16])
def test_lattice_bit_exact_batched(r, gated, mode, B):
    d, n = 640, 1000
    announce(f"batched lattice gated={gated} mode={mode} B={B} d={d} n={n} r={r}")
    layer = make_lattice_layer(d, n, r, gated, seed=31 + r)
    x = make_lattice_tokens(d, B, seed=41 + B)
    ref = oracle.forward(layer, x, mode)
    h = _pi().upload_layer(layer, "cuda", max_batch=16)
    idx, count, y = run_forward(h, x, mode)
    check_idx_valid(idx, count, n)
    assert count == ref["count"] and np.array_equal(idx, ref["idx"])
    assert _bitwise(y, ref["y"]), "y differs bitwise from the oracle"
    if mode == "predicted":
        pidx, _, z = run_predict(h, x)
        assert np.array_equal(pidx, ref["idx"])
        assert np.array_equal(z.astype(np.float64), ref["z"])
    h.close()


@pytest.mark.parametrize("B", [2, 16])
def test_lattice_forward_masked_batched(B):
    d, n, r = 640, 1000, 128
    announce(f"batched forward_masked lattice B={B}")
    layer = make_lattice_layer(d, n, r, True, seed=5)
    x = make_lattice_tokens(d, B, seed=6)
    h = _pi().upload_layer(layer, "cuda", max_batch=16)
    y0 = run_masked(h, x, [])
    assert np.all(y0 == 0) and not np.signbit(y0).any(), "an empty list must write +0.0"
    rng = np.random.default_rng(B)
    for sel in ([0], [n - 1], list(range(n)), sorted(rng.choice(n, 333, replace=False).tolist())):
        y = run_masked(h, x, sel)
        assert _bitwise(y, oracle.forward_masked(layer, x, sel)["y"]), f"list of {len(sel)}"
    h.close()


def test_lattice_tau_not_half_exact_mode():
    """Exact mode thresholds the pre-activation at 0 whatever the predictor's tau."""
    d, n, r = 640, 1000, 128
    announce("exact mode with tau = 0.8, batch 1 and 4")
    layer = make_lattice_layer(d, n, r, True, seed=8, tau=0.8)
    for B in (1, 4):
        x = make_lattice_tokens(d, B, seed=9)
        ref = oracle.forward(layer, x, "exact")
        h = _pi().upload_layer(layer, "cuda", max_batch=4)
        idx, count, y = run_forward(h, x, "exact")
        assert count == ref["count"] and np.array_equal(idx, ref["idx"])
        assert _bitwise(y, ref["y"])
        h.close()


def test_lattice_many_down_segments():
    """d = 16384 gives 8 down chunks; n = 17000 makes each chunk longer than one LDS segment."""
    d, n, r = 16384, 17000, 128
    announce(f"batched lattice d={d} n={n}: multi-segment down chunks")
    layer = make_lattice_layer(d, n, r, False, seed=12, w_nonzero=0.25, down_nonzero=1 / 64)
    x = make_lattice_tokens(d, 3, seed=13)
    h = _pi().upload_layer(layer, "cuda", max_batch=4)
    for mode in ("dense", "exact"):
        ref = oracle.forward(layer, x, mode)
        idx, count, y = run_forward(h, x, mode)
        assert count == ref["count"] and np.array_equal(idx, ref["idx"]), mode
        assert _bitwise(y, ref["y"]), mode
    sel = list(range(0, n, 2))
    assert _bitwise(run_masked(h, x, sel), oracle.forward_masked(layer, x, sel)["y"])
    h.close()


SMALL = LayerConfig(
    name="small-f16", cfg_id=90, workload="small gated ReLU FFN fp16 d=1024 n=3000 r=256",
    d_model=1024, d_ffn=3000, rank=256, gated=True, w_dtype="f16", p_dtype="f16", act_dtype="f16",
    n_layers=1, tokens=64, density=0.10, zipf_s=1.1, batches=(1, 16))


@pytest.mark.parametrize("B", [3, 16])
@pytest.mark.parametrize("mode", ["predicted", "exact"])
def test_random_layer_batched(B, mode):
    cfg = SMALL
    announce(f"random fp16 layer d={cfg.d_model} n={cfg.d_ffn} r={cfg.rank} mode={mode} B={B}")
    layer = make_layer(cfg, 0)
    x = make_tokens(cfg, 0, B, start=7)
    h = _pi().upload_layer(layer, "cuda", max_batch=16)
    idx, count, y = run_forward(h, x, mode)
    check_idx_valid(idx, count, layer.d_ffn)
    if mode == "predicted":
        vals = oracle.predictor_logits(x, layer.p1, layer.p2, layer.b_p)
        band = oracle.GUARD_SAFETY * oracle.prob_band_predictor(x, layer.p1, layer.p2, layer.b_p)
        rig = oracle.guard_band_predictor(x, layer.p1, layer.p2, layer.b_p) / oracle.GUARD_SAFETY
        thr = oracle.threshold_logit(layer.tau)
        pidx, _, z = run_predict(h, x)
        assert np.array_equal(pidx, idx)
        assert np.array_equal(idx, np.flatnonzero((z > np.float32(thr)).any(axis=0)))   # own decisions
        err = np.abs(z.astype(np.float64) - vals)
        assert np.all(err <= rig), "logit outside the rigorous fp32 bound"
        assert np.all(err <= band / oracle.GUARD_SAFETY), "logit outside the probabilistic fp32 bound"
        # the batch's list is the union of the per-token lists
        union = set()
        for t in range(B):
            union |= set(run_predict(h, x[t:t + 1])[0].tolist())
        assert idx.tolist() == sorted(union)
    else:
        pre = oracle.dense_weights(layer.w_gate, layer.s_gate)
        vals = x.astype(np.float64) @ pre.T + layer.b
        band, thr = oracle.GUARD_SAFETY * oracle.prob_band_exact(x, pre, layer.b), 0.0
    check_decisions(idx, layer.d_ffn, vals, band, thr)
    ref = oracle.forward_masked(layer, x, idx)["y64"]
    assert rel_l2_rows(y, ref).max() <= 1e-3
    if mode == "exact":
        # a token's exact-mode output does not depend on its batch mates (batch 1 runs the vector path)
        for t in range(B):
            _, _, yt = run_forward(h, x[t:t + 1], mode)
            assert rel_l2_rows(y[t:t + 1], yt).max() <= 1e-3
    h.close()


def test_batched_determinism_and_graph_replay():
    cfg = SMALL
    announce("batched path: repeated calls and graph replay")
    layer = make_layer(cfg, 0)
    x = make_tokens(cfg, 0, 16, start=30)
    pi = _pi()
    h = pi.upload_layer(layer, "cuda", max_batch=16)
    a = run_forward(h, x, "predicted")
    b = run_forward(h, x, "predicted")
    assert np.array_equal(a[0], b[0]) and _bitwise(a[2], b[2])
    xt = torch.from_numpy(x).cuda()
    y = torch.empty_like(xt)
    idx = torch.empty(layer.d_ffn, dtype=torch.int32, device="cuda")
    count = torch.empty(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        h.forward(xt, y, "predicted", idx, count)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            h.forward(xt, y, "predicted", idx, count)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        count.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert _bitwise(y.cpu().numpy(), a[2]), f"replay {rep}"
        assert int(count.item()) == a[1] and np.array_equal(idx[:a[1]].cpu().numpy(), a[0])
        h.forward(xt[:4], y[:4], "exact")   # eager work between replays
        torch.cuda.synchronize()
    h.close()
