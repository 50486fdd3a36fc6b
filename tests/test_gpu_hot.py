"""GPU parity of the hot set (pi_ffn_set_hot): the profile's hot neurons are computed on every
predicted-mode call without their predictor rows being read, and the predictor decides the rest.
Integer-lattice layers give bit-exact lists, logits and outputs against the oracle's predicted
mode with the same hot set; a random LLaMA-7B-shaped layer is profiled on calibration tokens
(exact-ReLU firing counts) and checked with the guard band."""

import numpy as np
import pytest

import oracle
from synth import config_by_name, make_lattice_layer, make_lattice_tokens, make_layer, make_tokens

from gpu_util import announce, check_decisions, check_idx_valid, dev_tensor, rel_l2_rows, run_forward, run_predict

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pi():
    import activation_sparse_decode_relu_amd as pi
    return pi


def _bitwise(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


def _words(mask):
    from activation_sparse_decode_relu_amd.hotset import hot_words
    return torch.from_numpy(hot_words(mask).view(np.int32)).cuda()


@pytest.mark.parametrize("d,n,w_dtype,gated", [(4096, 11008, "f16", True), (8192, 5000, "q4g32", False),
                                               (512, 1000, "f16", False), (8192, 3001, "f16", True)])
@pytest.mark.parametrize("density", [0.02, 0.5, 1.0])
def test_lattice_hot_set_bit_exact(d, n, w_dtype, gated, density):
    announce(f"hot set lattice d={d} n={n} {w_dtype} gated={gated} density={density}")
    layer = make_lattice_layer(d, n, 128, gated, w_dtype=w_dtype, seed=d + n + 11)
    hot = np.random.default_rng(n + int(100 * density)).random(n) < density
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    h.set_hot(_words(hot))
    for t in range(2):
        x = make_lattice_tokens(d, 1, seed=300 + t)
        ref = oracle.forward(layer, x, "predicted", hot=hot)
        idx, count, y = run_forward(h, x, "predicted")
        check_idx_valid(idx, count, n)
        assert count == ref["count"] and np.array_equal(idx, ref["idx"]), f"token {t}"
        assert _bitwise(y, ref["y"]), f"token {t}: y differs bitwise"
        pidx, _, z = run_predict(h, x)
        assert np.array_equal(pidx, ref["idx"])
        assert np.all(np.isposinf(z[:, hot])), "hot neurons' logits read +inf"
        assert np.array_equal(z[:, ~hot].astype(np.float64), ref["z"][:, ~hot])
    h.set_hot(None)                          # back to the plain predicted mode
    x = make_lattice_tokens(d, 1, seed=310)
    ref = oracle.forward(layer, x, "predicted")
    idx, count, y = run_forward(h, x, "predicted")
    assert np.array_equal(idx, ref["idx"]) and _bitwise(y, ref["y"])
    h.close()


def test_set_hot_validation():
    pi = _pi()
    announce("hot set: argument checks")
    layer = make_lattice_layer(512, 1000, 128, True, seed=320)
    words = _words(np.ones(1000, dtype=bool))
    hb = pi.upload_layer(layer, "cuda", max_batch=4)          # batches run elsewhere: unsupported
    with pytest.raises(pi.PiError) as e:
        hb.set_hot(words)
    assert e.value.status == 4
    hb.set_hot(None)
    hb.close()
    h = pi.upload_layer(layer, "cuda", max_batch=1)
    with pytest.raises(pi.PiError) as e:
        h.set_hot(torch.zeros(64, dtype=torch.uint8, device="cuda")[1:])   # bytes, not words: the binding
    assert e.value.status == 1
    # the library's own check, past the binding: an address 2 bytes into a large enough word buffer
    room = torch.zeros(words.numel() + 1, dtype=torch.int32, device="cuda")
    assert pi.LIB.pi_ffn_set_hot(h.handle, room.data_ptr() + 2) == 1
    assert "aligned" in pi.last_error()
    h.close()


def test_profiled_hot_set_random_layer():
    pi = _pi()
    from activation_sparse_decode_relu_amd.hotset import firing_counts, hot_set
    cfg = config_by_name("llama7b")
    announce("hot set: profile a random LLaMA-7B layer on calibration tokens, check against the oracle")
    layer = make_layer(cfg, 2)
    h = pi.upload_layer(layer, "cuda", max_batch=1)
    cal = 64
    hot = hot_set(firing_counts(h, dev_tensor(make_tokens(cfg, 2, cal, start=128))), cal, 0.99)
    assert hot.sum() > 0
    assert np.mean(layer.p[hot]) > 0.9        # the profiled set is the generator's always-firing head, about
    h.set_hot(_words(hot))
    thr = oracle.threshold_logit(layer.tau)
    x = make_tokens(cfg, 2, 4, start=0)
    cold = np.flatnonzero(~hot)
    for t in range(4):
        xt = x[t:t + 1]
        idx, count, y = run_forward(h, xt, "predicted")
        check_idx_valid(idx, count, layer.d_ffn)
        sel = np.zeros(layer.d_ffn, dtype=bool)
        sel[idx] = True
        assert np.all(sel[hot]), "every hot neuron is selected"
        pidx, _, z = run_predict(h, xt)
        assert np.array_equal(pidx, idx) and np.array_equal(idx, np.flatnonzero(z[0] > np.float32(thr)))
        zo = oracle.predictor_logits(xt, layer.p1, layer.p2, layer.b_p)
        band = oracle.GUARD_SAFETY * oracle.prob_band_predictor(xt, layer.p1, layer.p2, layer.b_p)
        check_decisions(np.flatnonzero(sel[cold]), cold.size, zo[:, cold], band[:, cold], thr)
        ref = oracle.forward_masked(layer, xt, idx)["y64"]
        assert rel_l2_rows(y, ref).max() <= 1e-3
    h.close()
