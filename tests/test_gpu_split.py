"""GPU parity of the one-token split path (fp16 activations and predictor; fp16 rows with d a
multiple of 512 up to 8192, int4 group-32 rows with d = 2048, 4096, 6144 or 8192) against the
CPU oracle.  The path is k_act (each wave: its neurons' mask source, decisions, mask bits, and
the gate / up rows of the selected ones) and k_down (column slice x list chunk tiles over the
global list, the last tile of a slice adding the chunks' partials into y).

Integer-lattice layers make every sum exact, so the index list, the logits and y must match the
oracle bit for bit.  Shapes cover ragged neuron counts (a partly used last mask word), every
mode (predicted, exact, dense, a caller's list), list chunks longer than one LDS segment,
workspaces shared between layers of different sizes, and graph replay.
"""

import numpy as np
import pytest

import oracle
from synth import config_by_name, make_lattice_layer, make_lattice_tokens, make_layer, make_tokens

from gpu_util import (announce, check_decisions, check_idx_valid, rel_l2_rows, run_forward, run_masked,
                      run_predict)

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


@pytest.mark.parametrize("d,n,r,gated", [
    (512, 1000, 128, True),      # one slice, 64 chunks; a ragged last mask word
    (1536, 11000, 256, False),   # three slices
    (4096, 11008, 1024, True),   # the LLaMA-7B shape
    (2048, 20000, 64, True),
    (512, 1, 64, True),          # a single neuron
    (1024, 37, 64, False),       # fewer neurons than one mask word
])
def test_lattice_bit_exact_split(d, n, r, gated):
    announce(f"split path lattice d={d} n={n} r={r} gated={gated}")
    layer = make_lattice_layer(d, n, r, gated, seed=d + n)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    for t in range(3):
        x = make_lattice_tokens(d, 1, seed=50 + t)
        ref = oracle.forward(layer, x, "predicted")
        idx, count, y = run_forward(h, x, "predicted")
        check_idx_valid(idx, count, n)
        assert count == ref["count"] and np.array_equal(idx, ref["idx"]), f"token {t}"
        assert _bitwise(y, ref["y"]), f"token {t}: y differs bitwise"
        pidx, _, z = run_predict(h, x)
        assert np.array_equal(pidx, ref["idx"])
        assert np.array_equal(z.astype(np.float64), ref["z"])
    h.close()


@pytest.mark.parametrize("d,n,r,gated", [
    (5120, 1000, 128, True),
    (6144, 11000, 512, False),
    (7168, 3000, 1024, False),   # the OPT-30B width and predictor rank
    (8192, 20000, 256, True),
    (5120, 40000, 128, False),
    (5120, 1000, 2048, True),    # a predictor rank above 1024
])
def test_lattice_bit_exact_split_wide(d, n, r, gated):
    announce(f"split path lattice d={d} n={n} r={r} gated={gated}")
    layer = make_lattice_layer(d, n, r, gated, seed=d + n + r)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    for t in range(2):
        x = make_lattice_tokens(d, 1, seed=60 + t)
        ref = oracle.forward(layer, x, "predicted")
        idx, count, y = run_forward(h, x, "predicted")
        check_idx_valid(idx, count, n)
        assert count == ref["count"] and np.array_equal(idx, ref["idx"]), f"token {t}"
        assert _bitwise(y, ref["y"]), f"token {t}: y differs bitwise"
        pidx, _, z = run_predict(h, x)
        assert np.array_equal(pidx, ref["idx"])
        assert np.array_equal(z.astype(np.float64), ref["z"])
    h.close()


@pytest.mark.parametrize("d,n,r,gated", [
    (4096, 3000, 128, True),     # gated int4
    (8192, 5000, 256, False),    # the Falcon-40B width
    (8192, 33000, 1024, False),
    (2048, 1000, 64, True),      # one int4 chunk per lane
])
def test_lattice_bit_exact_split_int4(d, n, r, gated):
    announce(f"split path int4 lattice d={d} n={n} r={r} gated={gated}")
    layer = make_lattice_layer(d, n, r, gated, w_dtype="q4g32", seed=d + n + r + 1)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    assert h.launch_plan(1, "predicted") == ("pred_hidden", "group", "down")
    for t in range(2):
        x = make_lattice_tokens(d, 1, seed=70 + t)
        ref = oracle.forward(layer, x, "predicted")
        idx, count, y = run_forward(h, x, "predicted")
        check_idx_valid(idx, count, n)
        assert count == ref["count"] and np.array_equal(idx, ref["idx"]), f"token {t}"
        assert _bitwise(y, ref["y"]), f"token {t}: y differs bitwise"
        pidx, _, z = run_predict(h, x)
        assert np.array_equal(pidx, ref["idx"])
        assert np.array_equal(z.astype(np.float64), ref["z"])
    h.close()


def test_lattice_split_wide_nothing_selected():
    d, n, r = 8192, 3000, 256
    announce("split path d=8192: no neuron selected")
    layer = make_lattice_layer(d, n, r, False, seed=79)
    layer.b_p = np.full(n, -1000.0, dtype=np.float32)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    idx, count, y = run_forward(h, make_lattice_tokens(d, 1, seed=80), "predicted")
    assert count == 0
    assert np.all(y == 0) and not np.signbit(y).any()
    h.close()


def test_lattice_split_nothing_selected():
    """Every logit below the threshold: the list is empty and y is +0.0."""
    d, n, r = 1024, 3000, 128
    announce("split path d=1024: no neuron selected")
    layer = make_lattice_layer(d, n, r, True, seed=77)
    layer.b_p = np.full(n, -1000.0, dtype=np.float32)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    x = make_lattice_tokens(d, 1, seed=78)
    idx, count, y = run_forward(h, x, "predicted")
    assert count == 0
    assert np.all(y == 0) and not np.signbit(y).any()
    h.close()


def test_random_llama7b_layer_split_and_graph_replay():
    cfg = config_by_name("llama7b")
    announce("split path: random LLaMA-7B layer, guard-band parity and graph replay")
    layer = make_layer(cfg, 3)
    pi = _pi()
    h = pi.upload_layer(layer, "cuda", max_batch=1)
    x = make_tokens(cfg, 3, 1, start=11)
    idx, count, y = run_forward(h, x, "predicted")
    check_idx_valid(idx, count, layer.d_ffn)
    zo = oracle.predictor_logits(x, layer.p1, layer.p2, layer.b_p)
    band = oracle.GUARD_SAFETY * oracle.prob_band_predictor(x, layer.p1, layer.p2, layer.b_p)
    check_decisions(idx, layer.d_ffn, zo, band, oracle.threshold_logit(layer.tau))
    ref = oracle.forward_masked(layer, x, idx)["y64"]
    assert rel_l2_rows(y, ref).max() <= 1e-3
    xt = torch.from_numpy(x).cuda()
    yt = torch.empty_like(xt)
    it = torch.empty(layer.d_ffn, dtype=torch.int32, device="cuda")
    ct = torch.empty(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        h.forward(xt, yt, "predicted", it, ct)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            h.forward(xt, yt, "predicted", it, ct)
    torch.cuda.synchronize()
    for rep in range(3):
        yt.fill_(float("nan"))
        ct.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert _bitwise(yt.cpu().numpy(), y), f"replay {rep}"
        assert int(ct.item()) == count and np.array_equal(it[:count].cpu().numpy(), idx)
        h.forward(xt, yt, "exact")   # eager work between replays
        torch.cuda.synchronize()
    h.close()


def test_launch_plan_reports_the_kernels():
    pi = _pi()
    announce("launch plans of the one-token, batched and vector paths")
    big = make_lattice_layer(4096, 11008, 1024, True, seed=1)
    h = pi.upload_layer(big, "cuda", max_batch=16)
    assert h.launch_plan(1, "predicted") == ("pred_hidden", "group", "down")
    assert h.launch_plan(1, "exact") == ("group", "down")
    assert h.launch_plan(1, "dense") == ("group", "down")
    assert h.launch_plan(4, "predicted") == ("pred_hidden", "group", "down", "finish")
    assert h.launch_plan(16, "dense") == ("group", "down", "finish")
    h.close()
    odd = make_lattice_layer(576, 1000, 128, True, seed=2)      # d not a multiple of 512: the vector path
    h = pi.upload_layer(odd, "cuda", max_batch=1)
    assert h.launch_plan(1, "predicted") == ("pred_hidden", "group", "finish")
    h.close()


@pytest.mark.parametrize("d,w_dtype", [(512, "f16"), (8192, "f16"), (4096, "q4g32")])
def test_shared_workspace_smaller_layer_after_larger(d, w_dtype):
    """A layer whose n leaves the last mask word partly unused (n % 32 = 8), run on a workspace a
    larger layer has just filled with selected neurons: its list must not pick up the larger
    layer's bits beyond n."""
    pi = _pi()
    announce(f"shared workspace: n=2000 then n=1000, d={d} {w_dtype}")
    big = make_lattice_layer(d, 2000, 128, True, w_dtype=w_dtype, seed=91)
    big.b_p = np.full(2000, 1000.0, dtype=np.float32)     # every neuron of the larger layer fires
    small = make_lattice_layer(d, 1000, 128, True, w_dtype=w_dtype, seed=92)
    hb = pi.upload_layer(big, "cuda", max_batch=1)
    hs = pi.upload_layer(small, "cuda", max_batch=1, workspace=hb.workspace)
    xb = make_lattice_tokens(d, 1, seed=93)
    idx_b, count_b, _ = run_forward(hb, xb, "predicted")
    assert count_b == 2000
    for t in range(2):
        x = make_lattice_tokens(d, 1, seed=94 + t)
        ref = oracle.forward(small, x, "predicted")
        idx, count, y = run_forward(hs, x, "predicted")
        check_idx_valid(idx, count, 1000)
        assert count == ref["count"] and np.array_equal(idx, ref["idx"]), f"token {t}"
        assert _bitwise(y, ref["y"]), f"token {t}"
        pidx, pcount, _ = run_predict(hs, x)
        assert pcount == ref["count"] and np.array_equal(pidx, ref["idx"])
        run_forward(hb, xb, "predicted")                   # the larger layer again, in between
    hs.close()
    hb.close()


@pytest.mark.parametrize("d,n,w_dtype,gated", [
    (512, 1000, "f16", True), (4096, 11008, "f16", False), (8192, 3000, "f16", True),
    (4096, 3000, "q4g32", False), (8192, 2000, "q4g32", True),
])
@pytest.mark.parametrize("mode", ["exact", "dense"])
def test_lattice_split_exact_and_dense(d, n, w_dtype, gated, mode):
    announce(f"split path lattice {mode} d={d} n={n} {w_dtype} gated={gated}")
    layer = make_lattice_layer(d, n, 64, gated, w_dtype=w_dtype, seed=d + n + 5)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    assert h.launch_plan(1, mode) == ("group", "down")
    for t in range(2):
        x = make_lattice_tokens(d, 1, seed=120 + t)
        ref = oracle.forward(layer, x, mode)
        idx, count, y = run_forward(h, x, mode)
        check_idx_valid(idx, count, n)
        assert count == ref["count"] and np.array_equal(idx, ref["idx"]), f"token {t}"
        assert _bitwise(y, ref["y"]), f"token {t}: y differs bitwise"
    h.close()


@pytest.mark.parametrize("d,n,w_dtype", [(512, 3000, "f16"), (8192, 5000, "f16"), (8192, 4000, "q4g32")])
def test_lattice_split_forward_masked(d, n, w_dtype):
    announce(f"split path forward_masked d={d} n={n} {w_dtype}")
    layer = make_lattice_layer(d, n, 64, True, w_dtype=w_dtype, seed=d + n + 6)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    x = make_lattice_tokens(d, 1, seed=130)
    rng = np.random.default_rng(131)
    for sel in ([], [0], [n - 1], sorted(rng.choice(n, n // 7, replace=False).tolist()), list(range(n))):
        y = run_masked(h, x, sel)
        ref = oracle.forward_masked(layer, x, sel)["y"]
        assert _bitwise(y, ref), f"list of {len(sel)}"
        if not sel:
            assert not np.signbit(y).any(), "an empty list must write +0.0"
    h.close()


def test_lattice_split_long_chunks():
    """Dense mode on a narrow, very wide layer: every list chunk spans several LDS segments."""
    d, n = 512, 150000      # one slice, 64 chunks of ~2344 neurons
    announce(f"split path dense d={d} n={n}: chunks over several segments")
    layer = make_lattice_layer(d, n, 64, False, seed=140, w_nonzero=0.05, down_nonzero=1 / 256)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    x = make_lattice_tokens(d, 1, seed=141)
    for mode in ("dense", "exact"):
        ref = oracle.forward(layer, x, mode)
        idx, count, y = run_forward(h, x, mode)
        assert count == ref["count"] and np.array_equal(idx, ref["idx"]), mode
        assert _bitwise(y, ref["y"]), mode
    h.close()
