"""GPU parity of the wave-independent one-token predicted kernels (fp16
activations and predictor, batch 1) against the CPU oracle: one wave per neuron
for fp16 rows with d a multiple of 512 up to 4096; a wave pair per neuron (each
wave half of d and of r, r <= 1024) for fp16 rows with d a multiple of 1024 from
5120 to 8192 and for int4 group-32 rows with d = 4096 or 8192.

Integer-lattice layers make every sum exact, so the index list, the logits and
y must match the oracle bit for bit.  Shapes cover workgroups of one 8-neuron
unit (small n), of 5-6 units (n spread over 256 workgroups) and of the
64-neuron maximum (n large enough that 256 workgroups would not suffice), and
d from 512 to 4096 including a non-power-of-two multiple of 512.
"""

import numpy as np
import pytest

import oracle
from synth import config_by_name, make_lattice_layer, make_lattice_tokens, make_layer, make_tokens

from gpu_util import announce, check_decisions, check_idx_valid, rel_l2_rows, run_forward, run_predict

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
    (512, 1000, 128, True),      # 125 units: one unit per workgroup, ragged last unit
    (1536, 11000, 256, False),   # 1375 units over 256 workgroups (5-6 units each)
    (4096, 11008, 1024, True),   # the LLaMA-7B shape
    (2048, 20000, 64, True),     # 2500 units: 313 workgroups of 7-8 units (64 neurons)
])
def test_lattice_bit_exact_wave(d, n, r, gated):
    announce(f"wave kernel lattice d={d} n={n} r={r} gated={gated}")
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
    (5120, 1000, 128, True),     # one unit per workgroup: pairs of 2 neurons, two pairs idle
    (6144, 11000, 512, False),   # 5-6 units per workgroup
    (7168, 3000, 1024, False),   # the OPT-30B width and predictor rank
    (8192, 20000, 256, True),    # 9-10 units per workgroup: 18-20 neurons per pair, mask bits across words
    (5120, 40000, 128, False),   # 15-16 units per workgroup: up to 32 neurons per pair
    (5120, 1000, 2048, True),    # r above 1024: the vector path
])
def test_lattice_bit_exact_wave_pairs(d, n, r, gated):
    announce(f"wave-pair kernel lattice d={d} n={n} r={r} gated={gated}")
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
    (4096, 3000, 128, True),     # gated int4, one chunk per lane of each half row
    (8192, 5000, 256, False),    # the Falcon-40B width, 2-3 units per workgroup
    (8192, 33000, 1024, False),  # 16 units per workgroup: 32 neurons per pair, several steps per pair
])
def test_lattice_bit_exact_wave_pairs_int4(d, n, r, gated):
    announce(f"wave-pair kernel int4 lattice d={d} n={n} r={r} gated={gated}")
    layer = make_lattice_layer(d, n, r, gated, w_dtype="q4g32", seed=d + n + r + 1)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    assert h.launch_plan(1, "predicted") == ("pred_hidden", "group", "finish")
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


def test_lattice_wave_pairs_nothing_selected():
    d, n, r = 8192, 3000, 256
    announce("wave-pair kernel: no neuron selected")
    layer = make_lattice_layer(d, n, r, False, seed=79)
    layer.b_p = np.full(n, -1000.0, dtype=np.float32)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    idx, count, y = run_forward(h, make_lattice_tokens(d, 1, seed=80), "predicted")
    assert count == 0
    assert np.all(y == 0) and not np.signbit(y).any()
    h.close()


def test_lattice_wave_nothing_selected():
    """Every logit below the threshold: the list is empty and y is +0.0."""
    d, n, r = 1024, 3000, 128
    announce("wave kernel: no neuron selected")
    layer = make_lattice_layer(d, n, r, True, seed=77)
    layer.b_p = np.full(n, -1000.0, dtype=np.float32)
    h = _pi().upload_layer(layer, "cuda", max_batch=1)
    x = make_lattice_tokens(d, 1, seed=78)
    idx, count, y = run_forward(h, x, "predicted")
    assert count == 0
    assert np.all(y == 0) and not np.signbit(y).any()
    h.close()


def test_random_llama7b_layer_wave_and_graph_replay():
    cfg = config_by_name("llama7b")
    announce("wave kernel: random LLaMA-7B layer, guard-band parity and graph replay")
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
        h.forward(xt, yt, "exact")   # eager work (the vector kernel) between replays
        torch.cuda.synchronize()
    h.close()


def test_launch_plan_reports_the_kernels():
    pi = _pi()
    announce("launch plans of the one-token, batched and vector paths")
    big = make_lattice_layer(4096, 11008, 1024, True, seed=1)
    h = pi.upload_layer(big, "cuda", max_batch=16)
    assert h.launch_plan(1, "predicted") == ("pred_hidden", "group", "finish")
    assert h.launch_plan(4, "predicted") == ("pred_hidden", "group", "down", "finish")
    assert h.launch_plan(1, "exact") == ("group", "finish")
    assert h.launch_plan(16, "dense") == ("group", "down", "finish")
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
