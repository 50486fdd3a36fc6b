"""pi_ffn_forward_static (the allocation-free entry point, working in the library's static
scratch array) against pi_ffn_forward on handles with their own workspaces: two calls in a row,
the second on a smaller layer, must give bit-identical index lists and outputs, and both match
the oracle bit for bit on integer-lattice layers."""

import numpy as np
import pytest

import oracle
from synth import make_lattice_layer, make_lattice_tokens

from gpu_util import announce, dev_tensor, run_forward

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _static(h, x, mode):
    n = h.desc.d_ffn
    xt = dev_tensor(x)
    y = torch.full_like(xt, float("nan"))
    idx = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    count = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    h.forward_static(xt, y, mode, idx, count)
    return y, idx, count


def _bitwise(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("mode", ["predicted", "exact"])
def test_static_matches_handle_forward_two_calls(mode):
    import activation_sparse_decode_relu_amd as pi
    announce(f"static scratch forward, {mode}: LLaMA-7B-sized lattice layer, then a smaller batched one")
    big = make_lattice_layer(4096, 11008, 1024, True, seed=201)         # one token: the split path
    small = make_lattice_layer(512, 1000, 128, False, seed=202)          # four tokens: the matrix-core path
    hb = pi.upload_layer(big, "cuda", max_batch=1)
    hs = pi.upload_layer(small, "cuda", max_batch=4)
    xb, xs = make_lattice_tokens(4096, 1, seed=203), make_lattice_tokens(512, 4, seed=204)
    ref_b, ref_s = run_forward(hb, xb, mode), run_forward(hs, xs, mode)
    for rep in range(2):
        outs = [_static(hb, xb, mode), _static(hs, xs, mode)]     # two calls in a row, the second smaller
        torch.cuda.synchronize()
        for (y, idx, count), (ridx, rcount, ry), layer, x in zip(outs, (ref_b, ref_s), (big, small), (xb, xs)):
            c = int(count.item())
            assert c == rcount and np.array_equal(idx[:c].cpu().numpy(), ridx), f"repeat {rep}"
            assert _bitwise(y.cpu().numpy(), ry), f"repeat {rep}: y differs from pi_ffn_forward"
            ref = oracle.forward(layer, x, mode)
            assert c == ref["count"] and _bitwise(y.cpu().numpy(), ref["y"])
    hs.close()
    hb.close()


def test_static_rejects_oversized_descriptor():
    import activation_sparse_decode_relu_amd as pi
    announce("static scratch forward: oversized descriptor")
    layer = make_lattice_layer(512, 1000, 128, True, seed=205)
    h = pi.upload_layer(layer, "cuda", max_batch=1)
    h.desc.max_batch = 16
    h.desc.d_ffn = 1 << 22      # the workspace this would need exceeds the static scratch
    x = dev_tensor(make_lattice_tokens(512, 1, seed=206))
    y = torch.empty_like(x)
    with pytest.raises(pi.PiError) as e:
        h.forward_static(x, y, "predicted")
    assert e.value.status == 2
    h.close()
