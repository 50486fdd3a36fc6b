"""Host-side argument checks of the Python binding (no GPU).

The C ABI sees bare addresses: it checks alignment, but a host address or a buffer too small for
what a call writes would reach a kernel.  The binding checks every tensor argument first (a
contiguous torch tensor on the layer's device, of the call's dtype, with the bytes the call reads
or writes) and raises PiError(PI_ERR_INVALID).  Here the layer object has no handle (NULL, which
the library itself rejects with "handle is NULL"), so an argument that got past the binding would
show up as the library's message instead of the binding's.
"""

from types import SimpleNamespace

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pi = pytest.importorskip("activation_sparse_decode_relu_amd")

D, N, R, B = 128, 96, 64, 3
NULL_STREAM = SimpleNamespace(cuda_stream=0)   # stands in for a torch stream: no GPU to ask for one


def _layer(act="f16", device="cpu"):
    lay = object.__new__(pi.FFNLayer)
    lay.desc = pi.make_desc(D, N, R, True, 4, "f16", "f16", act)
    lay.handle = None
    lay.device = torch.device(device)
    lay.weights = pi.PiWeights()
    return lay


def _args(act=torch.float16):
    x = torch.zeros(B, D, dtype=act)
    return dict(x=x, y=torch.zeros(B, D, dtype=act), idx=torch.zeros(N, dtype=torch.int32),
                count=torch.zeros(1, dtype=torch.int32))


def _rejects(fn, *needles):
    with pytest.raises(pi.PiError) as e:
        fn()
    assert e.value.status == pi.binding.PI_ERR_INVALID
    msg = str(e.value)
    assert "handle is NULL" not in msg, "a bad argument reached the library"
    for s in needles:
        assert s in msg, msg


def _reaches_library(fn):
    with pytest.raises(pi.PiError) as e:
        fn()
    assert e.value.status == pi.binding.PI_ERR_INVALID and "handle is NULL" in str(e.value)


def test_valid_arguments_reach_the_library():
    lay, a, s = _layer(), _args(), NULL_STREAM
    _reaches_library(lambda: lay.forward(a["x"], a["y"], "dense", a["idx"], a["count"], stream=s))
    _reaches_library(lambda: lay.forward(a["x"], a["y"], "exact", stream=s))   # no list requested
    _reaches_library(lambda: lay.forward(a["x"], None, "dense", stream=s))     # NULL y: the library decides
    _reaches_library(lambda: lay.predict(a["x"], a["idx"], a["count"], torch.zeros(B, N), stream=s))
    _reaches_library(lambda: lay.forward_masked(a["x"], a["idx"][:1], a["count"], a["y"], stream=s))
    _reaches_library(lambda: lay.set_hot(torch.zeros((N + 31) // 32, dtype=torch.int32)))
    _reaches_library(lambda: lay.set_hot(None))
    lay32, a32 = _layer("f32"), _args(torch.float32)
    _reaches_library(lambda: lay32.forward(a32["x"], a32["y"], "dense", stream=s))


def test_x_is_checked():
    lay, a = _layer(), _args()
    y = a["y"]
    _rejects(lambda: lay.forward(a["x"].float(), y, "dense"), "x is torch.float32", "torch.float16")
    _rejects(lambda: lay.forward(torch.zeros(D, B, dtype=torch.float16).t(), y, "dense"), "x is not contiguous")
    _rejects(lambda: lay.forward(torch.zeros(D, dtype=torch.float16), y, "dense"), f"[B][{D}]")
    _rejects(lambda: lay.forward(torch.zeros(B, D + 64, dtype=torch.float16), y, "dense"), f"[B][{D}]")
    _rejects(lambda: lay.forward(np.zeros((B, D), np.float16), y, "dense"), "torch tensor", "ndarray")
    _rejects(lambda: lay.forward(None, y, "dense"), "[B]")


def test_y_and_list_sizes_are_checked():
    lay, a = _layer(), _args()
    x = a["x"]
    _rejects(lambda: lay.forward(x, a["y"][:B - 1], "dense"), "y holds", str(B * D * 2))
    _rejects(lambda: lay.forward(x, a["y"].float(), "dense"), "y is torch.float32")
    _rejects(lambda: lay.forward(x, a["y"], "dense", a["idx"][:N - 1], a["count"]), "idx holds", str(4 * N))
    _rejects(lambda: lay.forward(x, a["y"], "dense", a["idx"].long(), a["count"]), "idx is torch.int64")
    _rejects(lambda: lay.forward(x, a["y"], "dense", a["idx"], a["count"][:0]), "count holds 0 bytes")
    _rejects(lambda: lay.forward_static(x, a["y"], "dense", a["idx"][:N - 1], a["count"]), "idx holds")
    _rejects(lambda: lay.predict(x, a["idx"], a["count"], torch.zeros(B, N - 1)), "logits_dbg holds")
    _rejects(lambda: lay.predict(x, a["idx"], a["count"], torch.zeros(B, N, dtype=torch.float64)),
             "logits_dbg is torch.float64")
    _rejects(lambda: lay.forward_masked(x, a["idx"][:0], a["count"], a["y"]), "idx holds 0 bytes")
    _rejects(lambda: lay.forward_masked(x, a["idx"], a["count"], a["y"][:1]), "y holds")


def test_device_is_checked():
    # a CUDA layer (torch.device needs no GPU to name one) given host tensors
    lay, a = _layer(device="cuda:0"), _args()
    _rejects(lambda: lay.forward(a["x"], a["y"], "dense"), "x is on cpu", "cuda:0")
    _rejects(lambda: lay.set_hot(torch.zeros(4, dtype=torch.int32)), "hot_words is on cpu")


def test_hot_words_are_checked():
    lay = _layer()
    words = (N + 31) // 32
    _rejects(lambda: lay.set_hot(torch.zeros(words - 1, dtype=torch.int32)), "hot_words holds")
    _rejects(lambda: lay.set_hot(torch.zeros(4 * words, dtype=torch.uint8)), "hot_words is torch.uint8")


def test_weights_must_be_cuda_tensors():
    desc = pi.make_desc(D, N, R, True, 1, "f16", "f16", "f16")
    with pytest.raises(pi.PiError) as e:
        pi.FFNLayer(desc, {"w_up": torch.zeros(N, D, dtype=torch.float16)})
    assert e.value.status == pi.binding.PI_ERR_INVALID and "CUDA" in str(e.value)
    with pytest.raises(pi.PiError):
        pi.probe_read(torch.zeros(64, dtype=torch.int32), torch.zeros(1, dtype=torch.int32))


def test_weight_bytes_follow_the_header_layouts():
    f16 = pi.binding._weight_bytes(pi.make_desc(D, N, R, True, 1, "f16", "f16", "f16"))
    assert f16 == dict(w_gate=N * D * 2, w_up=N * D * 2, w_down_t=N * D * 2, s_gate=0, s_up=0, s_down=0,
                       b=4 * N, p1=R * D * 2, p2=N * R * 2, b_p=4 * N)
    q4 = pi.binding._weight_bytes(pi.make_desc(D, N, R, False, 1, "q4g32", "f32", "f16"))
    assert q4["w_up"] == N * D // 2 and q4["s_up"] == N * (D // 32) * 2
    assert q4["p1"] == R * D * 4 and q4["p2"] == N * R * 4
    f32 = pi.binding._weight_bytes(pi.make_desc(D, N, 0, True, 1, "f32", "f16", "f32"))
    assert f32["w_down_t"] == N * D * 4 and f32["p1"] == 0 and f32["p2"] == 0
