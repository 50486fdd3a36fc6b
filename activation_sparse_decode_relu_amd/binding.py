"""ctypes binding of libpi_ffn.so (the C ABI declared in include/pi_ffn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory and streams.  If the
library is not built, importing this module raises ImportError: there is no
fallback.

The C ABI sees bare addresses: it checks their alignment, but it cannot tell
host memory from device memory or see how large a buffer is, and a kernel that
reads a host address or writes past a buffer faults the GPU.  So before an
address is passed, the binding checks that each tensor is a contiguous CUDA
tensor on the layer's device, of the dtype and with at least the bytes the
call reads or writes; a failed check raises PiError(PI_ERR_INVALID) and
nothing is enqueued.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PI_FFN_LIB", os.path.join(PKG_DIR, "libpi_ffn.so"))

PI_OK, PI_ERR_INVALID, PI_ERR_WORKSPACE, PI_ERR_HIP, PI_ERR_UNSUPPORTED = range(5)
PI_F32, PI_F16, PI_Q4G32 = range(3)
PI_MASK_PREDICTED, PI_MASK_EXACT_RELU, PI_MASK_DENSE = range(3)
PI_PHASE_PRED_HIDDEN, PI_PHASE_GROUP, PI_PHASE_DOWN, PI_PHASE_FINISH, PI_PHASE_COUNT = range(5)

DTYPES = {"f32": PI_F32, "f16": PI_F16, "q4g32": PI_Q4G32}
MODES = {"predicted": PI_MASK_PREDICTED, "exact": PI_MASK_EXACT_RELU, "dense": PI_MASK_DENSE}
PHASES = {"pred_hidden": PI_PHASE_PRED_HIDDEN, "group": PI_PHASE_GROUP, "down": PI_PHASE_DOWN,
          "finish": PI_PHASE_FINISH}
STATUS_NAMES = {0: "PI_OK", 1: "PI_ERR_INVALID", 2: "PI_ERR_WORKSPACE", 3: "PI_ERR_HIP", 4: "PI_ERR_UNSUPPORTED"}

ABI_VERSION = 8   # PI_FFN_ABI_VERSION of the header this binding follows
STATIC_SCRATCH_BYTES = 16 << 20   # PI_FFN_STATIC_SCRATCH_BYTES

EXPORTED = ("pi_ffn_abi_version", "pi_last_error", "pi_ffn_workspace_bytes", "pi_ffn_create",
            "pi_ffn_destroy", "pi_ffn_predict", "pi_ffn_forward", "pi_ffn_forward_masked",
            "pi_ffn_forward_static", "pi_probe_read", "pi_ffn_set_hot", "pi_ffn_launch_plan",
            "pi_ffn_profile_next")


class PiDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ffn", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("gated", ctypes.c_int32), ("max_batch", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("p_dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("tau", ctypes.c_float)]


class PiWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("w_gate", "w_up", "w_down_t", "s_gate", "s_up", "s_down", "b", "p1", "p2", "b_p")]


class PiError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                          "or `python activation_sparse_decode_relu_amd/_build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    lib.pi_ffn_abi_version.restype = i32
    lib.pi_ffn_abi_version.argtypes = []
    lib.pi_last_error.restype = ctypes.c_char_p
    lib.pi_last_error.argtypes = []
    lib.pi_ffn_workspace_bytes.restype = st
    lib.pi_ffn_workspace_bytes.argtypes = [ctypes.POINTER(PiDesc), ctypes.POINTER(ctypes.c_size_t)]
    lib.pi_ffn_create.restype = st
    lib.pi_ffn_create.argtypes = [ctypes.POINTER(PiDesc), ctypes.POINTER(PiWeights), vp, ctypes.c_size_t, vp,
                                  ctypes.POINTER(vp)]
    lib.pi_ffn_destroy.restype = st
    lib.pi_ffn_destroy.argtypes = [vp]
    lib.pi_ffn_predict.restype = st
    lib.pi_ffn_predict.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.pi_ffn_forward.restype = st
    lib.pi_ffn_forward.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp]
    lib.pi_ffn_forward_masked.restype = st
    lib.pi_ffn_forward_masked.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.pi_ffn_forward_static.restype = st
    lib.pi_ffn_forward_static.argtypes = [ctypes.POINTER(PiDesc), ctypes.POINTER(PiWeights), vp, i32, i32, vp, vp, vp,
                                          vp]
    lib.pi_probe_read.restype = st
    lib.pi_probe_read.argtypes = [vp, ctypes.c_size_t, vp, i32, vp]
    lib.pi_ffn_set_hot.restype = st
    lib.pi_ffn_set_hot.argtypes = [vp, vp]
    lib.pi_ffn_launch_plan.restype = st
    lib.pi_ffn_launch_plan.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_uint32)]
    lib.pi_ffn_profile_next.restype = st
    lib.pi_ffn_profile_next.argtypes = [vp, i32, vp, vp]
    got = lib.pi_ffn_abi_version()
    if got != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {got}, this binding expects {ABI_VERSION}; rebuild it")
    return lib


LIB = _load()


def last_error() -> str:
    return LIB.pi_last_error().decode()


def check(status: int) -> None:
    if status != PI_OK:
        raise PiError(status, last_error())


def make_desc(d_model, d_ffn, rank, gated, max_batch, w_dtype, p_dtype, act_dtype, tau=0.5) -> PiDesc:
    def dt(v):
        return DTYPES[v] if isinstance(v, str) else int(v)
    return PiDesc(int(d_model), int(d_ffn), int(rank), int(bool(gated)), int(max_batch), dt(w_dtype),
                  dt(p_dtype), dt(act_dtype), float(tau))


def workspace_bytes(desc: PiDesc) -> int:
    out = ctypes.c_size_t(0)
    check(LIB.pi_ffn_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return int(out.value)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


_ACT_TORCH = {PI_F32: "float32", PI_F16: "float16"}   # act_dtype -> torch dtype of x and y
_ELEM_BYTES = {PI_F32: 4, PI_F16: 2}


def _invalid(msg: str) -> PiError:
    return PiError(PI_ERR_INVALID, msg)


def _arg(t, name: str, device, nbytes: int = 0, dtype: Optional[str] = None) -> None:
    """Raise PiError(PI_ERR_INVALID) unless `t` (None passes: the library decides whether the
    argument may be NULL) is a contiguous torch tensor on `device`, of torch dtype `dtype` if
    given, holding at least `nbytes` bytes."""
    if t is None:
        return
    import torch
    if not isinstance(t, torch.Tensor):
        raise _invalid(f"{name} must be a torch tensor, not {type(t).__name__}")
    if t.device != device:
        raise _invalid(f"{name} is on {t.device}, the layer is on {device}")
    if not t.is_contiguous():
        raise _invalid(f"{name} is not contiguous")
    if dtype is not None and t.dtype != getattr(torch, dtype):
        raise _invalid(f"{name} is {t.dtype}, expected torch.{dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise _invalid(f"{name} holds {have} bytes, the call needs {nbytes}")


def _weight_bytes(desc: PiDesc) -> dict:
    """Bytes each weight tensor holds under the header's layouts (the descriptor is valid: the
    library has accepted it)."""
    n, d, r = desc.d_ffn, desc.d_model, desc.rank
    row = {PI_F32: 4 * d, PI_F16: 2 * d, PI_Q4G32: d // 2}[desc.w_dtype]
    scales = n * (d // 32) * 2 if desc.w_dtype == PI_Q4G32 else 0
    pe = _ELEM_BYTES.get(desc.p_dtype, 0)
    return dict(w_gate=n * row, w_up=n * row, w_down_t=n * row, s_gate=scales, s_up=scales, s_down=scales,
                b=4 * n, p1=r * d * pe, p2=n * r * pe, b_p=4 * n)


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) or None


class FFNLayer:
    """One layer bound to device tensors: a handle of the C library.

    `tensors` maps w_gate, w_up, w_down_t, s_gate, s_up, s_down, b, p1, p2, b_p
    to CUDA tensors (or None).  The layer keeps references to them and to its
    workspace for as long as the handle lives.
    """

    def __init__(self, desc: PiDesc, tensors: dict, workspace=None, stream=None):
        import torch
        self.desc = desc
        self.tensors = dict(tensors)
        need = workspace_bytes(desc)
        given = [t for t in self.tensors.values() if t is not None]
        if not given or not isinstance(given[0], torch.Tensor) or given[0].device.type != "cuda":
            raise _invalid("the weights must be CUDA tensors")
        self.device = given[0].device
        sizes = _weight_bytes(desc)
        for k, t in self.tensors.items():
            if k not in sizes:
                raise _invalid(f"unknown weight tensor {k!r}")
            _arg(t, k, self.device, sizes[k])
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        _arg(workspace, "workspace", self.device)
        self.workspace = workspace
        w = PiWeights(*[_ptr(self.tensors.get(k)) for k, _ in PiWeights._fields_])
        self.weights = w
        handle = ctypes.c_void_p()
        check(LIB.pi_ffn_create(ctypes.byref(desc), ctypes.byref(w), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream),
                                ctypes.byref(handle)))
        self.handle = handle

    def close(self) -> None:
        if getattr(self, "handle", None) is not None and self.handle.value:
            check(LIB.pi_ffn_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _x(self, x) -> int:
        """Check x [B][d] (act dtype) and return B."""
        _arg(x, "x", self.device, dtype=_ACT_TORCH.get(self.desc.act_dtype))
        if x is None or x.dim() != 2 or x.shape[1] != self.desc.d_model:
            shape = None if x is None else tuple(x.shape)
            raise _invalid(f"x must be [B][{self.desc.d_model}], got {shape}")
        return int(x.shape[0])

    def _y(self, y, B: int) -> None:
        _arg(y, "y", self.device, B * self.desc.d_model * _ELEM_BYTES.get(self.desc.act_dtype, 0),
             _ACT_TORCH.get(self.desc.act_dtype))

    def _list(self, idx, count, idx_entries: int) -> None:
        _arg(idx, "idx", self.device, 4 * idx_entries, "int32")
        _arg(count, "count", self.device, 4, "int32")

    def predict(self, x, idx, count, logits_dbg=None, stream=None) -> None:
        B = self._x(x)
        self._list(idx, count, self.desc.d_ffn)
        _arg(logits_dbg, "logits_dbg", self.device, 4 * B * self.desc.d_ffn, "float32")
        check(LIB.pi_ffn_predict(self.handle, _ptr(x), int(x.shape[0]), _ptr(idx), _ptr(count),
                                 _ptr(logits_dbg), _stream(stream)))

    def forward(self, x, y, mode="predicted", idx_out=None, count_out=None, stream=None) -> None:
        m = MODES[mode] if isinstance(mode, str) else int(mode)
        self._y(y, self._x(x))
        self._list(idx_out, count_out, self.desc.d_ffn)
        check(LIB.pi_ffn_forward(self.handle, _ptr(x), int(x.shape[0]), m, _ptr(y), _ptr(idx_out),
                                 _ptr(count_out), _stream(stream)))

    def forward_static(self, x, y, mode="predicted", idx_out=None, count_out=None, stream=None) -> None:
        """pi_ffn_forward_static with this layer's descriptor and weights (the handle's workspace
        is not used: the call works in the library's static scratch array)."""
        m = MODES[mode] if isinstance(mode, str) else int(mode)
        self._y(y, self._x(x))
        self._list(idx_out, count_out, self.desc.d_ffn)
        check(LIB.pi_ffn_forward_static(ctypes.byref(self.desc), ctypes.byref(self.weights), _ptr(x),
                                        int(x.shape[0]), m, _ptr(y), _ptr(idx_out), _ptr(count_out),
                                        _stream(stream)))

    def forward_masked(self, x, idx, count, y, stream=None) -> None:
        """idx holds the list on the device; its length *count is not read on the host, so only
        the first entry's room is checked here."""
        self._y(y, self._x(x))
        self._list(idx, count, 1)
        check(LIB.pi_ffn_forward_masked(self.handle, _ptr(x), int(x.shape[0]), _ptr(idx), _ptr(count),
                                        _ptr(y), _stream(stream)))

    def set_hot(self, hot_words=None) -> None:
        """pi_ffn_set_hot: hot_words (int32 device tensor, ceil(n / 32) words, bit i = neuron i) are
        computed on every predicted-mode call; None clears the set.  The layer keeps a reference."""
        _arg(hot_words, "hot_words", self.device, 4 * ((self.desc.d_ffn + 31) // 32), "int32")
        check(LIB.pi_ffn_set_hot(self.handle, _ptr(hot_words)))
        self.hot_words = hot_words

    def launch_plan(self, batch: int, mode="predicted"):
        """The phases a forward call with this batch and mode launches, in launch order."""
        m = MODES[mode] if isinstance(mode, str) else int(mode)
        out = ctypes.c_uint32(0)
        check(LIB.pi_ffn_launch_plan(self.handle, int(batch), m, ctypes.byref(out)))
        return tuple(name for name, p in sorted(PHASES.items(), key=lambda kv: kv[1]) if out.value & (1 << p))

    def profile_next(self, phase, start_event, stop_event) -> None:
        p = PHASES[phase] if isinstance(phase, str) else int(phase)
        def handle(ev):
            if ev is None:
                return None
            return int(getattr(ev, "cuda_event", ev))    # a torch event or a raw hipEvent_t
        s0, s1 = handle(start_event), handle(stop_event)
        check(LIB.pi_ffn_profile_next(self.handle, p, s0, s1))


_TENSOR_NAMES = ("w_gate", "w_up", "w_down_t", "s_gate", "s_up", "s_down", "b", "p1", "p2", "b_p")


def upload_layer(layer, device="cuda", max_batch=1, workspace=None, stream=None,
                 with_predictor=True) -> FFNLayer:
    """Copy a host layer (numpy arrays, neuron-major) to `device` and bind a handle."""
    import torch
    tensors = {}
    for name in _TENSOR_NAMES:
        arr = getattr(layer, name, None)
        if arr is None or (not with_predictor and name in ("p1", "p2", "b_p")):
            tensors[name] = None
            continue
        tensors[name] = torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    rank = layer.rank if (with_predictor and layer.p1 is not None) else 0
    desc = make_desc(layer.d_model, layer.d_ffn, rank, layer.gated, max_batch, layer.w_dtype,
                     layer.p_dtype, layer.act_dtype, layer.tau)
    return FFNLayer(desc, tensors, workspace=workspace, stream=stream)


def probe_read(buf, sums, stream=None) -> None:
    """pi_probe_read: read every byte of the device tensor `buf` once; sums (uint32 device tensor)
    receives one word-sum per workgroup."""
    import torch
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda":
        raise _invalid("buf must be a CUDA tensor")
    _arg(buf, "buf", buf.device)
    _arg(sums, "sums", buf.device, 4, "int32")
    check(LIB.pi_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sums), int(sums.numel()),
                            _stream(stream)))
