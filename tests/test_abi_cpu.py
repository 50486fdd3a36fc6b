"""The C ABI library loads, exports every declared symbol, and validates on the host (CPU only)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pi_ffn.h")


def _pi():
    import activation_sparse_decode_relu_amd as pi
    return pi


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|pi_status|int32_t)\s+(pi_\w+)\s*\(", text, re.M)))


def test_header_declares_the_api():
    names = declared_functions()
    assert {"pi_ffn_create", "pi_ffn_predict", "pi_ffn_forward", "pi_ffn_forward_masked",
            "pi_ffn_destroy", "pi_ffn_workspace_bytes", "pi_last_error"} <= set(names)


def test_library_exports_every_declared_symbol():
    pi = _pi()
    for name in declared_functions():
        assert hasattr(pi.LIB, name), f"{name} is declared in pi_ffn.h but not exported"
    assert set(declared_functions()) == set(pi.EXPORTED)
    assert pi.LIB.pi_ffn_abi_version() == 8


def test_struct_layouts_match_header():
    pi = _pi()
    assert ctypes.sizeof(pi.PiDesc) == 9 * 4
    assert ctypes.sizeof(pi.PiWeights) == 10 * ctypes.sizeof(ctypes.c_void_p)


def _desc(**kw):
    pi = _pi()
    base = dict(d_model=4096, d_ffn=11008, rank=1024, gated=1, max_batch=1, w_dtype="f16", p_dtype="f16",
                act_dtype="f16", tau=0.5)
    base.update(kw)
    return pi.make_desc(**base)


@pytest.mark.parametrize("bad", [dict(d_model=100), dict(d_model=0), dict(d_ffn=0), dict(rank=65),
                                 dict(rank=-64), dict(max_batch=0), dict(max_batch=65), dict(w_dtype=7),
                                 dict(p_dtype=2), dict(act_dtype=2), dict(tau=0.0), dict(tau=1.0),
                                 dict(gated=1, w_dtype="q4g32", d_model=96)])
def test_invalid_descriptors(bad):
    pi = _pi()
    with pytest.raises(pi.PiError) as e:
        pi.workspace_bytes(_desc(**bad))
    assert e.value.status == 1
    assert pi.last_error()


def test_workspace_grows_with_batch_and_rank():
    pi = _pi()
    b1 = pi.workspace_bytes(_desc(max_batch=1))
    b16 = pi.workspace_bytes(_desc(max_batch=16))
    b64 = pi.workspace_bytes(_desc(max_batch=64))
    r0 = pi.workspace_bytes(_desc(rank=0))
    assert b64 > b16 > b1 > r0 > 0
    assert b1 % 256 == 0


@pytest.mark.parametrize("bad", [dict(w_dtype="q4g32"), dict(act_dtype="f32"), dict(d_model=4096 + 64)])
def test_more_than_16_tokens_needs_the_matrix_core_shape(bad):
    """Past 16 tokens only fp16 weights and activations with d a multiple of 128 are supported."""
    pi = _pi()
    assert pi.workspace_bytes(_desc(max_batch=64)) > 0
    with pytest.raises(pi.PiError) as e:
        pi.workspace_bytes(_desc(max_batch=17, **bad))
    assert e.value.status == 4


def _create(desc, weights, ws_ptr=None, ws_bytes=0):
    pi = _pi()
    handle = ctypes.c_void_p()
    st = pi.LIB.pi_ffn_create(ctypes.byref(desc), ctypes.byref(weights), ws_ptr, ws_bytes, None,
                              ctypes.byref(handle))
    return st, handle


def _weights(**kw):
    pi = _pi()
    fake = 0x10000
    base = dict(w_gate=fake, w_up=fake, w_down_t=fake, s_gate=None, s_up=None, s_down=None, b=fake,
                p1=fake, p2=fake, b_p=fake)
    base.update(kw)
    return pi.PiWeights(*[base[k] for k, _ in pi.PiWeights._fields_])


@pytest.mark.parametrize("bad", [dict(w_gate=None), dict(w_up=None), dict(b=None), dict(p1=None),
                                 dict(s_up=0x10000), dict(w_down_t=0x10004)])
def test_create_rejects_bad_weights_before_any_gpu_call(bad):
    st, handle = _create(_desc(), _weights(**bad))
    assert st == 1 and not handle.value


def test_create_rejects_small_or_misaligned_workspace():
    pi = _pi()
    need = pi.workspace_bytes(_desc())
    st, _ = _create(_desc(), _weights(), None, need)
    assert st == 2
    st, _ = _create(_desc(), _weights(), 0x10000, need - 1)
    assert st == 2
    st, _ = _create(_desc(), _weights(), 0x10080, need)
    assert st == 2


def test_null_handle_calls_are_invalid():
    pi = _pi()
    assert pi.LIB.pi_ffn_forward(None, 0x1000, 1, 0, 0x1000, None, None, None) == 1
    assert pi.LIB.pi_ffn_predict(None, 0x1000, 1, 0x1000, 0x1000, None, None) == 1
    assert pi.LIB.pi_ffn_forward_masked(None, 0x1000, 1, 0x1000, 0x1000, 0x1000, None) == 1
    assert pi.LIB.pi_ffn_destroy(None) == 1
    assert pi.LIB.pi_ffn_profile_next(None, 0, None, None) == 1
    assert pi.LIB.pi_ffn_launch_plan(None, 1, 0, None) == 1
    assert pi.LIB.pi_ffn_set_hot(None, None) == 1


def test_package_fails_loudly_without_library(tmp_path):
    import subprocess
    import sys
    env = dict(os.environ, PI_FFN_LIB=str(tmp_path / "missing.so"))
    res = subprocess.run([sys.executable, "-c", "import activation_sparse_decode_relu_amd"], cwd=ROOT, env=env,
                         capture_output=True, text=True)
    assert res.returncode != 0 and "ImportError" in res.stderr


def test_static_forward_rejects_before_any_gpu_call():
    """The allocation-free entry point validates on the host: bad descriptors and weights, and a
    descriptor whose workspace exceeds the static scratch, return before anything is enqueued."""
    pi = _pi()
    lib = pi.LIB
    d = _desc()
    assert lib.pi_ffn_forward_static(None, ctypes.byref(_weights()), 0x1000, 1, 0, 0x1000, None, None, None) == 1
    assert lib.pi_ffn_forward_static(ctypes.byref(d), ctypes.byref(_weights(w_gate=None)), 0x1000, 1, 0, 0x1000,
                                     None, None, None) == 1
    big = _desc(d_model=8192, d_ffn=28672, max_batch=16)      # Llama2-70B shape at 16 tokens: ~130 MB
    assert pi.workspace_bytes(big) > pi.binding.STATIC_SCRATCH_BYTES
    assert lib.pi_ffn_forward_static(ctypes.byref(big), ctypes.byref(_weights()), 0x1000, 1, 0, 0x1000, None, None,
                                     None) == 2
    assert "static scratch" in pi.last_error()


def test_static_scratch_fits_the_one_token_workloads():
    """The static scratch holds the workspace of every batch-1 workload shape."""
    pi = _pi()
    for dm, n, w in ((4096, 11008, "f16"), (7168, 28672, "f16"), (8192, 32768, "q4g32"), (8192, 28672, "f16")):
        assert pi.workspace_bytes(_desc(d_model=dm, d_ffn=n, w_dtype=w)) <= pi.binding.STATIC_SCRATCH_BYTES


def test_probe_read_validates_on_the_host():
    pi = _pi()
    assert pi.LIB.pi_probe_read(None, 16, 0x1000, 1, None) == 1
    assert pi.LIB.pi_probe_read(0x1008, 16, 0x1000, 1, None) == 1      # misaligned
    assert pi.LIB.pi_probe_read(0x1000, 20, 0x1000, 1, None) == 1      # not whole 16-byte units
    assert pi.LIB.pi_probe_read(0x1000, 16, 0x1000, 0, None) == 1


def test_header_is_plain_c(tmp_path):
    """The boundary is a C ABI: pi_ffn.h compiles as C99 (and as C++) with every warning an error,
    and a C caller can name every declared entry point."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = declared_functions()
    src = tmp_path / "use.c"
    src.write_text('#include "pi_ffn.h"\n'
                   "typedef void (*any_fn)(void);\n"
                   "any_fn entry_points[] = {\n" + "".join(f"  (any_fn){n},\n" for n in names) + "};\n")
    for lang, std in (("c", "-std=c99"), ("c++", "-std=c++17")):
        r = subprocess.run([cc, "-x", lang, std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I",
                            os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
        assert r.returncode == 0, f"{lang}: {r.stderr}"


def test_c_caller_links_and_runs(tmp_path):
    """A plain C99 program links libpi_ffn.so and calls it with no Python in between: the ABI
    version, a workspace size equal to the one the binding reads, and host-side rejections with
    their messages (no call here reaches a GPU)."""
    import shutil
    import subprocess
    pi = _pi()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    expect = pi.workspace_bytes(pi.make_desc(4096, 11008, 1024, True, 1, "f16", "f16", "f16", 0.5))
    src = tmp_path / "caller.c"
    src.write_text(r'''#include <stdio.h>
#include <string.h>
#include "pi_ffn.h"

int main(void) {
  pi_ffn_desc d = {.d_model = 4096, .d_ffn = 11008, .rank = 1024, .gated = 1, .max_batch = 1,
                   .w_dtype = PI_F16, .p_dtype = PI_F16, .act_dtype = PI_F16, .tau = 0.5f};
  size_t bytes = 0;
  if (pi_ffn_abi_version() != PI_FFN_ABI_VERSION) return 10;
  if (pi_ffn_workspace_bytes(&d, &bytes) != PI_OK || bytes == 0) return 11;
  printf("%zu\n", bytes);
  d.d_model = 100;
  if (pi_ffn_workspace_bytes(&d, &bytes) != PI_ERR_INVALID) return 12;
  if (strstr(pi_last_error(), "d_model") == NULL) return 13;
  if (pi_ffn_forward(NULL, NULL, 1, PI_MASK_DENSE, NULL, NULL, NULL, NULL) != PI_ERR_INVALID) return 14;
  if (strstr(pi_last_error(), "handle") == NULL) return 15;
  return 0;
}
''')
    exe = tmp_path / "caller"
    libdir = os.path.dirname(pi.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                        "-o", str(exe), f"-L{libdir}", "-lpi_ffn", f"-Wl,-rpath,{libdir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.returncode, run.stderr)
    assert int(run.stdout.strip()) == expect
