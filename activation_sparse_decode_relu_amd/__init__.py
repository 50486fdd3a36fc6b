"""Activation-sparse ReLU FFN decode on MI355X (gfx950).

The compute lives in libpi_ffn.so (hand-written HIP kernels behind the C ABI in
include/pi_ffn.h); this package is its thin Python binding.
"""

from .binding import (  # noqa: F401
    DTYPES,
    EXPORTED,
    FFNLayer,
    LIB,
    LIB_PATH,
    MODES,
    PHASES,
    PiDesc,
    PiError,
    PiWeights,
    check,
    last_error,
    make_desc,
    probe_read,
    upload_layer,
    workspace_bytes,
)
