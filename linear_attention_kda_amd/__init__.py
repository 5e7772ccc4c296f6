"""MI355X-native Kimi Delta Attention (KDA) chunkwise forward pass.

The computation lives in hand-written HIP kernels for gfx950 behind a C ABI
(include/kda.h, built as linear_attention_kda_amd/libkda.so).  This package is
the thin Python binding over that ABI: argument marshalling only.  Importing
it does not load the library or touch the GPU; the first call does, and it
fails loudly when the library has not been built.
"""
from .binding import (  # noqa: F401
    KDA_BF16,
    KDA_FP32,
    KdaError,
    fwd,
    fwd_check,
    library_path,
    load_library,
)
