"""MoE FFN-service layer (the FFN side of Attention-FFN Disaggregation) on
AMD Instinct MI355X: hand-written HIP kernels for gfx950 behind a C ABI
(include/afd_ffn.h), with a thin ctypes/torch binding."""
from . import _ffi
from ._ffi import AfdError, load_library
from .layer import FfnLayer, quantize_fp8_128x128, quantize_fp8_1x128

__all__ = ["FfnLayer", "AfdError", "load_library", "quantize_fp8_1x128",
           "quantize_fp8_128x128", "_ffi"]
