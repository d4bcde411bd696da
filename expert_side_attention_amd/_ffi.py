"""ctypes binding of libafd_ffn.so (include/afd_ffn.h).

Argument marshalling only: every step of the layer runs in the library's
HIP kernels.  Functions keep the C names; non-zero status codes raise
``AfdError`` carrying the library's message.  There is no fallback: if the
library is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libafd_ffn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "afd_ffn.h")

AFD_FFN_ABI_VERSION = 3
AFD_OK, AFD_ERR_INVALID_ARG, AFD_ERR_UNSUPPORTED = 0, 1, 2
AFD_ERR_CAPACITY, AFD_ERR_OUT_OF_MEMORY, AFD_ERR_HIP = 3, 4, 5
AFD_MODE_F32, AFD_MODE_BF16, AFD_MODE_W8A8_E4M3 = 0, 1, 2
AFD_FFN_STATIC_SCRATCH_BYTES = 128 << 20
STAGES = ("router", "dispatch", "quant", "gate_up", "down", "combine", "gate_up_big",
          "down_big", "single", "ffn")
STAGE_INDEX = {n: i for i, n in enumerate(STAGES)}

_STATUS_NAMES = {0: "AFD_OK", 1: "AFD_ERR_INVALID_ARG", 2: "AFD_ERR_UNSUPPORTED",
                 3: "AFD_ERR_CAPACITY", 4: "AFD_ERR_OUT_OF_MEMORY", 5: "AFD_ERR_HIP"}


class AfdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class afd_ffn_config(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("mode", ctypes.c_uint32),
                ("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_shared", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("has_router_bias", ctypes.c_int32),
                ("single_launch", ctypes.c_int32), ("split_gemms", ctypes.c_int32)]


class afd_ffn_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "router_b", "gate_w", "up_w", "down_w", "gate_s", "up_s",
        "down_s", "sh_gate_w", "sh_up_w", "sh_down_w", "sh_gate_s", "sh_up_s",
        "sh_down_s")]


class afd_ffn_trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_ids", "topk_w", "counts", "offsets", "perm", "slot_row", "x_q",
        "x_s", "logits", "z_q", "z_s", "num_tiles", "sync_timeouts")]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m expert_side_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    sig = {
        "afd_ffn_create": (ctypes.c_int, [ctypes.POINTER(afd_ffn_config),
                                          ctypes.POINTER(afd_ffn_weights),
                                          ctypes.POINTER(P)]),
        "afd_ffn_forward": (ctypes.c_int, [P, P, P, I64, P]),
        "afd_ffn_forward_traced": (ctypes.c_int, [P, P, P, I64, P,
                                                  ctypes.POINTER(afd_ffn_trace)]),
        "afd_ffn_destroy": (None, [P]),
        "afd_ffn_forward_static": (ctypes.c_int, [ctypes.POINTER(afd_ffn_config),
                                                  ctypes.POINTER(afd_ffn_weights),
                                                  P, P, I64, P]),
        "afd_quant_fp8_1x128": (ctypes.c_int, [P, I64, I64, P, P, P]),
        "afd_quant_fp8_128x128": (ctypes.c_int, [P, I64, I64, P, P, P]),
        "afd_quant_fp8_1x128_f32": (ctypes.c_int, [P, I64, I64, P, P, P]),
        "afd_ffn_profile_enable": (ctypes.c_int, [P, U32]),
        "afd_ffn_profile_read": (ctypes.c_int, [P, ctypes.POINTER(ctypes.c_double),
                                                ctypes.POINTER(ctypes.c_int64)]),
        "afd_ffn_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions include/afd_ffn.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:int|void|const char \*)\s*(afd_\w+)\s*\(",
                                 text, re.M)))


def _check(rc: int):
    if rc != AFD_OK:
        raise AfdError(rc, load_library().afd_ffn_last_error().decode())


# ---- the C entry points, same names -------------------------------------
def afd_ffn_create(cfg: afd_ffn_config, w: afd_ffn_weights) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().afd_ffn_create(ctypes.byref(cfg), ctypes.byref(w),
                                         ctypes.byref(h)))
    return h


def afd_ffn_forward(h, hidden: int, out: int, T: int, stream: int):
    _check(load_library().afd_ffn_forward(h, hidden, out, T, stream))


def afd_ffn_forward_traced(h, hidden: int, out: int, T: int, stream: int,
                           trace: afd_ffn_trace):
    _check(load_library().afd_ffn_forward_traced(h, hidden, out, T, stream,
                                                 ctypes.byref(trace)))


def afd_ffn_forward_static(cfg: afd_ffn_config, w: afd_ffn_weights, hidden: int, out: int,
                           T: int, stream: int):
    _check(load_library().afd_ffn_forward_static(ctypes.byref(cfg), ctypes.byref(w), hidden,
                                                 out, T, stream))


def afd_ffn_destroy(h):
    load_library().afd_ffn_destroy(h)


def afd_quant_fp8_1x128(x: int, rows: int, cols: int, q: int, s: int, stream: int):
    _check(load_library().afd_quant_fp8_1x128(x, rows, cols, q, s, stream))


def afd_quant_fp8_1x128_f32(x: int, rows: int, cols: int, q: int, s: int, stream: int):
    _check(load_library().afd_quant_fp8_1x128_f32(x, rows, cols, q, s, stream))


def afd_quant_fp8_128x128(w: int, rows: int, cols: int, q: int, s: int, stream: int):
    _check(load_library().afd_quant_fp8_128x128(w, rows, cols, q, s, stream))


def afd_ffn_profile_enable(h, stage_mask: int):
    _check(load_library().afd_ffn_profile_enable(h, stage_mask))


def afd_ffn_profile_read(h):
    ms = (ctypes.c_double * len(STAGES))()
    n = (ctypes.c_int64 * len(STAGES))()
    _check(load_library().afd_ffn_profile_read(h, ms, n))
    return {STAGES[i]: (ms[i], n[i]) for i in range(len(STAGES))}


def afd_ffn_last_error() -> str:
    return load_library().afd_ffn_last_error().decode()
