"""ctypes loader for libsagebwd.so (the HIP kernels behind the C ABI in include/sagebwd.h).

There is no fallback: if the library is missing the import fails loudly.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsagebwd.so")

SAGEBWD_FP16 = 0
SAGEBWD_BF16 = 1
DQ_AUTO, DQ_SPILL, DQ_ATOMIC = 0, 1, 2
LAYOUT_BHND, LAYOUT_BNHD = 0, 1
FMT_INT8, FMT_FP8 = 0, 1   # sagebwd_fmt
SPLIT_SAGEBWD, SPLIT_QATTN = 0, 1   # sagebwd_split

# Quantisation tile shapes of the kernels (include/sagebwd.h); the backward's P and dS tiles
# span one query block (blk rows) by BWD_P_TILE_K and min(blk, BWD_DS_TILE_K) keys.
FWD_TILE_Q = 32
BWD_P_TILE_K = 16
BWD_DS_TILE_K = 64
QATTN_FWD_TILE_K = 64

STATUS = {
    0: "SAGEBWD_OK", -1: "SAGEBWD_ERR_NULL", -2: "SAGEBWD_ERR_SHAPE", -3: "SAGEBWD_ERR_UNSUPPORTED",
    -4: "SAGEBWD_ERR_ALIGN", -5: "SAGEBWD_ERR_WORKSPACE", -6: "SAGEBWD_ERR_HIP", -7: "SAGEBWD_ERR_SCRATCH",
}

NOALLOC_SCRATCH_BYTES = 16 << 20   # SAGEBWD_NOALLOC_SCRATCH_BYTES


class Params(ctypes.Structure):
    """Mirror of sagebwd_params."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
        ("blk", ctypes.c_int32), ("causal", ctypes.c_int32), ("qk_norm", ctypes.c_int32),
        ("k_smooth", ctypes.c_int32), ("eps", ctypes.c_float), ("sm_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32), ("dq_mode", ctypes.c_int32), ("q_smooth", ctypes.c_int32),
        ("layout", ctypes.c_int32), ("qk_gain", ctypes.c_int32), ("normed_grads", ctypes.c_int32),
        ("fmt", ctypes.c_int32), ("split", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_SIZE = ctypes.c_size_t
_ST = ctypes.c_int

SIGNATURES = {
    "sagebwd_prologue_workspace_bytes": (_SIZE, [ctypes.POINTER(Params)]),
    "sagebwd_quant_prologue": (_ST, [ctypes.POINTER(Params)] + [_P] * 16 + [_P, _SIZE, _P]),
    "sagebwd_quant_prologue_noalloc": (_ST, [ctypes.POINTER(Params)] + [_P] * 16 + [_P]),
    "sagebwd_forward": (_ST, [ctypes.POINTER(Params)] + [_P] * 10 + [_P]),
    "sagebwd_backward_workspace_bytes": (_SIZE, [ctypes.POINTER(Params)]),
    "sagebwd_backward": (_ST, [ctypes.POINTER(Params)] + [_P] * 21 + [_P, _SIZE, _P]),
    "sagebwd_backward_part": (_ST, [ctypes.POINTER(Params), ctypes.c_int32] + [_P] * 21 + [_P, _SIZE, _P]),
    "sagebwd_status_string": (ctypes.c_char_p, [_ST]),
    "sagebwd_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libsagebwd.so once; raise if it has not been built.

    torch is imported first so that the library binds to the HIP runtime torch already
    loaded. Both runtimes carry the soname libamdhip64.so.7, but torch asks for it as
    libamdhip64.so; if the library were loaded first, torch would bring a second HIP/HSA
    runtime into the process and the library's runtime would find no device.
    """
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m bit_trainable_attention_amd.build`")
        import torch  # noqa: F401  (binds the HIP runtime; see above)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
