"""ctypes view of the C ABI declared in include/fa_gfx950.h.

Loading fails loudly (FaLibraryMissing) when libfa_gfx950.so has not been built:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_gfx950.so")
# check build: every buffer->LDS load batch waited for as soon as it is issued
SERIAL_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_gfx950_serial.so")

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE_TOO_SMALL = 3
FA_ERR_HIP = 4
FA_BWD_PHASE_PRE = 1
FA_BWD_PHASE_MAIN = 2
FA_BWD_PHASE_POST = 4
FA_BWD_PHASE_ALL = 7
FA_DTYPE_BF16 = 0
FA_DTYPE_F32 = 1


class FaLibraryMissing(RuntimeError):
    pass


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status_str(status)} ({status})")


Strides = c_int64 * 3


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("o", c_void_p), ("lse", c_void_p),
        ("q_stride", Strides), ("k_stride", Strides), ("v_stride", Strides), ("o_stride", Strides),
        ("batch", c_int32), ("seqlen_q", c_int32), ("seqlen_k", c_int32), ("num_heads", c_int32),
        ("head_dim", c_int32),
        ("cu_seqlens_q", c_void_p), ("cu_seqlens_k", c_void_p),
        ("max_seqlen_q", c_int32), ("max_seqlen_k", c_int32), ("total_q", c_int32), ("total_k", c_int32),
        ("softmax_scale", c_float), ("causal", c_int32), ("o_dtype", c_int32),
    ]


class FwdTuning(ctypes.Structure):
    _fields_ = [("exp2_poly_per16", c_int32), ("rescale_threshold_log2", c_int32),
                ("q_tiles_per_workgroup", c_int32), ("key_splits", c_int32)]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("o", c_void_p), ("dout", c_void_p),
        ("lse", c_void_p), ("dq", c_void_p), ("dk", c_void_p), ("dv", c_void_p),
        ("q_stride", Strides), ("k_stride", Strides), ("v_stride", Strides), ("o_stride", Strides),
        ("do_stride", Strides), ("dq_stride", Strides), ("dk_stride", Strides), ("dv_stride", Strides),
        ("batch", c_int32), ("seqlen_q", c_int32), ("seqlen_k", c_int32), ("num_heads", c_int32),
        ("head_dim", c_int32),
        ("cu_seqlens_q", c_void_p), ("cu_seqlens_k", c_void_p),
        ("max_seqlen_q", c_int32), ("max_seqlen_k", c_int32), ("total_q", c_int32), ("total_k", c_int32),
        ("softmax_scale", c_float), ("causal", c_int32), ("deterministic", c_int32), ("grad_dtype", c_int32),
    ]


_lib = None

# name -> (restype, argtypes) for every entry point of include/fa_gfx950.h
SIGNATURES = {
    "fa_fwd_workspace_size": (c_int32, [POINTER(FwdArgs), POINTER(FwdTuning), POINTER(c_size_t)]),
    "fa_fwd": (c_int32, [POINTER(FwdArgs), POINTER(FwdTuning), c_void_p, c_size_t, c_void_p]),
    "fa_fwd_build_schedule": (c_int32, [POINTER(FwdArgs), POINTER(FwdTuning), c_void_p, c_size_t, c_void_p]),
    "fa_fwd_tile_rows": (c_int32, [POINTER(FwdTuning)]),
    "fa_exp2_probe": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p]),
    "fa_bwd_workspace_size": (c_int32, [POINTER(BwdArgs), POINTER(c_size_t)]),
    "fa_bwd": (c_int32, [POINTER(BwdArgs), c_void_p, c_size_t, c_void_p]),
    "fa_bwd_phases": (c_int32, [POINTER(BwdArgs), c_int32, c_void_p, c_size_t, c_void_p]),
    "fa_bwd_noalloc": (c_int32, [POINTER(BwdArgs), c_void_p]),
    "fa_bwd_noalloc_scratch_bytes": (c_size_t, []),
    "fa_status_str": (c_char_p, [c_int32]),
    "fa_version": (c_char_p, []),
}


def load(path: str):
    """A handle on the library at `path` with every entry point's signature set."""
    if not os.path.exists(path):
        raise FaLibraryMissing(
            f"{path} is not built; run `python -m tiled_exact_attention_bf16_amd.build_lib` "
            "(there is no fallback implementation)")
    handle = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib():
    """The loaded library (built in place by build_lib.py); raises if it is missing."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def status_str(status: int) -> str:
    return lib().fa_status_str(status).decode()


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)
