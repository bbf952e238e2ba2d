"""ctypes loader for libsas.so (the C ABI declared in include/sas.h).

The library is loaded on first use.  If it has not been built the loader
raises immediately: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsas.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "sas.h")

SAS_BF16 = 0
SAS_FP32 = 1

SAS_GATE_SOFTMAX = 0
SAS_GATE_SIGMOID = 1
SAS_GATE_RAW = 2
SAS_GATE_INNER = 0
SAS_GATE_OUTER = 1
GATE_ACTS = {"softmax": SAS_GATE_SOFTMAX, "sigmoid": SAS_GATE_SIGMOID, "raw": SAS_GATE_RAW}
GATE_POS = {"inner": SAS_GATE_INNER, "outer": SAS_GATE_OUTER}
SAS_GATE_SOFT = 0
SAS_GATE_HARD_STE = 1
GATE_RANK = {"soft": SAS_GATE_SOFT, "hard_ste": SAS_GATE_HARD_STE}

SAS_OK = 0
SAS_E_INVALID = -1
SAS_E_UNSUPPORTED = -2
SAS_E_WORKSPACE = -3
SAS_E_CAPACITY = -4
SAS_E_HIP = -5

STATUS_NAMES = {SAS_OK: "SAS_OK", SAS_E_INVALID: "SAS_E_INVALID",
                SAS_E_UNSUPPORTED: "SAS_E_UNSUPPORTED", SAS_E_WORKSPACE: "SAS_E_WORKSPACE",
                SAS_E_CAPACITY: "SAS_E_CAPACITY", SAS_E_HIP: "SAS_E_HIP"}


class SasProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("budget_k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("o_dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("gate_act", ctypes.c_int32), ("gate_pos", ctypes.c_int32),
                ("gate_rank", ctypes.c_int32), ("n_score_heads", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("total_tokens", ctypes.c_int64)]


class SasDecodeProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("pool_blocks", ctypes.c_int32), ("budget_k", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float)]


_P = ctypes.POINTER(SasProblem)
_PD = ctypes.POINTER(SasDecodeProblem)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32

SIGNATURES = {
    "sas_abi_version": ([], _i32),
    "sas_last_error": ([], ctypes.c_char_p),
    "sas_gate_threshold": ([_P, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp], _i32),
    "sas_gated_attn_fwd": ([_P, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp], _i32),
    "sas_gated_attn_bwd_workspace_size": ([_P, _i32], ctypes.c_size_t),
    "sas_gated_attn_bwd": ([_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                            _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp], _i32),
    "sas_gated_attn_bwd_dq": ([_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                               _vp, _vp, ctypes.c_size_t, _vp], _i32),
    "sas_gated_attn_bwd_dkdv": ([_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                 _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp], _i32),
    "sas_decode_select": ([_PD, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp], _i32),
    "sas_decode_workspace_size": ([_PD, _i32], ctypes.c_size_t),
    "sas_decode_attn": ([_PD, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                         ctypes.c_size_t, _vp, _vp], _i32),
    "sas_decode_attn_noalloc": ([_PD, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                 _vp], _i32),
}
DECODE_SCRATCH_BYTES = 32 << 20   # SAS_DECODE_SCRATCH_BYTES

_lib = None


class SasError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


def lib():
    """The loaded library (raises if libsas.so has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m gated_block_sparse_attn_amd.build` "
                "(the HIP library is the only implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def header_symbols():
    """Names of the functions declared in include/sas.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(sas_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def check(status: int) -> None:
    if status != SAS_OK:
        msg = lib().sas_last_error()
        raise SasError(status, msg.decode() if msg else "")
