"""ctypes declarations of liblsh.so (include/lsh.h)."""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "liblsh.so")

LSH_OK, LSH_ERR_INVALID, LSH_ERR_UNSUPPORTED, LSH_ERR_WORKSPACE, LSH_ERR_NO_DEVICE, LSH_ERR_HIP = range(6)
LSH_F32, LSH_BF16 = 0, 1
ABI_VERSION = 1

# Every function the header declares, with (restype, argtypes).
c_i64 = ctypes.c_int64
c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("q", c_vp), ("k", c_vp), ("v", c_vp), ("o", c_vp), ("lse", c_vp),
        ("dtype", c_i32), ("reserved", c_i32),
        ("B", c_i64), ("Sq", c_i64), ("Skv", c_i64), ("H", c_i64), ("D", c_i64),
        ("q_stride", c_i64 * 3), ("k_stride", c_i64 * 3), ("v_stride", c_i64 * 3),
        ("o_stride", c_i64 * 3),
        ("scale", ctypes.c_float),
    ]


class AttnBwdArgs(ctypes.Structure):
    _fields_ = [
        ("q", c_vp), ("k", c_vp), ("v", c_vp), ("dout", c_vp), ("o", c_vp), ("lse", c_vp),
        ("dq", c_vp), ("dk", c_vp), ("dv", c_vp),
        ("dtype", c_i32), ("reserved", c_i32),
        ("B", c_i64), ("Sq", c_i64), ("Skv", c_i64), ("H", c_i64), ("D", c_i64),
        ("q_stride", c_i64 * 3), ("k_stride", c_i64 * 3), ("v_stride", c_i64 * 3),
        ("do_stride", c_i64 * 3), ("o_stride", c_i64 * 3), ("dq_stride", c_i64 * 3),
        ("dk_stride", c_i64 * 3), ("dv_stride", c_i64 * 3),
        ("scale", ctypes.c_float),
    ]


_ARGS_P = ctypes.POINTER(AttnArgs)
_BWD_P = ctypes.POINTER(AttnBwdArgs)
SIGNATURES = {
    "lsh_abi_version": (ctypes.c_int, []),
    "lsh_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "lsh_last_error": (ctypes.c_char_p, []),
    "lsh_device_check": (ctypes.c_int, []),
    "lsh_attn_fwd": (ctypes.c_int, [_ARGS_P, c_vp]),
    "lsh_attn_fwd_chunked": (ctypes.c_int, [_ARGS_P, ctypes.POINTER(c_i32), c_i32, c_vp,
                                            ctypes.c_size_t, c_vp, c_vp]),
    "lsh_attn_fwd_chunked_workspace": (ctypes.c_size_t, [_ARGS_P]),
    "lsh_attn_partial": (ctypes.c_int, [_ARGS_P, c_vp]),
    "lsh_attn_partial_accumulate": (ctypes.c_int, [_ARGS_P, c_vp]),
    "lsh_lse_merge": (ctypes.c_int, [c_vp, c_vp, c_i32, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "lsh_head_permute": (ctypes.c_int, [c_vp, c_vp, c_i32, c_i64, c_i64, c_i64, c_i64, c_i32, c_i32, c_vp]),
    "lsh_attn_fwd_blocksparse": (ctypes.c_int, [_ARGS_P, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "lsh_attn_fwd_blocksparse_workspace": (ctypes.c_size_t, [_ARGS_P]),
    "lsh_attn_fwd_blocksparse_noalloc": (ctypes.c_int, [_ARGS_P, c_vp, c_vp]),
    "lsh_attn_bwd": (ctypes.c_int, [_BWD_P, c_vp, ctypes.c_size_t, c_vp]),
    "lsh_attn_bwd_workspace": (ctypes.c_size_t, [_BWD_P]),
}

_lock = threading.Lock()
_lib = None


class LshError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads liblsh.so once. Raises RuntimeError if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build the HIP library first "
                "(python -m long_sequence_head_amd.build)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.lsh_abi_version() != ABI_VERSION:
            raise RuntimeError("liblsh.so ABI version mismatch")
        _lib = lib
        return lib


def check(fn: str, status: int):
    if status != LSH_OK:
        lib = load()
        raise LshError(fn, status, lib.lsh_last_error().decode() or lib.lsh_status_str(status).decode())
