"""ctypes view of ``libmla_decode.so`` (the C ABI in ``include/mla_decode.h``).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any entry point.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_decode.so")
# the debug build (-DMLA_DEBUG: device-side precondition checks, see build.py)
DEBUG_LIB_PATH = os.path.join(_PKG, "libmla_decode_debug.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_CAPACITY = 3
MLA_ERR_PRECONDITION = 4
MLA_ERR_DEVICE = 5
MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3 = 1

_c_i32, _c_i64, _c_f32, _c_p, _c_sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                       ctypes.c_void_p, ctypes.c_size_t)

# name -> (restype, argtypes), in the order of include/mla_decode.h
SIGNATURES = {
    "mla_abi_version": (_c_i32, []),
    "mla_status_string": (ctypes.c_char_p, [_c_i32]),
    "mla_last_error_message": (ctypes.c_char_p, []),
    "mla_build_block_table": (_c_i32, [_c_p, _c_i32, _c_i64, _c_p, _c_p, _c_i32, _c_i32, _c_p,
                                       _c_i32, _c_i32, _c_i32, _c_p]),
    "mla_plan_splits": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p]),
    "mla_build_table_and_plan": (_c_i32, [_c_p, _c_i32, _c_i64, _c_p, _c_p, _c_i32, _c_i32, _c_p,
                                          _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_p,
                                          _c_p, _c_p]),
    "mla_plan_fixed_splits": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p]),
    "mla_plan_fixed_packed": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p]),
    "mla_fixed_split_parts_bound": (_c_i32, [_c_i32, _c_i32, _c_i32]),
    "mla_max_total_splits": (_c_i32, [_c_i32, _c_i32]),
    "mla_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32]),
    "mla_partial_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32]),
    "mla_device_num_cus": (_c_i32, []),
    "mla_decode": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_p, _c_i32, _c_i64, _c_p, _c_i32,
                            _c_p, _c_p, _c_i32, _c_p, _c_f32, _c_i32, _c_p, _c_p, _c_p, _c_i32,
                            _c_p, _c_p, _c_p]),
    "mla_decode_q8": (_c_i32, [_c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_p, _c_i64, _c_p, _c_i32,
                               _c_p, _c_p, _c_i32, _c_p, _c_f32, _c_i32, _c_p, _c_p, _c_p,
                               _c_i32, _c_p, _c_p, _c_p]),
    "mla_merge_states": (_c_i32, [_c_p, _c_p, _c_i32, _c_p, _c_i32, _c_i32, _c_i32, _c_p, _c_p,
                                  _c_p]),
    "mla_decode_time_next_launch": (_c_i32, [_c_p, _c_p]),
    "mla_decode_static": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_p, _c_i32, _c_i64, _c_p,
                                   _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_f32, _c_i32, _c_p, _c_p,
                                   _c_p, _c_p]),
    "mla_set_kv_buffer": (_c_i32, [_c_p, _c_i64, _c_p, _c_i32, _c_p, _c_i32, _c_i64, _c_p, _c_p]),
    "mla_quantize_q_fp8": (_c_i32, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
}

_lib = None
_debug_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def load(path: str) -> ctypes.CDLL:
    """Load one build of the library and declare every entry point's types."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m paged_kv_mla_req_amd.build`")
    handle = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def debug_lib() -> ctypes.CDLL:
    """The debug build (a separate copy of the library, for tests of its
    precondition checks); raises if it has not been built."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = load(DEBUG_LIB_PATH)
    return _debug_lib


def check(status: int) -> None:
    if status != MLA_OK:
        msg = lib().mla_last_error_message().decode() or lib().mla_status_string(status).decode()
        raise MLAError(status, msg)
