"""ctypes binding of libbased.so (declarations in include/based.h). Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbased.so")

BASED_OK = 0
BASED_ERR_INVALID_ARGUMENT = 1
BASED_ERR_UNSUPPORTED = 2
BASED_ERR_HIP = 3
BASED_ERR_OUT_OF_MEMORY = 4
BASED_ERR_WORKSPACE_TOO_SMALL = 5
BASED_BF16 = 0
BASED_F32 = 1

# Every symbol include/based.h declares, with its ctypes signature.
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
SIGNATURES = {
    "based_abi_version": (ctypes.c_int, []),
    "based_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "based_last_error_detail": (ctypes.c_char_p, []),
    "based_forward_workspace_bytes": (ctypes.c_size_t, [_i64] * 5),
    "based_forward": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_float, _vp,
                                     ctypes.c_int, _vp]),
    "based_forward_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_float, _vp,
                                             ctypes.c_int, _vp]),
    "based_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "based_forward_ws": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_float, _vp,
                                        ctypes.c_int, _vp, ctypes.c_size_t, _vp]),
    "based_forward_plan": (ctypes.c_int, [_i64] * 6 + [ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                                        ctypes.POINTER(ctypes.c_size_t)]),
    "based_timer_create": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(_vp)]),
    "based_timer_destroy": (None, [_vp]),
    "based_timer_reset": (None, [_vp]),
    "based_timer_set_kernel_mask": (None, [_vp, ctypes.c_uint]),
    "based_timer_read": (ctypes.c_int, [_vp, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_double)]),
    "based_kernel_name": (ctypes.c_char_p, [ctypes.c_int]),
    "based_device_info": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                         ctypes.POINTER(ctypes.c_int)]),
    "based_forward_ex": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_float, _vp,
                                        ctypes.c_int, _vp, ctypes.c_size_t, _i64, _vp, _vp]),
    "based_feature_dim": (_i64, [_i64]),
    "based_forward_state": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_float, _vp,
                                           ctypes.c_int, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "based_decode_step": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_float, _vp, _vp, _vp,
                                         ctypes.c_int, _vp]),
}

_lib = None


class BasedError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)}): {detail}")


def lib() -> ctypes.CDLL:
    """Load libbased.so (built in-tree by taylor_feature_map_amd.build). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m taylor_feature_map_amd.build`")
        cdll = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(cdll, name)
            fn.restype = res
            fn.argtypes = args
        _lib = cdll
    return _lib


def status_string(status: int) -> str:
    return lib().based_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status != BASED_OK:
        raise BasedError(status, where, lib().based_last_error_detail().decode())
