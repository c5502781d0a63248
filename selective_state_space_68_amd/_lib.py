"""ctypes view of libssm.so (the C ABI declared in include/ssm.h).

Only argument marshalling lives here: every step of the computation runs in the
library's gfx950 kernels.  The library is loaded on first use; a missing or
unloadable library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssm.so")

SSM_OK = 0
SSM_ERR_INVALID_ARG = 1
SSM_ERR_UNSUPPORTED = 2
SSM_ERR_HIP = 3
SSM_ERR_TOO_LARGE = 4

SSM_F32 = 0
SSM_BF16 = 1

SSM_SCAN_AUTO = 0
SSM_SCAN_SEQUENTIAL = 1
SSM_SCAN_CHUNKED = 2
SSM_SCAN_TOKSEQ = 3
SSM_SCAN_AP = 16

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/ssm.h and include/ssm_calib.h
SIGNATURES = {
    "ssm_selective_scan_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp,
                                      _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]),
    "ssm_selective_scan_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _int]),
    "ssm_selective_scan_fwd_from_state": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp,
                                                 _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]),
    "ssm_selective_scan_fwd_variant": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp,
                                              _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp, _int, _int]),
    "ssm_selective_scan_fwd_kernel": (_int, [_i64, _i64, _i64, _i64, _int, _int, _int, _int, _int, _int]),
    "ssm_selective_scan_fwd_zoh": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp,
                                          _i64, _i64, _i64, _i64, _int, _vp]),
    "ssm_state_update_zoh": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp,
                                    _i64, _i64, _i64, _int, _vp]),
    "ssm_causal_conv1d_fwd": (_int, [_vp, _vp, _vp, _i64, _int, _vp, _i64, _i64, _i64, _int, _vp]),
    "ssm_selective_scan_fwd_conv": (_int, [_vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp,
                                           _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp, _int]),
    "ssm_state_update": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp,
                                _i64, _i64, _i64, _int, _vp]),
    "ssm_selective_scan_bwd_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _int]),
    "ssm_selective_scan_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]),
    "ssm_selective_scan_fwd_save": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp,
                                           _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]),
    "ssm_selective_scan_bwd_saved_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _int]),
    "ssm_selective_scan_bwd_saved": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp,
                                            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]),
    "ssm_ssd_scan_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64, _int]),
    "ssm_ssd_scan_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp,
                                _i64, _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]),
    "ssm_ssd_scan_fwd_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp,
                                        _i64, _i64, _i64, _i64, _i64, _int, _vp]),
    "ssm_status_string": (ctypes.c_char_p, [_int]),
    "ssm_calib_copy": (_int, [_vp, _vp, _sz, _vp]),
    "ssm_calib_alu": (_int, [_int, _vp, _i64, _int, _vp]),
    "ssm_calib_alu_ops": (_i64, [_i64, _int]),
    "ssm_version": (_int, []),
}

_lock = threading.Lock()
_lib = None


class SsmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libssm.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m selective_state_space_68_amd.build_lib` "
                "(or __graft_entry__.build()); there is no fallback implementation")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().ssm_status_string(int(status)).decode()


def check(status: int) -> None:
    if status != SSM_OK:
        raise SsmError(status, status_string(status))
