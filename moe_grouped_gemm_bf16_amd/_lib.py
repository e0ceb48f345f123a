"""ctypes view of libmgemm.so (the C ABI declared in include/mgemm.h).

Loading never falls back to anything: if the library is missing or broken,
importing raises, naming the file and how to build it.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmgemm.so")

# status codes of mg_status
MG_OK, MG_ERR_NULL, MG_ERR_SHAPE, MG_ERR_ALIGN, MG_ERR_DEVICE, MG_ERR_LAUNCH, MG_ERR_OFFSETS = range(7)

# name -> (restype, argtypes); the exported symbols of include/mgemm.h
_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "mgemm_fwd": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _vp]),
    "mgemm_dgrad": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _vp]),
    "kgemm_wgrad": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp]),
    "kgemm_wgrad_noalloc": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp]),
    "mgemm_fwd_swiglu": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _i64, _vp]),
    "mgemm_fwd_swiglu_gu": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _i64,
                                   _vp]),
    "mgemm_dgrad_swiglu": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _vp]),
    "mg_moe_combine": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i64, _vp]),
    "mgemm_list": (_i32, [_vp, _i32, _vp]),
    "mgemm_fwd_mx": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _vp]),
    "mg_mx_scales_blocked": (_i32, [_vp, _vp, _i64, _i64, _i64, _vp]),
    "kgemm_wgrad_mx": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp]),
    "kgemm_wgrad_mx_tm": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp]),
    "mg_check_list_host": (_i32, [_vp, _i32]),
    "mg_status_str": (ctypes.c_char_p, [_i32]),
    "mg_abi_version": (_i32, []),
    "mg_check_offsets_host": (_i32, [_vp, _i32, _i64]),
}


class GemmDesc(ctypes.Structure):
    """mg_gemm_desc of include/mgemm.h: one group of mgemm_list."""
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("m", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("lda", ctypes.c_int32), ("ldb", ctypes.c_int32), ("ldd", ctypes.c_int32)]


assert ctypes.sizeof(GemmDesc) == 48


class MgemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python moe_grouped_gemm_bf16_amd/build.py` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.mg_abi_version() != 1:
        raise ImportError(f"{LIB_PATH}: unexpected ABI version {lib.mg_abi_version()}")
    return lib


LIB = _load()


def status_str(status: int) -> str:
    return LIB.mg_status_str(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != MG_OK:
        raise MgemmError(status, what)
