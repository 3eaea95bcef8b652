"""ctypes declarations of liblowrank.so (the C ABI in include/lowrank.h).

Argument marshalling only: every computation happens in the library.  Loading
fails loudly when the shared library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblowrank.so")

LR_OK, LR_ERR_ARG, LR_ERR_DTYPE, LR_ERR_ALIGN, LR_ERR_WORKSPACE, LR_ERR_CAPACITY, \
    LR_ERR_HIP, LR_ERR_UNSUPPORTED = range(8)
LR_F32, LR_BF16 = 0, 1
LR_FULL, LR_STAGE1_ONLY, LR_STAGE2_ONLY = 0, 1, 2

# every symbol include/lowrank.h declares, with (restype, argtypes)
_i64, _u, _sz, _p, _pi32 = C.c_int64, C.c_uint, C.c_size_t, C.c_void_p, C.c_void_p
SIGNATURES = {
    "lowrank_linear_forward": (C.c_int, [C.c_int, _i64, _i64, _i64, _i64, _p, _i64, _p, _i64,
                                         _p, _i64, _p, _i64, _p, _i64, _u, _p, _sz, _p]),
    "kv_remap_gather": (C.c_int, [C.c_int, _p, _i64, _i64, _pi32, _i64, _pi32, _i64, _p, _i64,
                                  _p]),
    "lowrank_prepare_decode": (C.c_int, [_i64, _pi32, _pi32, _i64, _i64, _i64, _pi32, _pi32,
                                         _pi32, _pi32, _pi32, _pi32, _pi32, _i64]),
    "lowrank_workspace_bytes": (C.c_size_t, [C.c_int, C.c_int, _i64, _i64, _i64, _i64, _i64]),
    "lowrank_status_string": (C.c_char_p, [C.c_int]),
    "lowrank_version": (C.c_int, []),
}

_lib = None


class LowrankError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, status_string(status), status))


def load():
    """Load liblowrank.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("liblowrank.so is not built (%s); run `python -m "
                           "rank_decomposed_amd.build`" % LIB_PATH)
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(s: int) -> str:
    return load().lowrank_status_string(int(s)).decode()


def check(status: int, where: str):
    if status != LR_OK:
        raise LowrankError(status, where)
