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
    LR_ERR_HIP, LR_ERR_UNSUPPORTED, LR_ERR_WAIT = range(9)
LR_DEFAULT_WAIT_LIMIT = 1 << 20
LR_NOALLOC_SCRATCH_BYTES = 8 << 20
LR_F32, LR_BF16 = 0, 1
LR_FULL, LR_STAGE1_ONLY, LR_STAGE2_ONLY = 0, 1, 2
LR_PACKED_WEIGHTS = 4
LR_PREFILL_FUSED = 8

# every symbol include/lowrank.h declares, with (restype, argtypes)
_i64, _u, _sz, _p, _pi32 = C.c_int64, C.c_uint, C.c_size_t, C.c_void_p, C.c_void_p
SIGNATURES = {
    "lowrank_linear_forward": (C.c_int, [C.c_int, _i64, _i64, _i64, _i64, _p, _i64, _p, _i64,
                                         _p, _i64, _p, _i64, _p, _i64, _u, _p, _sz, _p]),
    "kv_remap_gather": (C.c_int, [C.c_int, _p, _i64, _i64, _pi32, _i64, _pi32, _i64, _p, _i64,
                                  _p]),
    "lowrank_prepare_decode": (C.c_int, [_i64, _pi32, _pi32, _i64, _i64, _i64, _pi32, _pi32,
                                         _pi32, _pi32, _pi32, _pi32, _pi32, _i64]),
    "lowrank_prepare_prefill": (C.c_int, [_i64, _pi32, _pi32, _pi32, _i64, _i64, _i64, _i64,
                                          _pi32, _pi32, _pi32, _pi32, _pi32, _pi32, _pi32,
                                          _pi32, _pi32, _i64]),
    "lowrank_workspace_bytes": (C.c_size_t, [C.c_int, C.c_int, _i64, _i64, _i64, _i64, _i64]),
    "lowrank_status_string": (C.c_char_p, [C.c_int]),
    "lowrank_version": (C.c_int, []),
    "lowrank_abi_sizeof": (C.c_size_t, [C.c_int]),
    "lowrank_rope_table": (C.c_int, [_i64, _i64, C.c_float, _p, _p]),
    "lowrank_decode_step_workspace_bytes": (C.c_size_t, [_p, _p]),
    "lowrank_layer_decode_step": (C.c_int, [_p, _p, _p, _p, _sz, _p]),
    "lowrank_decode_step_fused_workspace_bytes": (C.c_size_t, [_p, _p]),
    "lowrank_layer_decode_step_fused": (C.c_int, [_p, _p, _p, _p, _sz, _p]),
    "lowrank_prefill_step_workspace_bytes": (C.c_size_t, [_p, _p]),
    "lowrank_layer_prefill_step": (C.c_int, [_p, _p, _p, _p, _sz, _p]),
    "lowrank_packed_bytes": (C.c_size_t, [_i64, _i64]),
    "lowrank_group_workspace_bytes": (C.c_size_t, [_i64, C.c_int, _p]),
    "lowrank_linear_forward_group": (C.c_int, [_i64, C.c_int, _p, _u, _p, _sz, _p]),
    "lowrank_pack_factor": (C.c_int, [_p, _i64, _i64, _i64, _p, _i64, _p]),
    "lowrank_workspace_check": (C.c_int, [_p, _sz, _p, _p]),
    "lowrank_linear_forward_noalloc": (C.c_int, [C.c_int, _i64, _i64, _i64, _i64, _p, _i64, _p,
                                                 _i64, _p, _i64, _p, _i64, _p, _i64, _u, _p]),
    "lowrank_set_wait_limit": (None, [C.c_uint32]),
}


class LayerWeights(C.Structure):
    """lr_layer_weights (include/lowrank.h)."""
    _fields_ = [("d_model", C.c_int64), ("n_heads", C.c_int64), ("n_kv_heads", C.c_int64),
                ("head_dim", C.c_int64), ("d_ffn", C.c_int64), ("eps", C.c_float),
                ("Ut", C.c_void_p * 7), ("ldu", C.c_int64 * 7), ("Vt", C.c_void_p * 7),
                ("ldv", C.c_int64 * 7), ("r", C.c_int64 * 7), ("attn_norm", C.c_void_p),
                ("ffn_norm", C.c_void_p), ("rope", C.c_void_p), ("rope_max_pos", C.c_int64),
                ("mlp", C.c_int64)]


class PrefillState(C.Structure):
    """lr_prefill_state (include/lowrank.h)."""
    _fields_ = [("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("pool_rows", C.c_int64),
                ("pool_ld", C.c_int64), ("slot_mapping", C.c_void_p), ("remap", C.c_void_p),
                ("seq_off", C.c_void_p), ("tok_seq", C.c_void_p), ("pos", C.c_void_p),
                ("n_valid", C.c_void_p), ("T", C.c_int64), ("S", C.c_int64), ("cap", C.c_int64),
                ("max_seq_rows", C.c_int64)]


class Linear(C.Structure):
    """lr_linear (include/lowrank.h)."""
    _fields_ = [("d_in", C.c_int64), ("r", C.c_int64), ("d_out", C.c_int64),
                ("x", C.c_void_p), ("ldx", C.c_int64), ("Ut", C.c_void_p), ("ldu", C.c_int64),
                ("Vt", C.c_void_p), ("ldv", C.c_int64), ("y", C.c_void_p), ("ldy", C.c_int64),
                ("y_acc", C.c_void_p), ("ld_acc", C.c_int64), ("t_io", C.c_void_p),
                ("ldt", C.c_int64)]


class DecodeState(C.Structure):
    """lr_decode_state (include/lowrank.h)."""
    _fields_ = [("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("pool_rows", C.c_int64),
                ("pool_ld", C.c_int64), ("slot_mapping", C.c_void_p), ("remap", C.c_void_p),
                ("seq_off", C.c_void_p), ("pos", C.c_void_p), ("n_valid", C.c_void_p),
                ("B", C.c_int64), ("cap", C.c_int64), ("max_seq_rows", C.c_int64)]

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
