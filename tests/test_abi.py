"""The C ABI library loads, exports every symbol include/lowrank.h declares,
and rejects bad arguments on the host before launching anything (CPU only:
no call here reaches a kernel launch)."""
import ctypes
import ctypes as C
import os
import re

import pytest

import rank_decomposed_amd as lr
from rank_decomposed_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "lowrank.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:lr_status|size_t|const char\*|int)\s+(\w+)\s*\(", text, re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = header_functions()
    for n in ("lowrank_linear_forward", "kv_remap_gather", "lowrank_prepare_decode",
              "lowrank_prepare_prefill", "lowrank_layer_prefill_step",
              "lowrank_workspace_bytes", "lowrank_status_string", "lowrank_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = lr.load()
    for n in header_functions():
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_status_strings_and_version():
    assert lr.lowrank_status_string(0) == "ok"
    for s in range(1, 8):
        assert lr.lowrank_status_string(s) not in ("ok", "unknown status")
    assert lr.lowrank_status_string(99) == "unknown status"
    assert lr.lowrank_version() >= 100


A16 = 1 << 20      # fake 16-byte-aligned "device" addresses: never dereferenced,
A2 = A16 + 2       # every call below fails validation before any launch


def _fwd(**kw):
    args = dict(dt=_lib.LR_BF16, T=4, d_in=64, r=16, d_out=32, x=A16, ldx=64, Ut=A16, ldu=64,
                Vt=A16, ldv=16, y=A16, ldy=32, t=None, ldt=0, flags=0, ws=None, wsb=0, st=None)
    args.update(kw)
    return lr.load().lowrank_linear_forward(
        args["dt"], args["T"], args["d_in"], args["r"], args["d_out"], args["x"], args["ldx"],
        args["Ut"], args["ldu"], args["Vt"], args["ldv"], args["y"], args["ldy"], args["t"],
        args["ldt"], args["flags"], args["ws"], args["wsb"], args["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), _lib.LR_ERR_DTYPE),
    (dict(T=0), _lib.LR_ERR_ARG),
    (dict(d_in=-1), _lib.LR_ERR_ARG),
    (dict(r=0), _lib.LR_ERR_ARG),
    (dict(x=None), _lib.LR_ERR_ARG),
    (dict(Vt=None), _lib.LR_ERR_ARG),
    (dict(ldx=63), _lib.LR_ERR_ARG),
    (dict(ldv=8), _lib.LR_ERR_ARG),
    (dict(flags=3), _lib.LR_ERR_ARG),
    (dict(flags=1), _lib.LR_ERR_ARG),           # stage-only needs t_io
    (dict(flags=2), _lib.LR_ERR_ARG),
    (dict(x=A2), _lib.LR_ERR_ALIGN),
    (dict(ldx=68, ldu=68), _lib.LR_ERR_ALIGN),  # bf16 ld must be a multiple of 8
    (dict(ldv=20), _lib.LR_ERR_ALIGN),
    (dict(t=A16 + 1, ldt=16), _lib.LR_ERR_ALIGN),
    (dict(ws=None, wsb=0), _lib.LR_ERR_WORKSPACE),   # decode path needs scratch
    (dict(ws=A16, wsb=16), _lib.LR_ERR_WORKSPACE),
    (dict(ws=A16 + 16, wsb=1 << 30), _lib.LR_ERR_WORKSPACE),  # not 256-aligned
    # decode path: 32-bit tile offsets need every ld below 2^24 elements
    (dict(ldx=1 << 24, ws=A16, wsb=1 << 30), _lib.LR_ERR_UNSUPPORTED),
    (dict(ldv=1 << 24, ws=A16, wsb=1 << 30), _lib.LR_ERR_UNSUPPORTED),
])
def test_linear_rejects_bad_arguments(kw, status):
    assert _fwd(**kw) == status


def test_workspace_sizes():
    # decode path: split-K partials plus the bf16 hi/lo copy of t
    assert lr.lowrank_workspace_bytes(0, lr.LR_BF16, 64, 4096, 1228, 4096) > 0
    # fused prefill keeps t on chip: no workspace
    assert lr.lowrank_workspace_bytes(0, lr.LR_BF16, 1023, 4096, 819, 4096) == 0
    # from 1024 rows on t is parked in the workspace: bf16 [T, round_up(r, 8)],
    # past the decode path's control area (8 blocks of 4096 words), which a
    # workspace shared with decode calls keeps for them
    ctl = 8 * 4096 * 4
    assert lr.lowrank_workspace_bytes(0, lr.LR_BF16, 16384, 4096, 819, 4096) == ctl + 16384 * 824 * 2
    # rank tile too large for LDS: t parked in the workspace as bf16
    assert lr.lowrank_workspace_bytes(0, lr.LR_BF16, 4096, 640, 1494, 640) >= ctl + 4096 * 1496 * 2
    assert lr.lowrank_workspace_bytes(0, lr.LR_F32, 4, 512, 128, 512) >= ctl + 4 * 128 * 4
    assert lr.lowrank_workspace_bytes(0, lr.LR_BF16, 0, 4096, 1228, 4096) == 0


def test_gather_rejects_bad_arguments():
    g = lr.load().kv_remap_gather
    assert g(5, A16, 10, 8, A16, 4, None, 8, A16, 8, None) == _lib.LR_ERR_DTYPE
    assert g(_lib.LR_BF16, None, 10, 8, A16, 4, None, 8, A16, 8, None) == _lib.LR_ERR_ARG
    assert g(_lib.LR_BF16, A16, 0, 8, A16, 4, None, 8, A16, 8, None) == _lib.LR_ERR_ARG
    assert g(_lib.LR_BF16, A16, 10, 4, A16, 4, None, 8, A16, 8, None) == _lib.LR_ERR_ARG
    assert g(_lib.LR_BF16, A16, 10, 8, A16, 4, None, 8, A16, 4, None) == _lib.LR_ERR_ARG
    assert g(_lib.LR_BF16, A16 + 1, 10, 8, A16, 4, None, 8, A16, 8, None) == _lib.LR_ERR_ALIGN
    assert g(_lib.LR_BF16, A16, 10, 8, A16 + 2, 4, None, 8, A16, 8, None) == _lib.LR_ERR_ALIGN
    assert g(_lib.LR_F32, A16 + 2, 10, 8, A16, 4, None, 8, A16, 8, None) == _lib.LR_ERR_ALIGN


def test_struct_layouts_match_the_library():
    import ctypes
    lib = lr.load()
    assert lib.lowrank_abi_sizeof(0) == ctypes.sizeof(lr.LayerWeights)
    assert lib.lowrank_abi_sizeof(1) == ctypes.sizeof(lr.DecodeState)
    assert lib.lowrank_abi_sizeof(2) == ctypes.sizeof(_lib.Linear)
    assert lib.lowrank_abi_sizeof(3) == ctypes.sizeof(lr.PrefillState)
    assert lib.lowrank_abi_sizeof(4) == 0


def test_decode_step_rejects_bad_arguments():
    import ctypes
    lib = lr.load()
    w, s = lr.LayerWeights(), lr.DecodeState()
    h = ctypes.c_void_p(A16)
    # all-zero structs: rejected by the host checks before any launch
    assert lib.lowrank_layer_decode_step(None, ctypes.byref(s), h, None, 0, None) == _lib.LR_ERR_ARG
    assert lib.lowrank_layer_decode_step(ctypes.byref(w), ctypes.byref(s), h, None, 0,
                                         None) == _lib.LR_ERR_ARG
    assert lib.lowrank_decode_step_workspace_bytes(ctypes.byref(w), ctypes.byref(s)) == 0
    assert lib.lowrank_rope_table(7, 10, 10000.0, A16, None) == _lib.LR_ERR_ARG
    assert lib.lowrank_rope_table(64, 0, 10000.0, A16, None) == _lib.LR_ERR_ARG


def _group(n=2, T=4, flags=0, ws=A16, wsb=1 << 30, **kw):
    arr = (_lib.Linear * max(n, 1))()
    for a in arr:
        a.d_in, a.r, a.d_out = 64, 16, 32
        a.x, a.ldx, a.Ut, a.ldu, a.Vt, a.ldv, a.y, a.ldy = A16, 64, A16, 64, A16, 16, A16, 32
    for k, v in kw.items():
        setattr(arr[0], k, v)
    return lr.load().lowrank_linear_forward_group(T, n, ctypes.cast(arr, ctypes.c_void_p), flags,
                                                  ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), _lib.LR_ERR_ARG),
    (dict(n=9), _lib.LR_ERR_ARG),
    (dict(T=65), _lib.LR_ERR_ARG),
    (dict(T=0), _lib.LR_ERR_ARG),
    (dict(flags=1), _lib.LR_ERR_ARG),                 # only LR_PACKED_WEIGHTS is a group flag
    (dict(x=None), _lib.LR_ERR_ARG),
    (dict(Vt=None), _lib.LR_ERR_ARG),                 # stage 1 only needs t_io
    (dict(y=None), _lib.LR_ERR_ARG),
    (dict(ldu=60), _lib.LR_ERR_ARG),
    (dict(x=A2), _lib.LR_ERR_ALIGN),
    (dict(ldv=20), _lib.LR_ERR_ALIGN),
    (dict(ws=None), _lib.LR_ERR_WORKSPACE),
    (dict(wsb=1024), _lib.LR_ERR_WORKSPACE),
    (dict(ldx=1 << 24), _lib.LR_ERR_UNSUPPORTED),
])
def test_group_rejects_bad_arguments(kw, status):
    assert _group(**kw) == status


def test_group_workspace_bounds():
    # a group's workspace holds the fixed control area (which single calls
    # use too) once, plus every member's scratch; a launch splits stage 1
    # into fewer K ranges the more row blocks its members have, so a member
    # needs no more partials inside a group than alone
    arr = (_lib.Linear * 3)()
    shapes = [(4096, 1228, 4096), (4096, 1228, 4096), (4096, 1791, 11008)]
    for a, (d_in, r, d_out) in zip(arr, shapes):
        a.d_in, a.r, a.d_out = d_in, r, d_out
    g = lr.load().lowrank_group_workspace_bytes(8, 3, ctypes.cast(arr, ctypes.c_void_p))
    singles = [lr.lowrank_workspace_bytes(0, lr.LR_BF16, 8, *sh) for sh in shapes]
    ctl = 8 * 4096 * 4
    assert all(s > ctl for s in singles)
    assert g > ctl
    assert g - ctl <= sum(s - ctl for s in singles)
    assert lr.load().lowrank_group_workspace_bytes(65, 3, ctypes.cast(arr, ctypes.c_void_p)) == 0


def _valid_step_structs():
    # LLaMA-7B-shaped layer at ratio 0.2 with fake aligned addresses: passes
    # every host check, so the calls below stop at the check named by each case
    w, s = lr.LayerWeights(), lr.DecodeState()
    w.d_model, w.n_heads, w.n_kv_heads, w.head_dim, w.d_ffn, w.eps = 4096, 32, 32, 128, 11008, 1e-5
    dims = [(4096, 4096)] * 4 + [(4096, 11008)] * 2 + [(11008, 4096)]
    for k, (a, b) in enumerate(dims):
        r = int(0.2 * a * b) // (a + b)
        w.Ut[k], w.Vt[k], w.r[k] = A16, A16, r
        w.ldu[k], w.ldv[k] = (a + 7) // 8 * 8, (r + 7) // 8 * 8
    w.attn_norm = w.ffn_norm = w.rope = A16
    w.rope_max_pos = 4112
    s.k_pool = s.v_pool = s.slot_mapping = s.remap = s.seq_off = s.pos = s.n_valid = A16
    s.pool_rows, s.pool_ld = 300000, 416
    s.B, s.cap, s.max_seq_rows = 64, 64 * 4112, 4112
    return w, s


@pytest.mark.parametrize("field,value,status", [
    (None, None, _lib.LR_ERR_WORKSPACE),          # valid; no workspace given
    ("B", 65, _lib.LR_ERR_UNSUPPORTED),           # projections run on the decode path
    ("head_dim", 96, _lib.LR_ERR_UNSUPPORTED),
    ("pool_ld", 409, _lib.LR_ERR_ALIGN),
    ("n_heads", 33, _lib.LR_ERR_ARG),             # not a multiple of n_kv_heads
    ("rope", A16 + 8, _lib.LR_ERR_ALIGN),         # rotary epilogue reads 16-byte quads
    ("mlp", 2, _lib.LR_ERR_ARG),                  # neither SwiGLU nor ReLU
])
def test_decode_step_host_checks(field, value, status):
    w, s = _valid_step_structs()
    if field is not None:
        setattr(w if hasattr(w, field) and field not in ("B", "pool_ld") else s, field, value)
    lib = lr.load()
    assert lib.lowrank_layer_decode_step(C.byref(w), C.byref(s), C.c_void_p(A16), None, 0,
                                         None) == status
    if field is None:
        assert lib.lowrank_decode_step_workspace_bytes(C.byref(w), C.byref(s)) > 0


def test_decode_step_relu_mlp_needs_no_up_projection():
    # a non-GLU layer leaves slot 5 empty and still passes every host check
    w, s = _valid_step_structs()
    w.mlp = lr.LR_MLP_RELU
    w.Ut[5] = w.Vt[5] = None
    w.r[5] = 0
    lib = lr.load()
    assert lib.lowrank_layer_decode_step(C.byref(w), C.byref(s), C.c_void_p(A16), None, 0,
                                         None) == _lib.LR_ERR_WORKSPACE
    relu_ws = lib.lowrank_decode_step_workspace_bytes(C.byref(w), C.byref(s))
    w.mlp = lr.LR_MLP_SWIGLU
    assert lib.lowrank_layer_decode_step(C.byref(w), C.byref(s), C.c_void_p(A16), None, 0,
                                         None) == _lib.LR_ERR_ARG     # SwiGLU needs slot 5
    w2, s2 = _valid_step_structs()
    assert 0 < relu_ws < lib.lowrank_decode_step_workspace_bytes(C.byref(w2), C.byref(s2))


def _valid_prefill_state(T=300, S=4):
    _, s = _valid_step_structs()
    p = lr.PrefillState()
    p.k_pool, p.v_pool, p.pool_rows, p.pool_ld = s.k_pool, s.v_pool, s.pool_rows, s.pool_ld
    p.slot_mapping = p.remap = p.seq_off = p.tok_seq = p.pos = p.n_valid = A16
    p.T, p.S, p.cap, p.max_seq_rows = T, S, 4 * 4112, 4112
    return p


@pytest.mark.parametrize("field,value,status", [
    (None, None, _lib.LR_ERR_WORKSPACE),          # valid; no workspace given
    ("tok_seq", None, _lib.LR_ERR_ARG),
    ("S", 256, _lib.LR_ERR_UNSUPPORTED),          # rotary epilogue stages S + 1 offsets
    ("T", 0, _lib.LR_ERR_ARG),
])
def test_prefill_step_host_checks(field, value, status):
    w, _ = _valid_step_structs()
    p = _valid_prefill_state()
    if field is not None:
        setattr(p, field, value)
    lib = lr.load()
    assert lib.lowrank_layer_prefill_step(C.byref(w), C.byref(p), C.c_void_p(A16), None, 0,
                                          None) == status
    if field is None:
        # 300 tokens take the prefill path: more scratch than a 64-token chunk
        small = lib.lowrank_prefill_step_workspace_bytes(C.byref(w), C.byref(_valid_prefill_state(64)))
        assert lib.lowrank_prefill_step_workspace_bytes(C.byref(w), C.byref(p)) > small > 0
