"""rank_decomposed_amd -- the low-rank decomposed hot path on AMD MI355X.

Python binding of liblowrank.so with the C ABI's names.  The functions only
marshal arguments (shapes, leading dimensions, pointers, the current HIP
stream) from PyTorch tensors; every step of the computation runs in the
library's HIP kernels (or, for the preparation stage, its host C++ code).
PyTorch provides device memory and streams.

Layout reminder (include/lowrank.h): x [T, d_in], Ut = U_r^T [r, d_in],
Vt = V_r^T [d_out, r], y [T, d_out], t [T, r] fp32; row-major with explicit
leading dimensions, so tensor-parallel shares are plain slices
(``Ut[:, rows]``, ``Vt[cols, :]``).
"""
from __future__ import annotations

import ctypes as C
import weakref

import numpy as np

from . import _lib
from ._lib import (LR_BF16, LR_DEFAULT_WAIT_LIMIT, LR_ERR_WAIT, LR_F32, LR_FULL,
                   LR_NOALLOC_SCRATCH_BYTES, LR_PACKED_WEIGHTS, LR_PREFILL_FUSED,
                   LR_STAGE1_ONLY, LR_STAGE2_ONLY, LowrankError, load,
                   status_string)

__all__ = [
    "lowrank_linear_forward", "kv_remap_gather", "lowrank_prepare_decode", "lowrank_prepare_prefill",
    "lowrank_workspace_bytes", "lowrank_status_string", "lowrank_version",
    "LR_F32", "LR_BF16", "LR_FULL", "LR_STAGE1_ONLY", "LR_STAGE2_ONLY", "LR_PACKED_WEIGHTS",
    "LR_PREFILL_FUSED",
    "LowrankError", "load", "PackedFactor", "pack_factor", "lowrank_packed_bytes",
    "lowrank_linear_forward_group", "lowrank_group_workspace_bytes", "lowrank_workspace_check",
    "lowrank_set_wait_limit", "LR_DEFAULT_WAIT_LIMIT", "LR_ERR_WAIT",
    "lowrank_linear_forward_noalloc", "LR_NOALLOC_SCRATCH_BYTES",
]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LR_BF16
    if t.dtype == torch.float32:
        return LR_F32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _ld(t) -> int:
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with unit column stride")
    return int(t.stride(0)) if t.shape[0] > 1 else max(int(t.stride(0)), int(t.shape[1]))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return C.c_void_p(s.cuda_stream)


def lowrank_workspace_bytes(which: int, dtype: int, T_or_B: int, d_in: int, r: int,
                            d_out: int = 0, cap: int = 0) -> int:
    return int(load().lowrank_workspace_bytes(which, dtype, T_or_B, d_in, r, d_out, cap))


def lowrank_status_string(s: int) -> str:
    return status_string(s)


def lowrank_version() -> int:
    return int(load().lowrank_version())


def lowrank_workspace_check(workspace, stream=None, raise_on_wait=True) -> int:
    """Synchronise the stream and read the decode path's wait-error words of
    a workspace (see lowrank.h).  Returns the bit mask of control blocks whose
    bounded wait gave up (0 when none; the control area is then cleared);
    raises LowrankError(LR_ERR_WAIT) for a nonzero mask unless
    raise_on_wait is False."""
    mask = C.c_uint32(0)
    nbytes = workspace.numel() * workspace.element_size()
    st = load().lowrank_workspace_check(_ptr(workspace), nbytes, C.byref(mask),
                                        _stream(stream, workspace.device))
    if st == LR_ERR_WAIT and not raise_on_wait:
        return int(mask.value)
    _lib.check(st, "lowrank_workspace_check")
    return int(mask.value)


_watched = None  # decode-path workspaces seen while watching (test hook)


def watch_workspaces(on: bool = True) -> None:
    """Record every workspace a decode-path call uses from now on (weakly),
    so that check_watched_workspaces() can run lowrank_workspace_check on
    each; off drops the record."""
    global _watched
    _watched = weakref.WeakValueDictionary() if on else None


def _note(workspace) -> None:
    if _watched is not None and workspace is not None:
        _watched[workspace.data_ptr()] = workspace


def check_watched_workspaces() -> None:
    """lowrank_workspace_check on every recorded workspace still alive
    (raises LowrankError(LR_ERR_WAIT) if a bounded wait gave up)."""
    if _watched is None:
        return
    for ws in list(_watched.values()):
        lowrank_workspace_check(ws)


def lowrank_set_wait_limit(polls: int) -> None:
    """Polls a bounded wait of the decode path makes before it gives up, for
    launches issued from now on (LR_DEFAULT_WAIT_LIMIT restores the default)."""
    load().lowrank_set_wait_limit(int(polls))


class PackedFactor:
    """A bf16 factor W[N, K] in the fragment-packed layout of lowrank.h: a
    view (base element offset, N, K, block pitch in steps) of a flat bf16
    device tensor.  ``cols(k0, k1)`` and ``rows(n0, n1)`` give the
    tensor-parallel share views (k0 a multiple of 32, n0 of 16)."""

    def __init__(self, storage, N: int, K: int, pitch: int, offset: int = 0):
        self.storage, self.N, self.K, self.pitch, self.offset = storage, N, K, pitch, offset
        self.shape = (N, K)
        self.dtype = storage.dtype
        self.device = storage.device

    def data_ptr(self) -> int:
        return self.storage.data_ptr() + 2 * self.offset

    def cols(self, k0: int, k1: int) -> "PackedFactor":
        if k0 % 32 or not 0 <= k0 < k1 <= self.K:
            raise ValueError("column share must start at a multiple of 32")
        return PackedFactor(self.storage, self.N, k1 - k0, self.pitch, self.offset + k0 // 32 * 512)

    def rows(self, n0: int, n1: int) -> "PackedFactor":
        if n0 % 16 or not 0 <= n0 < n1 <= self.N:
            raise ValueError("row share must start at a multiple of 16")
        return PackedFactor(self.storage, n1 - n0, self.K, self.pitch,
                            self.offset + n0 // 16 * self.pitch * 512)


def lowrank_packed_bytes(N: int, K: int) -> int:
    return int(load().lowrank_packed_bytes(N, K))


def pack_factor(W, stream=None) -> PackedFactor:
    """Fragment-packed copy of a row-major bf16 device matrix W[N, K]."""
    torch = _torch()
    N, K = (int(v) for v in W.shape)
    pitch = (K + 31) // 32
    out = torch.empty(lowrank_packed_bytes(N, K) // 2, dtype=torch.bfloat16, device=W.device)
    st = load().lowrank_pack_factor(_ptr(W), N, K, _ld(W), _ptr(out), pitch,
                                    _stream(stream, W.device))
    _lib.check(st, "lowrank_pack_factor")
    return PackedFactor(out, N, K, pitch)


def _wld(w) -> int:
    return w.pitch if isinstance(w, PackedFactor) else _ld(w)


def lowrank_linear_forward(x, Ut, Vt, y=None, t_io=None, flags: int = LR_FULL, workspace=None,
                           stream=None):
    """y = (x U_r) V_r (or one stage of it, see lowrank.h).  Tensors on one
    HIP device; Ut = U_r^T [r, d_in], Vt = V_r^T [d_out, r]; t_io fp32 [T, r].
    Ut / Vt may be PackedFactor views (bf16, T <= 64), which sets
    LR_PACKED_WEIGHTS.  Returns y (allocated when not given and a stage 2 runs)."""
    torch = _torch()
    lib = load()
    ref = x if x is not None else t_io
    dev = ref.device
    if isinstance(Ut, PackedFactor) or isinstance(Vt, PackedFactor):
        flags |= LR_PACKED_WEIGHTS
    mode = flags & ~(LR_PACKED_WEIGHTS | LR_PREFILL_FUSED)
    if mode == LR_STAGE2_ONLY:
        T, r = t_io.shape
        d_in = int(Ut.shape[1]) if Ut is not None else 1
        dt = _dtype_code(Vt)
    else:
        T, d_in = x.shape
        r = int(Ut.shape[0])
        dt = _dtype_code(x)
    d_out = int(Vt.shape[0]) if Vt is not None else 1
    if y is None and mode != LR_STAGE1_ONLY:
        y = torch.empty((T, d_out), dtype=Vt.dtype, device=dev)
    need = 0 if flags & LR_PREFILL_FUSED else lowrank_workspace_bytes(0, dt, T, d_in, r, d_out)
    if workspace is None and need > 0:
        # zero-filled: the decode kernel's counters must start at zero (it
        # leaves them at zero when it finishes)
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.lowrank_linear_forward(
        dt, T, d_in, r, d_out,
        _ptr(x), _ld(x) if x is not None else 0,
        _ptr(Ut), _wld(Ut) if Ut is not None else 0,
        _ptr(Vt), _wld(Vt) if Vt is not None else 0,
        _ptr(y), _ld(y) if y is not None else 0,
        _ptr(t_io), _ld(t_io) if t_io is not None else 0,
        flags, _ptr(workspace), ws_bytes, _stream(stream, dev))
    _lib.check(st, "lowrank_linear_forward")
    if dt == LR_BF16 and T <= 64:
        _note(workspace)
    return y


def lowrank_linear_forward_noalloc(x, Ut, Vt, y=None, t_io=None, flags: int = LR_FULL,
                                   stream=None):
    """lowrank_linear_forward with the library's fixed scratch instead of a
    workspace (no device allocation by the library; y must then be given or
    is allocated here by the caller's framework).  See lowrank.h."""
    torch = _torch()
    lib = load()
    ref = x if x is not None else t_io
    dev = ref.device
    if isinstance(Ut, PackedFactor) or isinstance(Vt, PackedFactor):
        flags |= LR_PACKED_WEIGHTS
    mode = flags & ~(LR_PACKED_WEIGHTS | LR_PREFILL_FUSED)
    if mode == LR_STAGE2_ONLY:
        T, r = t_io.shape
        d_in = int(Ut.shape[1]) if Ut is not None else 1
        dt = _dtype_code(Vt)
    else:
        T, d_in = x.shape
        r = int(Ut.shape[0])
        dt = _dtype_code(x)
    d_out = int(Vt.shape[0]) if Vt is not None else 1
    if y is None and mode != LR_STAGE1_ONLY:
        y = torch.empty((T, d_out), dtype=Vt.dtype, device=dev)
    st = lib.lowrank_linear_forward_noalloc(
        dt, T, d_in, r, d_out,
        _ptr(x), _ld(x) if x is not None else 0,
        _ptr(Ut), _wld(Ut) if Ut is not None else 0,
        _ptr(Vt), _wld(Vt) if Vt is not None else 0,
        _ptr(y), _ld(y) if y is not None else 0,
        _ptr(t_io), _ld(t_io) if t_io is not None else 0,
        flags, _stream(stream, dev))
    _lib.check(st, "lowrank_linear_forward_noalloc")
    return y


def _group_structs(linears):
    arr = (_lib.Linear * len(linears))()
    for i, L in enumerate(linears):
        x, Ut, Vt = L.get("x"), L.get("Ut"), L.get("Vt")
        y, y_acc, t_io = L.get("y"), L.get("y_acc"), L.get("t_io")
        a = arr[i]
        a.d_in = int(x.shape[1]) if x is not None else 1
        a.r = int(Ut.shape[0]) if Ut is not None else int(t_io.shape[1])
        a.d_out = int(Vt.shape[0]) if Vt is not None else 1
        if Ut is not None:
            a.x, a.ldx = x.data_ptr(), _ld(x)
            a.Ut, a.ldu = Ut.data_ptr(), _wld(Ut)
        if Vt is not None:
            a.Vt, a.ldv = Vt.data_ptr(), _wld(Vt)
        if y is not None:
            a.y, a.ldy = y.data_ptr(), _ld(y)
        if y_acc is not None:
            a.y_acc, a.ld_acc = y_acc.data_ptr(), _ld(y_acc)
        if t_io is not None:
            a.t_io, a.ldt = t_io.data_ptr(), _ld(t_io)
    return arr


def lowrank_group_workspace_bytes(T: int, linears) -> int:
    arr = _group_structs(linears)
    return int(load().lowrank_group_workspace_bytes(T, len(linears), C.cast(arr, C.c_void_p)))


def lowrank_linear_forward_group(linears, workspace=None, stream=None):
    """n independent bf16 decode linears over the same T <= 64 rows in one
    launch.  Each entry: dict with x [T, d_in], Ut, Vt (None: stage 1 only),
    y (allocated when missing and neither y_acc nor stage-1-only), y_acc
    (fp32, added to), t_io (fp32).  Without x and Ut an entry is stage 2
    only, from its t_io.  Ut / Vt may be PackedFactor views (then all of them
    must be).  Returns the list of y (None where not written)."""
    torch = _torch()
    lib = load()
    ref = next(L.get("x") if L.get("Ut") is not None else L["t_io"] for L in linears)
    T = int(ref.shape[0])
    dev = ref.device
    packed = any(isinstance(L.get(k), PackedFactor) for L in linears for k in ("Ut", "Vt"))
    for L in linears:
        if L.get("Vt") is not None and L.get("y") is None and L.get("y_acc") is None:
            L["y"] = torch.empty((T, int(L["Vt"].shape[0])), dtype=torch.bfloat16, device=dev)
    arr = _group_structs(linears)
    need = int(lib.lowrank_group_workspace_bytes(T, len(linears), C.cast(arr, C.c_void_p)))
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.lowrank_linear_forward_group(T, len(linears), C.cast(arr, C.c_void_p),
                                          LR_PACKED_WEIGHTS if packed else 0, _ptr(workspace),
                                          ws_bytes, _stream(stream, dev))
    _lib.check(st, "lowrank_linear_forward_group")
    _note(workspace)
    return [L.get("y") for L in linears]


def kv_remap_gather(src, remap, dst, n_valid=None, row_elems=None, stream=None):
    """dst[j] = src[remap[j]] (zero row for invalid indices) for j < n_valid
    (device int32 scalar tensor, or all rows of remap when None)."""
    lib = load()
    re = int(row_elems if row_elems is not None else src.shape[1])
    st = lib.kv_remap_gather(_dtype_code(src), _ptr(src), int(src.shape[0]), _ld(src),
                             _ptr(remap), int(remap.numel()), _ptr(n_valid), re, _ptr(dst),
                             _ld(dst), _stream(stream, src.device))
    _lib.check(st, "kv_remap_gather")
    return dst


def lowrank_prepare_decode(lengths, tables, block: int, cap: int, want_runs: bool = False):
    """Host preparation stage: returns a dict of numpy int32 arrays remap[cap],
    seq_off[B+1], pos[B], slot_mapping[B] and ints n_valid, n_runs (plus
    runs[n_runs, 3] when want_runs)."""
    lib = load()
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    B = lengths.shape[0]
    if isinstance(tables, np.ndarray) and tables.ndim == 2:
        tab = np.ascontiguousarray(tables, dtype=np.int32)
    else:
        width = max((len(t) for t in tables), default=1)
        tab = np.full((B, max(width, 1)), -1, dtype=np.int32)
        for i, t in enumerate(tables):
            tab[i, :len(t)] = t
    remap = np.empty(cap, np.int32)
    seq_off = np.empty(B + 1, np.int32)
    pos = np.empty(max(B, 1), np.int32)
    slots = np.empty(max(B, 1), np.int32)
    nv = np.zeros(1, np.int32)
    nr = np.zeros(1, np.int32)
    max_runs = int(tab.size) if want_runs else 0
    runs = np.empty((max(max_runs, 1), 3), np.int32)

    def P(a):
        return a.ctypes.data_as(C.c_void_p)

    st = lib.lowrank_prepare_decode(B, P(lengths), P(tab), tab.shape[1], block, cap, P(remap),
                                    P(seq_off), P(pos), P(slots), P(nv), P(nr),
                                    P(runs) if want_runs else None, max_runs)
    _lib.check(st, "lowrank_prepare_decode")
    out = {"remap": remap, "seq_off": seq_off, "pos": pos[:B], "slot_mapping": slots[:B],
           "n_valid": int(nv[0]), "n_runs": int(nr[0])}
    if want_runs:
        out["runs"] = runs[:out["n_runs"]].copy()
    return out


def lowrank_prepare_prefill(lengths, chunks, tables, block: int, cap: int, max_tokens=None,
                            want_runs: bool = False):
    """Host preparation stage of a chunked-prefill step: sequence i has
    lengths[i] cached tokens and appends chunks[i] new ones.  Returns a dict
    of numpy int32 arrays remap[cap], seq_off[S+1], tok_seq[n], pos[n],
    slot_mapping[n] (n = sum of chunks) and ints n_valid, n_tokens, n_runs
    (plus runs[n_runs, 3] when want_runs)."""
    lib = load()
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    chunks = np.ascontiguousarray(chunks, dtype=np.int32)
    S = lengths.shape[0]
    if isinstance(tables, np.ndarray) and tables.ndim == 2:
        tab = np.ascontiguousarray(tables, dtype=np.int32)
    else:
        width = max((len(t) for t in tables), default=1)
        tab = np.full((S, max(width, 1)), -1, dtype=np.int32)
        for i, t in enumerate(tables):
            tab[i, :len(t)] = t
    mt = int(chunks.sum()) if max_tokens is None else int(max_tokens)
    remap = np.empty(cap, np.int32)
    seq_off = np.empty(S + 1, np.int32)
    tok_seq = np.empty(max(mt, 1), np.int32)
    pos = np.empty(max(mt, 1), np.int32)
    slots = np.empty(max(mt, 1), np.int32)
    nt, nv, nr = (np.zeros(1, np.int32) for _ in range(3))
    max_runs = int(tab.size) if want_runs else 0
    runs = np.empty((max(max_runs, 1), 3), np.int32)

    def P(a):
        return a.ctypes.data_as(C.c_void_p)

    st = lib.lowrank_prepare_prefill(S, P(lengths), P(chunks), P(tab), tab.shape[1], block, cap,
                                     mt, P(remap), P(seq_off), P(tok_seq), P(pos), P(slots),
                                     P(nt), P(nv), P(nr), P(runs) if want_runs else None,
                                     max_runs)
    _lib.check(st, "lowrank_prepare_prefill")
    n = int(nt[0])
    out = {"remap": remap, "seq_off": seq_off, "tok_seq": tok_seq[:n], "pos": pos[:n],
           "slot_mapping": slots[:n], "n_valid": int(nv[0]), "n_tokens": n,
           "n_runs": int(nr[0])}
    if want_runs:
        out["runs"] = runs[:out["n_runs"]].copy()
    return out


# ------------------------------------------------------------------ decode step
from ._lib import DecodeState, LayerWeights, PrefillState  # noqa: E402

LR_MLP_SWIGLU, LR_MLP_RELU = 0, 1  # lr_layer_weights.mlp
LINEARS = ("q", "k", "v", "o", "gate", "up", "down")
__all__ += ["LayerWeights", "DecodeState", "PrefillState", "layer_weights", "decode_state",
            "prefill_state", "lowrank_prefill_step_workspace_bytes", "lowrank_layer_prefill_step",
            "lowrank_rope_table", "lowrank_decode_step_workspace_bytes",
            "lowrank_layer_decode_step", "lowrank_decode_step_fused_workspace_bytes",
            "lowrank_layer_decode_step_fused", "LINEARS", "LR_MLP_SWIGLU", "LR_MLP_RELU"]


def lowrank_rope_table(head_dim: int, max_pos: int, theta: float, table, stream=None):
    """Fill table (device float [max_pos, head_dim/2, 2]) with cos/sin."""
    _lib.check(load().lowrank_rope_table(head_dim, max_pos, theta, _ptr(table),
                                         _stream(stream, table.device)), "lowrank_rope_table")
    return table


def layer_weights(cfg: dict, Ut: dict, Vt: dict, attn_norm, ffn_norm, rope, rope_max_pos: int):
    """Build lr_layer_weights from tensors: Ut[name] = U_r^T [r, d_in] and
    Vt[name] = V_r^T [d_out, r] bf16 views (name in LINEARS).  cfg["mlp"] is
    "swiglu" (default) or "relu"; a ReLU MLP takes fc1 as "gate" and fc2 as
    "down" and needs no "up".  The returned struct keeps references to the
    tensors it points to."""
    w = LayerWeights()
    w.d_model, w.n_heads, w.n_kv_heads = cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"]
    w.head_dim, w.d_ffn = cfg["head_dim"], cfg["d_ffn"]
    w.eps = cfg.get("eps", 1e-5)
    w.mlp = {"swiglu": LR_MLP_SWIGLU, "relu": LR_MLP_RELU}[cfg.get("mlp", "swiglu")]
    for k, name in enumerate(LINEARS):
        if w.mlp == LR_MLP_RELU and name == "up":
            continue
        u, v = Ut[name], Vt[name]
        w.Ut[k], w.ldu[k] = u.data_ptr(), _ld(u)
        w.Vt[k], w.ldv[k] = v.data_ptr(), _ld(v)
        w.r[k] = u.shape[0]
    w.attn_norm, w.ffn_norm = attn_norm.data_ptr(), ffn_norm.data_ptr()
    w.rope, w.rope_max_pos = rope.data_ptr(), rope_max_pos
    w._keep = (Ut, Vt, attn_norm, ffn_norm, rope)
    return w


def decode_state(k_pool, v_pool, slot_mapping, remap, seq_off, pos, n_valid, max_seq_rows: int):
    """Build lr_decode_state from device tensors (pools [pool_rows, pool_ld]
    bf16; int32 prep arrays; n_valid a 1-element int32 tensor)."""
    s = DecodeState()
    s.k_pool, s.v_pool = k_pool.data_ptr(), v_pool.data_ptr()
    s.pool_rows, s.pool_ld = k_pool.shape[0], _ld(k_pool)
    s.slot_mapping, s.remap, s.seq_off = slot_mapping.data_ptr(), remap.data_ptr(), seq_off.data_ptr()
    s.pos, s.n_valid = pos.data_ptr(), n_valid.data_ptr()
    s.B, s.cap, s.max_seq_rows = slot_mapping.numel(), remap.numel(), max_seq_rows
    s._keep = (k_pool, v_pool, slot_mapping, remap, seq_off, pos, n_valid)
    return s


def lowrank_decode_step_workspace_bytes(w: LayerWeights, s: DecodeState) -> int:
    return int(load().lowrank_decode_step_workspace_bytes(C.byref(w), C.byref(s)))


def lowrank_layer_decode_step(w: LayerWeights, s: DecodeState, h, workspace, stream=None):
    """One decoder layer in place on h (fp32 [B, d_model])."""
    nbytes = workspace.numel() * workspace.element_size()
    _lib.check(load().lowrank_layer_decode_step(C.byref(w), C.byref(s), _ptr(h), _ptr(workspace),
                                                nbytes, _stream(stream, h.device)),
               "lowrank_layer_decode_step")
    _note(workspace)
    return h


def lowrank_decode_step_fused_workspace_bytes(w: LayerWeights, s: DecodeState) -> int:
    return int(load().lowrank_decode_step_fused_workspace_bytes(C.byref(w), C.byref(s)))


def lowrank_layer_decode_step_fused(w: LayerWeights, s: DecodeState, h, workspace, stream=None):
    """lowrank_layer_decode_step with the reconstruction folded into the
    attention, in place on h (fp32 [B, d_model])."""
    nbytes = workspace.numel() * workspace.element_size()
    _lib.check(load().lowrank_layer_decode_step_fused(C.byref(w), C.byref(s), _ptr(h),
                                                      _ptr(workspace), nbytes,
                                                      _stream(stream, h.device)),
               "lowrank_layer_decode_step_fused")
    _note(workspace)
    return h


def prefill_state(k_pool, v_pool, slot_mapping, remap, seq_off, tok_seq, pos, n_valid,
                  max_seq_rows: int):
    """Build lr_prefill_state from device tensors (pools [pool_rows, pool_ld]
    bf16; int32 prep arrays of lowrank_prepare_prefill; n_valid a 1-element
    int32 tensor)."""
    s = PrefillState()
    s.k_pool, s.v_pool = k_pool.data_ptr(), v_pool.data_ptr()
    s.pool_rows, s.pool_ld = k_pool.shape[0], _ld(k_pool)
    s.slot_mapping, s.remap, s.seq_off = slot_mapping.data_ptr(), remap.data_ptr(), seq_off.data_ptr()
    s.tok_seq, s.pos, s.n_valid = tok_seq.data_ptr(), pos.data_ptr(), n_valid.data_ptr()
    s.T, s.S, s.cap = slot_mapping.numel(), seq_off.numel() - 1, remap.numel()
    s.max_seq_rows = max_seq_rows
    s._keep = (k_pool, v_pool, slot_mapping, remap, seq_off, tok_seq, pos, n_valid)
    return s


def lowrank_prefill_step_workspace_bytes(w: LayerWeights, s: PrefillState) -> int:
    return int(load().lowrank_prefill_step_workspace_bytes(C.byref(w), C.byref(s)))


def lowrank_layer_prefill_step(w: LayerWeights, s: PrefillState, h, workspace, stream=None):
    """One decoder layer over a chunk of prompt tokens, in place on h [T, d]
    (fp32, tokens in sequence order); causal attention over each token's
    cached and earlier chunk rows."""
    nbytes = workspace.numel() * workspace.element_size()
    _lib.check(load().lowrank_layer_prefill_step(C.byref(w), C.byref(s), _ptr(h), _ptr(workspace),
                                                 nbytes, _stream(stream, h.device)),
               "lowrank_layer_prefill_step")
    if s.T <= 64:  # projections on the decode path: its control area leads the workspace
        _note(workspace)
    return h
