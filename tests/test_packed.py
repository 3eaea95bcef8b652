"""Fragment-packed factors (lowrank.h, LR_PACKED_WEIGHTS).

CPU: the layout written out in numpy from its definition, its round trip, and
the host-side checks of the two entry points.  GPU: lowrank_pack_factor bit for
bit against the numpy layout, and the decode path on packed factors against
the row-major path (bit for bit: the same fragments meet the same MFMAs in the
same order) and against the fp64 oracle, including tensor-parallel share views.
"""
import numpy as np
import pytest

import rank_decomposed_amd as lr
import synth
from rank_decomposed_amd import _lib

A16 = 1 << 20   # fake aligned "device" address: never dereferenced (host checks fail first)


def pack_numpy(w: np.ndarray, pitch: int) -> np.ndarray:
    """W [N, K] (any dtype) -> flat packed array per the layout definition:
    element (n, k) at ((b*pitch + s)*64 + lane)*8 + e, b = n//16, s = k//32,
    lane = n%16 + 16*((k%32)//8), e = k%8; zero elsewhere."""
    N, K = w.shape
    nb = (N + 15) // 16
    out = np.zeros(nb * pitch * 512, dtype=w.dtype)
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    idx = (((n // 16) * pitch + k // 32) * 64 + n % 16 + 16 * ((k % 32) // 8)) * 8 + k % 8
    out[idx] = w
    return out


def unpack_numpy(p: np.ndarray, N: int, K: int, pitch: int) -> np.ndarray:
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    idx = (((n // 16) * pitch + k // 32) * 64 + n % 16 + 16 * ((k % 32) // 8)) * 8 + k % 8
    return p[idx]


@pytest.mark.parametrize("N,K,pitch", [(16, 32, 1), (37, 70, 3), (5, 100, 7), (64, 64, 2)])
def test_layout_round_trip_and_padding(N, K, pitch):
    w = np.arange(1, N * K + 1, dtype=np.int64).reshape(N, K)
    p = pack_numpy(w, pitch)
    assert np.array_equal(unpack_numpy(p, N, K, pitch), w)
    # every element lands in a distinct slot; all other slots are zero
    assert np.count_nonzero(p) == N * K
    # a 16x32 step is one contiguous 1 KiB (512 elements) run
    b, s = (N - 1) // 16, (K - 1) // 32
    run = p[(b * pitch + s) * 512:(b * pitch + s + 1) * 512]
    assert w[N - 1, K - 1] in run


def test_share_views_are_offsets():
    # the column share starting at a multiple of 32 and the row share starting
    # at a multiple of 16 are plain offsets into the packed array
    N, K, pitch = 48, 96, 3
    w = np.arange(1, N * K + 1, dtype=np.int64).reshape(N, K)
    p = pack_numpy(w, pitch)
    k0, n0 = 32, 16
    cols = p[k0 // 32 * 512:]
    assert np.array_equal(unpack_numpy(cols, N, K - k0, pitch), w[:, k0:])
    rows = p[n0 // 16 * pitch * 512:]
    assert np.array_equal(unpack_numpy(rows, N - n0, K, pitch), w[n0:, :])


def test_packed_bytes():
    assert lr.lowrank_packed_bytes(1228, 4096) == 77 * 128 * 1024
    assert lr.lowrank_packed_bytes(16, 1) == 1024
    assert lr.lowrank_packed_bytes(0, 5) == 0


@pytest.mark.parametrize("args,status", [
    ((None, 16, 32, 32, A16, 1), _lib.LR_ERR_ARG),
    ((A16, 16, 32, 32, None, 1), _lib.LR_ERR_ARG),
    ((A16, 0, 32, 32, A16, 1), _lib.LR_ERR_ARG),
    ((A16, 16, 64, 32, A16, 2), _lib.LR_ERR_ARG),       # ld < K
    ((A16, 16, 64, 64, A16, 1), _lib.LR_ERR_ARG),       # pitch < ceil(K/32)
    ((A16 + 2, 16, 32, 32, A16, 1), _lib.LR_ERR_ALIGN),
    ((A16, 16, 32, 36, A16, 1), _lib.LR_ERR_ALIGN),     # ld not a multiple of 8
])
def test_pack_rejects_bad_arguments(args, status):
    assert lr.load().lowrank_pack_factor(*args, None) == status


def _fwd(**kw):
    a = dict(dt=_lib.LR_BF16, T=4, d_in=64, r=16, d_out=32, x=A16, ldx=64, Ut=A16, ldu=2,
             Vt=A16, ldv=1, y=A16, ldy=32, t=None, ldt=0, flags=lr.LR_PACKED_WEIGHTS, ws=A16,
             wsb=1 << 30)
    a.update(kw)
    return lr.load().lowrank_linear_forward(
        a["dt"], a["T"], a["d_in"], a["r"], a["d_out"], a["x"], a["ldx"], a["Ut"], a["ldu"],
        a["Vt"], a["ldv"], a["y"], a["ldy"], a["t"], a["ldt"], a["flags"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ldu=1), _lib.LR_ERR_ARG),                    # pitch < ceil(d_in / 32)
    (dict(ldv=0), _lib.LR_ERR_ARG),
    (dict(dt=_lib.LR_F32), _lib.LR_ERR_UNSUPPORTED),
    (dict(T=65), _lib.LR_ERR_UNSUPPORTED),
    (dict(Ut=A16 + 2), _lib.LR_ERR_ALIGN),
    (dict(flags=lr.LR_PACKED_WEIGHTS | 3), _lib.LR_ERR_ARG),
    (dict(ldu=1 << 16), _lib.LR_ERR_UNSUPPORTED),      # 32-bit tile offsets
])
def test_packed_forward_rejects_bad_arguments(kw, status):
    assert _fwd(**kw) == status


# ---------------------------------------------------------------- GPU
gpu = pytest.mark.gpu


@gpu
@pytest.mark.parametrize("N,K,extra", [(1228, 4096, 0), (45, 300, 8), (16, 8, 0), (33, 1100, 16)])
def test_pack_factor_bit_exact(N, K, extra):
    import torch
    from gpu_util import bits, padded
    w = synth.bf16_bits(synth.gaussian(synth.seed_of(40, 0, 0, 0) + N, (N, K)))
    ld = (K + 7) // 8 * 8 + extra
    dw = padded(w, ld, "bf16")          # NaN padding must not leak into the packed copy
    p = lr.pack_factor(dw)
    torch.cuda.synchronize()
    got = bits(p.storage)
    assert np.array_equal(got, pack_numpy(w, (K + 31) // 32))


@gpu
@pytest.mark.parametrize("T", [1, 3, 8, 16, 17, 32, 33, 48, 64])
@pytest.mark.parametrize("shape", [(1024, 300, 768), (520, 45, 1100), (96, 7, 40), (11008, 90, 200),
                                   (256, 70, 8200)])     # wide output: 64-row stage-2 tiles at T > 32
def test_packed_decode_matches_row_major_and_oracle(T, shape):
    import torch
    import oracle
    from gpu_util import bits, dev, make_linear, maxrel, to_f64
    d_in, r, d_out = shape
    c = make_linear(5000 + T + d_in, T, d_in, r, d_out, "bf16", fast=True, ld_extra=8)
    pu, pv = lr.pack_factor(c["dUt"]), lr.pack_factor(c["dVt"])
    t1 = torch.empty((T, r), dtype=torch.float32, device=dev())
    t2 = torch.empty_like(t1)
    y1 = lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], t_io=t1)
    y2 = lr.lowrank_linear_forward(c["dx"], pu, pv, t_io=t2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y1), bits(y2))
    assert np.array_equal(to_f64(t1), to_f64(t2))
    tr, yr = oracle.linear(c["x"], c["U"], c["V"])
    assert maxrel(to_f64(t2), tr) <= 1e-5
    assert maxrel(to_f64(y2), yr) <= 2e-2


@gpu
@pytest.mark.parametrize("T", [4, 64])
def test_packed_tensor_parallel_share_views(T):
    # one of 4 shares: U_r input rows [k0, k1) (stage 1), V_r output columns
    # [n0, n1) (stage 2), both as views into the packed factors
    import torch
    import oracle
    from gpu_util import dev, make_linear, maxrel, to_f64
    d_in, r, d_out, P, s = 1024, 200, 768, 4, 2
    c = make_linear(6000 + T, T, d_in, r, d_out, "bf16", fast=True)
    pu, pv = lr.pack_factor(c["dUt"]), lr.pack_factor(c["dVt"])
    wi, wo = d_in // P, d_out // P
    t_s = torch.empty((T, r), dtype=torch.float32, device=dev())
    lr.lowrank_linear_forward(c["dx"][:, s * wi:(s + 1) * wi], pu.cols(s * wi, (s + 1) * wi), None,
                              t_io=t_s, flags=lr.LR_STAGE1_ONLY)
    tr, _ = oracle.linear(c["x"], c["U"], c["V"])
    t_full = torch.from_numpy(tr.astype(np.float32)).to(dev())
    y_s = lr.lowrank_linear_forward(None, None, pv.rows(s * wo, (s + 1) * wo), t_io=t_full,
                                    flags=lr.LR_STAGE2_ONLY)
    torch.cuda.synchronize()
    assert maxrel(to_f64(t_s), oracle.tp_share_stage1(c["x"], c["U"], s, P)) <= 1e-5
    ref_y = oracle.tp_share_stage2(tr.astype(np.float32).astype(np.float64), c["V"], s, P)
    assert maxrel(to_f64(y_s), ref_y) <= 2e-2
