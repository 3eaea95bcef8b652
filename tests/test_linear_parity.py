"""lowrank_linear_forward on the GPU against the fp64 oracle.

Bar: max|gpu - ref| / max|ref| <= 1e-5 (fp32) and <= 2e-2 (bf16); bit-exact on
integer-valued cases.  Leading-dimension padding is NaN-filled, so any
unmasked read of it fails the test."""
import numpy as np
import pytest
import torch

import oracle
import rank_decomposed_amd as lr
import synth
from gpu_util import bits, control_counters, dev, ld_for, make_linear, maxrel, padded, to_dev, to_f64

pytestmark = pytest.mark.gpu
BF16_TOL, F32_TOL = 2e-2, 1e-5


def _run(case, T, dtype, flags=lr.LR_FULL, with_t=False):
    d = dev()
    r = case["dUt"].shape[0]
    t_io = torch.full((T, r), float("nan"), dtype=torch.float32, device=d) if with_t else None
    y = lr.lowrank_linear_forward(case["dx"], case["dUt"], case["dVt"], t_io=t_io, flags=flags)
    torch.cuda.synchronize()
    return y, t_io


def test_config1_fp32_512_r128_T4():
    # 512 x 512, r = 128, 4 tokens, SVD factors with sqrt(sigma) on both sides
    c = make_linear(synth.seed_of(1), 4, 512, 128, 512, "f32", fast=False,
                    svd_weight_seed=synth.seed_of(1, 0, 0, synth.KIND_W))
    y, t = _run(c, 4, "f32", with_t=True)
    tr, yr = oracle.linear(c["x"], c["U"], c["V"])
    assert maxrel(to_f64(t), tr) <= F32_TOL
    assert maxrel(to_f64(y), yr) <= F32_TOL


@pytest.mark.parametrize("T", [1, 2, 7, 16, 17, 33, 64])
def test_fp32_ragged_tokens(T):
    c = make_linear(11 + T, T, 200, 37, 130, "f32", fast=True, ld_extra=3)
    y, _ = _run(c, T, "f32")
    assert maxrel(to_f64(y), oracle.linear(c["x"], c["U"], c["V"])[1]) <= F32_TOL


@pytest.mark.parametrize("T", [1, 3, 8, 16, 17, 32, 33, 48, 64])
@pytest.mark.parametrize("shape", [(1024, 300, 768), (520, 45, 1100), (96, 7, 40)])
def test_bf16_decode_path(T, shape):
    d_in, r, d_out = shape
    c = make_linear(1000 + T + d_in, T, d_in, r, d_out, "bf16", fast=True, ld_extra=8)
    y, t = _run(c, T, "bf16", with_t=True)
    tr, yr = oracle.linear(c["x"], c["U"], c["V"])
    assert maxrel(to_f64(t), tr) <= 1e-5          # t stays fp32 on the decode path
    assert maxrel(to_f64(y), yr) <= BF16_TOL


@pytest.mark.parametrize("T", [65, 130, 1000])
@pytest.mark.parametrize("shape", [(512, 300, 700), (1300, 1250, 1280), (40, 33, 72)])
def test_bf16_prefill_path(T, shape):
    d_in, r, d_out = shape
    c = make_linear(2000 + T + r, T, d_in, r, d_out, "bf16", fast=True, ld_extra=8)
    y, _ = _run(c, T, "bf16")
    assert maxrel(to_f64(y), oracle.linear(c["x"], c["U"], c["V"])[1]) <= BF16_TOL


@pytest.mark.parametrize("T", [1024, 1300])
@pytest.mark.parametrize("shape", [(512, 300, 700), (1300, 1250, 1280), (40, 33, 72),
                                   (2000, 257, 300)])
def test_bf16_prefill_large_tile_path(T, shape):
    # from 1024 rows on both stages run on the 256-row GEMM: ragged rows
    # (1300), ragged rank and output columns against 128/256-wide tiles, a
    # ragged last k-tile (d_in 1300, 2000; r 33, 257, 300) and K < 64 (d_in 40)
    d_in, r, d_out = shape
    c = make_linear(2500 + T + r, T, d_in, r, d_out, "bf16", fast=True, ld_extra=8)
    y, _ = _run(c, T, "bf16")
    y_t, t = _run(c, T, "bf16", with_t=True)
    tr, yr = oracle.linear(c["x"], c["U"], c["V"])
    assert maxrel(to_f64(y), yr) <= BF16_TOL
    assert maxrel(to_f64(t), tr) <= 1e-5
    # stage 2 multiplies the same bf16 t whether or not t_io is requested
    assert np.array_equal(bits(y_t), bits(y))


@pytest.mark.parametrize("T,shape", [(2600, (512, 300, 2100)), (3333, (1040, 700, 1000))])
def test_bf16_prefill_grouped_tile_order(T, shape):
    # the large-tile GEMM lists tiles four row tiles at a time: 11 and 14 row
    # tiles (two full groups and a partial one of 3 or 2 rows) against 9 / 4
    # output column tiles and 2 / 3-6 rank column tiles, with a ragged last
    # 64-deep k-tile in stage 1 (d_in 1040); every output tile must be
    # computed exactly once (outputs start as NaN)
    d_in, r, d_out = shape
    c = make_linear(3900 + T + r, T, d_in, r, d_out, "bf16", fast=True, ld_extra=8)
    y = torch.full((T, d_out), float("nan"), dtype=torch.bfloat16, device=dev())
    t = torch.full((T, r), float("nan"), dtype=torch.float32, device=dev())
    lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], y=y, t_io=t)
    torch.cuda.synchronize()
    tr, yr = oracle.linear(c["x"], c["U"], c["V"])
    assert maxrel(to_f64(t), tr) <= 1e-5
    assert maxrel(to_f64(y), yr) <= BF16_TOL


@pytest.mark.parametrize("T,shape", [(1100, (3003, 96, 320)), (1024, (4096, 409, 512)),
                                     (2000, (11008, 597, 4096)), (1024, (1200, 1100, 1300))])
def test_bf16_prefill_split_k(T, shape):
    # a stage 1 with few 128-column tiles splits d_in into ranges summed in
    # order: a ragged last range with a ragged last k-tile (3003), eight
    # 512-deep ranges (4096), the MLP down projection's d_in (11008), two
    # ranges before a wide rank (1200 -> 1100).  Fused y, y through an fp32
    # t_io, and stage 1 alone must agree
    d_in, r, d_out = shape
    c = make_linear(3100 + T + r, T, d_in, r, d_out, "bf16", fast=True, ld_extra=8)
    y, _ = _run(c, T, "bf16")
    y_t, t = _run(c, T, "bf16", with_t=True)
    t1 = torch.empty((T, r), dtype=torch.float32, device=dev())
    lr.lowrank_linear_forward(c["dx"], c["dUt"], None, t_io=t1, flags=lr.LR_STAGE1_ONLY)
    torch.cuda.synchronize()
    tr, yr = oracle.linear(c["x"], c["U"], c["V"])
    assert maxrel(to_f64(y), yr) <= BF16_TOL
    assert maxrel(to_f64(t), tr) <= 1e-5
    assert np.array_equal(t1.cpu().numpy(), t.cpu().numpy())
    assert np.array_equal(bits(y_t), bits(y))


@pytest.mark.parametrize("T,shape", [(5000, (8200, 3300, 3400)), (5000, (8200, 1600, 1700))])
def test_bf16_prefill_split_tail(T, shape):
    # launches whose last round of 256-row tiles is part-filled split that
    # round's tiles over K (fp32 partials summed in range order by a second
    # kernel): 260 tiles of 256 x 256 in stage 1 and 280 in stage 2 of the
    # first shape, 260 of 256 x 128 in stage 1 of the second, with ragged
    # rows (5000), ragged columns (3300, 3400, 1600) and a ragged last k-tile
    # in the last of four 2112-deep ranges (d_in 8200).  Every output element
    # is written once (y starts as NaN); seeded rows, the first and the last
    # included, against the oracle; a repeat call and a graph replay give the
    # same bits.
    d_in, r, d_out = shape
    c = make_linear(3600 + r, T, d_in, r, d_out, "bf16", fast=True, ld_extra=8)
    y = torch.full((T, d_out), float("nan"), dtype=torch.bfloat16, device=dev())
    ws = torch.zeros(lr.lowrank_workspace_bytes(0, lr.LR_BF16, T, d_in, r, d_out),
                     dtype=torch.uint8, device=dev())
    lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], y=y, workspace=ws)
    y2 = lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], workspace=ws)
    torch.cuda.synchronize()
    assert not torch.isnan(y.float()).any()
    assert np.array_equal(bits(y), bits(y2))
    rows = np.sort(np.random.default_rng(3600 + r).choice(T, 200, replace=False))
    rows[0], rows[-1] = 0, T - 1
    _, yr = oracle.linear(c["x"][rows], c["U"], c["V"])
    assert maxrel(to_f64(y)[rows], yr) <= BF16_TOL
    y3 = torch.full_like(y, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], y=y3, workspace=ws)
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(y3), bits(y)), rep
        y3.fill_(float("nan"))
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [5, 24, 64, 200, 1100])
@pytest.mark.parametrize("shape", [(640, 96, 320), (650, 100, 330)])
def test_bf16_stage_flags(T, shape):
    # stage 1 alone into an fp32 t, then stage 2 alone from it (on the decode
    # path t is re-laid in the packed bf16 operand layout in between); the
    # second shape has a ragged last k-step in both stages
    d_in, r, d_out = shape
    c = make_linear(3000 + T + r, T, d_in, r, d_out, "bf16", fast=True)
    d = dev()
    t = torch.empty((T, r), dtype=torch.float32, device=d)
    lr.lowrank_linear_forward(c["dx"], c["dUt"], None, t_io=t, flags=lr.LR_STAGE1_ONLY)
    y = lr.lowrank_linear_forward(None, None, c["dVt"], t_io=t, flags=lr.LR_STAGE2_ONLY)
    torch.cuda.synchronize()
    tr, yr = oracle.linear(c["x"], c["U"], c["V"])
    assert maxrel(to_f64(t), tr) <= 1e-5
    assert maxrel(to_f64(y), yr) <= BF16_TOL


@pytest.mark.parametrize("T", [1, 9, 64, 100, 300])
def test_integer_cases_bit_exact(T):
    # entries in {-1, 0, 1}, d_in <= 16, r <= 8: every partial sum is an integer
    # of magnitude <= 128, exactly representable in bf16, so the result is exact
    g = synth.seed_of(9, 0, 0, 0) + T
    x = synth.ternary(g, (T, 16))
    U = synth.ternary(g + 1, (16, 8))
    V = synth.ternary(g + 2, (8, 40))
    dx = padded(synth.bf16_bits(x), 24, "bf16")
    du = padded(synth.bf16_bits(np.ascontiguousarray(U.T)), 24, "bf16")
    dv = padded(synth.bf16_bits(np.ascontiguousarray(V.T)), 16, "bf16")
    t = torch.empty((T, 8), dtype=torch.float32, device=dev())
    y = lr.lowrank_linear_forward(dx, du, dv, t_io=t if T <= 64 else None)
    torch.cuda.synchronize()
    tr, yr = oracle.linear(x, U, V)
    assert np.array_equal(bits(y), synth.bf16_bits(yr))
    if T <= 64:
        assert np.array_equal(to_f64(t), tr)


@pytest.mark.parametrize("T", [1, 64, 128])
def test_signed_permutation_7b_shape_bit_exact(T):
    # q-shaped 4096 -> 1228 -> 4096: U_r has one +-1 per column, V_r at most
    # 128 +-1 entries per column; with integer x in [-2, 2] every sum is an
    # integer < 256, exact in bf16
    g = np.random.default_rng(synth.seed_of(9, 1, 0, 0) + T)
    d, r = 4096, 1228
    U = np.zeros((d, r))
    U[g.permutation(d)[:r], np.arange(r)] = g.choice([-1.0, 1.0], r)
    V = np.zeros((r, d))
    for n in range(d):
        rows = g.choice(r, 3, replace=False)
        V[rows, n] = g.choice([-1.0, 1.0], 3)
    x = g.integers(-2, 3, size=(T, d)).astype(np.float64)
    dx = to_dev(synth.bf16_bits(x), "bf16")
    du = to_dev(synth.bf16_bits(np.ascontiguousarray(U.T)), "bf16")
    dv = padded(synth.bf16_bits(np.ascontiguousarray(V.T)), 1232, "bf16")
    y = lr.lowrank_linear_forward(dx, du, dv)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), synth.bf16_bits(oracle.linear(x, U, V)[1]))


@pytest.mark.parametrize("T", [1, 24, 64])
def test_decode_workspace_returns_to_zero_and_is_deterministic(T):
    c = make_linear(4000 + T, T, 2048, 700, 1536, "bf16", fast=True)
    need = lr.lowrank_workspace_bytes(0, lr.LR_BF16, T, 2048, 700, 1536)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    outs = [bits(lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], workspace=ws))
            for _ in range(3)]
    torch.cuda.synchronize()
    counters = control_counters(ws)
    assert not counters.any(), np.nonzero(counters)   # counters, flags and error word at zero
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    _, yr = oracle.linear(c["x"], c["U"], c["V"])
    assert maxrel(synth.bf16_value(outs[0]), yr) <= BF16_TOL


@pytest.mark.parametrize("T", [8, 64, 256])
def test_graph_replay_matches_eager(T):
    # captured once, replayed with new inputs copied into the captured buffers
    c = make_linear(5000 + T, T, 1024, 300, 2048, "bf16", fast=True)
    d = dev()
    need = lr.lowrank_workspace_bytes(0, lr.LR_BF16, T, 1024, 300, 2048)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=d)
    y = torch.empty((T, 2048), dtype=torch.bfloat16, device=d)
    x = c["dx"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lr.lowrank_linear_forward(x, c["dUt"], c["dVt"], y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lr.lowrank_linear_forward(x, c["dUt"], c["dVt"], y=y, workspace=ws)
    for rep in range(3):
        xn = make_linear(5100 + 10 * rep + T, T, 1024, 300, 2048, "bf16", fast=True)
        x.copy_(xn["dx"])
        g.replay()
        torch.cuda.synchronize()
        got = bits(y)
        eager = bits(lr.lowrank_linear_forward(x, c["dUt"], c["dVt"], workspace=ws))
        torch.cuda.synchronize()
        assert np.array_equal(got, eager), rep
        _, yr = oracle.linear(xn["x"], c["U"], c["V"])
        assert maxrel(synth.bf16_value(got), yr) <= BF16_TOL


def test_decode_workspace_shared_across_shapes():
    # one workspace serves calls of different shapes in turn: the data one call
    # leaves in it must never sit where a later call keeps its counters (a
    # call with few row blocks followed by one with many, split-K on both)
    d = dev()
    shapes = [(64, 4096, 300, 512), (1, 8192, 1100, 1200), (33, 2048, 600, 640),
              (1, 8192, 1100, 1200), (8, 11008, 90, 200)]
    need = max(lr.lowrank_workspace_bytes(0, lr.LR_BF16, *s) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=d)
    for i, (T, d_in, r, d_out) in enumerate(shapes):
        c = make_linear(7000 + i, T, d_in, r, d_out, "bf16", fast=True)
        y_shared = lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], workspace=ws)
        y_fresh = lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"])
        torch.cuda.synchronize()
        assert np.array_equal(bits(y_shared), bits(y_fresh)), (T, d_in, r, d_out)
        assert maxrel(to_f64(y_shared), oracle.linear(c["x"], c["U"], c["V"])[1]) <= BF16_TOL
    counters = control_counters(ws)
    assert not counters.any(), np.nonzero(counters)   # every counter and flag back at zero


@pytest.mark.parametrize("T,shape", [(1024, (512, 300, 700)), (2100, (1300, 1194, 1280)),
                                     (4100, (4096, 819, 4096))])
def test_bf16_prefill_forced_fused(T, shape):
    # LR_PREFILL_FUSED keeps t on chip at row counts that otherwise take the
    # two large-tile GEMMs: a ragged last 64-row tile (2100, 4100), the
    # largest rank whose tile fits in LDS (1194 -> 1216 columns), ragged
    # d_in and d_out; both realizations meet the oracle's tolerance
    d_in, r, d_out = shape
    c = make_linear(4700 + T + r, T, d_in, r, d_out, "bf16", fast=True, ld_extra=8)
    y = torch.full((T, d_out), float("nan"), dtype=torch.bfloat16, device=dev())
    lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], y=y, flags=lr.LR_PREFILL_FUSED)
    y2, _ = _run(c, T, "bf16")
    torch.cuda.synchronize()
    _, yr = oracle.linear(c["x"], c["U"], c["V"])
    assert maxrel(to_f64(y), yr) <= BF16_TOL
    assert maxrel(to_f64(y2), yr) <= BF16_TOL


def test_bf16_prefill_forced_fused_refusals():
    # a rank tile past LDS, a requested t_io, a stage-only call and decode
    # row counts are refused before anything runs
    d = dev()
    x = torch.zeros((1024, 512), dtype=torch.bfloat16, device=d)
    for T, r, kw in [(1024, 1300, {}), (1024, 300, {"t_io": True}),
                     (1024, 300, {"stage1": True}), (64, 300, {})]:
        ut = torch.zeros((r, 512), dtype=torch.bfloat16, device=d)
        vt = torch.zeros((640, ld_for(r, 8)), dtype=torch.bfloat16, device=d)[:, :r]
        y = torch.full((T, 640), float("nan"), dtype=torch.bfloat16, device=d)
        t = torch.zeros((T, r), dtype=torch.float32, device=d)
        flags = lr.LR_PREFILL_FUSED | (lr.LR_STAGE1_ONLY if kw.get("stage1") else 0)
        with pytest.raises(lr.LowrankError) as err:
            lr.lowrank_linear_forward(x[:T], ut, vt, y=y, flags=flags,
                                      t_io=t if kw else None)
        assert err.value.status == lr._lib.LR_ERR_UNSUPPORTED, (T, r, kw)
        torch.cuda.synchronize()
        assert torch.isnan(y.float()).all()


@pytest.mark.parametrize("T", [1, 16, 17, 64])
def test_bf16_stage2_only_reads_strided_fp32_t(T):
    # stage 2 alone from a caller's fp32 t whose rows are padded with NaN past
    # r (ragged last k-step: r = 100): the padding must never reach y.  Up to
    # 16 tokens the tiles also form the bf16 residual of t, so y matches the
    # fp64 product of the fp32 t nearly to fp32 accuracy
    r, d_out = 100, 330
    c = make_linear(5100 + T, T, 640, r, d_out, "bf16", fast=True, ld_extra=8)
    g = torch.Generator(device="cpu").manual_seed(T)
    t = torch.full((T, r + 12), float("nan"), dtype=torch.float32)
    t[:, :r] = torch.randn((T, r), generator=g)
    t = t.to(dev())[:, :r]
    y = lr.lowrank_linear_forward(None, None, c["dVt"], t_io=t, flags=lr.LR_STAGE2_ONLY)
    torch.cuda.synchronize()
    yr = to_f64(t) @ c["V"]
    assert maxrel(to_f64(y), yr) <= BF16_TOL
    if T <= 16:   # t carried as bf16 hi + lo: only y's own bf16 rounding remains
        assert maxrel(to_f64(y), yr) <= 1e-2
