"""lowrank_linear_forward_group on the GPU: several independent decode
linears in one launch match the fp64 oracle (stage-1-only and accumulate
members included), and give bit for bit what separate calls give where both
split the stage-1 reduction alike (d_in under 1024 here: one or two K ranges
either way)."""
import functools

import numpy as np
import pytest
import torch

import oracle
import rank_decomposed_amd as lr
import synth
from gpu_util import bits, control_counters, dev, ld_for, make_linear, maxrel, padded, to_f64

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2
SHAPES = [(1024, 300, 1024), (1024, 96, 256), (1024, 120, 256)]     # q-, k-, v-like


def _cases(T, seed, shapes=SHAPES):
    return [make_linear(seed + i, T, d_in, r, d_out, "bf16", fast=True, ld_extra=8)
            for i, (d_in, r, d_out) in enumerate(shapes)]


@pytest.mark.parametrize("T", [1, 8, 16, 17, 33, 64])
def test_group_matches_separate_calls_and_oracle(T):
    cs = _cases(T, 8000 + T)
    x = cs[0]["dx"]                      # one input for all members, as q, k, v share it
    for c in cs[1:]:
        c["x"] = cs[0]["x"]
    ts = [torch.empty((T, c["dUt"].shape[0]), dtype=torch.float32, device=dev()) for c in cs]
    ys = lr.lowrank_linear_forward_group(
        [dict(x=x, Ut=c["dUt"], Vt=c["dVt"], t_io=t) for c, t in zip(cs, ts)])
    sep_t = [torch.empty_like(t) for t in ts]
    sep = [lr.lowrank_linear_forward(x, c["dUt"], c["dVt"], t_io=t) for c, t in zip(cs, sep_t)]
    torch.cuda.synchronize()
    for c, y, t, ys_, ts_ in zip(cs, ys, ts, sep, sep_t):
        assert np.array_equal(bits(y), bits(ys_))
        assert np.array_equal(to_f64(t), to_f64(ts_))
        tr, yr = oracle.linear(cs[0]["x"], c["U"], c["V"])
        assert maxrel(to_f64(t), tr) <= 1e-5
        assert maxrel(to_f64(y), yr) <= BF16_TOL


@pytest.mark.parametrize("T", [4, 40])
def test_group_mixed_members(T):
    # member 0: full; member 1: stage 1 only (the latent of a k projection);
    # member 2: accumulates into an fp32 residual
    cs = _cases(T, 8100 + T, [(640, 200, 640), (640, 64, 128), (640, 150, 512)])
    x = cs[0]["dx"]
    d = dev()
    t1 = torch.full((T, 64), float("nan"), dtype=torch.float32, device=d)
    g = torch.Generator(device="cpu").manual_seed(T)
    acc0 = torch.randn((T, 512), generator=g, dtype=torch.float32)
    acc = acc0.clone().to(d)
    ys = lr.lowrank_linear_forward_group([dict(x=x, Ut=cs[0]["dUt"], Vt=cs[0]["dVt"]),
                                          dict(x=x, Ut=cs[1]["dUt"], t_io=t1),
                                          dict(x=x, Ut=cs[2]["dUt"], Vt=cs[2]["dVt"], y_acc=acc)])
    torch.cuda.synchronize()
    xv = cs[0]["x"]
    assert maxrel(to_f64(ys[0]), oracle.linear(xv, cs[0]["U"], cs[0]["V"])[1]) <= BF16_TOL
    assert ys[1] is None and ys[2] is None
    assert maxrel(to_f64(t1), oracle.linear(xv, cs[1]["U"], cs[1]["V"])[0]) <= 1e-5
    added = to_f64(acc) - acc0.double().numpy()
    assert maxrel(added, oracle.linear(xv, cs[2]["U"], cs[2]["V"])[1]) <= BF16_TOL


@pytest.mark.parametrize("T", [40, 64])
def test_group_tall_stage2_tiles(T):
    # three members with a ragged last stage-2 tile (4100 output rows) at
    # more than 32 tokens; member 1 accumulates into an fp32 residual.
    # Outputs start as NaN.
    cs = _cases(T, 8200 + T, [(512, 100, 4100), (512, 60, 4100), (512, 130, 4100)])
    x = cs[0]["dx"]
    d = dev()
    y0 = torch.full((T, 4100), float("nan"), dtype=torch.bfloat16, device=d)
    y2 = torch.full((T, 4100), float("nan"), dtype=torch.bfloat16, device=d)
    g = torch.Generator(device="cpu").manual_seed(T)
    acc0 = torch.randn((T, 4100), generator=g, dtype=torch.float32)
    acc = acc0.clone().to(d)
    lr.lowrank_linear_forward_group([dict(x=x, Ut=cs[0]["dUt"], Vt=cs[0]["dVt"], y=y0),
                                     dict(x=x, Ut=cs[1]["dUt"], Vt=cs[1]["dVt"], y_acc=acc),
                                     dict(x=x, Ut=cs[2]["dUt"], Vt=cs[2]["dVt"], y=y2)])
    sep = [lr.lowrank_linear_forward(x, c["dUt"], c["dVt"]) for c in (cs[0], cs[2])]
    torch.cuda.synchronize()
    xv = cs[0]["x"]
    for c, y, s in zip((cs[0], cs[2]), (y0, y2), sep):
        yr = oracle.linear(xv, c["U"], c["V"])[1]
        assert maxrel(to_f64(y), yr) <= BF16_TOL
        # stage-2 tiles split k over the waves alike and sum the waves in one
        # fixed order: grouped equals separate bit for bit
        assert np.array_equal(bits(y), bits(s))
    added = to_f64(acc) - acc0.double().numpy()
    assert maxrel(added, oracle.linear(xv, cs[1]["U"], cs[1]["V"])[1]) <= BF16_TOL


@pytest.mark.parametrize("T", [1, 32])
def test_group_packed_matches_row_major(T):
    cs = _cases(T, 8200 + T)
    x = cs[0]["dx"]
    rm = lr.lowrank_linear_forward_group([dict(x=x, Ut=c["dUt"], Vt=c["dVt"]) for c in cs])
    pk = lr.lowrank_linear_forward_group([dict(x=x, Ut=lr.pack_factor(c["dUt"]),
                                               Vt=lr.pack_factor(c["dVt"])) for c in cs])
    torch.cuda.synchronize()
    for a, b in zip(rm, pk):
        assert np.array_equal(bits(a), bits(b))


def test_group_and_single_calls_share_a_workspace():
    d = dev()
    cs = _cases(8, 8300)
    x = cs[0]["dx"]
    ws = torch.zeros(4 << 20, dtype=torch.uint8, device=d)
    lin = [dict(x=x, Ut=c["dUt"], Vt=c["dVt"]) for c in cs]
    assert lr.lowrank_group_workspace_bytes(8, lin) <= ws.numel()
    for rep in range(3):
        y0 = lr.lowrank_linear_forward(x, cs[0]["dUt"], cs[0]["dVt"], workspace=ws)
        ys = lr.lowrank_linear_forward_group(lin, workspace=ws)
        y2 = lr.lowrank_linear_forward(x, cs[2]["dUt"], cs[2]["dVt"], workspace=ws)
        torch.cuda.synchronize()
        ref = [lr.lowrank_linear_forward(x, c["dUt"], c["dVt"]) for c in cs]
        torch.cuda.synchronize()
        assert np.array_equal(bits(y0), bits(ref[0]))
        assert np.array_equal(bits(y2), bits(ref[2]))
        for a, b in zip(ys, ref):
            assert np.array_equal(bits(a), bits(b))
        for L in lin:
            L.pop("y", None)
    assert not control_counters(ws).any()      # every counter back at zero


def test_group_graph_replay():
    d = dev()
    cs = _cases(16, 8400)
    x = cs[0]["dx"].clone()
    ws = torch.zeros(4 << 20, dtype=torch.uint8, device=d)
    ys = [torch.empty((16, c["dVt"].shape[0]), dtype=torch.bfloat16, device=d) for c in cs]
    lin = [dict(x=x, Ut=c["dUt"], Vt=c["dVt"], y=y) for c, y in zip(cs, ys)]
    lr.lowrank_linear_forward_group(lin, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(d)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lr.lowrank_linear_forward_group(lin, workspace=ws, stream=s)
    gen = torch.Generator(device=d).manual_seed(5)
    for rep in range(3):
        x.copy_(torch.randn(x.shape, generator=gen, device=d).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [bits(y) for y in ys]
        ref = [bits(lr.lowrank_linear_forward(x, c["dUt"], c["dVt"])) for c in cs]
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)


@functools.lru_cache(maxsize=8)
def _share_factors(seed, d_in, r, d_out, P):
    U, V = synth.fast_factors(seed, d_in, d_out, r)
    return U[:d_in // P], V[:, :d_out // P]


def _share(seed, T, d_in, r, d_out, P):
    """Share 0 of P of a rank-r decomposition of a d_in x d_out weight: the
    first d_in / P rows of U_r and the first d_out / P columns of V_r (so r
    may exceed both share widths), as make_linear returns them."""
    U, V = _share_factors(seed, d_in, r, d_out, P)
    wi = d_in // P
    x = synth.tokens(seed + 1 + T, T, wi)
    xs, xv = synth.quantize(x, "bf16")
    us, uv = synth.quantize(np.ascontiguousarray(U.T), "bf16")
    vs, vv = synth.quantize(np.ascontiguousarray(V.T), "bf16")
    return {"x": xv, "U": uv.T, "V": vv.T, "dx": padded(xs, ld_for(wi, 8), "bf16"),
            "dUt": padded(us, ld_for(wi, 8), "bf16"), "dVt": padded(vs, ld_for(r, 8), "bf16")}


@pytest.mark.parametrize("T", [1, 16, 17, 64])
def test_group_stage2_only_members(T):
    # a tensor-parallel share's stage 2: each member multiplies its own fp32
    # rank-space t (which the shares would have summed) by its V_r columns.
    # Three stage-2-only members (one packed split for all) against separate
    # stage-2-only calls, bit for bit, and against the oracle from that t
    cs = [_share(8500, T, 2560, 1024, 2560, 4), _share(8510, T, 2560, 1494, 6912, 4),
          make_linear(8520 + T, T, 640, 120, 130, "bf16", fast=True, ld_extra=8)]
    d = dev()
    g = torch.Generator(device="cpu").manual_seed(100 + T)
    ts = [torch.randn((T, c["dUt"].shape[0]), generator=g, dtype=torch.float32).to(d)
          for c in cs]
    ys = [torch.full((T, c["dVt"].shape[0]), float("nan"), dtype=torch.bfloat16, device=d)
          for c in cs]
    lr.lowrank_linear_forward_group([dict(Vt=c["dVt"], t_io=t, y=y)
                                     for c, t, y in zip(cs, ts, ys)])
    sep = [lr.lowrank_linear_forward(None, None, c["dVt"], t_io=t, flags=lr.LR_STAGE2_ONLY)
           for c, t in zip(cs, ts)]
    torch.cuda.synchronize()
    for c, t, y, s in zip(cs, ts, ys, sep):
        assert np.array_equal(bits(y), bits(s))
        assert maxrel(to_f64(y), to_f64(t) @ c["V"]) <= BF16_TOL


@pytest.mark.parametrize("T", [8, 64])
def test_group_share_pattern_stage1_then_stage2(T):
    # q, k, v of one share: stage 1 alone for all three (one launch, one x),
    # then stage 2 alone for all three from the fp32 t (one launch), packed
    # factors; equals the fused per-linear result of the oracle
    cs = [_share(8600 + i, T, 2560, 1024, 2560, 4) for i in range(3)]
    x = cs[0]["dx"]
    d = dev()
    ts = [torch.full((T, 1024), float("nan"), dtype=torch.float32, device=d) for _ in cs]
    s1 = [dict(x=x, Ut=lr.pack_factor(c["dUt"]), t_io=t) for c, t in zip(cs, ts)]
    s2 = [dict(Vt=lr.pack_factor(c["dVt"]), t_io=t) for c, t in zip(cs, ts)]
    need = max(lr.lowrank_group_workspace_bytes(T, s1), lr.lowrank_group_workspace_bytes(T, s2))
    ws = torch.zeros(need, dtype=torch.uint8, device=d)
    lr.lowrank_linear_forward_group(s1, workspace=ws)
    ys = lr.lowrank_linear_forward_group(s2, workspace=ws)
    torch.cuda.synchronize()
    # a launch where no linear waits counts nothing: its control words stay zero
    assert not control_counters(ws).any()
    for c, t, y in zip(cs, ts, ys):
        tr, yr = oracle.linear(cs[0]["x"], c["U"], c["V"])
        assert maxrel(to_f64(t), tr) <= 1e-5
        assert maxrel(to_f64(y), yr) <= BF16_TOL
