"""The decode path's bounded wait and its control area (GPU).

A stage-2 tile waits for the rank-r intermediate t of its linear (DeInfer/en
§2.A: the upward projection needs the whole downward one).  The wait is
bounded; one that gives up leaves an error word that lowrank_workspace_check
reports, and the kernel still returns every counter to zero, so the next
call on the same workspace is exact.  Forced here from the host with a
spin limit of zero polls (every kernel runs to its end).  Also: a workspace
reused by calls on different inputs gives each call its own result, bit for
bit what a fresh workspace gives."""
import numpy as np
import pytest
import torch

import oracle
import rank_decomposed_amd as lr
import synth
from gpu_util import bits, control_counters, dev, make_linear, maxrel, padded, to_f64

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2


def _ws(T, d_in, r, d_out):
    return torch.zeros(lr.lowrank_workspace_bytes(0, lr.LR_BF16, T, d_in, r, d_out),
                       dtype=torch.uint8, device=dev())


def _give_up(fn):
    """Run fn with waits that give up at once (the default restored after)."""
    try:
        lr.lowrank_set_wait_limit(0)
        out = fn()
        torch.cuda.synchronize()
    finally:
        lr.lowrank_set_wait_limit(lr.LR_DEFAULT_WAIT_LIMIT)
    return out


@pytest.mark.parametrize("T", [1, 64])
def test_give_up_is_reported_and_the_next_call_is_exact(T):
    # the gate shape at ratio 0.6: stage 1 streams 14.7 MB, long enough that
    # stage-2 tiles resident beside it reach their wait first
    c = make_linear(9100 + T, T, 4096, 1791, 11008, "bf16", fast=True)
    ws = _ws(T, 4096, 1791, 11008)
    ref = lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"])
    torch.cuda.synchronize()
    assert lr.lowrank_workspace_check(ws) == 0
    _give_up(lambda: lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], workspace=ws))
    # no check in between: the counters are back at zero, so this call is exact
    y = lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(ref))
    # the error word stays until it is read; reading it clears the area
    assert lr.lowrank_workspace_check(ws, raise_on_wait=False) == 1
    assert lr.lowrank_workspace_check(ws) == 0
    y = lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(ref))
    assert maxrel(to_f64(y), oracle.linear(c["x"], c["U"], c["V"])[1]) <= BF16_TOL


def test_give_up_in_a_group_names_its_members():
    T = 8
    shapes = [(4096, 1791, 11008), (4096, 1791, 11008)]
    cs = [make_linear(9150 + i, T, *s, "bf16", fast=True) for i, s in enumerate(shapes)]
    x = cs[0]["dx"]
    members = lambda: [dict(x=x, Ut=c["dUt"], Vt=c["dVt"]) for c in cs]
    ws = torch.zeros(lr.lowrank_group_workspace_bytes(T, members()), dtype=torch.uint8,
                     device=dev())
    ref = lr.lowrank_linear_forward_group(members())
    _give_up(lambda: lr.lowrank_linear_forward_group(members(), workspace=ws))
    mask = lr.lowrank_workspace_check(ws, raise_on_wait=False)
    assert mask != 0 and mask & ~0b11 == 0
    with pytest.raises(lr.LowrankError):           # a give-up raises by default
        _give_up(lambda: lr.lowrank_linear_forward_group(members(), workspace=ws))
        lr.lowrank_workspace_check(ws)
    assert lr.lowrank_workspace_check(ws) == 0
    got = lr.lowrank_linear_forward_group(members(), workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("T", [1, 16, 33, 64])
def test_workspace_reused_across_inputs(T):
    # t lives at the same workspace address in every call: each call must
    # read the t of its own stage 1
    c = make_linear(9200 + T, T, 4096, 1228, 4096, "bf16", fast=True)
    x2v = synth.tokens(9300 + T, T, 4096)
    xs2, x2 = synth.quantize(x2v, "bf16")
    dx2 = padded(xs2, 4096, "bf16")
    ws = _ws(T, 4096, 1228, 4096)
    outs = []
    for i in range(6):
        x = c["dx"] if i % 2 == 0 else dx2
        outs.append(lr.lowrank_linear_forward(x, c["dUt"], c["dVt"], workspace=ws))
    r1 = lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"])
    r2 = lr.lowrank_linear_forward(dx2, c["dUt"], c["dVt"])
    torch.cuda.synchronize()
    for i, y in enumerate(outs):
        assert np.array_equal(bits(y), bits(r1 if i % 2 == 0 else r2)), i
    assert maxrel(to_f64(outs[1]), oracle.linear(x2, c["U"], c["V"])[1]) <= BF16_TOL


def test_one_workspace_serves_every_path_in_turn():
    # The decode path keeps its counters in the workspace's control area; the
    # other paths park t there too (large-tile prefill GEMMs; the unfused
    # prefill for a rank tile too large for the fused kernel; fp32), past
    # that area, so decode calls before and after them on one workspace give
    # what a fresh workspace gives, with no clearing in between.
    dec = make_linear(9400, 8, 4096, 1228, 4096, "bf16", fast=True)
    big = make_linear(9410, 1024, 1024, 300, 768, "bf16", fast=True)
    unf = make_linear(9420, 100, 2048, 1500, 2048, "bf16", fast=True)
    f32 = make_linear(9430, 4, 512, 96, 256, "f32", fast=True)
    calls = [(dec, lr.LR_BF16), (big, lr.LR_BF16), (unf, lr.LR_BF16), (f32, lr.LR_F32)]
    need = max(lr.lowrank_workspace_bytes(0, dt, c["dx"].shape[0], c["dx"].shape[1],
                                          c["dUt"].shape[0], c["dVt"].shape[0])
               for c, dt in calls)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    ref = [lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"]) for c, _ in calls]
    torch.cuda.synchronize()
    for i in [0, 1, 0, 2, 0, 3, 0]:
        c = calls[i][0]
        print(f"shared workspace: call {i} T={c['dx'].shape[0]}", flush=True)
        y = lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), bits(ref[i])), i
        assert not control_counters(ws).any(), i
    assert lr.lowrank_workspace_check(ws) == 0
    for (c, _), y in zip(calls, ref):
        tol = 1e-5 if y.dtype == torch.float32 else BF16_TOL
        assert maxrel(to_f64(y), oracle.linear(c["x"], c["U"], c["V"])[1]) <= tol
