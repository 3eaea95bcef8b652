"""lowrank_linear_forward_noalloc (the library's fixed per-GPU scratch in place
of a workspace) against lowrank_linear_forward with a fresh workspace: two
calls in a row, the second smaller, then a prefill-path call and a request
larger than the scratch, which must be refused before anything runs."""
import numpy as np
import pytest
import torch

import oracle
import rank_decomposed_amd as lr
from rank_decomposed_amd import _lib
from gpu_util import bits, control_counters, dev, make_linear, maxrel, to_f64

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2


def _both(T, d_in, r, d_out, seed):
    c = make_linear(seed, T, d_in, r, d_out, "bf16", fast=True, ld_extra=8)
    need = lr.lowrank_workspace_bytes(0, lr.LR_BF16, T, d_in, r, d_out)
    assert need <= lr.LR_NOALLOC_SCRATCH_BYTES
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev())
    t_ref = torch.full((T, r), float("nan"), dtype=torch.float32, device=dev())
    y_ref = lr.lowrank_linear_forward(c["dx"], c["dUt"], c["dVt"], t_io=t_ref, workspace=ws)
    t = torch.full((T, r), float("nan"), dtype=torch.float32, device=dev())
    y = torch.full((T, d_out), float("nan"), dtype=torch.bfloat16, device=dev())
    lr.lowrank_linear_forward_noalloc(c["dx"], c["dUt"], c["dVt"], y=y, t_io=t)
    torch.cuda.synchronize()
    if need:
        assert not control_counters(ws).any()
    return c, y, t, y_ref, t_ref


def test_noalloc_matches_workspace_call_twice_then_smaller():
    # the MLP gate projection of a 7B decoder at 64 tokens, then the attention
    # q projection at 16 tokens: the second call reuses the scratch the first
    # left behind
    for T, shape, seed in [(64, (4096, 1791, 11008), 7100), (16, (4096, 1228, 4096), 7200)]:
        print(f"noalloc T={T} shape={shape}", flush=True)
        c, y, t, y_ref, t_ref = _both(T, *shape, seed)
        assert np.array_equal(bits(y), bits(y_ref)), (T, shape)
        assert np.array_equal(t.cpu().numpy(), t_ref.cpu().numpy()), (T, shape)
        tr, yr = oracle.linear(c["x"], c["U"], c["V"])
        assert maxrel(to_f64(t), tr) <= 1e-5
        assert maxrel(to_f64(y), yr) <= BF16_TOL


def test_noalloc_prefill_rows_and_repeat():
    # 300 rows run the prefill GEMMs (no scratch needed); a decode call after
    # it must still find the control words at zero
    for T, shape, seed in [(300, (1024, 300, 768), 7300), (8, (1024, 300, 768), 7400),
                           (8, (1024, 300, 768), 7400)]:
        print(f"noalloc T={T} shape={shape}", flush=True)
        _, y, t, y_ref, t_ref = _both(T, *shape, seed)
        assert np.array_equal(bits(y), bits(y_ref)), (T, shape)
        assert np.array_equal(t.cpu().numpy(), t_ref.cpu().numpy()), (T, shape)


def test_noalloc_refuses_requests_beyond_the_scratch():
    T, d_in, r, d_out = 1024, 4096, 1228, 4096
    need = lr.lowrank_workspace_bytes(0, lr.LR_BF16, T, d_in, r, d_out)
    assert need > lr.LR_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, d_in), dtype=torch.bfloat16, device=dev())
    ut = torch.zeros((r, d_in), dtype=torch.bfloat16, device=dev())
    vt = torch.zeros((d_out, r), dtype=torch.bfloat16, device=dev())
    y = torch.full((T, d_out), float("nan"), dtype=torch.bfloat16, device=dev())
    with pytest.raises(_lib.LowrankError) as err:
        lr.lowrank_linear_forward_noalloc(x, ut, vt, y=y)
    assert err.value.status == _lib.LR_ERR_CAPACITY
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all()      # refused before any kernel ran
