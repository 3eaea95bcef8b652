"""Helpers of the GPU tests: device tensors from seeded numpy inputs, and the
error metric max|gpu - ref| / max|ref|."""
import numpy as np
import torch

import synth


def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def to_dev(stor: np.ndarray, dtype: str):
    """Upload a synth.quantize storage array (uint16 bf16 bits or float32)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(stor).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(stor, dtype=np.float32))
    return t.to(dev())


def padded(stor: np.ndarray, ld: int, dtype: str, fill_nan: bool = True):
    """Device [rows, ld] buffer holding stor in its first columns; the padding
    is NaN so that any unmasked read of it poisons the result.  Returns the
    [rows, cols] view."""
    rows, cols = stor.shape
    if dtype == "bf16":
        full = np.full((rows, ld), 0x7FC0 if fill_nan else 0, dtype=np.uint16)
    else:
        full = np.full((rows, ld), np.nan if fill_nan else 0.0, dtype=np.float32)
    full[:, :cols] = stor
    return to_dev(full, dtype)[:, :cols]


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def maxrel(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def ld_for(n: int, extra: int = 0) -> int:
    return (n + 7) // 8 * 8 + extra


def make_linear(seed: int, T: int, d_in: int, r: int, d_out: int, dtype: str, fast: bool,
                ld_extra: int = 0, svd_weight_seed=None):
    """Seeded x, U_r, V_r quantised to dtype; returns exact fp64 values (math
    orientation) and device tensors x[T,d_in], Ut[r,d_in], Vt[d_out,r]."""
    if fast:
        U, V = synth.fast_factors(seed, d_in, d_out, r)
    else:
        W = synth.dense_weight(seed if svd_weight_seed is None else svd_weight_seed, d_in, d_out)
        U, V = synth.svd_factors(W, r)
    x = synth.tokens(seed + 1, T, d_in)
    xs, xv = synth.quantize(x, dtype)
    us, uv = synth.quantize(np.ascontiguousarray(U.T), dtype)     # [r, d_in]
    vs, vv = synth.quantize(np.ascontiguousarray(V.T), dtype)     # [d_out, r]
    dx = padded(xs, ld_for(d_in, ld_extra), dtype)
    du = padded(us, ld_for(d_in, ld_extra), dtype)
    dv = padded(vs, ld_for(r, ld_extra), dtype)
    return {"x": xv, "U": uv.T, "V": vv.T, "dx": dx, "dUt": du, "dVt": dv}


def control_counters(ws):
    """Every word of a decode-path workspace's eight control blocks (4096
    uint32 words each): counters, flags and error words, all back at zero
    after every call."""
    return ws[:8 * 16384].view(torch.int32).cpu().numpy().reshape(8, 4096)
