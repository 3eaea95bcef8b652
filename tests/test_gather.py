"""kv_remap_gather on the GPU against the oracle, bit for bit: every row
width class (one 16-byte chunk per lane and a 2-byte tail, rows past 2 KiB,
4- and 2-byte accesses for unaligned pitches), invalid remap entries (zero
rows), live counts of zero, partial and past the capacity, and the rows and
columns the call must leave untouched."""
import numpy as np
import pytest
import torch

import oracle
import rank_decomposed_amd as lr
import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu
SENTINEL = {torch.bfloat16: 0xABCD, torch.float32: 0x7FBADBAD}


def _case(seed, dtype, row_elems, src_ld, dst_ld, src_rows, cap):
    g = synth.rng(seed)
    nbits = np.uint16 if dtype == torch.bfloat16 else np.uint32
    sbits = g.integers(0, np.iinfo(nbits).max, size=(src_rows, src_ld), dtype=np.uint64).astype(nbits)
    remap = g.integers(0, src_rows, size=cap).astype(np.int32)
    bad = g.choice(cap, max(1, cap // 50), replace=False)
    remap[bad[::3]] = -1
    remap[bad[1::3]] = src_rows + g.integers(0, 1000, len(bad[1::3]))   # past the pool
    remap[bad[2::3]] = np.iinfo(np.int32).min
    sint = np.int16 if dtype == torch.bfloat16 else np.int32
    src = torch.from_numpy(sbits.view(sint)).to(dev()).view(dtype)
    dbits = np.full((cap, dst_ld), SENTINEL[dtype], dtype=nbits)
    dst = torch.from_numpy(dbits.view(sint)).to(dev()).view(dtype)
    return sbits, remap, src, dst, dbits


def _bits(t):
    sint = torch.int16 if t.dtype == torch.bfloat16 else torch.int32
    un = np.uint16 if t.dtype == torch.bfloat16 else np.uint32
    return t.view(sint).cpu().numpy().view(un)


@pytest.mark.parametrize("dtype,row_elems,src_ld,dst_ld,cap,nv", [
    (torch.bfloat16, 409, 416, 416, 40000, 37001),    # latent rows: 16-byte chunks + 2-byte tail
    (torch.bfloat16, 1024, 1024, 1032, 9000, None),   # 2 KiB rows, no tail
    (torch.bfloat16, 1025, 1032, 1040, 3000, 2999),   # past 2 KiB: per-chunk loop
    (torch.bfloat16, 7, 9, 11, 5000, 4000),            # unaligned pitch: 2-byte accesses
    (torch.float32, 409, 412, 420, 20000, 19999),     # 4-byte tail
    (torch.float32, 3, 3, 5, 7000, 7000),              # 4-byte accesses
    (torch.bfloat16, 409, 416, 416, 1000, 0),         # nothing live
    (torch.bfloat16, 64, 64, 64, 1000, 5000),         # live count past the capacity: clamped
])
def test_gather_bit_exact(dtype, row_elems, src_ld, dst_ld, cap, nv):
    src_rows = 3 * cap // 2 + 7
    sbits, remap, src, dst, dbits = _case(1000 + row_elems + cap, dtype, row_elems, src_ld,
                                          dst_ld, src_rows, cap)
    n_valid = None if nv is None else torch.tensor([nv], dtype=torch.int32, device=dev())
    lr.kv_remap_gather(src, torch.from_numpy(remap).to(dev()), dst, n_valid=n_valid,
                       row_elems=row_elems)
    torch.cuda.synchronize()
    got = _bits(dst)
    exp = oracle.remap_gather(sbits[:, :row_elems], remap, n_valid=nv,
                              dst_init=dbits[:, :row_elems])
    assert np.array_equal(got[:, :row_elems], exp)
    assert np.all(got[:, row_elems:] == SENTINEL[dtype])     # past row_elems: untouched
