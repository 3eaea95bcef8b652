"""Parity at the workloads' full sizes, on the launch configurations the bench
times, against the fp64 oracle: every output where the oracle is cheap
(decode, tensor-parallel shares at T = 64), seeded samples of rows or
sequences where it is not (prefill rows are independent; so are sequences
of the decode step), and the remap gather bit for bit."""
import functools

import numpy as np
import pytest
import torch

import oracle
import rank_decomposed_amd as lr
import synth
from gpu_util import bits, dev, maxrel, to_f64
from synth.decode_step import DecodeStepInputs

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2
SHAPES_7B = {"q": (4096, 4096), "gate": (4096, 11008), "down": (11008, 4096)}
SHAPES_13B = {"q": (5120, 5120), "gate": (5120, 13824), "down": (13824, 5120)}


@functools.lru_cache(maxsize=16)
def factors(cfg_id, role, d_in, d_out, rho):
    """bf16 bits of Ut, Vt and their fp64 values (math orientation)."""
    r = oracle.rank_for_ratio(rho, d_in, d_out)
    U, V = synth.fast_factors(synth.seed_of(cfg_id, 0, synth.ROLES.index(role), synth.KIND_W),
                              d_in, d_out, r)
    ub, vb = synth.bf16_bits(U.T), synth.bf16_bits(V.T)
    return ub, vb, synth.bf16_value(ub).T, synth.bf16_value(vb).T


def up(b, ld=None):
    rows, cols = b.shape
    ld = ld or (cols + 7) // 8 * 8
    full = np.zeros((rows, ld), np.uint16)
    full[:, :cols] = b
    t = torch.from_numpy(full.view(np.int16)).view(torch.bfloat16).to(dev())
    return t[:, :cols]


@pytest.mark.parametrize("role", ["q", "gate", "down"])
def test_decode_7b_ratio06_all_tokens(role):
    # LLaMA-7B projections at parameter ratio 0.6, T = 1, 8, 32, 64: every output
    d_in, d_out = SHAPES_7B[role]
    ub, vb, U, V = factors(2, role, d_in, d_out, 0.6)
    dUt, dVt = up(ub), up(vb)
    for T in (1, 8, 32, 64):
        x = synth.tokens(synth.seed_of(2, 0, 0, synth.KIND_X) + T, T, d_in)
        xb = synth.bf16_bits(x)
        t = torch.empty((T, U.shape[1]), dtype=torch.float32, device=dev())
        y = lr.lowrank_linear_forward(up(xb), dUt, dVt, t_io=t)
        torch.cuda.synchronize()
        tr, yr = oracle.linear(synth.bf16_value(xb), U, V)
        et, ey = maxrel(to_f64(t), tr), maxrel(to_f64(y), yr)
        print("decode %s T=%d: t err %.2e, y err %.2e" % (role, T, et, ey))
        assert et <= 1e-5 and ey <= BF16_TOL


@pytest.mark.parametrize("rho", [0.4, 0.2])
@pytest.mark.parametrize("role", ["q", "gate", "down"])
def test_prefill_7b_16384_rows_sampled(role, rho):
    # 8 x 2048 = 16384 rows on the two large-tile GEMMs; 384 seeded rows checked
    d_in, d_out = SHAPES_7B[role]
    ub, vb, U, V = factors(3, role, d_in, d_out, rho)
    M = 16384
    seed = synth.seed_of(3, 0, synth.ROLES.index(role), synth.KIND_X)
    x = synth.hash_bf16_rows_torch(seed, M, d_in, dev())
    y = lr.lowrank_linear_forward(x, up(ub), up(vb))
    torch.cuda.synchronize()
    rows = np.sort(synth.rng(seed).choice(M, 384, replace=False))
    rows[0], rows[-1] = 0, M - 1
    _, yr = oracle.linear(synth.hash_rows(seed, rows, d_in), U, V)
    got = to_f64(y[torch.from_numpy(rows).to(dev())])
    err = maxrel(got, yr)
    print("prefill %s rho=%.1f: sampled y err %.2e" % (role, rho, err))
    assert err <= BF16_TOL


@pytest.mark.parametrize("T", [64, 4096])
@pytest.mark.parametrize("role", ["q", "gate", "down"])
def test_tensor_parallel_share_13b(role, T):
    # one of 8 shares of LLaMA-13B projections at ratio 0.4: U_r split by
    # input rows (stage 1 -> partial rank-r intermediate), V_r by output
    # columns (stage 2), passed as plain sub-matrices of the full factors
    d_in, d_out = SHAPES_13B[role]
    ub, vb, U, V = factors(4, role, d_in, d_out, 0.4)
    dUt, dVt = up(ub), up(vb)
    r = U.shape[1]
    seed = synth.seed_of(4, 0, synth.ROLES.index(role), synth.KIND_X) + T
    rows = np.arange(T) if T <= 64 else np.sort(synth.rng(seed).choice(T, 256, replace=False))
    x = synth.hash_bf16_rows_torch(seed, T, d_in, dev())
    xv = synth.hash_rows(seed, rows, d_in)
    P, s = 8, 3
    wi, wo = d_in // P, d_out // P
    t_s = torch.empty((T, r), dtype=torch.float32, device=dev())
    lr.lowrank_linear_forward(x[:, s * wi:(s + 1) * wi], dUt[:, s * wi:(s + 1) * wi], None,
                              t_io=t_s, flags=lr.LR_STAGE1_ONLY)
    # stage 2 on the share's output columns, fed the oracle's full t (the value
    # the exchange across shares would deliver)
    tr_rows, _ = oracle.linear(xv, U, V)
    t_in = np.zeros((T, r), np.float32)
    t_in[rows] = tr_rows.astype(np.float32)
    t_dev = torch.from_numpy(t_in).to(dev())
    y_s = lr.lowrank_linear_forward(None, None, dVt[s * wo:(s + 1) * wo], t_io=t_dev,
                                    flags=lr.LR_STAGE2_ONLY)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).to(dev())
    ref_t = oracle.tp_share_stage1(xv, U, s, P)
    ref_y = oracle.tp_share_stage2(t_in[rows].astype(np.float64), V, s, P)
    et = maxrel(to_f64(t_s[idx]), ref_t)
    ey = maxrel(to_f64(y_s[idx]), ref_y)
    print("TP share %s T=%d: t_s err %.2e, y_s err %.2e" % (role, T, et, ey))
    assert et <= 1e-5 and ey <= BF16_TOL
    # the share's partial is exactly its slice of the contraction: summing the
    # eight partials (the all-reduce) gives x U_r
    if T == 64:
        tot = np.zeros((T, r))
        for sh in range(P):
            part = torch.empty((T, r), dtype=torch.float32, device=dev())
            lr.lowrank_linear_forward(x[:, sh * wi:(sh + 1) * wi], dUt[:, sh * wi:(sh + 1) * wi],
                                      None, t_io=part, flags=lr.LR_STAGE1_ONLY)
            tot += to_f64(part)
        assert maxrel(tot, tr_rows) <= 1e-5


@functools.lru_cache(maxsize=1)
def step_inputs():
    return DecodeStepInputs(device=dev())


def test_remap_gather_decode_step_shape_bit_exact():
    # cap = 64 x 4112 rows of 409 bf16 latents in a 416-wide pool
    si = step_inputs()
    pool = si.device_pool(0, 0)
    prep = lr.lowrank_prepare_decode(si.lengths, si.tables, si.block, si.cap)
    remap = prep["remap"].copy()
    g = synth.rng(99)
    bad = g.choice(prep["n_valid"], 64, replace=False)
    remap[bad[:32]] = -1
    remap[bad[32:]] = si.pool_rows + g.integers(0, 1000, 32)     # out of range
    nv = torch.tensor([prep["n_valid"]], dtype=torch.int32, device=dev())
    r = si.ranks["k"]
    dst = torch.full((si.cap, 416), -21555, dtype=torch.int16, device=dev())  # 0xABCD
    dst = dst.view(torch.bfloat16)
    lr.kv_remap_gather(pool, torch.from_numpy(remap).to(dev()), dst, n_valid=nv, row_elems=r)
    torch.cuda.synchronize()
    got = bits(dst)
    sample = np.unique(np.concatenate([bad, g.choice(prep["n_valid"], 4000, replace=False),
                                       [0, prep["n_valid"] - 1]]))
    src_rows = np.where((remap[sample] >= 0) & (remap[sample] < si.pool_rows), remap[sample], 0)
    src_vals = synth.bf16_bits(synth.hash_rows(si.pool_seed(0, 0), src_rows, si.pool_ld))
    exp = oracle.remap_gather(src_vals, np.where(remap[sample] == src_rows, np.arange(len(sample)),
                                                 -1).astype(np.int32))
    assert np.array_equal(got[sample, :r], exp[:, :r])
    assert np.all(got[prep["n_valid"]:] == 0xABCD)        # past n_valid: untouched
    assert np.all(got[sample, r:] == 0xABCD)              # past row_elems: untouched


def sampled_sequences(lengths):
    """8 seeded sequences of the 64, the shortest and the longest among them."""
    rest = np.setdiff1d(np.arange(len(lengths)), [np.argmin(lengths), np.argmax(lengths)])
    pick = np.random.default_rng(2024).choice(rest, 6, replace=False)
    return [int(np.argmin(lengths)), int(np.argmax(lengths))] + sorted(int(i) for i in pick)


@functools.lru_cache(maxsize=1)
def decode_step_reference():
    """fp64 oracle of the 32-layer step on the sampled sequences (computed
    once for both step variants; a few minutes of host time)."""
    si = DecodeStepInputs(device=None)
    c = si.cfg
    seqs = sampled_sequences(si.lengths)
    layers = (si.layer_values(li) for li in range(c["n_layers"]))
    pools_k = [si.pool_rows_for(li, 0, seqs) for li in range(c["n_layers"])]
    pools_v = [si.pool_rows_for(li, 1, seqs) for li in range(c["n_layers"])]
    sub_tables = [si.tables[i] for i in seqs]
    return seqs, oracle.decode_step(si.h0[seqs], layers, pools_k, pools_v, sub_tables,
                                    si.lengths[seqs], si.block, c)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fused", [False, True])
def test_decode_step_32_layers_sampled_sequences(fused):
    # fused: the reconstruction inside the attention (lowrank_layer_decode_step_fused)
    si = step_inputs()
    c = si.cfg
    d = dev()
    rope = torch.empty((si.max_seq_rows, c["head_dim"] // 2, 2), dtype=torch.float32, device=d)
    lr.lowrank_rope_table(c["head_dim"], si.max_seq_rows, 10000.0, rope)
    prep = lr.lowrank_prepare_decode(si.lengths, si.tables, si.block, si.cap)
    dp = {k: torch.from_numpy(np.ascontiguousarray(prep[k])).to(d)
          for k in ("remap", "seq_off", "pos", "slot_mapping")}
    nv = torch.tensor([prep["n_valid"]], dtype=torch.int32, device=d)
    h = torch.from_numpy(si.h0.astype(np.float32)).to(d)
    ws = None
    for li in range(c["n_layers"]):
        Ut, Vt, g1, g2 = si.device_layer(li)
        w = lr.layer_weights(c, Ut, Vt, g1, g2, rope, si.max_seq_rows)
        pk, pv = si.device_pool(li, 0), si.device_pool(li, 1)
        st = lr.decode_state(pk, pv, dp["slot_mapping"], dp["remap"], dp["seq_off"], dp["pos"],
                             nv, si.max_seq_rows)
        if ws is None:
            size = (lr.lowrank_decode_step_fused_workspace_bytes if fused
                    else lr.lowrank_decode_step_workspace_bytes)
            ws = torch.zeros(size(w, st), dtype=torch.uint8, device=d)
        (lr.lowrank_layer_decode_step_fused if fused else lr.lowrank_layer_decode_step)(w, st, h, ws)
        torch.cuda.synchronize()
        print("layer %d done" % li, flush=True)
        del pk, pv, w, st, Ut, Vt
    got = to_f64(h)
    seqs, ref = decode_step_reference()
    for k, i in enumerate(seqs):
        err = maxrel(got[i], ref[k])
        print("32-layer decode step%s, sequence %d (L=%d): max rel err %.2e"
              % (" (fused)" if fused else "", i, si.lengths[i], err))
        assert err <= BF16_TOL
