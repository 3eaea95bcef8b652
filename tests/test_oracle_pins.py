"""Pins of the fp64 oracle against what the mathematics fixes (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
swapped operand, the wrong half of the spectrum, sigma on one side only, an
off-by-one in the paging) fails at least one test here.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from golden_io import linear_cases, paging_case


def _rel(a, b):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300)


# ------------------------------------------------------------------ linear
@pytest.mark.parametrize("case", linear_cases(), ids=lambda c: c["name"])
def test_linear_hand_worked(case):
    t, y = oracle.linear(case["x"], case["U"], case["V"])
    assert np.array_equal(t, case["t"])
    assert np.array_equal(y, case["y"])


@pytest.mark.parametrize("seed", range(6))
def test_linear_brute_force_loops(seed):
    g = np.random.default_rng(seed)
    T, d_in, r, d_out = g.integers(1, 4), g.integers(1, 9), g.integers(1, 5), g.integers(1, 9)
    x = g.standard_normal((T, d_in))
    U = g.standard_normal((d_in, r))
    V = g.standard_normal((r, d_out))
    t, y = oracle.linear(x, U, V)
    tl, yl = oracle.linear_loops(x.tolist(), U.tolist(), V.tolist())
    assert np.allclose(t, tl, rtol=1e-13, atol=1e-13)
    assert np.allclose(y, yl, rtol=1e-13, atol=1e-13)


def test_associativity():
    g = np.random.default_rng(1)
    x = g.standard_normal((5, 48))
    U = g.standard_normal((48, 7))
    V = g.standard_normal((7, 40))
    _, y = oracle.linear(x, U, V)
    assert _rel(y, x @ (U @ V)) <= 1e-12


@pytest.mark.parametrize("shape", [(24, 24), (16, 40), (40, 16)])
def test_full_rank_reconstruction(shape):
    W = synth.dense_weight(7, *shape)
    r = min(shape)
    U, V, _ = oracle.truncated_factors(W, r)
    assert np.max(np.abs(U @ V - W)) <= 1e-12 * np.max(np.abs(W))
    x = synth.tokens(8, 3, shape[0])
    _, y = oracle.linear(x, U, V)
    assert _rel(y, x @ W) <= 1e-12


@pytest.mark.parametrize("r", [1, 5, 12, 23])
def test_eckart_young(r):
    W = synth.dense_weight(11, 24, 36)
    U, V, _ = oracle.truncated_factors(W, r)
    # singular values from an independent route: eigenvalues of W W^T
    lam = np.sort(np.linalg.eigvalsh(W @ W.T))[::-1]
    err = np.sum((W - U @ V) ** 2)
    assert abs(err - lam[r:].sum()) <= 1e-9 * lam.sum()
    # best rank-r: keeping any other r singular triplets is strictly worse
    P, s, Qt = np.linalg.svd(W, full_matrices=False)
    keep = np.arange(1, r + 1)
    alt = (P[:, keep] * s[keep]) @ Qt[keep]
    assert np.sum((W - alt) ** 2) > err


def test_factor_balance():
    W = synth.dense_weight(12, 20, 30)
    U, V, _ = oracle.truncated_factors(W, 6)
    lam = np.sort(np.linalg.eigvalsh(W @ W.T))[::-1][:6]
    sig = np.sqrt(lam)
    # sqrt(sigma) on each side: U^T U = diag(sigma) = V V^T
    assert np.allclose(U.T @ U, np.diag(sig), atol=1e-12)
    assert np.allclose(V @ V.T, np.diag(sig), atol=1e-12)


def test_rank_for_ratio_table():
    table = {(0.6, 4096, 4096): 1228, (0.6, 4096, 11008): 1791, (0.6, 11008, 4096): 1791,
             (0.4, 4096, 4096): 819, (0.4, 4096, 11008): 1194, (0.2, 4096, 4096): 409,
             (0.2, 4096, 11008): 597, (0.4, 5120, 5120): 1024, (0.4, 5120, 13824): 1494}
    for (rho, a, b), r in table.items():
        got = oracle.rank_for_ratio(rho, a, b)
        assert got == r, (rho, a, b)
        # closed-form bracket, in exact integers: r(a+b) <= rho*a*b < (r+1)(a+b)
        num = int(round(rho * 10)) * a * b
        assert 10 * r * (a + b) <= num < 10 * (r + 1) * (a + b)


def test_tp_shard_sum_and_concat():
    g = np.random.default_rng(3)
    x = g.standard_normal((4, 64))
    U = g.standard_normal((64, 9))
    V = g.standard_normal((9, 32))
    t, y = oracle.linear(x, U, V)
    parts = [oracle.tp_share_stage1(x, U, s, 8) for s in range(8)]
    assert _rel(sum(parts), t) <= 1e-13
    ys = [oracle.tp_share_stage2(t, V, s, 8) for s in range(8)]
    assert _rel(np.concatenate(ys, axis=1), y) <= 1e-13
    # a share only sees its own rows: zeroing the others changes nothing
    x2 = np.zeros_like(x)
    x2[:, 16:24] = x[:, 16:24]
    assert np.array_equal(oracle.tp_share_stage1(x2, U, 2, 8), parts[2])


# ------------------------------------------------------------------ paging
def test_prepare_hand_worked():
    c = paging_case()
    out = oracle.prepare_decode(c["tables"], c["len"], c["block"], c["cap"])
    for k in ("remap", "seq_off", "pos", "slot_mapping"):
        assert np.array_equal(out[k], c[k]), k
    assert out["n_valid"] == c["n_valid"]
    assert out["n_runs"] == c["n_runs"]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prepare_coverage_and_maximal_runs(seed):
    lengths = synth.decode_lengths(seed, 12, 1, 300)
    tables, nblocks = synth.block_tables(seed + 100, lengths, block=16)
    cap = int(sum(lengths) + len(lengths) + 37)
    out = oracle.prepare_decode(tables, lengths, 16, cap)
    off = out["seq_off"]
    assert off[0] == 0 and np.array_equal(np.diff(off), np.asarray(lengths) + 1)
    assert out["n_valid"] == off[-1]
    assert np.all(out["remap"][out["n_valid"]:] == -1)
    seen = set()
    for i, L in enumerate(lengths):
        for p in range(L + 1):
            phys = tables[i][p // 16] * 16 + p % 16
            assert out["remap"][off[i] + p] == phys
            seen.add(int(phys))
        assert out["slot_mapping"][i] == tables[i][L // 16] * 16 + L % 16
        assert out["pos"][i] == L
    assert len(seen) == out["n_valid"]           # no physical row used twice
    # runs are maximal: segment count = 1 + number of physical breaks
    breaks = 0
    for i, L in enumerate(lengths):
        nb = (L + 1 + 15) // 16
        breaks += 1 + sum(1 for b in range(1, nb) if tables[i][b] != tables[i][b - 1] + 1)
    assert out["n_runs"] == breaks
    for src, dst, n in out["runs"]:
        assert np.array_equal(out["remap"][dst:dst + n], np.arange(src, src + n))


def test_prepare_single_block_runs_is_block_table():
    # every other physical block: no two blocks adjacent, so each run is one block
    tables = [np.array([8, 2, 6], np.int32), np.array([0, 4], np.int32)]
    lengths = [40, 20]
    out = oracle.prepare_decode(tables, lengths, 16, 80)
    assert out["n_runs"] == 5
    exp = [src // 16 for src, _, _ in out["runs"]]
    assert exp == [8, 2, 6, 0, 4]


def test_prepare_capacity_error():
    with pytest.raises(ValueError):
        oracle.prepare_decode([np.array([0], np.int32)], [15], 16, 15)


def test_gather_against_loops_and_identities():
    g = np.random.default_rng(5)
    src = g.integers(0, 65536, size=(11, 5)).astype(np.uint16)
    remap = np.array([3, -1, 10, 11, 0, 7, -5, 2], dtype=np.int32)
    init = np.full((8, 5), 0xABCD, np.uint16)
    for nv in (None, 0, 5, 8, 100):
        a = oracle.remap_gather(src, remap, nv, init)
        b = np.array(oracle.remap_gather_loops(src.tolist(), remap.tolist(), nv, init.tolist()),
                     dtype=np.uint16)
        assert np.array_equal(a, b)
    ident = oracle.remap_gather(src, np.arange(11, dtype=np.int32))
    assert np.array_equal(ident, src)
    z = oracle.remap_gather(src, remap)
    assert np.all(z[[1, 3, 6]] == 0)
    kept = oracle.remap_gather(src, remap, 5, init)
    assert np.all(kept[5:] == 0xABCD)


# ------------------------------------------------------------------ decoder
def test_rmsnorm_closed_forms():
    g = np.linspace(0.5, 1.5, 16)
    # constant vector c: h/sqrt(c^2+eps)*g; eps = 0 gives sign(c) g
    assert np.allclose(oracle.rmsnorm(np.full(16, -3.0), g, eps=0.0), -g, atol=1e-15)
    # [3, 4] with unit gain: mean square 12.5
    out = oracle.rmsnorm(np.array([3.0, 4.0]), np.ones(2), eps=0.0)
    assert np.allclose(out, [3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], atol=1e-15)
    h = np.random.default_rng(0).standard_normal((3, 64))
    o = oracle.rmsnorm(h, np.ones(64), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(o * o, axis=-1)), 1.0)
    assert np.allclose(oracle.rmsnorm(7.0 * h, np.ones(64), eps=0.0), o)


def test_rope_closed_forms():
    g = np.random.default_rng(2)
    x = g.standard_normal((5, 8))
    assert np.allclose(oracle.rope(x, np.zeros(5)), x, atol=0)
    # complex form: z_i = x_i + j x_{i+d/2} multiplied by exp(j p theta^(-2i/d))
    d, p = 8, np.arange(5) * 3.0
    z = x[:, :4] + 1j * x[:, 4:]
    w = z * np.exp(1j * np.multiply.outer(p, 10000.0 ** (-np.arange(0, d, 2) / d)))
    out = oracle.rope(x, p)
    assert np.allclose(out[:, :4], w.real, atol=1e-13)
    assert np.allclose(out[:, 4:], w.imag, atol=1e-13)
    # dot products depend only on the position difference
    a, b = g.standard_normal(8), g.standard_normal(8)
    d1 = oracle.rope(a[None], [10])[0] @ oracle.rope(b[None], [3])[0]
    d2 = oracle.rope(a[None], [107])[0] @ oracle.rope(b[None], [100])[0]
    assert abs(d1 - d2) < 1e-12
    assert np.allclose(oracle.rope(oracle.rope(x, p), p + 1), oracle.rope(x, 2 * p + 1))


def test_attention_special_cases():
    g = np.random.default_rng(4)
    H, hd = 4, 8
    q = g.standard_normal((H, hd))
    V1 = g.standard_normal((1, H, hd))
    K1 = g.standard_normal((1, H, hd))
    assert np.allclose(oracle.attention_one(q, K1, V1), V1[0])          # one row
    Kc = np.repeat(g.standard_normal((1, H, hd)), 6, axis=0)
    Vs = g.standard_normal((6, H, hd))
    assert np.allclose(oracle.attention_one(q, Kc, Vs), Vs.mean(axis=0))  # equal keys
    # a dominant score selects its value
    K = np.zeros((3, H, hd)); K[1] = 1000.0 * q / np.linalg.norm(q, axis=1, keepdims=True)
    assert np.allclose(oracle.attention_one(q, K, Vs[:3]), Vs[1], atol=1e-12)
    # grouped kv heads: Hkv = 1 means every query head reads the same kv head
    Kg, Vg = g.standard_normal((5, 1, hd)), g.standard_normal((5, 1, hd))
    o = oracle.attention_one(q, Kg, Vg)
    for h in range(H):
        s = Kg[:, 0] @ q[h] / np.sqrt(hd)
        p = np.exp(s - s.max()); p /= p.sum()
        assert np.allclose(o[h], p @ Vg[:, 0])


def test_silu_values():
    assert oracle.silu(0.0) == 0.0
    assert np.isclose(oracle.silu(1.0), 1.0 / (1.0 + np.exp(-1.0)))
    assert np.isclose(oracle.silu(-40.0), -40.0 * np.exp(-40.0), rtol=1e-10)


def _tiny_layer_weights(seed, d, dff, Hkv, hd, full_rank):
    dims = {"q": (d, d), "k": (d, Hkv * hd), "v": (d, Hkv * hd), "o": (d, d),
            "gate": (d, dff), "up": (d, dff), "down": (dff, d)}
    U, V, Wd = {}, {}, {}
    for i, role in enumerate(oracle.decoder.LINEARS):
        W = synth.dense_weight(seed + i, *dims[role])
        r = min(dims[role]) if full_rank else max(1, min(dims[role]) // 3)
        U[role], V[role], _ = oracle.truncated_factors(W, r)
        Wd[role] = W
    g = np.random.default_rng(seed)
    return {"U": U, "V": V, "g1": 1 + 0.1 * g.standard_normal(d),
            "g2": 1 + 0.1 * g.standard_normal(d)}, Wd


def test_relu_values():
    assert np.array_equal(oracle.relu([-3.0, -0.0, 0.0, 2.5]), [0.0, 0.0, 0.0, 2.5])
    z = np.linspace(-4, 4, 81)
    # relu(z) - relu(-z) = z and relu(z) + relu(-z) = |z|
    assert np.array_equal(oracle.relu(z) - oracle.relu(-z), z)
    assert np.array_equal(oracle.relu(z) + oracle.relu(-z), np.abs(z))


def _dense_layer(h, Wd, w, lat_x, L, cfg):
    """Textbook dense decoder layer from the token-level normed inputs of all
    L+1 positions (lat_x: rows that produced the cache): K = RoPE(x W_k)."""
    H, Hkv, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    x = oracle.rmsnorm(h, w["g1"])
    q = oracle.rope((x @ Wd["q"]).reshape(H, hd), np.full(H, L))
    X = np.vstack([lat_x, x[None]])
    K = (X @ Wd["k"]).reshape(L + 1, Hkv, hd)
    K = np.stack([oracle.rope(K[:, j], np.arange(L + 1)) for j in range(Hkv)], axis=1)
    Vv = (X @ Wd["v"]).reshape(L + 1, Hkv, hd)
    o = oracle.attention_one(q, K, Vv).reshape(-1)
    h = h + o @ Wd["o"]
    x2 = oracle.rmsnorm(h, w["g2"])
    if cfg.get("mlp") == "relu":       # OPT-style: fc2(max(fc1 x, 0))
        return h + np.maximum(x2 @ Wd["gate"], 0.0) @ Wd["down"]
    return h + (oracle.silu(x2 @ Wd["gate"]) * (x2 @ Wd["up"])) @ Wd["down"]


@pytest.mark.parametrize("Hkv,mlp", [(4, "swiglu"), (2, "swiglu"), (1, "swiglu"), (2, "relu")])
def test_decode_layer_full_rank_equals_dense(Hkv, mlp):
    d, dff, H, hd, L = 32, 48, 4, 8, 6
    cfg = {"n_heads": H, "n_kv_heads": Hkv, "head_dim": hd, "mlp": mlp}
    w, Wd = _tiny_layer_weights(100 * Hkv, d, dff, Hkv, hd, full_rank=True)
    g = np.random.default_rng(9)
    prev_x = g.standard_normal((L, d))          # normed inputs of earlier tokens
    lat_k, lat_v = prev_x @ w["U"]["k"], prev_x @ w["U"]["v"]
    h = g.standard_normal(d)
    out, lk, lv = oracle.decode_layer_seq(h, w, lat_k, lat_v, L, cfg)
    ref = _dense_layer(h, Wd, w, prev_x, L, cfg)
    assert _rel(out, ref) <= 1e-11
    assert np.allclose(lk, oracle.rmsnorm(h, w["g1"]) @ w["U"]["k"])


def test_decode_layer_placement_invariance_and_L0():
    d, dff, H, hd = 32, 48, 4, 8
    cfg = {"n_heads": H, "n_kv_heads": H, "head_dim": hd}
    w, _ = _tiny_layer_weights(5, d, dff, H, hd, full_rank=False)
    rk = w["U"]["k"].shape[1]
    g = np.random.default_rng(1)
    lengths = [5, 0, 9]
    B, block = 3, 4
    h = g.standard_normal((B, d))
    logical_k = [g.standard_normal((L, rk)) for L in lengths]
    logical_v = [g.standard_normal((L, rk)) for L in lengths]
    outs = []
    for seed in (0, 1):
        tables, nb = synth.block_tables(seed, np.array(lengths), block=block)
        pk = np.full((nb * block, rk), np.nan)
        pv = np.full((nb * block, rk), np.nan)
        for i, L in enumerate(lengths):
            for p in range(L):
                phys = oracle.logical_to_physical(tables[i], p, block)
                pk[phys], pv[phys] = logical_k[i][p], logical_v[i][p]
        outs.append(oracle.decode_layer(h, w, pk, pv, tables, lengths, block, cfg)[0])
    assert np.array_equal(outs[0], outs[1])
    assert np.all(np.isfinite(outs[0]))
    # L = 0: attention over the new row only, so o equals the new token's values
    x = oracle.rmsnorm(h[1], w["g1"])
    v_new = (x @ w["U"]["v"]) @ w["V"]["v"]
    h_attn = h[1] + (v_new @ w["U"]["o"]) @ w["V"]["o"]
    x2 = oracle.rmsnorm(h_attn, w["g2"])
    mlp = ((oracle.silu((x2 @ w["U"]["gate"]) @ w["V"]["gate"]) *
            ((x2 @ w["U"]["up"]) @ w["V"]["up"])) @ w["U"]["down"]) @ w["V"]["down"]
    assert _rel(outs[0][1], h_attn + mlp) <= 1e-12


@pytest.mark.parametrize("mlp,Hkv", [("swiglu", 4), ("relu", 2)])
def test_prefill_layer_equals_token_by_token_decode(mlp, Hkv):
    # a causal chunk is the same as decoding its tokens one after another,
    # each appending its latents before the next one runs
    d, dff, H, hd, L, c = 32, 48, 4, 8, 5, 4
    cfg = {"n_heads": H, "n_kv_heads": Hkv, "head_dim": hd, "mlp": mlp}
    w, _ = _tiny_layer_weights(300 + Hkv, d, dff, Hkv, hd, full_rank=False)
    g = np.random.default_rng(12)
    rk, rv = w["U"]["k"].shape[1], w["U"]["v"].shape[1]
    lat_k, lat_v = g.standard_normal((L, rk)), g.standard_normal((L, rv))
    Hin = g.standard_normal((c, d))
    out, lk, lv = oracle.prefill_layer_seq(Hin, w, lat_k, lat_v, L, cfg)
    ck, cv = lat_k, lat_v
    for j in range(c):
        o, k1, v1 = oracle.decode_layer_seq(Hin[j], w, ck, cv, L + j, cfg)
        assert _rel(out[j], o) <= 1e-12
        assert np.allclose(lk[j], k1) and np.allclose(lv[j], v1)
        ck, cv = np.vstack([ck, k1[None]]), np.vstack([cv, v1[None]])
    # L = 0, c = 1: attention over the token itself, as in the decode pin
    o1, _, _ = oracle.prefill_layer_seq(Hin[:1], w, lat_k[:0], lat_v[:0], 0, cfg)
    o2, _, _ = oracle.decode_layer_seq(Hin[0], w, lat_k[:0], lat_v[:0], 0, cfg)
    assert _rel(o1[0], o2) <= 1e-12


# ------------------------------------------------- multi-layer compositions
# decode_step, prefill_layer and prefill_step compose the single-layer
# functions pinned above over layers (the residual stream threaded from one
# layer to the next, each layer reading its own latent pools) and over
# sequences (each sequence's rows at its own offset).  Their pins: at full
# rank a stack of layers equals a dense textbook decoder run sequence by
# sequence, and a prefill step whose chunks are single tokens equals a
# decode step.  Every layer has distinct weights and distinct pools, and the
# pools' unused rows hold NaN, so a slip in the threading of h, the layer
# order, the pool of a layer or a sequence's row offset fails these tests
# (the last test below shows it does).

def _phys(table, p, block):
    return int(table[p // block]) * block + p % block


def _scatter_pool(rows_per_seq, tables, nblocks, block, width):
    """Pool [nblocks * block, width] holding each sequence's logical rows at
    their physical rows (NaN elsewhere)."""
    pool = np.full((nblocks * block, width), np.nan)
    for i, rows in enumerate(rows_per_seq):
        for p in range(rows.shape[0]):
            pool[_phys(tables[i], p, block)] = rows[p]
    return pool


def _decoder_case(seed, n_layers, lengths, cfg, full_rank, d=32, dff=48, block=4,
                  extra_rows=None):
    """Layers (factors + dense weights), per-layer normed inputs of the cached
    tokens, paged pools of their latents and the block tables.  extra_rows[i]
    rows beyond the cached ones are placed too (chunked prefill)."""
    H, Hkv, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    lengths = np.asarray(lengths)
    covered = lengths if extra_rows is None else lengths + np.asarray(extra_rows) - 1
    tables, nblocks = synth.block_tables(seed, np.maximum(covered, 0), block=block,
                                         slack_blocks=2)
    g = np.random.default_rng(seed)
    layers, dense, prev_x, pools_k, pools_v = [], [], [], [], []
    for li in range(n_layers):
        w, Wd = _tiny_layer_weights(seed + 31 * li + 1, d, dff, Hkv, hd, full_rank)
        px = [g.standard_normal((int(L), d)) for L in lengths]
        layers.append(w)
        dense.append(Wd)
        prev_x.append(px)
        rk, rv = w["U"]["k"].shape[1], w["U"]["v"].shape[1]
        pools_k.append(_scatter_pool([x @ w["U"]["k"] for x in px], tables, nblocks, block, rk))
        pools_v.append(_scatter_pool([x @ w["U"]["v"] for x in px], tables, nblocks, block, rv))
    return layers, dense, prev_x, pools_k, pools_v, tables


def _dense_decoder_token(h, dense, layers, prev_x_seq, L, cfg):
    """One new token through every layer of a dense textbook decoder."""
    for Wd, w, px in zip(dense, layers, prev_x_seq):
        h = _dense_layer(h, Wd, w, px, L, cfg)
    return h


@pytest.mark.parametrize("Hkv,mlp", [(4, "swiglu"), (2, "swiglu"), (1, "relu")])
def test_decode_step_full_rank_equals_dense_stack(Hkv, mlp):
    cfg = {"n_heads": 4, "n_kv_heads": Hkv, "head_dim": 8, "mlp": mlp}
    lengths = [6, 0, 11, 3]
    layers, dense, prev_x, pk, pv, tables = _decoder_case(700 + Hkv, 3, lengths, cfg, True)
    h0 = np.random.default_rng(70).standard_normal((len(lengths), 32))
    got = oracle.decode_step(h0, layers, pk, pv, tables, lengths, 4, cfg)
    for i, L in enumerate(lengths):
        ref = _dense_decoder_token(h0[i], dense, layers, [px[i] for px in prev_x], L, cfg)
        assert _rel(got[i], ref) <= 1e-11, i
    # a subset of sequences, in any order, gives those sequences' rows
    sub = oracle.decode_step(h0, layers, pk, pv, tables, lengths, 4, cfg, seqs=[2, 0])
    assert np.array_equal(sub, got[[2, 0]])


@pytest.mark.parametrize("Hkv,mlp", [(4, "swiglu"), (2, "relu")])
def test_prefill_step_full_rank_equals_dense_causal_stack(Hkv, mlp):
    # several sequences with different cached lengths and chunk lengths; in
    # the dense decoder, chunk token j of a sequence is one more decoded
    # token whose cache holds the cached rows and chunk tokens 0 .. j-1 of
    # the same layer
    cfg = {"n_heads": 4, "n_kv_heads": Hkv, "head_dim": 8, "mlp": mlp}
    lengths, chunks = [5, 0, 2], [3, 1, 4]
    layers, dense, prev_x, pk, pv, tables = _decoder_case(800 + Hkv, 3, lengths, cfg, True,
                                                          extra_rows=chunks)
    n = sum(chunks)
    h0 = np.random.default_rng(80).standard_normal((n, 32))
    got = oracle.prefill_step(h0, layers, pk, pv, tables, lengths, chunks, 4, cfg)
    t = 0
    for i, (L, c) in enumerate(zip(lengths, chunks)):
        Hc = h0[t:t + c].copy()
        for Wd, w, px in zip(dense, layers, prev_x):
            X = np.stack([oracle.rmsnorm(Hc[j], w["g1"]) for j in range(c)])
            Hc = np.stack([_dense_layer(Hc[j], Wd, w, np.vstack([px[i], X[:j]]), L + j, cfg)
                           for j in range(c)])
        assert _rel(got[t:t + c], Hc) <= 1e-11, i
        t += c
    # prefill_layer returns the new latents of each token: x U_k / x U_v of
    # its normed input, sequence by sequence
    _, nk, nv = oracle.prefill_layer(h0, layers[0], pk[0], pv[0], tables, lengths, chunks, 4, cfg)
    X0 = oracle.rmsnorm(h0, layers[0]["g1"])
    assert _rel(nk, X0 @ layers[0]["U"]["k"]) <= 1e-13
    assert _rel(nv, X0 @ layers[0]["U"]["v"]) <= 1e-13


@pytest.mark.parametrize("mlp", ["swiglu", "relu"])
def test_prefill_step_single_token_chunks_equal_decode_step(mlp):
    # low rank, 3 layers: with one new token per sequence a prefill step is a
    # decode step (two independently written paths)
    cfg = {"n_heads": 4, "n_kv_heads": 2, "head_dim": 8, "mlp": mlp}
    lengths = [9, 1, 0, 14, 4]
    layers, _, _, pk, pv, tables = _decoder_case(900, 3, lengths, cfg, False)
    h0 = np.random.default_rng(90).standard_normal((len(lengths), 32))
    a = oracle.prefill_step(h0, layers, pk, pv, tables, lengths, [1] * len(lengths), 4, cfg)
    b = oracle.decode_step(h0, layers, pk, pv, tables, lengths, 4, cfg)
    assert _rel(a, b) <= 1e-12
    assert np.all(np.isfinite(a))


def test_composition_pins_catch_planted_slips():
    # the comparisons above fail for plausible slips in the compositions,
    # planted here in local copies (the oracle itself is untouched)
    cfg = {"n_heads": 4, "n_kv_heads": 2, "head_dim": 8}
    lengths = [6, 2, 9]
    layers, dense, prev_x, pk, pv, tables = _decoder_case(950, 3, lengths, cfg, True)
    h0 = np.random.default_rng(95).standard_normal((len(lengths), 32))
    ref = np.stack([_dense_decoder_token(h0[i], dense, layers, [px[i] for px in prev_x], L, cfg)
                    for i, L in enumerate(lengths)])
    assert _rel(oracle.decode_step(h0, layers, pk, pv, tables, lengths, 4, cfg), ref) <= 1e-11

    def unthreaded():
        for li, w in enumerate(layers):
            out, _, _ = oracle.decode_layer(h0, w, pk[li], pv[li], tables, lengths, 4, cfg)
        return out

    def reversed_layers():
        h = h0
        for li in reversed(range(len(layers))):
            h, _, _ = oracle.decode_layer(h, layers[li], pk[li], pv[li], tables, lengths, 4, cfg)
        return h

    def rotated_pools():
        h = h0
        for li, w in enumerate(layers):
            lj = (li + 1) % len(layers)
            h, _, _ = oracle.decode_layer(h, w, pk[lj], pv[lj], tables, lengths, 4, cfg)
        return h

    for slip in (unthreaded, reversed_layers, rotated_pools):
        assert not _rel(slip(), ref) <= 1e-3, slip.__name__

    # prefill: every sequence reading the first rows (offset never advanced)
    chunks = [2, 3, 1]
    layers2, _, _, pk2, pv2, tables2 = _decoder_case(960, 2, lengths, cfg, False,
                                                     extra_rows=chunks)
    hp = np.random.default_rng(96).standard_normal((sum(chunks), 32))
    good = oracle.prefill_step(hp, layers2, pk2, pv2, tables2, lengths, chunks, 4, cfg)
    per_seq = []
    t = 0
    for i, (L, c) in enumerate(zip(lengths, chunks)):
        one = oracle.prefill_step(hp[t:t + c], layers2, pk2, pv2, [tables2[i]], [L], [c], 4, cfg)
        per_seq.append(one)
        t += c
    assert _rel(good, np.vstack(per_seq)) <= 1e-13
    slipped = np.vstack([oracle.prefill_step(hp[:c], layers2, pk2, pv2, [tables2[i]], [L], [c], 4,
                                             cfg)
                         for i, (L, c) in enumerate(zip(lengths, chunks))])
    assert not _rel(slipped, good) <= 1e-3
