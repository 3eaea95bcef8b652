"""Oracle: one decode step of a decoder whose every linear is decomposed, with
a paged cache of rank-r latents reconstructed each step (test infrastructure
only).

The pages: decomposed models must rebuild the KV cache while decoding, by
multiplying the cached low-rank rows by the upward projection matrices
(DeInfer/en §1 third bottleneck and §2.C "Graph Replay Stage"; DeInfer/es §1
"Incompatibilidad con CUDA Graph").  The layer around it is LLaMA-shaped:
MHA/GQA/MQA attention and a GLU or non-GLU MLP (DeInfer/en §2.D; DeInfer/es
§2 "Generalización").

Readings where the pages are silent (each is listed with its reason in the
design notes): the cache holds the pre-rotary latents x U_k and x U_v; rotary
is applied to the reconstructed keys (it cannot be folded into V_k); RMSNorm
eps = 1e-5; rotate-half rotary with base 10000; softmax scale 1/sqrt(head_dim);
the new token sits at position L (its cached length) and attends to all L + 1
rows; the GLU MLP is SwiGLU, the non-GLU one (OPT-style) is fc2(relu(fc1 x))
with fc1 and fc2 in the "gate" and "down" slots; fp64 throughout.
"""
from __future__ import annotations

import numpy as np

from .paging import logical_to_physical

LINEARS = ("q", "k", "v", "o", "gate", "up", "down")


def rmsnorm(h: np.ndarray, g: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) * g over the last axis."""
    h = np.asarray(h, np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * np.asarray(g, np.float64)


def rope(x: np.ndarray, pos, theta: float = 10000.0) -> np.ndarray:
    """Rotate-half rotary embedding on the last axis (head_dim d): for
    i < d/2, the pair (x_i, x_{i+d/2}) is rotated by the angle
    pos * theta^(-2i/d).  x has shape [..., n, d] with pos of shape [n]
    (or a scalar)."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-(2.0 * np.arange(half)) / d)
    ang = np.multiply.outer(np.asarray(pos, np.float64), inv)   # [n, half]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attention_one(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Single-query softmax attention per head.
    q[H, hd], K[n, Hkv, hd], V[n, Hkv, hd] -> o[H, hd]; query head h reads kv
    head h // (H / Hkv).  Scores are scaled by 1/sqrt(hd) and the row max is
    subtracted before exponentiation."""
    H, hd = q.shape
    Hkv = K.shape[1]
    grp = H // Hkv
    o = np.empty((H, hd))
    for h in range(H):
        kv = h // grp
        s = K[:, kv, :] @ q[h] / np.sqrt(hd)
        p = np.exp(s - s.max())
        p /= p.sum()
        o[h] = p @ V[:, kv, :]
    return o


def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def relu(z):
    z = np.asarray(z, np.float64)
    return np.maximum(z, 0.0)


def _lin(x, w, role):
    return (x @ w["U"][role]) @ w["V"][role]


def decode_layer_seq(h, w, lat_k, lat_v, L: int, cfg):
    """One decoder layer for one sequence's new token.

    h[d] residual stream; w: {'U': {role: U_r}, 'V': {role: V_r}, 'g1', 'g2'};
    lat_k[L, r_k], lat_v[L, r_v]: the cached latents in logical order; cfg:
    n_heads, n_kv_heads, head_dim, eps, rope_theta, mlp ("swiglu" by default,
    or "relu": fc1 in the "gate" slot, fc2 in "down", no "up").
    Returns (h_out[d], new_k_latent[r_k], new_v_latent[r_v])."""
    H, Hkv, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    eps, theta = cfg.get("eps", 1e-5), cfg.get("rope_theta", 10000.0)
    h = np.asarray(h, np.float64)
    x = rmsnorm(h, w["g1"], eps)
    q = _lin(x, w, "q").reshape(H, hd)
    q = rope(q, np.full(H, L), theta)          # every head at position L
    lk = x @ w["U"]["k"]
    lv = x @ w["U"]["v"]
    LK = np.vstack([np.asarray(lat_k, np.float64).reshape(L, lk.shape[0]), lk[None]])
    LV = np.vstack([np.asarray(lat_v, np.float64).reshape(L, lv.shape[0]), lv[None]])
    K = (LK @ w["V"]["k"]).reshape(L + 1, Hkv, hd)
    K = np.stack([rope(K[:, j, :], np.arange(L + 1), theta) for j in range(Hkv)], axis=1)
    V = (LV @ w["V"]["v"]).reshape(L + 1, Hkv, hd)
    o = attention_one(q, K, V).reshape(H * hd)
    h = h + _lin(o, w, "o")
    x2 = rmsnorm(h, w["g2"], eps)
    if cfg.get("mlp", "swiglu") == "relu":
        m = relu(_lin(x2, w, "gate"))
    else:
        m = silu(_lin(x2, w, "gate")) * _lin(x2, w, "up")
    h = h + _lin(m, w, "down")
    return h, lk, lv


def _logical_rows(pool, table, n: int, block: int):
    return np.stack([np.asarray(pool[logical_to_physical(table, p, block)], np.float64)
                     for p in range(n)]) if n else np.zeros((0, pool.shape[1]))


def decode_layer(h, w, pool_k, pool_v, tables, lengths, block: int, cfg, seqs=None):
    """One layer for the selected sequences (all by default).  pool_k/pool_v
    hold the cached latents (fp64 values, physical rows, possibly wider than
    r: only the first r_k / r_v columns are read).  Returns
    (h_out[len(seqs), d], new_k[len(seqs), r_k], new_v[len(seqs), r_v])."""
    seqs = range(len(lengths)) if seqs is None else seqs
    rk = w["U"]["k"].shape[1]
    rv = w["U"]["v"].shape[1]
    hs, nk, nv = [], [], []
    for i in seqs:
        L = int(lengths[i])
        lat_k = _logical_rows(pool_k, tables[i], L, block)[:, :rk]
        lat_v = _logical_rows(pool_v, tables[i], L, block)[:, :rv]
        ho, lk, lv = decode_layer_seq(h[i], w, lat_k, lat_v, L, cfg)
        hs.append(ho); nk.append(lk); nv.append(lv)
    return np.array(hs), np.array(nk), np.array(nv)


def decode_step(h, layers, pools_k, pools_v, tables, lengths, block: int, cfg, seqs=None):
    """All layers in order for the selected sequences: h[B, d] -> h[len(seqs), d].
    Each layer reads its own latent pools."""
    seqs = list(range(len(lengths))) if seqs is None else list(seqs)
    hcur = np.asarray(h, np.float64)[seqs]
    sub_len = [lengths[i] for i in seqs]
    sub_tab = [tables[i] for i in seqs]
    for li, w in enumerate(layers):
        hcur, _, _ = decode_layer(hcur, w, pools_k[li], pools_v[li], sub_tab, sub_len,
                                  block, cfg)
    return hcur


def prefill_layer_seq(H, w, lat_k, lat_v, L: int, cfg):
    """One decoder layer for a chunk of c new tokens of one sequence (the
    chunked-prefill step): H[c, d] residual rows of the tokens at positions
    L .. L + c - 1; lat_k[L, r_k], lat_v[L, r_v] the cached latents.  Token j
    attends causally to rows 0 .. L + j: the cached rows and the chunk's
    tokens up to itself.  Returns (H_out[c, d], new_k[c, r_k], new_v[c, r_v]).
    """
    Hn, Hkv, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    eps, theta = cfg.get("eps", 1e-5), cfg.get("rope_theta", 10000.0)
    H = np.asarray(H, np.float64)
    c = H.shape[0]
    X = np.stack([rmsnorm(H[j], w["g1"], eps) for j in range(c)])
    Q = (X @ w["U"]["q"]) @ w["V"]["q"]                      # [c, Hn * hd]
    lk = X @ w["U"]["k"]
    lv = X @ w["U"]["v"]
    LK = np.vstack([np.asarray(lat_k, np.float64).reshape(L, lk.shape[1]), lk])
    LV = np.vstack([np.asarray(lat_v, np.float64).reshape(L, lv.shape[1]), lv])
    K = (LK @ w["V"]["k"]).reshape(L + c, Hkv, hd)
    K = np.stack([rope(K[:, i, :], np.arange(L + c), theta) for i in range(Hkv)], axis=1)
    V = (LV @ w["V"]["v"]).reshape(L + c, Hkv, hd)
    out = np.empty_like(H)
    for j in range(c):
        q = rope(Q[j].reshape(Hn, hd), np.full(Hn, L + j), theta)
        o = attention_one(q, K[:L + j + 1], V[:L + j + 1]).reshape(Hn * hd)
        h = H[j] + _lin(o, w, "o")
        x2 = rmsnorm(h, w["g2"], eps)
        if cfg.get("mlp", "swiglu") == "relu":
            m = relu(_lin(x2, w, "gate"))
        else:
            m = silu(_lin(x2, w, "gate")) * _lin(x2, w, "up")
        out[j] = h + _lin(m, w, "down")
    return out, lk, lv


def prefill_layer(h, w, pool_k, pool_v, tables, lengths, chunks, block: int, cfg):
    """One layer of a chunked-prefill step over S sequences: h[n, d] holds the
    new tokens sequence by sequence (chunks[i] of them for sequence i, at
    positions lengths[i] ..).  Pools as in decode_layer.  Returns
    (h_out[n, d], new_k[n, r_k], new_v[n, r_v])."""
    rk = w["U"]["k"].shape[1]
    rv = w["U"]["v"].shape[1]
    hs, nk, nv = [], [], []
    t = 0
    for i in range(len(lengths)):
        L, c = int(lengths[i]), int(chunks[i])
        lat_k = _logical_rows(pool_k, tables[i], L, block)[:, :rk]
        lat_v = _logical_rows(pool_v, tables[i], L, block)[:, :rv]
        ho, lk, lv = prefill_layer_seq(np.asarray(h, np.float64)[t:t + c], w, lat_k, lat_v, L,
                                       cfg)
        hs.append(ho); nk.append(lk); nv.append(lv)
        t += c
    return np.vstack(hs), np.vstack(nk), np.vstack(nv)


def prefill_step(h, layers, pools_k, pools_v, tables, lengths, chunks, block: int, cfg):
    """All layers in order for one chunked-prefill step: h[n, d] -> h[n, d]."""
    hcur = np.asarray(h, np.float64)
    for li, w in enumerate(layers):
        hcur, _, _ = prefill_layer(hcur, w, pools_k[li], pools_v[li], tables, lengths, chunks,
                                   block, cfg)
    return hcur
