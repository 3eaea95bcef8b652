"""Seeded inputs of the 32-layer decode step at LLaMA-7B shape.

64 sequences with cached lengths uniform in [128, 4096], block 16, seeded
placement (see synth.block_tables); every linear decomposed at parameter
ratio 0.2.  Layer 0's factors follow the law of a truncated SVD of an
N(0, 1/d_in) weight (synth.fast_factors); layer l > 0 reuses them under a
seeded signed permutation of the rank components (same law, distinct bytes).
Norm weights 1 + 0.1 N(0,1), residual stream h0 ~ N(0,1), cached latents
~ N(0,1) from the counter-based generator, so a GPU materialises every pool
while the CPU side regenerates only the rows of the sequences it checks.

Only inputs are built here: no step of the method is computed.
"""
from __future__ import annotations

import functools
from fractions import Fraction

import numpy as np

from . import (DECODE_STEP_7B, KIND_LAT, KIND_LEN, KIND_NORM, KIND_PLACE, KIND_W, KIND_X,
               ROLES, bf16_bits, bf16_value, block_tables, decode_lengths, fast_factors,
               hash_bf16_rows_torch, hash_rows, rank_permutation, rng, seed_of, tokens)

CFG_ID = 5


def dims(c):
    dq, dkv = c["n_heads"] * c["head_dim"], c["n_kv_heads"] * c["head_dim"]
    return {"q": (c["d_model"], dq), "k": (c["d_model"], dkv), "v": (c["d_model"], dkv),
            "o": (dq, c["d_model"]), "gate": (c["d_model"], c["d_ffn"]),
            "up": (c["d_model"], c["d_ffn"]), "down": (c["d_ffn"], c["d_model"])}


def ranks(c):
    f = Fraction(str(c["rho"]))
    return {n: int((f * a * b) // (a + b)) for n, (a, b) in dims(c).items()}


def ld8(n):
    return (n + 7) // 8 * 8


@functools.lru_cache(maxsize=4)
def base_factor_bits(cfg_items):
    """bf16 bits of layer 0's Ut = U_r^T and Vt = V_r^T per role."""
    c = dict(cfg_items)
    out = {}
    for i, role in enumerate(ROLES):
        d_in, d_out = dims(c)[role]
        U, V = fast_factors(seed_of(CFG_ID, 0, i, KIND_W), d_in, d_out, ranks(c)[role])
        out[role] = (bf16_bits(U.T), bf16_bits(V.T))
    return out


class DecodeStepInputs:
    def __init__(self, cfg=None, n_layers=None, B=None, device=None):
        self.cfg = dict(cfg or DECODE_STEP_7B)
        if n_layers is not None:
            self.cfg["n_layers"] = n_layers
        if B is not None:
            self.cfg["B"] = B
        c = self.cfg
        self.key = tuple(sorted((k, v) for k, v in c.items() if k != "n_layers" and k != "B"))
        self.ranks = ranks(c)
        self.block = c["block"]
        self.lengths = decode_lengths(seed_of(CFG_ID, 0, 0, KIND_LEN), c["B"], c["len_lo"],
                                      c["len_hi"])
        self.tables, nblocks = block_tables(seed_of(CFG_ID, 0, 0, KIND_PLACE), self.lengths,
                                            self.block, slack_blocks=16)
        self.pool_rows = nblocks * self.block
        self.pool_ld = ld8(max(self.ranks["k"], self.ranks["v"]))
        self.max_seq_rows = (c["len_hi"] + 1 + 15) // 16 * 16
        self.cap = c["B"] * self.max_seq_rows
        self.h0 = tokens(seed_of(CFG_ID, 0, 0, KIND_X), c["B"], c["d_model"]).astype(
            np.float32).astype(np.float64)
        self.device = device

    # ---------------------------------------------------------------- host
    def perm(self, layer, role):
        i = ROLES.index(role)
        return rank_permutation(seed_of(CFG_ID, layer, i, KIND_W) + 7, self.ranks[role])

    def norms(self, layer):
        g = rng(seed_of(CFG_ID, layer, 0, KIND_NORM))
        g1 = bf16_bits(1.0 + 0.1 * g.standard_normal(self.cfg["d_model"]))
        g2 = bf16_bits(1.0 + 0.1 * g.standard_normal(self.cfg["d_model"]))
        return g1, g2

    def layer_values(self, layer):
        """fp64 values of layer `layer` in math orientation (oracle side)."""
        base = base_factor_bits(self.key)
        U, V = {}, {}
        for role in ROLES:
            ub, vb = base[role]
            u, v = bf16_value(ub).T, bf16_value(vb).T     # [d_in, r], [r, d_out]
            if layer > 0:
                p, s = self.perm(layer, role)
                u, v = u[:, p] * s[None, :], v[p, :] * s[:, None]
            U[role], V[role] = u, v
        g1, g2 = self.norms(layer)
        return {"U": U, "V": V, "g1": bf16_value(g1), "g2": bf16_value(g2)}

    def pool_seed(self, layer, kind):
        return seed_of(CFG_ID, layer, kind, KIND_LAT)

    def pool_rows_for(self, layer, kind, seqs):
        """SparsePool holding the physical rows the given sequences read."""
        rows = set()
        for i in seqs:
            t = self.tables[i]
            for p in range(int(self.lengths[i])):
                rows.add(int(t[p // self.block]) * self.block + p % self.block)
        rows = np.array(sorted(rows), dtype=np.int64)
        vals = hash_rows(self.pool_seed(layer, kind), rows, self.pool_ld)
        return SparsePool(dict(zip(rows.tolist(), vals)), self.pool_ld)

    # ---------------------------------------------------------------- device
    def device_layer(self, layer):
        """(Ut dict, Vt dict, g1, g2) as device bf16 tensors (views)."""
        import torch
        dev = self.device
        base = base_factor_bits(self.key)
        Ut, Vt = {}, {}
        for role in ROLES:
            ub, vb = base[role]
            r, d_in = ub.shape
            d_out = vb.shape[0]
            u = _dev_bits(ub, dev)
            v = _dev_bits(vb, dev)
            if layer > 0:
                p, s = self.perm(layer, role)
                pt = torch.from_numpy(p).to(dev)
                st = torch.from_numpy(s).to(dev).to(torch.bfloat16)
                u = u[pt] * st[:, None]
                v = v[:, pt] * st[None, :]
            uf = torch.zeros((r, ld8(d_in)), dtype=torch.bfloat16, device=dev)
            vf = torch.zeros((d_out, ld8(r)), dtype=torch.bfloat16, device=dev)
            uf[:, :d_in] = u
            vf[:, :r] = v
            Ut[role], Vt[role] = uf[:, :d_in], vf[:, :r]
        g1, g2 = self.norms(layer)
        return Ut, Vt, _dev_bits(g1, dev), _dev_bits(g2, dev)

    def device_pool(self, layer, kind):
        return hash_bf16_rows_torch(self.pool_seed(layer, kind), self.pool_rows, self.pool_ld,
                                    self.device)


class SparsePool:
    """Row-indexable stand-in for a pool of which only some rows are known."""

    def __init__(self, rows: dict, ld: int):
        self.rows, self.shape = rows, (max(rows) + 1 if rows else 0, ld)

    def __getitem__(self, r):
        return self.rows[int(r)]


def _dev_bits(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
