"""Seeded decode-step inputs for the GPU tests: numpy values (oracle side)
and device tensors (GPU side) built from the same synth arrays."""
import numpy as np
import torch

import oracle
import rank_decomposed_amd as lr
import synth
from gpu_util import dev, to_dev

DIMS = lambda c: {"q": (c["d_model"], c["n_heads"] * c["head_dim"]),
                  "k": (c["d_model"], c["n_kv_heads"] * c["head_dim"]),
                  "v": (c["d_model"], c["n_kv_heads"] * c["head_dim"]),
                  "o": (c["n_heads"] * c["head_dim"], c["d_model"]),
                  "gate": (c["d_model"], c["d_ffn"]), "up": (c["d_model"], c["d_ffn"]),
                  "down": (c["d_ffn"], c["d_model"])}


def ld8(n, extra=0):
    return (n + 7) // 8 * 8 + extra


def make_layer(cfg_id, layer, cfg, ranks, fast=False):
    """Factors (bf16) and norms of one layer: numpy values + device tensors."""
    vals = {"U": {}, "V": {}}
    Ut, Vt = {}, {}
    for i, name in enumerate(lr.LINEARS):
        d_in, d_out = DIMS(cfg)[name]
        r = ranks[name]
        seed = synth.seed_of(cfg_id, layer, i, synth.KIND_W)
        if fast:
            U, V = synth.fast_factors(seed, d_in, d_out, r)
        else:
            U, V = synth.svd_factors(synth.dense_weight(seed, d_in, d_out), r)
        ub, vb = synth.bf16_bits(U.T), synth.bf16_bits(V.T)
        vals["U"][name] = synth.bf16_value(ub).T
        vals["V"][name] = synth.bf16_value(vb).T
        Ut[name] = pad_dev(ub, ld8(d_in))
        Vt[name] = pad_dev(vb, ld8(r))
    g = synth.rng(synth.seed_of(cfg_id, layer, 0, synth.KIND_NORM))
    g1 = synth.bf16_bits(1.0 + 0.1 * g.standard_normal(cfg["d_model"]))
    g2 = synth.bf16_bits(1.0 + 0.1 * g.standard_normal(cfg["d_model"]))
    vals["g1"], vals["g2"] = synth.bf16_value(g1), synth.bf16_value(g2)
    return vals, Ut, Vt, to_dev(g1, "bf16"), to_dev(g2, "bf16")


def pad_dev(bits, ld):
    rows, cols = bits.shape
    full = np.zeros((rows, ld), np.uint16)
    full[:, :cols] = bits
    return to_dev(full, "bf16")[:, :cols]


class Step:
    """B sequences with given cached lengths, n_layers layers, paged latent
    pools with seeded placement.  ranks: one {name: r} for every layer, or a
    list with one per layer (per-layer ratios).  fused: run
    lowrank_layer_decode_step_fused (reconstruction inside the attention)."""

    def __init__(self, cfg_id, cfg, ranks, lengths, n_layers, block=16, fast=False,
                 max_seq_rows=None, cap=None, slack_blocks=3, fused=False):
        self.cfg, self.block, self.fused = cfg, block, fused
        self.lengths = np.asarray(lengths, dtype=np.int64)
        B = len(lengths)
        self.tables, nblocks = synth.block_tables(synth.seed_of(cfg_id, 0, 0, synth.KIND_PLACE),
                                                  self.lengths, block, slack_blocks=slack_blocks)
        self.pool_rows = nblocks * block
        self.max_seq_rows = max_seq_rows or int(self.lengths.max() + 1)
        self.cap = cap or int(B * ((self.max_seq_rows + 15) // 16 * 16))
        per_layer = ranks if isinstance(ranks, (list, tuple)) else [ranks] * n_layers
        self.pool_ld = ld8(max(max(rk["k"], rk["v"]) for rk in per_layer), 8)
        d = dev()
        self.layers, self.weights, self.pools_np_k, self.pools_np_v = [], [], [], []
        self.pools_k, self.pools_v = [], []
        self.rope = torch.empty((self.max_seq_rows, cfg["head_dim"] // 2, 2), dtype=torch.float32,
                                device=d)
        lr.lowrank_rope_table(cfg["head_dim"], self.max_seq_rows, 10000.0, self.rope)
        for li in range(n_layers):
            vals, Ut, Vt, g1, g2 = make_layer(cfg_id, li, cfg, per_layer[li], fast)
            self.layers.append(vals)
            self.weights.append(lr.layer_weights(cfg, Ut, Vt, g1, g2, self.rope,
                                                 self.max_seq_rows))
            for kind, store_np, store in ((0, self.pools_np_k, self.pools_k),
                                          (1, self.pools_np_v, self.pools_v)):
                g = synth.rng(synth.seed_of(cfg_id, li, kind, synth.KIND_LAT))
                bits = synth.bf16_bits(g.standard_normal((self.pool_rows, self.pool_ld)))
                store_np.append(synth.bf16_value(bits))
                store.append(to_dev(bits, "bf16"))
        h0 = synth.tokens(synth.seed_of(cfg_id, 0, 0, synth.KIND_X), B, cfg["d_model"])
        self.h0 = h0.astype(np.float32).astype(np.float64)
        self.h = torch.from_numpy(self.h0.astype(np.float32)).to(d)
        # preparation stage (host, product) -> fixed device buffers
        prep = lr.lowrank_prepare_decode(self.lengths, self.tables, block, self.cap)
        self.prep = prep
        self.dev_prep = {k: torch.from_numpy(np.ascontiguousarray(prep[k])).to(d)
                         for k in ("remap", "seq_off", "pos", "slot_mapping")}
        self.n_valid = torch.tensor([prep["n_valid"]], dtype=torch.int32, device=d)
        self.states = [lr.decode_state(self.pools_k[li], self.pools_v[li],
                                       self.dev_prep["slot_mapping"], self.dev_prep["remap"],
                                       self.dev_prep["seq_off"], self.dev_prep["pos"],
                                       self.n_valid, self.max_seq_rows)
                       for li in range(n_layers)]
        size = (lr.lowrank_decode_step_fused_workspace_bytes if fused
                else lr.lowrank_decode_step_workspace_bytes)
        nbytes = max(size(w, s) for w, s in zip(self.weights, self.states))
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=d)

    def run(self):
        step = lr.lowrank_layer_decode_step_fused if self.fused else lr.lowrank_layer_decode_step
        for w, s in zip(self.weights, self.states):
            step(w, s, self.h, self.ws)
        return self.h

    def oracle(self, seqs=None):
        return oracle.decode_step(self.h0, self.layers, self.pools_np_k, self.pools_np_v,
                                  self.tables, self.lengths, self.block, self.cfg, seqs)


class Prefill:
    """One chunked-prefill step: S sequences with cached lengths append
    chunks[i] prompt tokens each; n_layers layers; paged latent pools with
    seeded placement (the pools hold the cached rows' latents)."""

    def __init__(self, cfg_id, cfg, ranks, lengths, chunks, n_layers, block=16, fast=False):
        self.cfg, self.block = cfg, block
        self.lengths = np.asarray(lengths, dtype=np.int64)
        self.chunks = np.asarray(chunks, dtype=np.int64)
        rows = self.lengths + self.chunks
        # block_tables covers its lengths + 1 rows
        self.tables, nblocks = synth.block_tables(synth.seed_of(cfg_id, 0, 1, synth.KIND_PLACE),
                                                  rows - 1, block, slack_blocks=3)
        self.pool_rows = nblocks * block
        self.max_seq_rows = int(rows.max())
        self.cap = int(rows.sum() + 37)
        self.pool_ld = ld8(max(ranks["k"], ranks["v"]), 8)
        d = dev()
        self.rope = torch.empty((self.max_seq_rows, cfg["head_dim"] // 2, 2), dtype=torch.float32,
                                device=d)
        lr.lowrank_rope_table(cfg["head_dim"], self.max_seq_rows, 10000.0, self.rope)
        self.layers, self.weights = [], []
        self.pools_np_k, self.pools_np_v, self.pools_k, self.pools_v = [], [], [], []
        for li in range(n_layers):
            vals, Ut, Vt, g1, g2 = make_layer(cfg_id, li, cfg, ranks, fast)
            self.layers.append(vals)
            self.weights.append(lr.layer_weights(cfg, Ut, Vt, g1, g2, self.rope,
                                                 self.max_seq_rows))
            for kind, store_np, store in ((0, self.pools_np_k, self.pools_k),
                                          (1, self.pools_np_v, self.pools_v)):
                g = synth.rng(synth.seed_of(cfg_id, li, kind, synth.KIND_LAT))
                bits = synth.bf16_bits(g.standard_normal((self.pool_rows, self.pool_ld)))
                store_np.append(synth.bf16_value(bits))
                store.append(to_dev(bits, "bf16"))
        T = int(self.chunks.sum())
        h0 = synth.tokens(synth.seed_of(cfg_id, 0, 1, synth.KIND_X), T, cfg["d_model"])
        self.h0 = h0.astype(np.float32).astype(np.float64)
        self.h = torch.from_numpy(self.h0.astype(np.float32)).to(d)
        prep = lr.lowrank_prepare_prefill(self.lengths, self.chunks, self.tables, block, self.cap)
        self.prep = prep
        dp = {k: torch.from_numpy(np.ascontiguousarray(prep[k])).to(d)
              for k in ("remap", "seq_off", "tok_seq", "pos", "slot_mapping")}
        self.n_valid = torch.tensor([prep["n_valid"]], dtype=torch.int32, device=d)
        self.states = [lr.prefill_state(self.pools_k[li], self.pools_v[li], dp["slot_mapping"],
                                        dp["remap"], dp["seq_off"], dp["tok_seq"], dp["pos"],
                                        self.n_valid, self.max_seq_rows)
                       for li in range(n_layers)]
        self._dp = dp
        nbytes = max(lr.lowrank_prefill_step_workspace_bytes(w, s)
                     for w, s in zip(self.weights, self.states))
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=d)

    def run(self):
        for w, s in zip(self.weights, self.states):
            lr.lowrank_layer_prefill_step(w, s, self.h, self.ws)
        return self.h

    def oracle(self):
        return oracle.prefill_step(self.h0, self.layers, self.pools_np_k, self.pools_np_v,
                                   self.tables, self.lengths, self.chunks, self.block, self.cfg)
