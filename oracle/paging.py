"""Oracle: preparation stage and remap gather of the paged latent cache
(test infrastructure only).

The pages split KV-cache reconstruction into two stages so that it fits a
static graph (DeInfer/en §2.C "Integrating Paged KV Cache with CUDA Graphs";
DeInfer/es §2 "Etapa de Preparación" / "Etapa de Reproducción del Gráfico";
DeInfer/zh, the remapping table of the solution section):
  * preparation: scan the paged memory for physically contiguous blocks and
    emit a remapping index list (a new block table);
  * replay: copy those blocks into a compact contiguous buffer at a fixed
    address, then multiply it by the upward projections.

Reading taken where the pages are silent: a sequence with L cached tokens
decodes one new token at position L, so its compact segment holds L + 1 rows
(logical positions 0..L); segments are packed back to back; the remapping
list has one source row per destination row (-1 = no source, a zero row).
"""
from __future__ import annotations

import numpy as np


def logical_to_physical(table, p: int, block: int) -> int:
    """Physical pool row of logical position p under a block table."""
    return int(table[p // block]) * block + p % block


def contiguous_runs(table, n_rows: int, block: int):
    """Maximal runs of physically consecutive blocks covering the first n_rows
    logical rows.  Returns a list of (physical_start_row, logical_start_row,
    n_rows) tuples in logical order."""
    runs = []
    nb = (n_rows + block - 1) // block
    b = 0
    while b < nb:
        e = b + 1
        while e < nb and int(table[e]) == int(table[e - 1]) + 1:
            e += 1
        lo = b * block
        hi = min(e * block, n_rows)
        runs.append((int(table[b]) * block, lo, hi - lo))
        b = e
    return runs


def prepare_decode(tables, lengths, block: int, cap: int):
    """Preparation stage for one decode step over B sequences.

    Returns a dict of int32 arrays: remap[cap], seq_off[B+1], pos[B],
    slot_mapping[B], and the ints n_valid and n_runs, plus 'runs' (a list of
    (physical_start_row, dst_row, n_rows)).  Raises ValueError when the
    packed rows exceed cap."""
    B = len(lengths)
    seq_off = [0] * (B + 1)
    for i in range(B):
        seq_off[i + 1] = seq_off[i] + int(lengths[i]) + 1
    n_valid = seq_off[B]
    if n_valid > cap:
        raise ValueError("packed rows %d exceed capacity %d" % (n_valid, cap))
    remap = [-1] * cap
    runs = []
    pos, slots = [0] * B, [0] * B
    for i in range(B):
        n = int(lengths[i]) + 1
        for (src, lo, cnt) in contiguous_runs(tables[i], n, block):
            runs.append((src, seq_off[i] + lo, cnt))
            for k in range(cnt):
                remap[seq_off[i] + lo + k] = src + k
        pos[i] = int(lengths[i])
        slots[i] = logical_to_physical(tables[i], int(lengths[i]), block)
    return {
        "remap": np.array(remap, dtype=np.int32),
        "seq_off": np.array(seq_off, dtype=np.int32),
        "pos": np.array(pos, dtype=np.int32),
        "slot_mapping": np.array(slots, dtype=np.int32),
        "n_valid": n_valid,
        "n_runs": len(runs),
        "runs": runs,
    }


def prepare_prefill(tables, lengths, chunks, block: int, cap: int):
    """Preparation stage for one chunked-prefill step: sequence i has
    lengths[i] cached tokens and appends chunks[i] >= 1 new tokens at
    positions lengths[i] .. lengths[i] + chunks[i] - 1, so its compact
    segment holds lengths[i] + chunks[i] rows.  New tokens are numbered
    sequence by sequence in position order.

    Returns int32 arrays remap[cap], seq_off[S+1], tok_seq[n], pos[n],
    slot_mapping[n] and the ints n_valid, n_tokens, n_runs, plus 'runs'."""
    S = len(lengths)
    rows = [int(lengths[i]) + int(chunks[i]) for i in range(S)]
    seq_off = np.concatenate([[0], np.cumsum(rows, dtype=np.int64)]).astype(np.int64)
    n_valid = int(seq_off[-1])
    if n_valid > cap:
        raise ValueError("packed rows %d exceed capacity %d" % (n_valid, cap))
    remap = np.full(cap, -1, dtype=np.int64)
    runs = []
    tok_seq, pos, slots = [], [], []
    for i in range(S):
        for (src, lo, cnt) in contiguous_runs(tables[i], rows[i], block):
            runs.append((src, int(seq_off[i]) + lo, cnt))
            remap[seq_off[i] + lo: seq_off[i] + lo + cnt] = np.arange(src, src + cnt)
        for p in range(int(lengths[i]), rows[i]):
            tok_seq.append(i)
            pos.append(p)
            slots.append(logical_to_physical(tables[i], p, block))
    return {
        "remap": remap.astype(np.int32),
        "seq_off": seq_off.astype(np.int32),
        "tok_seq": np.array(tok_seq, dtype=np.int32),
        "pos": np.array(pos, dtype=np.int32),
        "slot_mapping": np.array(slots, dtype=np.int32),
        "n_valid": n_valid,
        "n_tokens": len(pos),
        "n_runs": len(runs),
        "runs": runs,
    }


def remap_gather(src: np.ndarray, remap: np.ndarray, n_valid=None, dst_init=None):
    """dst[j] = src[remap[j]] when 0 <= remap[j] < rows(src), else a zero
    row, for j < n_valid (all of remap when n_valid is None); rows at and
    beyond n_valid keep dst_init.  Works on any dtype (bit copy)."""
    src = np.asarray(src)
    remap = np.asarray(remap, dtype=np.int64)
    cap = remap.shape[0]
    nv = cap if n_valid is None else max(0, min(int(n_valid), cap))
    if dst_init is None:
        dst = np.zeros((cap,) + src.shape[1:], dtype=src.dtype)
    else:
        dst = np.array(dst_init, copy=True)
    idx = remap[:nv]
    ok = (idx >= 0) & (idx < src.shape[0])
    rows = np.take(src, np.where(ok, idx, 0), axis=0)
    rows[~ok] = 0
    dst[:nv] = rows
    return dst


def remap_gather_loops(src, remap, n_valid=None, dst_init=None):
    """remap_gather written as loops over rows (tiny cases)."""
    cap = len(remap)
    nv = cap if n_valid is None else max(0, min(int(n_valid), cap))
    out = [list(row) for row in dst_init] if dst_init is not None else \
        [[0] * len(src[0]) for _ in range(cap)]
    for j in range(nv):
        s = int(remap[j])
        if 0 <= s < len(src):
            out[j] = list(src[s])
        else:
            out[j] = [0] * len(src[0])
    return out
