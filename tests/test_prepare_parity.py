"""Preparation stage (host C++ in liblowrank) against the oracle: bit-exact
integer outputs on seeded placements at the decode-step workload's shape
(64 sequences, lengths uniform in [128, 4096], block 16) and on edge cases.
CPU only."""
import numpy as np
import pytest

import oracle
import rank_decomposed_amd as lr
import synth
from golden_io import paging_case


def _compare(lengths, tables, block, cap):
    ref = oracle.prepare_decode(tables, lengths, block, cap)
    got = lr.lowrank_prepare_decode(lengths, tables, block, cap, want_runs=True)
    for k in ("remap", "seq_off", "pos", "slot_mapping"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["n_valid"] == ref["n_valid"]
    assert got["n_runs"] == ref["n_runs"]
    assert [tuple(r) for r in got["runs"]] == ref["runs"]


def test_hand_worked_case():
    c = paging_case()
    _compare(c["len"], c["tables"], c["block"], c["cap"])


@pytest.mark.parametrize("seed", [0, 1])
def test_decode_step_workload(seed):
    # 64 sequences, L ~ U[128, 4096], block 16, cap = 64 * 4112 rows
    lengths = synth.decode_lengths(synth.seed_of(5, 0, 0, synth.KIND_LEN) + seed, 64)
    tables, _ = synth.block_tables(synth.seed_of(5, 0, 0, synth.KIND_PLACE) + seed, lengths,
                                   block=16)
    _compare(lengths, tables, 16, 64 * 4112)


@pytest.mark.parametrize("block", [1, 3, 16, 64])
def test_ragged_and_small(block):
    lengths = np.array([0, 1, 15, 16, 17, 100, 0])
    tables, _ = synth.block_tables(7, lengths, block=block, max_extent=3)
    cap = int(lengths.sum() + len(lengths)) + 5
    _compare(lengths, tables, block, cap)


def test_empty_batch_and_exact_capacity():
    _compare(np.array([], dtype=np.int64), [], 16, 4)
    lengths = np.array([31])
    tables, _ = synth.block_tables(0, lengths, block=16)
    _compare(lengths, tables, 16, 32)


def test_errors():
    with pytest.raises(lr.LowrankError) as e:
        lr.lowrank_prepare_decode(np.array([31]), [np.array([0, 1])], 16, 31)
    assert e.value.status == 5
    with pytest.raises(lr.LowrankError) as e:          # table too short
        lr.lowrank_prepare_decode(np.array([32]), [np.array([0, 1])], 16, 100)
    assert e.value.status == 1
    with pytest.raises(lr.LowrankError) as e:          # negative block index
        lr.lowrank_prepare_decode(np.array([3]), [np.array([-2])], 16, 100)
    assert e.value.status == 1


# ---------------------------------------------------------------- chunked prefill
def _prefill_case(seed, S, block, max_chunk):
    g = synth.rng(seed)
    lengths = g.integers(0, 300, S)
    chunks = g.integers(1, max_chunk + 1, S)
    # tables cover lengths + chunks rows (block_tables covers its lengths + 1)
    tables, _ = synth.block_tables(seed, lengths + chunks - 1, block=block, max_extent=4)
    return lengths, chunks, tables


@pytest.mark.parametrize("seed,block,max_chunk", [(0, 16, 64), (1, 3, 1), (2, 1, 9), (3, 64, 300)])
def test_prefill_against_oracle(seed, block, max_chunk):
    lengths, chunks, tables = _prefill_case(seed, 9, block, max_chunk)
    cap = int((lengths + chunks).sum()) + 7
    ref = oracle.prepare_prefill(tables, lengths, chunks, block, cap)
    got = lr.lowrank_prepare_prefill(lengths, chunks, tables, block, cap, want_runs=True)
    for k in ("remap", "seq_off", "tok_seq", "pos", "slot_mapping"):
        assert np.array_equal(got[k], ref[k]), k
    for k in ("n_valid", "n_tokens", "n_runs"):
        assert got[k] == ref[k], k
    assert [tuple(r) for r in got["runs"]] == ref["runs"]


def test_prefill_oracle_against_decode_oracle():
    # two oracle functions written independently: a chunk of c tokens lays out
    # the rows of a decode step at length L + c - 1, and its last token is that
    # step's new token; chunks of one are exactly a decode step
    lengths, chunks, tables = _prefill_case(11, 7, 16, 40)
    cap = int((lengths + chunks).sum())
    pf = oracle.prepare_prefill(tables, lengths, chunks, 16, cap)
    dc = oracle.prepare_decode(tables, lengths + chunks - 1, 16, cap)
    for k in ("remap", "seq_off"):
        assert np.array_equal(pf[k], dc[k]), k
    assert pf["runs"] == dc["runs"]
    last = np.cumsum(chunks) - 1
    assert np.array_equal(pf["pos"][last], dc["pos"])
    assert np.array_equal(pf["slot_mapping"][last], dc["slot_mapping"])
    assert np.array_equal(pf["tok_seq"], np.repeat(np.arange(7), chunks))
    one = oracle.prepare_prefill(tables, lengths, np.ones(7, np.int64), 16, cap)
    dec = oracle.prepare_decode(tables, lengths, 16, cap)
    for k in ("remap", "seq_off", "pos", "slot_mapping"):
        assert np.array_equal(one[k], dec[k]), k


def test_prefill_errors():
    tables = [np.array([0, 1, 2])]
    with pytest.raises(lr.LowrankError) as e:          # a chunk must hold a token
        lr.lowrank_prepare_prefill(np.array([3]), np.array([0]), tables, 16, 100)
    assert e.value.status == 1
    with pytest.raises(lr.LowrankError) as e:          # more new tokens than max_tokens
        lr.lowrank_prepare_prefill(np.array([3]), np.array([5]), tables, 16, 100, max_tokens=4)
    assert e.value.status == 5
    with pytest.raises(lr.LowrankError) as e:          # table too short for 3 + 46 rows
        lr.lowrank_prepare_prefill(np.array([3]), np.array([46]), tables, 16, 100)
    assert e.value.status == 1
