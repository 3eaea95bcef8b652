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
