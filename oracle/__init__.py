"""fp64 CPU oracle for the low-rank decomposed hot path.

TEST INFRASTRUCTURE, NOT PRODUCT.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
It shares no code with the HIP path (``rank_decomposed_amd``) and imports
nothing from it; both sides receive their inputs from ``synth``.

Every function is a plain, slow statement of what the method computes, in
float64, written from the pages (citation key: "DeInfer/en" = English
technical summary of *DeInfer: Efficient Parallel Inferencing for Decomposed
Large Language Models*, "DeInfer/es" the Spanish one, "DeInfer/zh" the
Chinese one).  Library primitives (matmul, SVD, take) serve as steps; there is
no blocking, fusion or reordering beyond the definitions.

Pins (``tests/test_oracle_pins.py`` and friends, ``-m "not gpu"``):
associativity, full-rank reconstruction, Eckart-Young, brute-force loops on
tiny shapes, hand-computed golden cases, shard-sum, gather identities,
paging coverage/maximality, RMSNorm/rotary/softmax closed forms, the
full-rank decoder layer against a dense textbook layer, a chunk of prefill
against token-by-token decode, and the multi-layer, multi-sequence
compositions (decode_step, prefill_layer, prefill_step) against a dense
textbook decoder stack at full rank plus prefill_step with single-token
chunks against decode_step.  Each function has at least one such pin.
"""
from .lowrank import (rank_for_ratio, truncated_factors, linear, linear_loops,
                      tp_share_stage1, tp_share_stage2)
from .paging import (logical_to_physical, contiguous_runs, prepare_decode, prepare_prefill,
                     remap_gather, remap_gather_loops)
from .decoder import (rmsnorm, rope, attention_one, silu, relu, decode_layer_seq,
                      decode_layer, decode_step, prefill_layer_seq, prefill_layer,
                      prefill_step)

__all__ = [
    "rank_for_ratio", "truncated_factors", "linear", "linear_loops",
    "tp_share_stage1", "tp_share_stage2",
    "logical_to_physical", "contiguous_runs", "prepare_decode", "prepare_prefill", "remap_gather",
    "remap_gather_loops",
    "rmsnorm", "rope", "attention_one", "silu", "relu", "decode_layer_seq",
    "decode_layer", "decode_step", "prefill_layer_seq", "prefill_layer", "prefill_step",
]
