"""lowrank_layer_prefill_step on the GPU against the fp64 oracle: chunks of
prompt tokens appended to a paged cache of rank-r latents, causal attention
over each token's cached and earlier chunk rows.  Chunks of at most 64
tokens take the decode path, larger ones the prefill path (fused kernel
below 1024 rows, large-tile GEMMs from 1024 on, with the residual add and
the MLP activation in their epilogues).  Bar: max|gpu - ref| /
max|ref| <= 2e-2 on the residual stream."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import maxrel, to_f64
from step_util import Prefill
from test_decode_step import TOL, ranks_for, small_cfg

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lengths,chunks,n_layers,mlp", [
    ([0, 5, 40, 100], [3, 1, 16, 20], 1, "swiglu"),      # 40 tokens: decode path
    ([10, 0, 300], [100, 64, 150], 2, "swiglu"),         # 314 tokens: fused prefill kernel
    ([7, 0, 120], [33, 90, 10], 1, "relu"),              # 133 tokens, non-GLU MLP
    ([50], [1100], 1, "swiglu"),                         # 1100 tokens: large-tile GEMMs
    ([20, 3], [700, 330], 1, "relu"),                    # 1030 tokens: relu in the epilogue
])
def test_prefill_step_against_oracle(lengths, chunks, n_layers, mlp):
    cfg = dict(small_cfg(4, 2, 64, d_ffn=512), mlp=mlp)
    st = Prefill(60 + len(lengths) + sum(chunks), cfg, ranks_for(cfg), lengths, chunks, n_layers)
    h = st.run()
    torch.cuda.synchronize()
    err = maxrel(to_f64(h), st.oracle())
    print("prefill chunks %s, %d layers, %s: max rel err %.2e" % (chunks, n_layers, mlp, err))
    assert err <= TOL
    # every chunk token's latents were appended at its slot (bf16 of x U_k)
    x = np.stack([oracle.rmsnorm(r, st.layers[0]["g1"]) for r in st.h0])
    lk = x @ st.layers[0]["U"]["k"]
    slots = torch.from_numpy(st.prep["slot_mapping"].astype(np.int64)).cuda()
    got = st.pools_k[0][slots, :lk.shape[1]]
    assert maxrel(to_f64(got), lk) <= 1e-2


@pytest.mark.parametrize("H,Hkv,hd", [(4, 4, 128), (8, 1, 64), (2, 2, 128)])
def test_prefill_attention_head_shapes(H, Hkv, hd):
    # head_dim 128 and 64, MHA and MQA; chunks spanning several 128-token
    # query blocks (200, 129) and cached rows spanning several 64-row key
    # tiles with ragged ends (130, 257)
    cfg = dict(small_cfg(H, Hkv, hd, d_ffn=384), mlp="swiglu")
    lengths, chunks = [0, 130, 257], [200, 129, 70]
    st = Prefill(90 + H + hd, cfg, ranks_for(cfg), lengths, chunks, 1)
    h = st.run()
    torch.cuda.synchronize()
    err = maxrel(to_f64(h), st.oracle())
    print("prefill H=%d Hkv=%d hd=%d: max rel err %.2e" % (H, Hkv, hd, err))
    assert err <= TOL


def test_prefill_step_graph_replays_match_eager():
    # two layers over 1050 tokens of three sequences (grouped stage 1 of q, k, v
    # and gate, up, split-K stage 1 of o and down, residual add and SwiGLU in
    # the GEMM epilogues, tiled attention) captured once:
    # every replay, with eager runs of the same step in between, equals the
    # eager result bit for bit
    cfg = dict(small_cfg(4, 2, 64, d_ffn=384), mlp="swiglu")
    st = Prefill(95, cfg, ranks_for(cfg), [30, 0, 200], [600, 300, 150], 2)
    h_in = st.h.clone()
    pk = [p.clone() for p in st.pools_k]
    pv = [p.clone() for p in st.pools_v]

    def reset():
        st.h.copy_(h_in)
        for li in range(len(pk)):
            st.pools_k[li].copy_(pk[li])
            st.pools_v[li].copy_(pv[li])

    reset()
    st.run()
    torch.cuda.synchronize()
    ref = st.h.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    for _ in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.h, ref)
        reset()
        st.run()
        torch.cuda.synchronize()
        assert torch.equal(st.h, ref)
