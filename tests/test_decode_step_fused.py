"""lowrank_layer_decode_step_fused on the GPU: the decode layer with the K/V
reconstruction expanded per 256-row block inside the attention.  Against the
fp64 oracle to the decode step's bar, against lowrank_layer_decode_step
(which stores the same bf16 K/V rows and differs only in the order of fp32
sums), and graph replays against eager execution bit for bit."""
import numpy as np
import pytest
import torch

import rank_decomposed_amd as lr
from gpu_util import maxrel, to_f64
from step_util import Step
from test_decode_step import TOL, ranks_for, small_cfg

pytestmark = pytest.mark.gpu

# sequences of 0 to 700 cached rows: one row, block-aligned rows (255 + 1 =
# 256), several 256-row blocks with ragged ends
LENGTHS = [0, 1, 15, 255, 40, 300, 511, 700]


@pytest.mark.parametrize("H,Hkv,hd", [(4, 4, 64), (4, 2, 64), (4, 4, 128), (8, 2, 64),
                                      (16, 2, 128), (2, 1, 128), (16, 16, 128), (32, 8, 64),
                                      (16, 4, 128), (16, 8, 128), (12, 6, 128), (10, 10, 128)])
def test_fused_layer_against_oracle_and_unfused(H, Hkv, hd):
    # items of one, two or four 256-column tiles: 16 x 128 columns make 8
    # tiles in two four-tile items (four XCDs per item); 4 x 128 with 4
    # query heads per kv head two-tile items of 16 heads; 8 x 128 with 2
    # query heads per kv head four-tile items of 16 heads; 6 x 128 and
    # 10 x 128 a last item with fewer tiles
    cfg = small_cfg(H, Hkv, hd)
    seed = 150 + H + Hkv + hd
    st = Step(seed, cfg, ranks_for(cfg), LENGTHS, n_layers=1, fused=True)
    h = st.run()
    torch.cuda.synchronize()
    err = maxrel(to_f64(h), st.oracle())
    ref = Step(seed, cfg, ranks_for(cfg), LENGTHS, n_layers=1).run()
    torch.cuda.synchronize()
    diff = maxrel(to_f64(h), to_f64(ref))
    print("fused layer H=%d Hkv=%d hd=%d: max rel err %.2e, vs unfused %.2e" % (H, Hkv, hd, err,
                                                                              diff))
    assert err <= TOL
    assert diff <= 1e-2


def test_fused_two_layers_graph_replays_match_eager():
    cfg = small_cfg(4, 2, 128, d_ffn=384)
    st = Step(171, cfg, ranks_for(cfg), [3, 260, 0, 511, 90], n_layers=2, fused=True)
    h_in = st.h.clone()
    pk = [p.clone() for p in st.pools_k]
    pv = [p.clone() for p in st.pools_v]

    def reset():
        st.h.copy_(h_in)
        for li in range(2):
            st.pools_k[li].copy_(pk[li])
            st.pools_v[li].copy_(pv[li])

    reset()
    eager = st.run().clone()
    torch.cuda.synchronize()
    assert maxrel(to_f64(eager), st.oracle()) <= TOL
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
        assert torch.equal(st.h, eager)
        reset()
        st.run()
        torch.cuda.synchronize()
        assert torch.equal(st.h, eager)


def test_fused_rejects_too_many_query_heads_per_tile():
    # 256 / 64 kv heads per column tile x 8 query heads each = 32 > 16
    cfg = small_cfg(8, 1, 64)
    with pytest.raises(Exception):
        Step(181, cfg, ranks_for(cfg), [4, 9], n_layers=1, fused=True).run()


def test_fused_pools_over_2gib_take_the_gather_path_bit_exactly():
    # pools under 2 GiB are read in place through the remap list; larger ones
    # are first gathered into the compact buffers.  The same rows embedded at
    # the start of >= 2 GiB pools must give the same output bit for bit
    cfg = small_cfg(4, 2, 128)
    st = Step(191, cfg, ranks_for(cfg), [3, 260, 0, 511, 90, 17], n_layers=1, fused=True)
    h_in = st.h.clone()
    small = st.run().clone()
    torch.cuda.synchronize()
    assert maxrel(to_f64(small), st.oracle()) <= TOL
    pk, pv = st.pools_k[0], st.pools_v[0]
    rows = (1 << 31) // (2 * pk.stride(0)) + 16
    big_k = torch.zeros((rows, pk.shape[1]), dtype=pk.dtype, device=pk.device)
    big_v = torch.zeros_like(big_k)
    big_k[: pk.shape[0]] = pk   # the cached rows, and the new token's row the first run appended
    big_v[: pv.shape[0]] = pv
    assert big_k.numel() * 2 >= 1 << 31
    s = st.states[0]
    dp = st.dev_prep
    st.states = [lr.decode_state(big_k, big_v, dp["slot_mapping"], dp["remap"], dp["seq_off"],
                                 dp["pos"], st.n_valid, st.max_seq_rows)]
    st.h.copy_(h_in)
    big = st.run()
    torch.cuda.synchronize()
    assert torch.equal(big, small)
    del big_k, big_v, s
    torch.cuda.empty_cache()
