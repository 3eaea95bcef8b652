"""lowrank_layer_decode_step on the GPU against the fp64 oracle (decode with
a paged cache of rank-r latents, remap gather, fixed-size reconstruction GEMM
and graph replay).  Bar: max|gpu - ref| / max|ref| <= 2e-2 on the residual
stream (bf16 arithmetic, fp32 residual)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import maxrel, to_f64
from step_util import Step

pytestmark = pytest.mark.gpu
TOL = 2e-2


def small_cfg(H, Hkv, hd, d_ffn=512):
    return {"d_model": H * hd, "n_heads": H, "n_kv_heads": Hkv, "head_dim": hd,
            "d_ffn": d_ffn, "eps": 1e-5}


def ranks_for(cfg, frac=3):
    dq, dkv = cfg["n_heads"] * cfg["head_dim"], cfg["n_kv_heads"] * cfg["head_dim"]
    d, f = cfg["d_model"], cfg["d_ffn"]
    return {"q": min(d, dq) // frac + 1, "k": min(d, dkv) // frac + 3,
            "v": min(d, dkv) // frac + 5, "o": min(d, dq) // frac + 2, "gate": min(d, f) // frac + 7,
            "up": min(d, f) // frac + 1, "down": min(d, f) // frac + 4}


@pytest.mark.parametrize("H,Hkv,hd", [(4, 4, 64), (4, 2, 64), (4, 4, 128), (8, 1, 64)])
def test_one_layer_against_oracle(H, Hkv, hd):
    cfg = small_cfg(H, Hkv, hd)
    st = Step(50 + H + Hkv + hd, cfg, ranks_for(cfg), [0, 1, 15, 16, 40, 300], n_layers=1)
    h = st.run()
    torch.cuda.synchronize()
    ref = st.oracle()
    err = maxrel(to_f64(h), ref)
    print("one layer H=%d Hkv=%d hd=%d max rel err %.2e" % (H, Hkv, hd, err))
    assert err <= TOL
    # the new tokens' latents were appended at their slots (bf16 of x U_k)
    x = oracle.rmsnorm(st.h0, st.layers[0]["g1"])
    lk = x @ st.layers[0]["U"]["k"]
    slots = st.prep["slot_mapping"]
    got = st.pools_k[0][torch.from_numpy(slots.astype(np.int64)).cuda(), :lk.shape[1]]
    assert maxrel(to_f64(got), lk) <= 1e-2


def test_three_layers_full_rank_against_oracle():
    cfg = small_cfg(4, 4, 64, d_ffn=384)
    full = {"q": 256, "k": 256, "v": 256, "o": 256, "gate": 256, "up": 256, "down": 256}
    st = Step(71, cfg, full, [3, 70, 129, 0, 255], n_layers=3)
    h = st.run()
    torch.cuda.synchronize()
    err = maxrel(to_f64(h), st.oracle())
    print("three layers full rank max rel err %.2e" % err)
    assert err <= TOL


def test_relu_mlp_layers_against_oracle():
    # non-GLU (OPT-style) MLP: fc2(relu(fc1 x)), fc1 and fc2 in the gate and
    # down slots, no up projection
    cfg = dict(small_cfg(4, 2, 64, d_ffn=640), mlp="relu")
    st = Step(81, cfg, ranks_for(cfg), [0, 9, 31, 64, 200], n_layers=2)
    h = st.run()
    torch.cuda.synchronize()
    err = maxrel(to_f64(h), st.oracle())
    print("relu mlp, two layers: max rel err %.2e" % err)
    assert err <= TOL


def test_per_layer_ratios_in_one_graph():
    # three layers at different ranks (ratios ~1/2, 1/3, 1/5 of full rank)
    # captured in one graph; replays match eager execution bit for bit and
    # the oracle to the bar
    cfg = small_cfg(4, 4, 64, d_ffn=448)
    ranks = [ranks_for(cfg, frac) for frac in (2, 3, 5)]
    st = Step(85, cfg, ranks, [4, 50, 0, 130], n_layers=3)
    h_in = st.h.clone()
    eager = st.run().clone()
    torch.cuda.synchronize()
    err = maxrel(to_f64(eager), st.oracle())
    print("per-layer ratios: max rel err %.2e" % err)
    assert err <= TOL
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st.h.copy_(h_in)
        st.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    for _ in range(3):
        st.h.copy_(h_in)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.h, eager)


def test_graph_replay_with_new_lengths_matches_eager():
    cfg = small_cfg(4, 2, 64)
    lengths = np.array([5, 33, 0, 100])
    # the pool holds the blocks of the largest step below (18 of 16 rows)
    st = Step(90, cfg, ranks_for(cfg), lengths, n_layers=2, max_seq_rows=160, cap=4 * 160,
              slack_blocks=6)
    h_in = st.h.clone()
    # capture the two layers once
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    import rank_decomposed_amd as lr
    for step, new_len in enumerate(([5, 33, 0, 100], [6, 34, 1, 101], [40, 2, 150, 7])):
        # host preparation for this step into the same device buffers; the
        # pools are reset to the seeded contents so each replay is comparable
        new_len = np.array(new_len)
        tables, _ = synth.block_tables(synth.seed_of(90, 0, step, synth.KIND_PLACE), new_len,
                                       16, slack_blocks=3)
        nb = st.pool_rows // 16
        assert max(t.max() for t in tables) < nb, step
        prep = lr.lowrank_prepare_decode(new_len, tables, 16, st.cap)
        for k in ("remap", "seq_off", "pos", "slot_mapping"):
            st.dev_prep[k].copy_(torch.from_numpy(np.ascontiguousarray(prep[k])))
        st.n_valid.fill_(prep["n_valid"])
        for li in range(2):
            st.pools_k[li].copy_(torch.from_numpy(synth.bf16_bits(st.pools_np_k[li]).view(np.int16))
                                 .view(torch.bfloat16).cuda())
            st.pools_v[li].copy_(torch.from_numpy(synth.bf16_bits(st.pools_np_v[li]).view(np.int16))
                                 .view(torch.bfloat16).cuda())
        st.h.copy_(h_in)
        g.replay()
        torch.cuda.synchronize()
        got = st.h.clone()
        st.h.copy_(h_in)
        for li in range(2):
            st.pools_k[li].copy_(torch.from_numpy(synth.bf16_bits(st.pools_np_k[li]).view(np.int16))
                                 .view(torch.bfloat16).cuda())
            st.pools_v[li].copy_(torch.from_numpy(synth.bf16_bits(st.pools_np_v[li]).view(np.int16))
                                 .view(torch.bfloat16).cuda())
        st.run()
        torch.cuda.synchronize()
        assert torch.equal(got, st.h), step
        ref = oracle.decode_step(st.h0, st.layers, st.pools_np_k, st.pools_np_v, tables, new_len,
                                 16, cfg)
        assert maxrel(to_f64(got), ref) <= TOL
