"""lowrank_layer_prefill_step on the GPU against the fp64 oracle: chunks of
prompt tokens appended to a paged cache of rank-r latents, causal attention
over each token's cached and earlier chunk rows.  Chunks of at most 64
tokens take the decode path, larger ones the prefill path (fused kernel
below 1024 rows, large-tile GEMMs from 1024 on).  Bar: max|gpu - ref| /
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
