"""Parity of the large-tile GEMM launches with ragged edges.

The small layer cases run every GEMM on 128 x 128 tiles; the full-size cases
reach the 256-wide tiles only with sizes that are multiples of 256.  Here one
MLP shard has 4000 tokens (15 full row tiles and 160 rows) and a local ffn of
3896 (15 full column tiles and 56 columns), so that the fc1 forward (bias +
GeLU, writing GeLU'(z) and GeLU(z)) and the fc2 dgrad with GeLU' run on
16 x 16 = 256 tiles of 256 x 256 whose last tile row and column are partial.
Every output is compared in full with the fp64 oracle of the rank's MLP
share.
"""
import numpy as np
import pytest

import synth
from oracle import layer as L
from oracle import shard as S
from tests.parity_util import assert_bf16, f64

SHAPE = synth.LayerShape(hidden=1024, heads=8, ffn=3896, seq=4000, micro_batch=1, tp=1)


@pytest.mark.gpu
def test_mlp_ragged_256_tiles(mtl):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import RankState, bf16_dev, host_f64

    print(f"mlp shard {SHAPE}", flush=True)
    inp = synth.layer_inputs(SHAPE, tp=1, rank=0)
    hb = synth.layer_tensor(SHAPE, "h")
    st = RankState(SHAPE, 1, 0, inp)
    h, dy = bf16_dev(hb), bf16_dev(inp["dy"])
    st.mlp_fwd(h)
    st.mlp_bwd(dy, h)
    torch.cuda.synchronize()
    g = {k: host_f64(getattr(st, k)) for k in ("gz", "a", "p_mlp", "p_dh", "dw1", "db1", "dw2", "db2")}
    del st
    torch.cuda.empty_cache()

    pr = {k: f64(inp[k]) for k in ("w1", "b1", "w2")}
    H, DY = f64(hb), f64(inp["dy"])
    fw = S.rank_mlp_forward(pr, H)
    assert_bf16("gz", g["gz"], L.gelu_grad(fw["z"]))
    assert_bf16("a", g["a"], fw["a"])
    assert_bf16("mlp partial", g["p_mlp"], fw["partial"])
    bw = S.rank_mlp_backward(pr, DY, H, fw["z"], fw["a"])
    assert_bf16("dh partial", g["p_dh"], bw["dh_partial"])
    for k in ("dw1", "db1", "dw2", "db2"):
        assert_bf16(k, g[k], bw[k])
