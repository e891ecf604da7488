"""The output projection's backward in two halves of its contraction, with a
ragged token count.

At hidden 8192 with TP=8 (local heads 8 of 128, o_l 1024) the data gradient
dO = dH . W_o^T has few output tiles and a contraction (hidden) at least 1.5x
the weight gradient's (tokens), so the library runs dO as two fp32 halves of
the hidden dimension beside dW_o on 256 x 256 tiles and the attention
backward's D pass sums the halves into bf16 dO.  Here the rank has 3000 tokens:
the last row tile of dO and the last k slabs of dW_o are partial, and the D
pass sees a ragged last block.  dO and dQKV (read from the call's scratch) are
compared in full with the fp64 oracle of the rank's attention backward, dW_o and
dW_qkv on sampled columns, dX on sampled rows, db_qkv and db_o in full.
"""
import numpy as np
import pytest

import synth
from oracle import layer as L
from tests.parity_util import assert_bf16, f64

SHAPE = synth.LayerShape(hidden=8192, heads=64, ffn=8192, seq=3000, micro_batch=1, tp=8)
ROWS = [0, 1, 255, 256, 1023, 2047, 2048, 2815, 2816, 2999]


def _cols(n, seed):
    rng = np.random.default_rng(seed)
    return sorted(set([0, 1, 255, 256, n - 1] + rng.choice(n, 8, replace=False).tolist()))


@pytest.mark.gpu
def test_proj_bwd_halves_ragged_tokens(mtl):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import RankState, bf16_dev, host_f64

    t = SHAPE.tp
    print(f"attention shard {SHAPE} rank 0", flush=True)
    inp = synth.layer_inputs(SHAPE, tp=t, rank=0, names=("x", "w_qkv", "b_qkv", "w_o", "w1", "b1", "w2"))
    dhb = synth.layer_tensor(SHAPE, "dh")
    st = RankState(SHAPE, t, 0, inp)
    x, dh = bf16_dev(inp["x"]), bf16_dev(dhb)
    st.attn_fwd(x)
    st.attn_bwd(dh, x)
    torch.cuda.synchronize()
    g = {k: host_f64(getattr(st, k)) for k in ("qkv", "p_dx", "dw_qkv", "db_qkv", "dw_o", "db_o")}
    off_do, off_dqkv = mtl.mtl_attn_bwd_scratch_layout(st.cfg)
    D = st.D
    sview = lambda off, cols: host_f64(st.scratch[off:off + D.S * cols * 2].view(torch.bfloat16).view(D.S, cols))
    g["do"], g["dqkv"] = sview(off_do, D.o_l), sview(off_dqkv, D.qkv_l)
    del st
    torch.cuda.empty_cache()

    p = {k: f64(inp[k]) for k in ("w_qkv", "b_qkv", "w_o")}
    X, DH = f64(inp["x"]), f64(dhb)
    lh = SHAPE.heads // t
    # the oracle's backward takes the device's QKV (checked by the layer tests), so
    # that this test's cost stays with the products it is about
    qkv = g["qkv"]
    o, _ = L.attention_forward(qkv, lh)
    do = DH @ p["w_o"].T
    assert_bf16("do", g["do"], do)
    dqkv = L.attention_backward(qkv, do, lh)
    assert_bf16("dqkv", g["dqkv"], dqkv)
    co = _cols(SHAPE.hidden, 1)
    assert_bf16("dw_o[:, cols]", g["dw_o"][:, co], o.T @ DH[:, co])
    assert_bf16("db_o", g["db_o"], DH.sum(axis=0))
    cq = _cols(3 * SHAPE.hidden // t, 2)
    assert_bf16("dw_qkv[:, cols]", g["dw_qkv"][:, cq], X.T @ dqkv[:, cq])
    assert_bf16("db_qkv", g["db_qkv"], dqkv.sum(axis=0))
    assert_bf16("dx partial[rows]", g["p_dx"][ROWS], dqkv[ROWS] @ p["w_qkv"].T)
