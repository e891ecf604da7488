"""Parity at the full workload sizes, in the launch configuration bench.py times.

One TP rank's shard of a 7B-class layer (hidden 4096, 32 heads, ffn 16384,
seq 4096, TP=4) and of a 96-layer-GPT-shaped layer (hidden 8192, 64 heads, ffn
32768, seq 4096, TP=8), rank 0.  Each block call of the C ABI is fed seeded
synthetic inputs (x and dY, plus independent H and dH for the MLP and
attention halves) and compared with the fp64 oracle of the rank's share:
QKV, attention output and log-sum-exp, the attention backward's dO and dQKV
(read from the call's scratch) and the bias gradients in full; the large GEMM
outputs on sampled rows (activations) or sampled columns (weight gradients),
which the oracle computes one by one.
"""
import numpy as np
import pytest

import synth
from oracle import layer as L
from tests.parity_util import assert_bf16, f64

ROWS = [0, 1, 63, 64, 127, 1000, 2047, 2048, 3001, 4095]
COLS = [0, 1, 7, 8, 255, 256, 511, 1023]


def _cols(n):
    rng = np.random.default_rng(5)
    extra = rng.choice(n, 8, replace=False).tolist()
    return sorted(set([c for c in COLS if c < n] + [n - 1] + extra))


@pytest.mark.gpu
@pytest.mark.parametrize("workload", ["7b-tp4", "gpt96l-tp8"])
def test_rank_shard_full_size(mtl, workload):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import RankState, bf16_dev, host_f64

    shape = synth.WORKLOADS[workload]
    t = shape.tp
    print(f"workload {workload} rank 0 of tp {t}", flush=True)
    inp = synth.layer_inputs(shape, tp=t, rank=0)
    hb = synth.layer_tensor(shape, "h")
    dhb = synth.layer_tensor(shape, "dh")
    st = RankState(shape, t, 0, inp)
    x, dy, h, dh = bf16_dev(inp["x"]), bf16_dev(inp["dy"]), bf16_dev(hb), bf16_dev(dhb)
    st.attn_fwd(x)
    st.mlp_fwd(h)
    st.mlp_bwd(dy, h)
    st.attn_bwd(dh, x)
    torch.cuda.synchronize()
    g = {k: host_f64(getattr(st, k)) for k in ("qkv", "o", "lse", "gz", "a", "p_attn", "p_mlp", "p_dh", "p_dx",
                                               "dw_qkv", "db_qkv", "dw_o", "db_o", "dw1", "db1", "dw2", "db2")}
    # the attention backward's own outputs, left in the scratch: dO and dQKV
    off_do, off_dqkv = mtl.mtl_attn_bwd_scratch_layout(st.cfg)
    D = st.D
    sview = lambda off, cols: host_f64(st.scratch[off:off + D.S * cols * 2].view(torch.bfloat16).view(D.S, cols))
    g["do"], g["dqkv"] = sview(off_do, D.o_l), sview(off_dqkv, D.qkv_l)
    del st
    torch.cuda.empty_cache()

    p = {k: f64(inp[k]) for k in ("w_qkv", "b_qkv", "w_o", "w1", "b1", "w2")}
    X, DY, H, DH = f64(inp["x"]), f64(inp["dy"]), f64(hb), f64(dhb)
    lh = shape.heads // t
    rows = ROWS

    # attention forward: qkv, o, lse in full; the partial on sampled rows
    qkv = X @ p["w_qkv"] + p["b_qkv"]
    assert_bf16("qkv", g["qkv"], qkv)
    o, lse = L.attention_forward(qkv, lh)
    assert_bf16("o", g["o"], o)
    assert_bf16("lse", g["lse"], lse)
    assert_bf16("attn partial[rows]", g["p_attn"][rows], o[rows] @ p["w_o"])

    # MLP forward on sampled rows
    z_r = H[rows] @ p["w1"] + p["b1"]
    a_r = L.gelu(z_r)
    assert_bf16("gz[rows]", g["gz"][rows], L.gelu_grad(z_r))
    assert_bf16("a[rows]", g["a"][rows], a_r)
    assert_bf16("mlp partial[rows]", g["p_mlp"][rows], a_r @ p["w2"])

    # MLP backward: dgrad partial on sampled rows, weight gradients on sampled columns
    dz_r = (DY[rows] @ p["w2"].T) * L.gelu_grad(z_r)
    assert_bf16("dh partial[rows]", g["p_dh"][rows], dz_r @ p["w1"].T)
    z_full = H @ p["w1"] + p["b1"]
    a_full = L.gelu(z_full)
    ch = _cols(shape.hidden)
    assert_bf16("dw2[:, cols]", g["dw2"][:, ch], a_full.T @ DY[:, ch])
    cf = _cols(shape.ffn // t)
    dz_c = (DY @ p["w2"][cf].T) * L.gelu_grad(z_full[:, cf])
    assert_bf16("dw1[:, cols]", g["dw1"][:, cf], H.T @ dz_c)
    dz_full = (DY @ p["w2"].T) * L.gelu_grad(z_full)
    assert_bf16("db1", g["db1"], dz_full.sum(axis=0))
    assert_bf16("db2", g["db2"], DY.sum(axis=0))
    del z_full, a_full, dz_full

    # attention backward: dO and dQKV in full, then the products that take them
    do = DH @ p["w_o"].T
    assert_bf16("do", g["do"], do)
    dqkv = L.attention_backward(qkv, do, lh)
    assert_bf16("dqkv", g["dqkv"], dqkv)
    co = _cols(shape.hidden)
    assert_bf16("dw_o[:, cols]", g["dw_o"][:, co], o.T @ DH[:, co])
    assert_bf16("db_o", g["db_o"], DH.sum(axis=0))
    cq = _cols(3 * shape.hidden // t)
    assert_bf16("dw_qkv[:, cols]", g["dw_qkv"][:, cq], X.T @ dqkv[:, cq])
    assert_bf16("db_qkv", g["db_qkv"], dqkv.sum(axis=0))
    assert_bf16("dx partial[rows]", g["p_dx"][rows], dqkv[rows] @ p["w_qkv"].T)


@pytest.mark.gpu
def test_fp8_rank_shard_full_size(mtl):
    """The fp8 variant of the 7B-class TP=4 rank 0 shard, in the launch
    configuration bench.py --precision fp8 times.  Every fp8 GEMM kind is
    checked where its operands are call inputs (so both sides quantise the same
    bf16 values to the same codes) against the fp64 product of the dequantised
    codes: qkv in full, GeLU'(z) and a on sampled rows, dw2 and dw_o on sampled
    columns, db1 (a column sum of the dgrad output dz) on sampled columns, and
    dO (read from the attention backward's scratch) in full."""
    import torch
    from oracle import fp8_layer as F8
    from megatron_tensor_transformer_layer_amd.layer import RankState, bf16_dev, host_f64

    shape = synth.WORKLOADS["7b-tp4"]
    t = shape.tp
    f_l, o_l = shape.ffn // t, shape.hidden // t
    print(f"fp8 workload 7b-tp4 rank 0 of tp {t}", flush=True)
    inp = synth.layer_inputs(shape, tp=t, rank=0)
    hb, dhb = synth.layer_tensor(shape, "h"), synth.layer_tensor(shape, "dh")
    zb = synth.bf16_round_bits(f64(synth.layer_tensor(shape, "dh", seed=3))[:, :f_l] * 2.0)
    ab = synth.layer_tensor(shape, "h", seed=4)[:, :f_l].copy()
    ob = synth.layer_tensor(shape, "x", seed=6)[:, :o_l].copy()
    st = RankState(shape, t, 0, inp, precision=mtl.MTL_PREC_FP8_HYBRID)
    x, dy, h, dh = bf16_dev(inp["x"]), bf16_dev(inp["dy"]), bf16_dev(hb), bf16_dev(dhb)
    st.attn_fwd(x)
    st.mlp_fwd(h)
    torch.cuda.synchronize()
    g = dict(qkv=host_f64(st.qkv), gz=host_f64(st.gz[ROWS]), a=host_f64(st.a[ROWS]))
    st.gz.copy_(bf16_dev(synth.bf16_round_bits(L.gelu_grad(f64(zb)))))  # the saved GeLU'(z) of an independent z
    st.a.copy_(bf16_dev(ab))
    st.o.copy_(bf16_dev(ob))
    st.mlp_bwd(dy, h)
    st.attn_bwd(dh, x)
    torch.cuda.synchronize()
    g.update(dw2=host_f64(st.dw2), db1=host_f64(st.db1), dw_o=host_f64(st.dw_o), db_o=host_f64(st.db_o))
    off_do, _ = mtl.mtl_attn_bwd_scratch_layout(st.cfg)
    g["do"] = host_f64(st.scratch[off_do:off_do + shape.seq * o_l * 2].view(torch.bfloat16).view(shape.seq, o_l))
    del st
    torch.cuda.empty_cache()
    print("device calls done", flush=True)

    q4, q5 = F8.q4, F8.q5
    p = {k: f64(inp[k]) for k in ("w_qkv", "b_qkv", "w1", "b1", "w2")}
    Xq = q4(f64(inp["x"]))
    assert_bf16("qkv", g["qkv"], Xq @ q4(p["w_qkv"]) + p["b_qkv"])
    del Xq
    z_r = q4(f64(hb))[ROWS] @ q4(p["w1"]) + p["b1"]
    assert_bf16("gz[rows]", g["gz"], L.gelu_grad(z_r))
    assert_bf16("a[rows]", g["a"], L.gelu(z_r))
    DYq = q5(f64(inp["dy"]))
    ch = _cols(shape.hidden)
    assert_bf16("dw2[:, cols]", g["dw2"][:, ch], q4(f64(ab)).T @ DYq[:, ch])
    cf = _cols(f_l)
    dz_c = (DYq @ q4(p["w2"])[cf].T) * L.gelu_grad(f64(zb)[:, cf])
    assert_bf16("db1[cols]", g["db1"][cf], dz_c.sum(axis=0))
    del DYq
    DH = f64(dhb)
    # dO = dH . w_o^T: the dgrad half of the output projection's fp8 pair launch
    assert_bf16("do", g["do"], q5(DH) @ q4(f64(inp["w_o"])).T)
    assert_bf16("dw_o[:, cols]", g["dw_o"][:, ch], q4(f64(ob)).T @ q5(DH)[:, ch])
    assert_bf16("db_o", g["db_o"], DH.sum(axis=0))


# The fp8 GEMMs of the 7B-class TP=4 rank (M, N, K, fmt A, fmt B, what it is),
# each launched alone as the layer calls launch them; operands k-contiguous.
FP8_GEMMS = [
    (4096, 3072, 4096, 0, 0, "qkv forward (with bias)"),
    (4096, 4096, 1024, 0, 0, "output projection forward"),
    (4096, 4096, 4096, 0, 0, "fc2 forward"),
    (4096, 4096, 4096, 1, 0, "fc1 dgrad"),
    (4096, 4096, 3072, 1, 0, "qkv dgrad"),
    (4096, 4096, 4096, 0, 1, "fc1 wgrad"),
    (4096, 3072, 4096, 0, 1, "qkv wgrad"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(FP8_GEMMS)))
def test_fp8_gemm_full_size_identical_codes(mtl, case):
    """Every fp8 GEMM shape of the 7B-class TP=4 rank whose operand inside the
    layer calls is an intermediate (and so differs from the oracle's in its last
    bits): here both operands are quantised from the same bf16 values on both
    sides (the cast is bit-exact), and the device product, through the same
    dispatch and tile choice, is compared with the fp64 product of the
    dequantised codes on sampled rows and columns, within the bf16 bound."""
    import torch
    from oracle import fp8_layer as F8
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev, host_f64
    M, N, K, fa, fb, what = FP8_GEMMS[case]
    print(f"fp8 gemm {what}: {M}x{N}x{K} formats {fa},{fb}", flush=True)
    ab = synth.mx_operand(M, K, "mx_a", 1.0, seed=40 + case)
    bb = synth.mx_operand(N, K, "mx_b", 1.0 if fb == 1 else synth.WEIGHT_STD, seed=60 + case)
    bias = synth.bf16_round_bits(np.random.default_rng(case).standard_normal(N) * synth.WEIGHT_STD) \
        if case == 0 else None
    dev = lambda bits: bf16_dev(bits)
    qa = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    qb = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    ra = torch.empty(4, dtype=torch.float32, device="cuda")
    rb = torch.empty(4, dtype=torch.float32, device="cuda")
    ws = torch.empty(mtl.MTL_FP8_AMAX_SCRATCH, dtype=torch.uint8, device="cuda")
    mtl.mtl_fp8_quantize(dev(ab), M, K, fa, ra, qa, None, ws)
    mtl.mtl_fp8_quantize(dev(bb), N, K, fb, rb, qb, None, ws)
    out = torch.empty(M, N, dtype=torch.float32 if fb == 1 else torch.bfloat16, device="cuda")
    mtl.mtl_fp8_gemm(M, N, K, qa, fa, ra, qb, fb, rb, None if bias is None else dev(bias), out)
    torch.cuda.synchronize()
    got = host_f64(out)
    q = lambda bits, f: (F8.q5 if f == 1 else F8.q4)(f64(bits))
    A, B = q(ab, fa), q(bb, fb)
    rows, cols = ROWS, _cols(N)
    add = 0.0 if bias is None else f64(bias)
    assert_bf16(f"{what} rows", got[rows], A[rows] @ B.T + add)
    assert_bf16(f"{what} cols", got[:, cols], A @ B[cols].T + (0.0 if bias is None else f64(bias)[cols]))
