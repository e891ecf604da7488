"""fp64 oracle of one tensor-parallel rank's layer share with MXFP4 GEMM operands.

Test infrastructure only (see the package docstring).

The site summary's precision list and deploy step 7 name 4-bit training
(NVFP4 on Blackwell) with no recipe; the reading here is OCP MXFP4 (see
``oracle.mxfp4``) applied the way microscaling formats are applied to
training: every GEMM of the four linears -- forward, dgrad and wgrad -- takes
both of its operands quantised to MXFP4 with the 32-element blocks running
along that product's contraction, and multiplies them exactly.  So the
forward x . W quantises x along its rows' features and W down its columns (its
input features); dgrad dY . W^T quantises dY along its features and W along
its rows' output features; wgrad X^T . dY quantises both down their token
columns.  Attention, softmax, GeLU, the biases, the reductions and the bias
gradients stay in full precision, as in ``oracle.fp8_layer``.

Every function takes the quantiser ``q`` (default: MXFP4 quant-dequant of a
matrix along its last axis) so that a test can pass the identity -- which must
give ``oracle.shard`` exactly -- or a quantiser that takes the bf16 value the
device stores first.
"""
from __future__ import annotations

import numpy as np

from . import layer as L
from . import mxfp4 as MX
from . import shard as S


def q_last(x):
    """MXFP4 quant-dequant of x [rows, k] in blocks of 32 along its last axis."""
    codes, scales = MX.quantize_fast(np.asarray(x, dtype=np.float64), "e2m1")
    return MX.dequantize(codes, scales, "e2m1")


def mm(a, b, q=q_last):
    """a @ b with both operands quantised along the contraction: a along its
    last axis, b along its first (b^T along its last)."""
    return q(a) @ q(np.asarray(b).T).T


def rank_attn_forward(pr: dict, x, local_heads: int, micro_batch: int = 1, q=q_last) -> dict:
    qkv = mm(x, pr["w_qkv"], q) + pr["b_qkv"]
    o, lse = L.attention_forward(qkv, local_heads, micro_batch)
    return dict(qkv=qkv, o=o, lse=lse, partial=mm(o, pr["w_o"], q))


def rank_mlp_forward(pr: dict, h, q=q_last) -> dict:
    z = mm(h, pr["w1"], q) + pr["b1"]
    a = L.gelu(z)
    return dict(z=z, a=a, partial=mm(a, pr["w2"], q))


def rank_mlp_backward(pr: dict, dy, h, z, a, q=q_last) -> dict:
    dz = mm(dy, pr["w2"].T, q) * L.gelu_grad(z)
    return dict(dz=dz, dw2=mm(np.asarray(a).T, dy, q), dw1=mm(np.asarray(h).T, dz, q), db1=dz.sum(axis=0),
                dh_partial=mm(dz, pr["w1"].T, q), db2=np.asarray(dy).sum(axis=0))


def rank_attn_backward(pr: dict, dh, x, qkv, local_heads: int, micro_batch: int = 1, q=q_last) -> dict:
    o, _ = L.attention_forward(qkv, local_heads, micro_batch)
    do = mm(dh, pr["w_o"].T, q)
    dqkv = L.attention_backward(qkv, do, local_heads, micro_batch)
    return dict(do=do, dw_o=mm(o.T, dh, q), db_o=np.asarray(dh).sum(axis=0), dqkv=dqkv,
                dw_qkv=mm(np.asarray(x).T, dqkv, q), db_qkv=dqkv.sum(axis=0), dx_partial=mm(dqkv, pr["w_qkv"].T, q))


def sharded_layer(p: dict, x, g, heads: int, tp: int, micro_batch: int = 1, residual: bool = False,
                  q=q_last) -> dict:
    """The whole layer as t MXFP4 rank shards plus the four reductions, in the
    order of ``oracle.shard.sharded_layer``."""
    S.check_divisible(x.shape[1], heads, p["w1"].shape[1], tp)
    lh = heads // tp
    prs = [S.shard_params(p, heads, tp, r) for r in range(tp)]
    att = [rank_attn_forward(pr, x, lh, micro_batch, q) for pr in prs]
    hh = S.reduce_partials([a["partial"] for a in att], p["b_o"], x if residual else None)
    mlp = [rank_mlp_forward(pr, hh, q) for pr in prs]
    y = S.reduce_partials([m["partial"] for m in mlp], p["b2"], hh if residual else None)
    mb = [rank_mlp_backward(pr, g, hh, m["z"], m["a"], q) for pr, m in zip(prs, mlp)]
    dh = S.reduce_partials([m["dh_partial"] for m in mb], None, g if residual else None)
    ab = [rank_attn_backward(pr, dh, x, a["qkv"], lh, micro_batch, q) for pr, a in zip(prs, att)]
    dx = S.reduce_partials([a["dx_partial"] for a in ab], None, dh if residual else None)
    return dict(y=y, h=hh, dh=dh, dx=dx, att=att, mlp=mlp, mlp_bwd=mb, attn_bwd=ab)
