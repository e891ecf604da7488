"""fp64 oracle of one tensor-parallel rank's layer share with fp8 GEMM operands.

Test infrastructure only (see the package docstring).

The site summary's MoE deploy step passes ``--fp8-format hybrid``; the pages
give no recipe beyond the name.  Readings (with those of ``oracle.fp8``):

* only the four linears' GEMMs (forward, dgrad and wgrad) take fp8 operands;
  attention, softmax, GeLU, biases, the reductions and the bias gradients
  stay in full precision;
* every GEMM operand is quantised per tensor with current scaling, then
  multiplied in fp64 as its dequantised value decode(code)/s (the device
  accumulates in fp32 and applies both 1/s in the epilogue);
* forward operands (activations, weights) are E4M3, gradient operands E5M2:
  dgrad = q5(gradient) . q4(W)^T, wgrad = q4(activation)^T . q5(gradient);
* "per tensor" is the tensor the rank holds: the rank's weight shard, the full
  X / H / dY / dH it receives, its local A, dZ, O, dO, dQKV.

This is the second reference for the fp8 path: it isolates GEMM and
accumulation error from quantisation error.  The first is the plain fp64
layer on the unquantised inputs (``oracle.shard``).

Each function takes the two quantisers as arguments (defaults: the real
quant-dequant), so a test can swap them for the identity -- which must give
``oracle.shard`` exactly -- or for a marker that shows which operands each
format reaches.
"""
from __future__ import annotations

import numpy as np

from . import fp8 as Q
from . import layer as L
from . import shard as S


def q4(x):
    """Quant-dequant to E4M3 (forward operands)."""
    return Q.quant_dequant(np.asarray(x, dtype=np.float64), Q.E4M3)


def q5(x):
    """Quant-dequant to E5M2 (gradient operands)."""
    return Q.quant_dequant(np.asarray(x, dtype=np.float64), Q.E5M2)


def rank_attn_forward(pr: dict, x, local_heads: int, micro_batch: int = 1, fq=q4) -> dict:
    qkv = fq(x) @ fq(pr["w_qkv"]) + pr["b_qkv"]
    o, lse = L.attention_forward(qkv, local_heads, micro_batch)
    return dict(qkv=qkv, o=o, lse=lse, partial=fq(o) @ fq(pr["w_o"]))


def rank_mlp_forward(pr: dict, h, fq=q4) -> dict:
    z = fq(h) @ fq(pr["w1"]) + pr["b1"]
    a = L.gelu(z)
    return dict(z=z, a=a, partial=fq(a) @ fq(pr["w2"]))


def rank_mlp_backward(pr: dict, dy, h, z, a, fq=q4, gq=q5) -> dict:
    dyq = gq(dy)
    dz = (dyq @ fq(pr["w2"]).T) * L.gelu_grad(z)
    dzq = gq(dz)
    return dict(dz=dz, dw2=fq(a).T @ dyq, dw1=fq(h).T @ dzq, db1=dz.sum(axis=0),
                dh_partial=dzq @ fq(pr["w1"]).T, db2=dy.sum(axis=0))


def rank_attn_backward(pr: dict, dh, x, qkv, local_heads: int, micro_batch: int = 1, fq=q4, gq=q5) -> dict:
    o, _ = L.attention_forward(qkv, local_heads, micro_batch)
    dhq = gq(dh)
    do = dhq @ fq(pr["w_o"]).T
    dqkv = L.attention_backward(qkv, do, local_heads, micro_batch)
    dqq = gq(dqkv)
    return dict(do=do, dw_o=fq(o).T @ dhq, db_o=dh.sum(axis=0), dqkv=dqkv, dw_qkv=fq(x).T @ dqq,
                db_qkv=dqkv.sum(axis=0), dx_partial=dqq @ fq(pr["w_qkv"]).T)


def sharded_layer(p: dict, x, g, heads: int, tp: int, micro_batch: int = 1, residual: bool = False, fq=q4,
                  gq=q5) -> dict:
    """The whole layer as t fp8 rank shards plus the four reductions, in the
    order of ``oracle.shard.sharded_layer``."""
    S.check_divisible(x.shape[1], heads, p["w1"].shape[1], tp)
    lh = heads // tp
    prs = [S.shard_params(p, heads, tp, r) for r in range(tp)]
    att = [rank_attn_forward(pr, x, lh, micro_batch, fq) for pr in prs]
    hh = S.reduce_partials([a["partial"] for a in att], p["b_o"], x if residual else None)
    mlp = [rank_mlp_forward(pr, hh, fq) for pr in prs]
    y = S.reduce_partials([m["partial"] for m in mlp], p["b2"], hh if residual else None)
    mb = [rank_mlp_backward(pr, g, hh, m["z"], m["a"], fq, gq) for pr, m in zip(prs, mlp)]
    dh = S.reduce_partials([m["dh_partial"] for m in mb], None, g if residual else None)
    ab = [rank_attn_backward(pr, dh, x, a["qkv"], lh, micro_batch, fq, gq) for pr, a in zip(prs, att)]
    dx = S.reduce_partials([a["dx_partial"] for a in ab], None, dh if residual else None)
    return dict(y=y, h=hh, dh=dh, dx=dx, att=att, mlp=mlp, mlp_bwd=mb, attn_bwd=ab)
