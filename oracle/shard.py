"""fp64 oracle of one tensor-parallel rank's share of the layer.

Test infrastructure only (see the package docstring).

Placement follows the tutorial's section 2.2: the QKV projection is split by
output columns (whole attention heads, heads/t per rank -- the tutorial's
section 4.2 example is 12 heads / TP 2 = 6), the first MLP linear by columns,
the output projection and second MLP linear by rows.  A row-parallel linear
yields a partial sum per rank; the t partials are added (the all-reduce) and
the row-parallel bias is added once, after the sum.  The divisibility rule
(hidden size and head count divisible by the TP degree; the tutorial's
3-heads-on-TP-8 example fails) is ``check_divisible``.
"""
from __future__ import annotations

import numpy as np

from . import layer as L


class ShapeError(ValueError):
    pass


def check_divisible(hidden: int, heads: int, ffn: int, tp: int, rank: int = 0) -> None:
    """Raise ShapeError unless the shard is well defined: every size positive,
    hidden % heads == 0, heads % tp == 0 (hence hidden % tp == 0), ffn % tp == 0
    and 0 <= rank < tp."""
    if min(hidden, heads, ffn, tp) <= 0:
        raise ShapeError("sizes must be positive")
    if hidden % heads:
        raise ShapeError(f"hidden {hidden} not divisible by heads {heads}")
    if heads % tp:
        raise ShapeError(f"heads {heads} not divisible by TP {tp}")
    if ffn % tp:
        raise ShapeError(f"ffn {ffn} not divisible by TP {tp}")
    if not 0 <= rank < tp:
        raise ShapeError(f"rank {rank} outside [0, {tp})")


def shard_params(p: dict, heads: int, tp: int, rank: int) -> dict:
    """Rank ``rank``'s slices of the full parameters (fp64 views).  b_o and b2 are
    returned whole: they belong to the sum, not to a rank."""
    h = p["w_qkv"].shape[0]
    f = p["w1"].shape[1]
    check_divisible(h, heads, f, tp, rank)
    c = 3 * h // tp
    o = h // tp
    m = f // tp
    return dict(
        w_qkv=p["w_qkv"][:, rank * c:(rank + 1) * c], b_qkv=p["b_qkv"][rank * c:(rank + 1) * c],
        w_o=p["w_o"][rank * o:(rank + 1) * o, :], b_o=p["b_o"],
        w1=p["w1"][:, rank * m:(rank + 1) * m], b1=p["b1"][rank * m:(rank + 1) * m],
        w2=p["w2"][rank * m:(rank + 1) * m, :], b2=p["b2"],
    )


def rank_attn_forward(pr: dict, x, local_heads: int, micro_batch: int = 1) -> dict:
    """Column-parallel QKV (+ its bias shard), causal attention over the local
    heads, row-parallel projection without bias -> partial [tokens, hidden]."""
    qkv = x @ pr["w_qkv"] + pr["b_qkv"]
    o, lse = L.attention_forward(qkv, local_heads, micro_batch)
    return dict(qkv=qkv, o=o, lse=lse, partial=o @ pr["w_o"])


def rank_mlp_forward(pr: dict, h) -> dict:
    """Column-parallel fc1 (+ bias shard) with GeLU, row-parallel fc2 without bias."""
    z = h @ pr["w1"] + pr["b1"]
    a = L.gelu(z)
    return dict(z=z, a=a, partial=a @ pr["w2"])


def reduce_partials(partials, bias=None, residual=None):
    """The all-reduce stand-in: sum of the t partials, plus the row-parallel bias
    once, plus an optional residual."""
    out = np.sum(np.stack(partials), axis=0)
    if bias is not None:
        out = out + bias
    if residual is not None:
        out = out + residual
    return out


def rank_mlp_backward(pr: dict, dy, h, z, a) -> dict:
    """Gradients of the rank's MLP share given dY (the full upstream gradient,
    which every rank holds): dz, dw2, dw1, db1, the dgrad partial dh_partial,
    and db2 = colsum(dY) (the same on every rank)."""
    da = dy @ pr["w2"].T
    dz = da * L.gelu_grad(z)
    return dict(dz=dz, dw2=a.T @ dy, dw1=h.T @ dz, db1=dz.sum(axis=0), dh_partial=dz @ pr["w1"].T,
                db2=dy.sum(axis=0))


def rank_attn_backward(pr: dict, dh, x, qkv, local_heads: int, micro_batch: int = 1) -> dict:
    """Gradients of the rank's attention share given dH (full, reduced): do,
    dw_o, db_o (= colsum(dH), the same on every rank), dqkv, dw_qkv, db_qkv and
    the dgrad partial dx_partial."""
    o, _ = L.attention_forward(qkv, local_heads, micro_batch)
    do = dh @ pr["w_o"].T
    dqkv = L.attention_backward(qkv, do, local_heads, micro_batch)
    return dict(do=do, dw_o=o.T @ dh, db_o=dh.sum(axis=0), dqkv=dqkv, dw_qkv=x.T @ dqkv,
                db_qkv=dqkv.sum(axis=0), dx_partial=dqkv @ pr["w_qkv"].T)


def sharded_layer(p: dict, x, g, heads: int, tp: int, micro_batch: int = 1, residual: bool = False) -> dict:
    """The whole layer computed as t rank shards plus four reductions (two
    forward, two backward).  Returns the reduced tensors (y, dx, h, dh) and the
    per-rank pieces (lists indexed by rank)."""
    h_dim = x.shape[1]
    f = p["w1"].shape[1]
    check_divisible(h_dim, heads, f, tp)
    lh = heads // tp
    prs = [shard_params(p, heads, tp, r) for r in range(tp)]
    att = [rank_attn_forward(pr, x, lh, micro_batch) for pr in prs]
    hh = reduce_partials([a["partial"] for a in att], p["b_o"], x if residual else None)
    mlp = [rank_mlp_forward(pr, hh) for pr in prs]
    y = reduce_partials([m["partial"] for m in mlp], p["b2"], hh if residual else None)
    mb = [rank_mlp_backward(pr, g, hh, m["z"], m["a"]) for pr, m in zip(prs, mlp)]
    dh = reduce_partials([m["dh_partial"] for m in mb], None, g if residual else None)
    ab = [rank_attn_backward(pr, dh, x, a["qkv"], lh, micro_batch) for pr, a in zip(prs, att)]
    dx = reduce_partials([a["dx_partial"] for a in ab], None, dh if residual else None)
    return dict(y=y, h=hh, dh=dh, dx=dx, att=att, mlp=mlp, mlp_bwd=mb, attn_bwd=ab)
