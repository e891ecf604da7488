"""Seeded synthetic inputs for one transformer layer's tensor-parallel shard.

Shared by the tests, ``__graft_entry__.smoke()`` and ``bench.py``.  This module
draws random numbers, rounds them once to bfloat16 and cuts them into shards; it
holds none of the layer's arithmetic.

Recipe (the same for every workload):

* Each tensor is drawn from its own PCG64 stream keyed ``[seed, tensor id,
  granule]``.  A tensor that is split across tensor-parallel ranks is drawn in
  *granules* along its split axis (one attention head for the QKV weight and
  bias and for the output-projection rows; ``gcd(ffn, 64)`` equal column/row
  blocks for the MLP), so a rank's shard can be drawn on its own and its values
  never depend on the TP degree.
* Activations and upstream gradients are N(0, 1); weights and biases are
  N(0, 0.02).  Draws are fp64 and are rounded once, round-to-nearest-even, to
  bfloat16; both the oracle and the device consume the same bits.
* The fused QKV weight is head-interleaved: columns ``[n*3d, (n+1)*3d)`` hold
  head n's query, key and value projections in that order, so a rank's column
  shard is one contiguous block of whole heads.
* MoE router logits are ``log w_e + Gumbel(0, 1)`` in fp32 with Zipf weights
  ``w_e = (e+1)^-1.1``; top-k of such logits is weighted sampling of k distinct
  experts without replacement (the Gumbel-max trick).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Stream identifiers; changing one changes that tensor's values.
_TID = {
    "x": 1, "w_qkv": 2, "b_qkv": 3, "w_o": 4, "b_o": 5, "w1": 6, "b1": 7,
    "w2": 8, "b2": 9, "dy": 10, "h": 11, "dh": 12,
    "moe_x": 20, "moe_w1": 21, "moe_w2": 22, "moe_dy": 23, "moe_gumbel": 24, "moe_wr": 25, "moe_dgates": 26,
    "cp_qkv": 27, "cp_dout": 28, "mx_a": 29, "mx_b": 30,
}

WEIGHT_STD = 0.02


# ---------------------------------------------------------------- bfloat16 bits
def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values once, to nearest-even, to bfloat16; return the bit patterns (uint16).

    ``frexp`` gives x = m * 2^e with 0.5 <= |m| < 1; bfloat16 keeps 8 significant
    bits, so ``rint(x * 2^(8-e))`` (ties to even) is the rounded significand.
    Every step is exact in fp64.  Below bf16's smallest normal the spacing is
    that of the subnormals; values past the largest finite bf16 become
    infinities."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)  # below 2^-126 the spacing is fixed (subnormals)
    y = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    with np.errstate(over="ignore"):
        f32 = y.astype(np.float32)  # exact, or +-inf past the largest bf16
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------- shapes
@dataclass(frozen=True)
class LayerShape:
    hidden: int
    heads: int
    ffn: int
    seq: int
    micro_batch: int = 1
    tp: int = 1

    @property
    def tokens(self) -> int:
        return self.seq * self.micro_batch

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads


@dataclass(frozen=True)
class MoeShape:
    tokens: int
    hidden: int
    ffn: int
    experts: int
    topk: int
    ep: int
    zipf_s: float = 1.1


# The workloads: a GPT-2-small layer split two ways (both shards on one device),
# one rank of a 7B-class layer at TP=4, one rank of a 96-layer-GPT-shaped layer
# at TP=8, one expert-parallel rank of a 256-expert top-8 MoE layer, and the fp8
# variant of the 7B-class rank.
WORKLOADS = {
    "gpt2-small-tp2": LayerShape(hidden=768, heads=12, ffn=3072, seq=512, micro_batch=1, tp=2),
    "7b-tp4": LayerShape(hidden=4096, heads=32, ffn=16384, seq=4096, micro_batch=1, tp=4),
    "gpt96l-tp8": LayerShape(hidden=8192, heads=64, ffn=32768, seq=4096, micro_batch=1, tp=8),
}
# One context-parallel rank's attention share: the local heads of the 7B-class
# rank (8 heads of 128) over a 32768-token sequence cut into 4 chunks.
@dataclass(frozen=True)
class CpShape:
    seq: int
    heads: int
    head_dim: int
    cp: int

    @property
    def chunk(self) -> int:
        return self.seq // self.cp


CP_WORKLOADS = {
    "cp4-seq32k-7b-tp4": CpShape(seq=32768, heads=8, head_dim=128, cp=4),
}
# A GEMM of the 7B-class TP=4 rank in MXFP4 or MXFP6: the fc1 forward, tokens x
# hidden times hidden x local ffn (4096 x 4096 x 4096).
@dataclass(frozen=True)
class MxShape:
    M: int
    N: int
    K: int
    elem: str = "e2m1"  # MXFP4; "e2m3" for MXFP6


MX_WORKLOADS = {
    "mxfp4-gemm-7b-tp4": MxShape(M=4096, N=4096, K=4096),
    "mxfp6-gemm-7b-tp4": MxShape(M=4096, N=4096, K=4096, elem="e2m3"),
}
MOE_WORKLOADS = {
    "moe-256e-top8-ep16": MoeShape(tokens=4096, hidden=7168, ffn=18432, experts=256, topk=8, ep=16),
}


# ---------------------------------------------------------------- draws
def _normal(seed: int, name: str, granule: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng([seed, _TID[name], granule])
    return rng.standard_normal(shape) * std


def _ffn_granules(ffn: int) -> int:
    return math.gcd(ffn, 64)


def _granules(shape: LayerShape, name: str) -> int:
    if name in ("w_qkv", "b_qkv", "w_o"):
        return shape.heads
    if name in ("w1", "b1", "w2"):
        return _ffn_granules(shape.ffn)
    return 1


def _draw_granules(shape: LayerShape, name: str, seed: int, lo: int, hi: int) -> np.ndarray:
    """fp64 values of granules [lo, hi) of tensor ``name``, concatenated on its split axis."""
    h, f, d = shape.hidden, shape.ffn, shape.head_dim
    g = _granules(shape, name)
    parts = []
    for i in range(lo, hi):
        if name == "w_qkv":
            parts.append(_normal(seed, name, i, (h, 3 * d), WEIGHT_STD))
        elif name == "b_qkv":
            parts.append(_normal(seed, name, i, (3 * d,), WEIGHT_STD))
        elif name == "w_o":
            parts.append(_normal(seed, name, i, (d, h), WEIGHT_STD))
        elif name == "w1":
            parts.append(_normal(seed, name, i, (h, f // g), WEIGHT_STD))
        elif name == "b1":
            parts.append(_normal(seed, name, i, (f // g,), WEIGHT_STD))
        elif name == "w2":
            parts.append(_normal(seed, name, i, (f // g, h), WEIGHT_STD))
        else:
            raise KeyError(name)
    axis = 1 if name in ("w_qkv", "w1") else 0
    return np.concatenate(parts, axis=axis)


_SPLIT = ("w_qkv", "b_qkv", "w_o", "w1", "b1", "w2")


def layer_tensor(shape: LayerShape, name: str, seed: int = 0, tp: int = 1, rank: int = 0) -> np.ndarray:
    """bf16 bits of one layer tensor, or of rank ``rank``'s shard of it when ``tp > 1``.

    Names: x, dy, h, dh ([tokens, hidden], N(0,1)); w_qkv [hidden, 3*hidden]; b_qkv
    [3*hidden]; w_o [hidden, hidden]; b_o [hidden]; w1 [hidden, ffn]; b1 [ffn];
    w2 [ffn, hidden]; b2 [hidden].  Column-parallel tensors (w_qkv, b_qkv, w1, b1)
    are split on their last axis, row-parallel ones (w_o, w2) on their first;
    x, dy, h, dh, b_o, b2 are not split."""
    h = shape.hidden
    if name in ("x", "dy", "h", "dh"):
        return bf16_round_bits(_normal(seed, name, 0, (shape.tokens, h), 1.0))
    if name in ("b_o", "b2"):
        return bf16_round_bits(_normal(seed, name, 0, (h,), WEIGHT_STD))
    if name not in _SPLIT:
        raise KeyError(name)
    g = _granules(shape, name)
    if g % tp != 0:
        full = _draw_granules(shape, name, seed, 0, g)
        axis = 1 if name in ("w_qkv", "w1") else 0
        n = full.shape[axis] // tp
        sl = [slice(None)] * full.ndim
        sl[axis] = slice(rank * n, (rank + 1) * n)
        return bf16_round_bits(full[tuple(sl)])
    per = g // tp
    return bf16_round_bits(_draw_granules(shape, name, seed, rank * per, (rank + 1) * per))


LAYER_NAMES = ("x", "w_qkv", "b_qkv", "w_o", "b_o", "w1", "b1", "w2", "b2", "dy")


def layer_inputs(shape: LayerShape, seed: int = 0, tp: int = 1, rank: int = 0, names=LAYER_NAMES) -> dict:
    """bf16 bits of every layer input (the rank's shard where split)."""
    return {n: layer_tensor(shape, n, seed, tp, rank) for n in names}


# ---------------------------------------------------------------- CP inputs
CP_QKV_STD = WEIGHT_STD * 64.0  # x ~ N(0,1) through a N(0, 0.02) projection over 4096 inputs


def cp_qkv(shape: CpShape, seed: int = 0) -> np.ndarray:
    """bf16 bits of the whole sequence's head-interleaved QKV [seq, 3*heads*d],
    N(0, CP_QKV_STD) (the spread of a QKV projection of N(0,1) activations);
    chunk j is rows [j*C, (j+1)*C).  Drawn per 4096-row granule."""
    from concurrent.futures import ThreadPoolExecutor
    width = 3 * shape.heads * shape.head_dim
    g = 4096
    out = np.empty((shape.seq, width), dtype=np.uint16)

    def fill(i):
        rows = min(g, shape.seq - i * g)
        out[i * g:i * g + rows] = bf16_round_bits(_normal(seed, "cp_qkv", i, (rows, width), CP_QKV_STD))

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(fill, range((shape.seq + g - 1) // g)))
    return out


def cp_dout(shape: CpShape, seed: int = 0) -> np.ndarray:
    """bf16 bits of one rank's output gradient dO [chunk, heads*d], N(0,1)."""
    return bf16_round_bits(_normal(seed, "cp_dout", 0, (shape.chunk, shape.heads * shape.head_dim), 1.0))


# ---------------------------------------------------------------- MXFP4 GEMM inputs
def mx_operand(rows: int, cols: int, name: str, std: float, seed: int = 0) -> np.ndarray:
    """bf16 bits of a K-contiguous GEMM operand [rows, cols] (name mx_a: the
    activations, N(0,1); mx_b: a weight stored [out, in], N(0, WEIGHT_STD)),
    drawn per 1024-row granule."""
    g = 1024
    out = np.empty((rows, cols), dtype=np.uint16)
    for i in range((rows + g - 1) // g):
        r = min(g, rows - i * g)
        out[i * g:i * g + r] = bf16_round_bits(_normal(seed, name, i, (r, cols), std))
    return out


# ---------------------------------------------------------------- MoE inputs
def moe_logits(shape: MoeShape, seed: int = 0) -> np.ndarray:
    """fp32 router logits [tokens, experts] = log(Zipf weight) + Gumbel(0,1)."""
    rng = np.random.default_rng([seed, _TID["moe_gumbel"], 0])
    u = rng.random((shape.tokens, shape.experts))
    gumbel = -np.log(-np.log(np.clip(u, 1e-300, None)))
    logw = -shape.zipf_s * np.log(np.arange(1, shape.experts + 1, dtype=np.float64))
    return (logw[None, :] + gumbel).astype(np.float32)


def moe_tokens(shape: MoeShape, seed: int = 0, name: str = "moe_x") -> np.ndarray:
    """bf16 bits of token activations (moe_x) or upstream gradient (moe_dy), [tokens, hidden], N(0,1)."""
    return bf16_round_bits(_normal(seed, name, 0, (shape.tokens, shape.hidden), 1.0))


def moe_expert_weight(shape: MoeShape, name: str, expert: int, seed: int = 0) -> np.ndarray:
    """bf16 bits of one expert's fc1 ([hidden, ffn], name moe_w1) or fc2 ([ffn, hidden], moe_w2) weight."""
    if name == "moe_w1":
        shp = (shape.hidden, shape.ffn)
    elif name == "moe_w2":
        shp = (shape.ffn, shape.hidden)
    else:
        raise KeyError(name)
    return bf16_round_bits(_normal(seed, name, expert, shp, WEIGHT_STD))


def router_weight(shape: MoeShape, seed: int = 0) -> np.ndarray:
    """bf16 bits of the router's weight [hidden, experts], N(0, WEIGHT_STD)."""
    return bf16_round_bits(_normal(seed, "moe_wr", 0, (shape.hidden, shape.experts), WEIGHT_STD))


def gate_grads(shape: MoeShape, seed: int = 0) -> np.ndarray:
    """fp32 upstream gradients of the gates [tokens, topk], N(0, 1)."""
    return _normal(seed, "moe_dgates", 0, (shape.tokens, shape.topk), 1.0).astype(np.float32)


def moe_expert_weight_device(shape: MoeShape, name: str, expert: int, seed: int = 0, device="cuda"):
    """A full-size expert weight drawn on the device (torch's Philox generator),
    N(0, WEIGHT_STD) rounded to bf16: a fast stand-in for experts whose values
    no check reads.  Not the numbers of moe_expert_weight."""
    import torch
    if name == "moe_w1":
        shp = (shape.hidden, shape.ffn)
    elif name == "moe_w2":
        shp = (shape.ffn, shape.hidden)
    else:
        raise KeyError(name)
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + _TID[name]) * 4099 + expert)
    return (torch.randn(shp, generator=g, device=device, dtype=torch.float32) * WEIGHT_STD).to(torch.bfloat16)
