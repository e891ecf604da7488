"""fp64 oracle of one (unsharded) transformer layer: forward and backward.

Test infrastructure only (see the package docstring).

The layer is the five pieces the tutorial's section 2.2 describes for tensor
parallelism -- fused QKV projection, self-attention, output projection, first
MLP linear, second MLP linear -- with these readings where the pages are silent:

* attention is causal scaled dot-product attention, scale 1/sqrt(d), d = hidden/heads;
* the MLP activation is GeLU in its exact form z*Phi(z) (Phi = normal CDF);
* every linear has a bias; there is no LayerNorm and no dropout;
* residual connections are optional (``residual=True`` adds X to the
  projection output and H to the MLP output);
* the fused QKV columns are head-interleaved: column n*3d + j*d + i is head n,
  component j in (q, k, v), index i;
* activations are row-major [tokens, features] with rows ordered
  [micro-batch][sequence]; attention never crosses micro-batch elements.

Loss convention for the backward pass: L = sum(Y * G) with G = dL/dY given.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

SQRT2 = math.sqrt(2.0)
INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


# ----------------------------------------------------------------- GeLU
def normal_cdf(z):
    return 0.5 * (1.0 + erf(z / SQRT2))


def normal_pdf(z):
    return INV_SQRT_2PI * np.exp(-0.5 * z * z)


def gelu(z):
    """GeLU(z) = z * Phi(z)."""
    return z * normal_cdf(z)


def gelu_grad(z):
    """d/dz [z * Phi(z)] = Phi(z) + z * phi(z)."""
    return normal_cdf(z) + z * normal_pdf(z)


# ----------------------------------------------------------------- attention
def head_slices(heads: int, d: int, n: int):
    """Column ranges of head n's q, k, v inside the head-interleaved QKV tensor."""
    base = n * 3 * d
    return slice(base, base + d), slice(base + d, base + 2 * d), slice(base + 2 * d, base + 3 * d)


def causal_softmax(s):
    """Row softmax of s with entries above the diagonal (key j > query i) masked out.

    Returns (P, lse) where lse[i] = log sum_{j<=i} exp(s[i, j])."""
    n = s.shape[0]
    s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


def attention_forward(qkv, heads: int, micro_batch: int = 1):
    """Causal self-attention over every head of a head-interleaved QKV tensor.

    qkv: [tokens, 3*heads*d]. Returns O [tokens, heads*d] (heads concatenated in
    order) and lse [heads, tokens]."""
    tokens = qkv.shape[0]
    d = qkv.shape[1] // (3 * heads)
    seq = tokens // micro_batch
    o = np.zeros((tokens, heads * d))
    lse = np.zeros((heads, tokens))
    scale = 1.0 / math.sqrt(d)
    for b in range(micro_batch):
        rows = slice(b * seq, (b + 1) * seq)
        for n in range(heads):
            sq, sk, sv = head_slices(heads, d, n)
            q, k, v = qkv[rows, sq], qkv[rows, sk], qkv[rows, sv]
            p, l = causal_softmax((q @ k.T) * scale)
            o[rows, n * d:(n + 1) * d] = p @ v
            lse[n, rows] = l
    return o, lse


def attention_backward(qkv, do, heads: int, micro_batch: int = 1):
    """Gradient of causal attention w.r.t. the QKV tensor, given dO.

    Per head: dV = P^T dO; dP = dO V^T; dS = P * (dP - rowsum(dP * P));
    dQ = dS K * scale; dK = dS^T Q * scale.  rowsum(dP * P) equals
    rowsum(dO * O) because O = P V."""
    tokens = qkv.shape[0]
    d = qkv.shape[1] // (3 * heads)
    seq = tokens // micro_batch
    dqkv = np.zeros_like(qkv)
    scale = 1.0 / math.sqrt(d)
    for b in range(micro_batch):
        rows = slice(b * seq, (b + 1) * seq)
        for n in range(heads):
            sq, sk, sv = head_slices(heads, d, n)
            q, k, v = qkv[rows, sq], qkv[rows, sk], qkv[rows, sv]
            p, _ = causal_softmax((q @ k.T) * scale)
            g = do[rows, n * d:(n + 1) * d]
            dv = p.T @ g
            dp = g @ v.T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dqkv[rows, sq] = (ds @ k) * scale
            dqkv[rows, sk] = (ds.T @ q) * scale
            dqkv[rows, sv] = dv
    return dqkv


# ----------------------------------------------------------------- the layer
PARAM_NAMES = ("w_qkv", "b_qkv", "w_o", "b_o", "w1", "b1", "w2", "b2")


def layer_forward(p: dict, x, heads: int, micro_batch: int = 1, residual: bool = False) -> dict:
    """Forward pass. p holds w_qkv [h,3h], b_qkv [3h], w_o [h,h], b_o [h], w1 [h,f],
    b1 [f], w2 [f,h], b2 [h] (fp64); x is [tokens, h].  Returns every
    intermediate: qkv, o, lse, u, h, z, a, y."""
    qkv = x @ p["w_qkv"] + p["b_qkv"]
    o, lse = attention_forward(qkv, heads, micro_batch)
    u = o @ p["w_o"] + p["b_o"]
    h = u + x if residual else u
    z = h @ p["w1"] + p["b1"]
    a = gelu(z)
    y = a @ p["w2"] + p["b2"]
    if residual:
        y = y + h
    return dict(qkv=qkv, o=o, lse=lse, u=u, h=h, z=z, a=a, y=y)


def layer_backward(p: dict, x, fwd: dict, g, heads: int, micro_batch: int = 1, residual: bool = False) -> dict:
    """Backward pass for L = sum(Y * g).  Returns dx and the gradient of every
    parameter (dw_qkv, db_qkv, dw_o, db_o, dw1, db1, dw2, db2) plus the
    intermediate gradients da, dz, dh, do, dqkv."""
    dw2 = fwd["a"].T @ g
    db2 = g.sum(axis=0)
    da = g @ p["w2"].T
    dz = da * gelu_grad(fwd["z"])
    dw1 = fwd["h"].T @ dz
    db1 = dz.sum(axis=0)
    dh = dz @ p["w1"].T
    if residual:
        dh = dh + g
    dw_o = fwd["o"].T @ dh
    db_o = dh.sum(axis=0)
    do = dh @ p["w_o"].T
    dqkv = attention_backward(fwd["qkv"], do, heads, micro_batch)
    dw_qkv = x.T @ dqkv
    db_qkv = dqkv.sum(axis=0)
    dx = dqkv @ p["w_qkv"].T
    if residual:
        dx = dx + dh
    return dict(dx=dx, dw_qkv=dw_qkv, db_qkv=db_qkv, dw_o=dw_o, db_o=db_o, dw1=dw1, db1=db1,
                dw2=dw2, db2=db2, da=da, dz=dz, dh=dh, do=do, dqkv=dqkv)


def layer_flops(hidden: int, heads: int, ffn: int, tokens: int, micro_batch: int = 1, tp: int = 1) -> dict:
    """Algorithmic FLOP of one TP rank's share of the layer (2*M*N*K per GEMM;
    causal attention counts key j <= query i only, i.e. seq*(seq+1)/2 score
    entries per head; backward attention is twice forward).  Elementwise work is
    not counted."""
    s, h, f = tokens, hidden, ffn
    seq = tokens // micro_batch
    gemm_fwd = 2 * s * h * (3 * h // tp) + 2 * s * (h // tp) * h + 2 * s * h * (f // tp) + 2 * s * (f // tp) * h
    pairs = micro_batch * seq * (seq + 1) // 2
    attn_fwd = 2 * 2 * pairs * (h // tp)  # QK^T and PV
    return dict(gemm=3 * gemm_fwd, attention=3 * attn_fwd, total=3 * gemm_fwd + 3 * attn_fwd,
                gemm_fwd=gemm_fwd, attention_fwd=attn_fwd)
