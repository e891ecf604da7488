"""fp64 oracle of one expert-parallel rank's MoE expert block.

Test infrastructure only (see the package docstring).

The site summary's MoE deploy step (step 6) fixes 256 experts, a top-8 router
and expert-parallel size 16; the guide's table of parallel strategies names
grouped GEMM as the MoE compute lever and its performance section asks for the
per-expert token distribution and the drop/capacity policy.  The pages print no
router formula, so the readings are:

* routing: the k experts with the largest fp32 logits, ties to the lower expert
  id, listed in slot order of decreasing logit;
* gates: softmax over the k selected logits;
* dropless (no capacity limit);
* rank r of ep holds experts [r*E/ep, (r+1)*E/ep) contiguously;
* the rank's assignments (token, slot) whose expert is local are grouped by
  expert, tokens ascending within an expert (a stable sort of the flattened
  (token, slot) list by expert id);
* expert MLP: GeLU(x W1_e) W2_e with no biases; the output row is scaled by its
  gate and a token's local outputs are summed in slot order (the rank's partial
  of the combine; the other ranks' experts arrive by all-to-all, which is not
  modelled).
"""
from __future__ import annotations

import numpy as np

from . import layer as L


def route_topk(logits, k: int):
    """Top-k expert ids per token (descending logit, ties -> lower id) and the
    softmax gates over the selected logits.  logits: [T, E] fp32.
    Returns (idx int32 [T, k], gates fp64 [T, k]).

    Non-finite logits follow the order of numpy's stable sort of the negated
    row: +inf first, -inf below every finite value, NaN below -inf (ties among
    NaNs and between -0 and +0 to the lower id).  A NaN among the selected
    logits, or a selection of only infinities of one sign, makes that row's
    gates NaN."""
    logits = np.asarray(logits)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    return order.astype(np.int32), e / e.sum(axis=1, keepdims=True)


def local_range(experts: int, ep: int, rank: int):
    n = experts // ep
    return rank * n, (rank + 1) * n


def permute(idx, experts: int, ep: int, rank: int):
    """Group the rank's local assignments by expert.

    Returns counts [E/ep], offsets [E/ep + 1] (exclusive prefix sum),
    perm_token [N] and perm_slot [N] (all int32), where N = offsets[-1]."""
    lo, hi = local_range(experts, ep, rank)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    tok = np.repeat(np.arange(T), k)
    slot = np.tile(np.arange(k), T)
    mine = (flat >= lo) & (flat < hi)
    e_loc = flat[mine] - lo
    order = np.argsort(e_loc, kind="stable")
    counts = np.bincount(e_loc, minlength=hi - lo).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return counts, offsets, tok[mine][order].astype(np.int32), slot[mine][order].astype(np.int32)


def expert_forward(x, w1, w2, offsets, perm_token):
    """Per-assignment expert MLP without gate: returns xp, z, a, ye (each [N, .]).
    w1: [E_local, h, f], w2: [E_local, f, h] (fp64)."""
    xp = x[perm_token]
    f = w1.shape[2]
    n = xp.shape[0]
    z = np.zeros((n, f))
    ye = np.zeros((n, x.shape[1]))
    for e in range(w1.shape[0]):
        r = slice(offsets[e], offsets[e + 1])
        z[r] = xp[r] @ w1[e]
    a = L.gelu(z)
    for e in range(w1.shape[0]):
        r = slice(offsets[e], offsets[e + 1])
        ye[r] = a[r] @ w2[e]
    return dict(xp=xp, z=z, a=a, ye=ye)


def combine(ye, gates, perm_token, perm_slot, tokens: int):
    """Y_t = sum over the rank's slots s of token t (ascending s) of g[t, s] * ye."""
    y = np.zeros((tokens, ye.shape[1]))
    order = np.lexsort((perm_slot, perm_token))  # by token, then slot
    for i in order:
        t, s = perm_token[i], perm_slot[i]
        y[t] += gates[t, s] * ye[i]
    return y


def moe_forward(x, w1, w2, logits, k: int, ep: int, rank: int) -> dict:
    experts = logits.shape[1]
    idx, gates = route_topk(logits, k)
    counts, offsets, ptok, pslot = permute(idx, experts, ep, rank)
    f = expert_forward(x, w1, w2, offsets, ptok)
    y = combine(f["ye"], gates, ptok, pslot, x.shape[0])
    return dict(idx=idx, gates=gates, counts=counts, offsets=offsets, perm_token=ptok, perm_slot=pslot, y=y, **f)


def moe_backward(x, w1, w2, fwd: dict, dy) -> dict:
    """Backward of the rank's partial Y given dY.  Returns dx [T, h] (the rank's
    partial), dw1, dw2 [E_local, ...], and dgates [T, k] (zero on slots whose
    expert is not local).  The gradient through the gate softmax into the
    logits is not part of this block."""
    ptok, pslot, offsets = fwd["perm_token"], fwd["perm_slot"], fwd["offsets"]
    g = fwd["gates"][ptok, pslot][:, None]
    dye = g * dy[ptok]
    dgates = np.zeros_like(fwd["gates"])
    dgates[ptok, pslot] = np.sum(fwd["ye"] * dy[ptok], axis=1)
    dw1 = np.zeros_like(w1)
    dw2 = np.zeros_like(w2)
    dxp = np.zeros_like(fwd["xp"])
    for e in range(w1.shape[0]):
        r = slice(offsets[e], offsets[e + 1])
        da = dye[r] @ w2[e].T
        dz = da * L.gelu_grad(fwd["z"][r])
        dw2[e] = fwd["a"][r].T @ dye[r]
        dw1[e] = fwd["xp"][r].T @ dz
        dxp[r] = dz @ w1[e].T
    dx = np.zeros_like(x)
    order = np.lexsort((pslot, ptok))
    for i in order:
        dx[ptok[i]] += dxp[i]
    return dict(dx=dx, dw1=dw1, dw2=dw2, dgates=dgates, dye=dye, dxp=dxp)


def moe_flops(counts, hidden: int, ffn: int) -> int:
    """Algorithmic FLOP of the rank's grouped GEMMs, forward + backward (12*N*h*f)."""
    return int(12 * int(np.sum(counts)) * hidden * ffn)
