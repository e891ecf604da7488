"""fp64 oracle of the MoE router: its linear, the backward of the gates into the
logits, and the load-balancing loss.

Test infrastructure only (see the package docstring).

The site summary's MoE deploy step (step 6) sets a top-8 router over 256
experts and `--moe-aux-loss-coeff 0.001`; the pages print no router or loss
formula.  The readings are:

* router linear: logits = x W_r in fp32 from bf16 operands, no bias,
  W_r [hidden, experts];
* routing and gates as in `oracle.moe.route_topk` (top-k of the logits, gates =
  softmax over the k selected logits); the gate backward is that softmax's
  backward: dl_j = g_j (dg_j - sum_i g_i dg_i) for selected j, 0 elsewhere;
* load-balancing loss, the Switch Transformer form (Fedus, Zoph and Shazeer,
  2021) with the assignment fraction taken over all T*k assignments:
      L = alpha * E * sum_e f_e P_e,  f_e = c_e / (T k),
      P_e = (1/T) sum_t softmax(logits_t)_e  (over all E experts),
  where c_e counts the assignments routed to expert e and is a constant of the
  backward (routing is not differentiable).  Balanced routing with uniform
  probabilities gives L = alpha exactly.
"""
from __future__ import annotations

import numpy as np


def softmax_rows(logits):
    """Row softmax over the last axis (max-subtracted), fp64."""
    l = np.asarray(logits, dtype=np.float64)
    e = np.exp(l - l.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def router_forward(x, w_r):
    """logits [T, E] = x [T, h] . w_r [h, E]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64)


def expert_counts(idx, experts: int):
    """Assignments per expert over all tokens and slots: c_e, int64 [E]."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=experts).astype(np.int64)


def aux_loss(logits, idx, coeff: float) -> float:
    """The load-balancing loss alpha * E * sum_e f_e P_e."""
    T, E = np.shape(logits)
    k = np.shape(idx)[1]
    f = expert_counts(idx, E) / (T * k)
    P = softmax_rows(logits).mean(axis=0)
    return float(coeff * E * np.sum(f * P))


def router_backward(x, w_r, logits, idx, gates, dgates, coeff: float) -> dict:
    """Gradients of  sum(dgates * gates) + aux_loss(logits)  (dgates the
    upstream gradient of the gates, idx and the counts held fixed):
    dlogits [T, E], dw_r = x^T dlogits [h, E], dx = dlogits w_r^T [T, h], and
    the loss value aux."""
    logits = np.asarray(logits, dtype=np.float64)
    gates = np.asarray(gates, dtype=np.float64)
    dgates = np.asarray(dgates, dtype=np.float64)
    T, E = logits.shape
    k = np.shape(idx)[1]
    # backward of the softmax over the selected logits
    inner = np.sum(gates * dgates, axis=1, keepdims=True)
    dl = np.zeros_like(logits)
    np.put_along_axis(dl, np.asarray(idx, dtype=np.int64), gates * (dgates - inner), axis=1)
    # backward of the load-balancing loss through the full softmax
    c = expert_counts(idx, E).astype(np.float64)
    p = softmax_rows(logits)
    q = np.sum(p * c, axis=1, keepdims=True)
    dl += coeff * E / (T * T * k) * p * (c - q)
    x = np.asarray(x, dtype=np.float64)
    w_r = np.asarray(w_r, dtype=np.float64)
    return dict(dlogits=dl, dw_r=x.T @ dl, dx=dl @ w_r.T, aux=aux_loss(logits, idx, coeff))
