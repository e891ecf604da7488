"""Pins of the router oracle (oracle/router.py) by things other than itself:

* central finite differences (fp64) of  sum(G * gates) + aux_loss  through
  the whole router -- logits, x and w_r -- with the routing held fixed (the
  test logits keep every top-k decision away from a tie, so the perturbations
  never change it);
* torch CPU autograd of the same loss built from torch's own softmax, gather
  and matmul;
* closed forms: perfectly balanced routing with equal logits gives
  aux_loss = alpha and no gradient from the loss; with k = E the gate gradient
  is the full softmax's backward (torch); the gate gradient of every token sums
  to zero (softmax is shift invariant).
A dropped term, a sign, a wrong normaliser (T, k or E) or a transposed operand
in the oracle fails one of them.
"""
import numpy as np
import pytest
import torch

from oracle import moe as M
from oracle import router as R

EPS = 1e-6
ALPHA = 0.001


def _problem(T=6, h=5, E=8, k=3, seed=0, alpha=ALPHA):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, h))
    w = rng.normal(size=(h, E))
    G = rng.normal(size=(T, k))
    logits = R.router_forward(x, w)
    srt = np.sort(logits, axis=1)
    assert np.min(np.diff(srt, axis=1)) > 1e-4  # no near-ties: the routing is stable under EPS
    idx, gates = M.route_topk(logits, k)
    return x, w, G, logits, idx, gates


def _loss_from_logits(l, idx, G, alpha):
    sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    gates = e / e.sum(axis=1, keepdims=True)
    return float(np.sum(G * gates) + R.aux_loss(l, idx, alpha))


def _fd(fn, arr):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + EPS
        up = fn()
        arr[i] = old - EPS
        dn = fn()
        arr[i] = old
        g[i] = (up - dn) / (2 * EPS)
    return g


@pytest.mark.parametrize("alpha", [ALPHA, 0.7])
def test_router_backward_matches_finite_differences(alpha):
    x, w, G, logits, idx, gates = _problem(alpha=alpha)
    bw = R.router_backward(x, w, logits, idx, gates, G, alpha)
    l = logits.copy()
    fd_l = _fd(lambda: _loss_from_logits(l, idx, G, alpha), l)
    assert np.max(np.abs(bw["dlogits"] - fd_l)) <= 1e-6 * max(1.0, np.max(np.abs(fd_l)))
    xx, ww = x.copy(), w.copy()
    fd_x = _fd(lambda: _loss_from_logits(xx @ ww, idx, G, alpha), xx)
    fd_w = _fd(lambda: _loss_from_logits(xx @ ww, idx, G, alpha), ww)
    assert np.max(np.abs(bw["dx"] - fd_x)) <= 1e-6 * max(1.0, np.max(np.abs(fd_x)))
    assert np.max(np.abs(bw["dw_r"] - fd_w)) <= 1e-6 * max(1.0, np.max(np.abs(fd_w)))


def test_router_matches_torch_autograd():
    T, h, E, k = 12, 7, 16, 4
    x, w, G, logits, idx, gates = _problem(T, h, E, k, seed=3)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    lt = xt @ wt
    it = torch.tensor(idx, dtype=torch.int64)
    g = torch.softmax(torch.gather(lt, 1, it), dim=1)
    counts = torch.bincount(it.reshape(-1), minlength=E).to(torch.float64)
    p = torch.softmax(lt, dim=1)
    aux = ALPHA * E * torch.sum(counts / (T * k) * p.mean(dim=0))
    (torch.sum(torch.tensor(G) * g) + aux).backward()
    bw = R.router_backward(x, w, logits, idx, gates, G, ALPHA)
    assert np.allclose(g.detach().numpy(), gates, rtol=0, atol=1e-15)
    assert abs(aux.item() - bw["aux"]) <= 1e-15
    assert np.allclose(xt.grad.numpy(), bw["dx"], rtol=1e-12, atol=1e-14)
    assert np.allclose(wt.grad.numpy(), bw["dw_r"], rtol=1e-12, atol=1e-14)


def test_balanced_routing_gives_alpha_and_no_loss_gradient():
    T, E, k = 8, 4, 2
    logits = np.zeros((T, E))
    # every expert gets exactly T*k/E assignments
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)], dtype=np.int32)
    assert np.all(R.expert_counts(idx, E) == T * k // E)
    assert R.aux_loss(logits, idx, 0.25) == pytest.approx(0.25, abs=1e-15)
    gates = np.full((T, k), 1.0 / k)
    bw = R.router_backward(np.ones((T, 3)), np.zeros((3, E)), logits, idx, gates, np.zeros((T, k)), 0.25)
    assert np.max(np.abs(bw["dlogits"])) == 0.0


def test_all_experts_selected_is_the_softmax_backward():
    T, E = 5, 6
    rng = np.random.default_rng(9)
    logits = rng.normal(size=(T, E))
    idx, gates = M.route_topk(logits, E)
    G = rng.normal(size=(T, E))
    bw = R.router_backward(np.eye(T), np.zeros((T, E)), logits, idx, gates, G, 0.0)
    lt = torch.tensor(logits, requires_grad=True)
    Gfull = np.zeros((T, E))
    np.put_along_axis(Gfull, idx.astype(np.int64), G, axis=1)
    (torch.softmax(lt, dim=1) * torch.tensor(Gfull)).sum().backward()
    assert np.allclose(bw["dlogits"], lt.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_gate_gradient_rows_sum_to_zero():
    x, w, G, logits, idx, gates = _problem(T=9, E=12, k=5, seed=4)
    bw = R.router_backward(x, w, logits, idx, gates, G, ALPHA)
    assert np.max(np.abs(bw["dlogits"].sum(axis=1))) <= 1e-15
