"""Pin: the oracle against independent library routines in torch CPU fp64 --
``scaled_dot_product_attention(is_causal=True)`` for the attention core,
``gelu(approximate='none')`` for the activation, and torch autograd through a
composition of library ops for every gradient."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import layer as L
from tests.oracle_util import tiny_params, rel_err


def _torch_layer(p, x, heads, mb, residual):
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tokens, h = x.shape
    d = h // heads
    seq = tokens // mb
    qkv = F.linear(xt, t["w_qkv"].T, t["b_qkv"])
    # head-interleaved columns: [tokens, heads, 3, d]
    q4 = qkv.view(mb, seq, heads, 3, d)
    q, k, v = (q4[:, :, :, j, :].permute(0, 2, 1, 3) for j in range(3))
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    o = o.permute(0, 2, 1, 3).reshape(tokens, h)
    u = F.linear(o, t["w_o"].T, t["b_o"])
    hh = u + xt if residual else u
    a = F.gelu(F.linear(hh, t["w1"].T, t["b1"]), approximate="none")
    y = F.linear(a, t["w2"].T, t["b2"])
    if residual:
        y = y + hh
    return t, xt, y


@pytest.mark.parametrize("residual", [False, True])
@pytest.mark.parametrize("mb,heads,h,f,seq", [(1, 4, 32, 48, 33), (2, 2, 16, 64, 9), (1, 3, 24, 24, 1)])
def test_layer_matches_torch_library(residual, mb, heads, h, f, seq):
    p = tiny_params(h, f, seed=11, scale=0.3)
    rng = np.random.default_rng(12)
    x = rng.standard_normal((mb * seq, h))
    g = rng.standard_normal((mb * seq, h))
    fwd = L.layer_forward(p, x, heads, mb, residual)
    grads = L.layer_backward(p, x, fwd, g, heads, mb, residual)
    t, xt, y = _torch_layer(p, x, heads, mb, residual)
    assert rel_err(fwd["y"], y.detach().numpy()) < 1e-12
    (y * torch.tensor(g)).sum().backward()
    for name in L.PARAM_NAMES:
        assert rel_err(grads["d" + name], t[name].grad.numpy()) < 1e-10, name
    assert rel_err(grads["dx"], xt.grad.numpy()) < 1e-10


def test_gelu_matches_torch_library():
    z = np.linspace(-8, 8, 4001)
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    gt = F.gelu(zt, approximate="none")
    gt.sum().backward()
    assert np.max(np.abs(L.gelu(z) - gt.detach().numpy())) < 1e-15
    assert np.max(np.abs(L.gelu_grad(z) - zt.grad.numpy())) < 1e-14


def test_lse_matches_torch_logsumexp():
    rng = np.random.default_rng(13)
    s = rng.standard_normal((7, 7)) * 3
    _, lse = L.causal_softmax(s)
    mask = torch.tril(torch.ones(7, 7, dtype=torch.bool))
    ref = torch.logsumexp(torch.tensor(s).masked_fill(~mask, float("-inf")), dim=1).numpy()
    assert np.max(np.abs(lse - ref)) < 1e-13
