"""Pin: the oracle's hand-written backward against central finite differences of
its forward (fp64, eps=1e-6, relative error <= 1e-6), for every input, weight and
bias, on tiny shapes.  Any dropped term, sign or transposed operand in a backward
formula fails here."""
import numpy as np
import pytest

from oracle import layer as L
from oracle import moe as M
from oracle import shard as S
from tests.oracle_util import tiny_params, rel_err

EPS = 1e-6


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


@pytest.mark.parametrize("residual", [False, True])
@pytest.mark.parametrize("mb", [1, 2])
def test_layer_backward_matches_finite_differences(residual, mb):
    h, heads, f, seq = 8, 2, 16, 5
    p = tiny_params(h, f, seed=3)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((seq * mb, h))
    g = rng.standard_normal((seq * mb, h))

    def loss():
        return float(np.sum(L.layer_forward(p, x, heads, mb, residual)["y"] * g))

    fwd = L.layer_forward(p, x, heads, mb, residual)
    grads = L.layer_backward(p, x, fwd, g, heads, mb, residual)
    for name in L.PARAM_NAMES:
        num = _fd(loss, p[name])
        assert rel_err(grads["d" + name], num) < 1e-6, name
    assert rel_err(grads["dx"], _fd(loss, x)) < 1e-6


def test_attention_backward_matches_finite_differences():
    heads, d, seq = 3, 4, 6
    rng = np.random.default_rng(5)
    qkv = rng.standard_normal((seq, 3 * heads * d))
    do = rng.standard_normal((seq, heads * d))

    def loss():
        return float(np.sum(L.attention_forward(qkv, heads)[0] * do))

    assert rel_err(L.attention_backward(qkv, do, heads), _fd(loss, qkv)) < 1e-6


@pytest.mark.parametrize("tp", [1, 2])
def test_rank_backward_matches_finite_differences(tp):
    """The sharded view's per-rank gradients are the gradients of the rank's own
    share of the loss (its partial contribution), checked per rank."""
    h, heads, f, seq = 8, 2, 16, 5
    p = tiny_params(h, f, seed=6)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((seq, h))
    hh = rng.standard_normal((seq, h))
    g = rng.standard_normal((seq, h))
    for r in range(tp):
        pr = {k: v.copy() for k, v in S.shard_params(p, heads, tp, r).items()}

        def mlp_loss():
            return float(np.sum(S.rank_mlp_forward(pr, hh)["partial"] * g))

        fw = S.rank_mlp_forward(pr, hh)
        bw = S.rank_mlp_backward(pr, g, hh, fw["z"], fw["a"])
        assert rel_err(bw["dw1"], _fd(mlp_loss, pr["w1"])) < 1e-6
        assert rel_err(bw["db1"], _fd(mlp_loss, pr["b1"])) < 1e-6
        assert rel_err(bw["dw2"], _fd(mlp_loss, pr["w2"])) < 1e-6
        assert rel_err(bw["dh_partial"], _fd(mlp_loss, hh)) < 1e-6

        def attn_loss():
            return float(np.sum(S.rank_attn_forward(pr, x, heads // tp)["partial"] * g))

        fa = S.rank_attn_forward(pr, x, heads // tp)
        ba = S.rank_attn_backward(pr, g, x, fa["qkv"], heads // tp)
        assert rel_err(ba["dw_qkv"], _fd(attn_loss, pr["w_qkv"])) < 1e-6
        assert rel_err(ba["db_qkv"], _fd(attn_loss, pr["b_qkv"])) < 1e-6
        assert rel_err(ba["dw_o"], _fd(attn_loss, pr["w_o"])) < 1e-6
        assert rel_err(ba["dx_partial"], _fd(attn_loss, x)) < 1e-6


def test_moe_backward_matches_finite_differences():
    T, h, f, E, k = 6, 4, 6, 4, 2
    rng = np.random.default_rng(8)
    x = rng.standard_normal((T, h))
    w1 = rng.standard_normal((E // 2, h, f)) * 0.5
    w2 = rng.standard_normal((E // 2, f, h)) * 0.5
    logits = rng.standard_normal((T, E)).astype(np.float32)
    dy = rng.standard_normal((T, h))
    fwd = M.moe_forward(x, w1, w2, logits, k, ep=2, rank=0)
    assert fwd["offsets"][-1] > 0
    bwd = M.moe_backward(x, w1, w2, fwd, dy)

    def loss():
        return float(np.sum(M.moe_forward(x, w1, w2, logits, k, ep=2, rank=0)["y"] * dy))

    assert rel_err(bwd["dx"], _fd(loss, x)) < 1e-6
    assert rel_err(bwd["dw1"], _fd(loss, w1)) < 1e-6
    assert rel_err(bwd["dw2"], _fd(loss, w2)) < 1e-6

    # dgates: perturb the gate values themselves (routing held fixed)
    gates = fwd["gates"].copy()

    def gate_loss():
        y = M.combine(fwd["ye"], gates, fwd["perm_token"], fwd["perm_slot"], T)
        return float(np.sum(y * dy))

    num = _fd(gate_loss, gates)
    assert rel_err(bwd["dgates"], num) < 1e-6
