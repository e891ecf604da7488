"""Pin: the sharded view against the unsharded layer (fp64).  Tensor parallelism
only moves work: the sum of the row-parallel partials plus the bias equals the
unsharded output, and the column/head shards concatenate to the full QKV, Z, A
and the full weight gradients (the guide's semantic-alignment table: compare
parameters regrouped by logical parameter, forward outputs and gradients)."""
import numpy as np
import pytest

from oracle import layer as L
from oracle import shard as S
from tests.oracle_util import tiny_params, rel_err


@pytest.mark.parametrize("tp", [1, 2, 4])
@pytest.mark.parametrize("residual", [False, True])
def test_sharded_equals_unsharded(tp, residual):
    h, heads, f, seq, mb = 16, 4, 32, 7, 1
    p = tiny_params(h, f, seed=21, scale=0.4)
    rng = np.random.default_rng(22)
    x = rng.standard_normal((seq * mb, h))
    g = rng.standard_normal((seq * mb, h))
    full = L.layer_forward(p, x, heads, mb, residual)
    fb = L.layer_backward(p, x, full, g, heads, mb, residual)
    sh = S.sharded_layer(p, x, g, heads, tp, mb, residual)
    assert rel_err(sh["y"], full["y"]) < 1e-12
    assert rel_err(sh["h"], full["h"]) < 1e-12
    assert rel_err(sh["dh"], fb["dh"]) < 1e-12
    assert rel_err(sh["dx"], fb["dx"]) < 1e-12
    # column/head shards concatenate to the full tensors
    cat = lambda lst, key, axis=1: np.concatenate([e[key] for e in lst], axis=axis)
    assert rel_err(cat(sh["att"], "qkv"), full["qkv"]) < 1e-12
    assert rel_err(cat(sh["att"], "o"), full["o"]) < 1e-12
    assert rel_err(cat(sh["att"], "lse", 0), full["lse"]) < 1e-12
    assert rel_err(cat(sh["mlp"], "z"), full["z"]) < 1e-12
    assert rel_err(cat(sh["mlp"], "a"), full["a"]) < 1e-12
    assert rel_err(cat(sh["mlp_bwd"], "dz"), fb["dz"]) < 1e-12
    assert rel_err(cat(sh["mlp_bwd"], "dw1"), fb["dw1"]) < 1e-12
    assert rel_err(cat(sh["mlp_bwd"], "db1", 0), fb["db1"]) < 1e-12
    assert rel_err(cat(sh["mlp_bwd"], "dw2", 0), fb["dw2"]) < 1e-12
    assert rel_err(cat(sh["attn_bwd"], "dw_o", 0), fb["dw_o"]) < 1e-12
    assert rel_err(cat(sh["attn_bwd"], "dqkv"), fb["dqkv"]) < 1e-12
    assert rel_err(cat(sh["attn_bwd"], "dw_qkv"), fb["dw_qkv"]) < 1e-12
    assert rel_err(cat(sh["attn_bwd"], "db_qkv", 0), fb["db_qkv"]) < 1e-12
    for r in range(tp):  # row-parallel bias gradients are the same on every rank
        assert rel_err(sh["mlp_bwd"][r]["db2"], fb["db2"]) < 1e-12
        assert rel_err(sh["attn_bwd"][r]["db_o"], fb["db_o"]) < 1e-12


def test_partials_sum_needs_bias_once():
    """Adding the row-parallel bias on every rank (t copies) breaks the sum: the
    reading 'bias once, after the sum' is the one that reproduces the layer."""
    h, heads, f, seq, tp = 8, 2, 16, 4, 2
    p = tiny_params(h, f, seed=23)
    x = np.random.default_rng(24).standard_normal((seq, h))
    full = L.layer_forward(p, x, heads)
    prs = [S.shard_params(p, heads, tp, r) for r in range(tp)]
    parts = [S.rank_attn_forward(pr, x, heads // tp)["partial"] for pr in prs]
    assert rel_err(S.reduce_partials(parts, p["b_o"]), full["u"]) < 1e-12
    wrong = S.reduce_partials([q + p["b_o"] for q in parts])
    assert rel_err(wrong, full["u"]) > 1e-3
