"""Pin: special cases where the oracle must reduce to something known exactly."""
import json
import math
import os

import numpy as np
import pytest

from oracle import layer as L
from oracle import moe as M
from oracle import shard as S
from tests.oracle_util import tiny_params, rel_err

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_single_token_attention_returns_v():
    rng = np.random.default_rng(31)
    heads, d = 3, 5
    qkv = rng.standard_normal((1, 3 * heads * d))
    o, lse = L.attention_forward(qkv, heads)
    for n in range(heads):
        _, _, sv = L.head_slices(heads, d, n)
        assert np.array_equal(o[0, n * d:(n + 1) * d], qkv[0, sv])
        # lse of a single score is the score itself
        sq, sk, _ = L.head_slices(heads, d, n)
        assert abs(lse[n, 0] - qkv[0, sq] @ qkv[0, sk] / math.sqrt(d)) < 1e-14


def test_zero_query_gives_prefix_mean_of_v():
    rng = np.random.default_rng(32)
    heads, d, seq = 2, 4, 9
    qkv = rng.standard_normal((seq, 3 * heads * d))
    for n in range(heads):
        sq, _, _ = L.head_slices(heads, d, n)
        qkv[:, sq] = 0.0
    o, lse = L.attention_forward(qkv, heads)
    for n in range(heads):
        _, _, sv = L.head_slices(heads, d, n)
        v = qkv[:, sv]
        prefix_mean = np.cumsum(v, axis=0) / np.arange(1, seq + 1)[:, None]
        assert rel_err(o[:, n * d:(n + 1) * d], prefix_mean) < 1e-14
        assert np.max(np.abs(lse[n] - np.log(np.arange(1, seq + 1)))) < 1e-14


def test_first_row_attends_only_to_itself_and_future_keys_do_not_matter():
    rng = np.random.default_rng(33)
    heads, d, seq = 2, 4, 6
    qkv = rng.standard_normal((seq, 3 * heads * d))
    o1, _ = L.attention_forward(qkv, heads)
    qkv2 = qkv.copy()
    qkv2[3:] = rng.standard_normal((seq - 3, 3 * heads * d))  # change rows >= 3
    o2, _ = L.attention_forward(qkv2, heads)
    assert np.array_equal(o1[:3], o2[:3])  # causality
    for n in range(heads):
        _, _, sv = L.head_slices(heads, d, n)
        assert np.allclose(o1[0, n * d:(n + 1) * d], qkv[0, sv], rtol=0, atol=1e-15)


def test_gelu_closed_forms():
    # Phi(1) = 0.8413447460685429..., phi(1) = 0.24197072451914337...
    assert L.gelu(0.0) == 0.0
    assert L.gelu_grad(0.0) == 0.5
    assert abs(L.gelu(1.0) - 0.8413447460685429) < 1e-15
    assert abs(L.gelu(-1.0) + 0.15865525393145707) < 1e-15
    assert abs(L.gelu_grad(1.0) - (0.8413447460685429 + 0.24197072451914337)) < 1e-15
    assert abs(L.gelu(10.0) - 10.0) < 1e-15 and abs(L.gelu(-10.0)) < 1e-20


def test_tp1_is_the_plain_layer():
    h, heads, f = 8, 2, 16
    p = tiny_params(h, f, seed=34)
    x = np.random.default_rng(35).standard_normal((5, h))
    pr = S.shard_params(p, heads, 1, 0)
    for k in p:
        assert np.array_equal(pr[k], p[k])
    a = S.rank_attn_forward(pr, x, heads)
    assert rel_err(a["partial"] + p["b_o"], L.layer_forward(p, x, heads)["u"]) < 1e-14


def test_moe_single_expert_is_dense_mlp_without_bias():
    rng = np.random.default_rng(36)
    T, h, f = 7, 6, 10
    x = rng.standard_normal((T, h))
    w1 = rng.standard_normal((1, h, f))
    w2 = rng.standard_normal((1, f, h))
    logits = rng.standard_normal((T, 1)).astype(np.float32)
    out = M.moe_forward(x, w1, w2, logits, k=1, ep=1, rank=0)
    assert np.all(out["gates"] == 1.0)
    assert rel_err(out["y"], L.gelu(x @ w1[0]) @ w2[0]) < 1e-14


def test_moe_identical_experts_sum_gates_to_one():
    rng = np.random.default_rng(37)
    T, h, f, E, k = 9, 4, 6, 8, 3
    x = rng.standard_normal((T, h))
    w1 = np.repeat(rng.standard_normal((1, h, f)), E, axis=0)
    w2 = np.repeat(rng.standard_normal((1, f, h)), E, axis=0)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    out = M.moe_forward(x, w1, w2, logits, k=k, ep=1, rank=0)
    assert rel_err(out["y"], L.gelu(x @ w1[0]) @ w2[0]) < 1e-13
    # the ep ranks' partials add up to the ep=1 result
    parts = [M.moe_forward(x, w1[r * 2:(r + 1) * 2], w2[r * 2:(r + 1) * 2], logits, k, ep=4, rank=r)["y"]
             for r in range(4)]
    assert rel_err(np.sum(parts, axis=0), out["y"]) < 1e-13


def test_divisibility_cases_from_the_pages():
    cases = json.load(open(os.path.join(GOLDEN, "divisibility.json")))
    for c in cases["dense"]:
        if c["ok"]:
            S.check_divisible(c["hidden"], c["heads"], c["ffn"], c["tp"])
            assert c["hidden"] // c["tp"] == c["hidden_per_rank"]
            assert c["heads"] // c["tp"] == c["heads_per_rank"]
        else:
            with pytest.raises(S.ShapeError):
                S.check_divisible(c["hidden"], c["heads"], c["ffn"], c["tp"])
    with pytest.raises(S.ShapeError):
        S.check_divisible(768, 12, 3072, 2, rank=2)
    with pytest.raises(S.ShapeError):
        S.check_divisible(768, 12, 3070, 4)
