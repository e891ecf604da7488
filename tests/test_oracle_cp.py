"""Pins of the context-parallel attention oracle (oracle/cp.py) against closed
forms, invariants of the causal mask across chunks, the log-sum-exp merge
identity, and (backward) linearity over the ranks and finite differences,
independent of the oracle's own code path."""
import math

import numpy as np
import pytest

from oracle import cp as CP
from oracle import layer as L


def _qkv(seed, seq, heads, d, std=1.0):
    return np.random.default_rng(seed).standard_normal((seq, 3 * heads * d)) * std


def test_chunk_rows_cover_the_sequence_once():
    seq, cp = 96, 4
    got = np.concatenate([np.arange(seq)[CP.chunk_rows(seq, cp, r)] for r in range(cp)])
    assert np.array_equal(got, np.arange(seq))
    with pytest.raises(ValueError):
        CP.chunk_rows(97, 4, 0)
    with pytest.raises(ValueError):
        CP.chunk_rows(96, 4, 4)


def test_cp1_is_plain_attention():
    qkv = _qkv(1, 40, 2, 8)
    o, lse = CP.rank_attention(qkv, 2, 1, 0)
    o_ref, lse_ref = L.attention_forward(qkv, 2)
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)


def test_constant_keys_give_prefix_mean_at_global_positions():
    """Equal keys make every visible score equal: query i (global index) gets
    the mean of V over tokens 0..i and lse = q.k/sqrt(d) + log(i+1).  A chunk
    masked by local instead of global positions fails this."""
    seq, cp, heads, d = 48, 4, 2, 4
    qkv = _qkv(2, seq, heads, d)
    for n in range(heads):
        _, sk, _ = L.head_slices(heads, d, n)
        qkv[:, sk] = qkv[0, sk]
    for r in range(cp):
        o, lse = CP.rank_attention(qkv, heads, cp, r)
        rows = CP.chunk_rows(seq, cp, r)
        for j, i in enumerate(range(rows.start, rows.stop)):
            for n in range(heads):
                sq, sk, sv = L.head_slices(heads, d, n)
                assert np.allclose(o[j, n * d:(n + 1) * d], qkv[: i + 1, sv].mean(axis=0), rtol=0, atol=1e-12)
                want = qkv[i, sq] @ qkv[0, sk] / math.sqrt(d) + math.log(i + 1)
                assert abs(lse[n, j] - want) < 1e-12


def test_later_chunks_do_not_matter_and_earlier_ones_do():
    seq, cp, heads, d = 64, 4, 2, 8
    qkv = _qkv(3, seq, heads, d)
    r = 2
    o, lse = CP.rank_attention(qkv, heads, cp, r)
    later = qkv.copy()
    later[CP.chunk_rows(seq, cp, 3)] = _qkv(4, seq // cp, heads, d)
    o2, lse2 = CP.rank_attention(later, heads, cp, r)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    earlier = qkv.copy()
    earlier[CP.chunk_rows(seq, cp, 0)] = _qkv(5, seq // cp, heads, d)
    o3, _ = CP.rank_attention(earlier, heads, cp, r)
    assert np.max(np.abs(o3 - o)) > 1e-3


def test_sampled_rows_match_full_attention():
    seq, heads, d = 70, 3, 8
    qkv = _qkv(6, seq, heads, d, std=1.5)
    rows = [0, 1, 17, 63, 64, 69]
    o, lse = CP.attention_rows(qkv, heads, rows)
    o_ref, lse_ref = L.attention_forward(qkv, heads)
    assert np.allclose(o, o_ref[rows], rtol=0, atol=1e-12)
    assert np.allclose(lse, lse_ref[:, rows], rtol=0, atol=1e-12)


def test_merge_of_chunk_partials_equals_the_rank_rows():
    """Rank r's rows equal the log-sum-exp merge of its queries' attention over
    each key chunk j <= r on its own (full for j < r, causal for j = r):
    L = log sum_j exp(L_j), O = sum_j exp(L_j - L) O_j."""
    seq, cp, heads, d = 64, 4, 2, 8
    qkv = _qkv(7, seq, heads, d, std=1.3)
    c = seq // cp
    scale = 1.0 / math.sqrt(d)
    for r in range(cp):
        o_ref, lse_ref = CP.rank_attention(qkv, heads, cp, r)
        q_rows = CP.chunk_rows(seq, cp, r)
        for n in range(heads):
            sq, sk, sv = L.head_slices(heads, d, n)
            parts = []
            for j in range(r + 1):
                kr = CP.chunk_rows(seq, cp, j)
                s = qkv[q_rows, sq] @ qkv[kr, sk].T * scale
                if j == r:
                    s = np.where(np.tril(np.ones((c, c), dtype=bool)), s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                z = e.sum(axis=1, keepdims=True)
                parts.append(((e / z) @ qkv[kr, sv], (m + np.log(z))[:, 0]))
            lse = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
            o = sum(np.exp(p[1] - lse)[:, None] * p[0] for p in parts)
            assert np.allclose(o, o_ref[:, n * d:(n + 1) * d], rtol=0, atol=1e-12)
            assert np.allclose(lse, lse_ref[n], rtol=0, atol=1e-12)


def test_backward_cp1_is_plain_attention_backward():
    seq, heads, d = 24, 2, 4
    qkv = _qkv(8, seq, heads, d)
    do = _qkv(9, seq, heads, d)[:, : heads * d]
    g = CP.rank_attention_backward(qkv, do, heads, 1, 0)
    ref = L.attention_backward(qkv, do, heads)
    for n in range(heads):
        sq, sk, sv = L.head_slices(heads, d, n)
        assert np.array_equal(g["dq"][:, n * d:(n + 1) * d], ref[:, sq])
        assert np.array_equal(g["dkv"][0][:, 2 * n * d:(2 * n + 1) * d], ref[:, sk])
        assert np.array_equal(g["dkv"][0][:, (2 * n + 1) * d:(2 * n + 2) * d], ref[:, sv])


def test_backward_shares_of_all_ranks_add_up_to_the_full_gradient():
    """Linearity in dO: every rank's dQ rows, and the dK/dV shares every rank
    hands each chunk summed over the ranks, give the backward of the whole
    sequence's dO."""
    seq, cp, heads, d = 64, 4, 2, 8
    c = seq // cp
    qkv = _qkv(10, seq, heads, d, std=1.2)
    do = _qkv(11, seq, heads, d)[:, : heads * d]
    ref = L.attention_backward(qkv, do, heads)
    dq = np.zeros((seq, heads * d))
    dkv = np.zeros((seq, 2 * heads * d))
    for r in range(cp):
        g = CP.rank_attention_backward(qkv, do[r * c:(r + 1) * c], heads, cp, r)
        dq[r * c:(r + 1) * c] = g["dq"]
        for j, part in enumerate(g["dkv"]):
            dkv[j * c:(j + 1) * c] += part
    for n in range(heads):
        sq, sk, sv = L.head_slices(heads, d, n)
        assert np.allclose(dq[:, n * d:(n + 1) * d], ref[:, sq], rtol=0, atol=1e-12)
        assert np.allclose(dkv[:, 2 * n * d:(2 * n + 1) * d], ref[:, sk], rtol=0, atol=1e-12)
        assert np.allclose(dkv[:, (2 * n + 1) * d:(2 * n + 2) * d], ref[:, sv], rtol=0, atol=1e-12)


def test_backward_by_finite_differences_through_the_rank_loss():
    """dq and the dkv shares are the gradient of <dO, O_rank> with respect to
    the rank's queries and each earlier chunk's keys and values."""
    seq, cp, heads, d, r = 32, 4, 1, 4, 2
    c = seq // cp
    qkv = _qkv(12, seq, heads, d)
    do = _qkv(13, c, heads, d)[:, : heads * d]
    g = CP.rank_attention_backward(qkv, do, heads, cp, r)
    loss = lambda t: float(np.sum(CP.rank_attention(t, heads, cp, r)[0] * do))
    sq, sk, sv = L.head_slices(heads, d, 0)
    eps = 1e-6
    for tok, col, want in [(r * c + 3, sq.start + 1, g["dq"][3, 1]), (5, sk.start + 2, g["dkv"][0][5, 2]),
                           (c + 7, sv.start, g["dkv"][1][7, d]), (r * c + 1, sk.start, g["dkv"][r][1, 0])]:
        p, m = qkv.copy(), qkv.copy()
        p[tok, col] += eps
        m[tok, col] -= eps
        fd = (loss(p) - loss(m)) / (2 * eps)
        assert abs(fd - want) < 1e-7 * max(1.0, abs(want)), (tok, col, fd, want)


def test_dq_rows_match_the_rank_backward():
    seq, cp, heads, d, r = 64, 4, 2, 8, 3
    c = seq // cp
    qkv = _qkv(14, seq, heads, d, std=1.3)
    do = _qkv(15, c, heads, d)[:, : heads * d]
    g = CP.rank_attention_backward(qkv, do, heads, cp, r)
    local = [0, 5, 15]
    got = CP.dq_rows(qkv, do[local], heads, [r * c + i for i in local])
    assert np.allclose(got, g["dq"][local], rtol=0, atol=1e-12)


@pytest.mark.parametrize("cp,rank,heads,d", [(4, 2, 2, 64), (3, 2, 1, 128), (2, 0, 3, 64)])
def test_dkv_rows_equal_the_rank_backward(cp, rank, heads, d):
    """The key-restricted backward gives the rank backward's dK/dV shares on
    every key row it sees (chunks 0..rank), including the diagonal chunk."""
    seq = 192
    rng = np.random.default_rng(31 + rank)
    qkv = rng.standard_normal((seq, 3 * heads * d)) * 1.3
    c = seq // cp
    do = rng.standard_normal((c, heads * d))
    ref = CP.rank_attention_backward(qkv, do, heads, cp, rank)
    full = np.concatenate(ref["dkv"], axis=0)  # key rows 0 .. (rank+1)*c - 1
    keys = list(range((rank + 1) * c))
    got = CP.dkv_rows(qkv, do, heads, cp, rank, keys, block=40)
    assert np.max(np.abs(got - full)) <= 1e-12 * max(1.0, np.max(np.abs(full)))
    with pytest.raises(ValueError):
        CP.dkv_rows(qkv, do, heads, cp, rank, [(rank + 1) * c])
    # a subset of heads gives those heads' columns
    last = heads - 1
    sub = CP.dkv_rows(qkv, do, heads, cp, rank, keys[::7], head_ids=[last], block=64)
    assert np.max(np.abs(sub - full[::7, 2 * last * d:(2 * last + 2) * d])) <= 1e-12 * max(1.0, np.max(np.abs(full)))
