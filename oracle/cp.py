"""fp64 oracle of one context-parallel rank's share of causal attention, forward
and backward.

Test infrastructure only (see the package docstring).

The guide ([guide] ai.lansai.wang/82226, the parallel-dimension table and the
tolerance section) says that context parallelism cuts the inputs and
activations along the sequence, that attention still needs the keys and values
held by the other ranks, and that masks must be re-checked at several sequence
lengths; the site summary ([site] navi2ai.com/sites/1106, its parallelism list
and deploy examples) sets `--context-parallel-size`.  Neither fixes how the
sequence is assigned to ranks.  Reading taken here: the S tokens are cut into
cp contiguous chunks of C = S/cp, rank r holds the queries of chunk r, and its
result is rows [rC, (r+1)C) of the causal attention over the whole sequence
(O and the row log-sum-exp), i.e. the plain definition.  Its backward is the
gradient that its rows' dO sends into the QKV of the sequence: the complete dQ
of its queries and a dK/dV share for every chunk up to its own.  How a device
splits that work over key chunks is not restated here.
"""
from __future__ import annotations

import math

import numpy as np

from . import layer as L


def chunk_rows(seq: int, cp: int, rank: int) -> slice:
    """Token rows held by CP rank `rank`: [rank*seq/cp, (rank+1)*seq/cp)."""
    if cp < 1 or seq % cp != 0:
        raise ValueError("seq must split into cp equal chunks")
    if not 0 <= rank < cp:
        raise ValueError("rank outside [0, cp)")
    c = seq // cp
    return slice(rank * c, (rank + 1) * c)


def rank_attention(qkv_full, heads: int, cp: int, rank: int):
    """O [C, heads*d] and lse [heads, C] of rank `rank`'s queries.

    Causal attention of a row depends only on the tokens up to it, so the full
    attention is evaluated over the prefix that ends with the rank's chunk and
    the rank's rows are taken from it."""
    qkv_full = np.asarray(qkv_full, dtype=np.float64)
    rows = chunk_rows(qkv_full.shape[0], cp, rank)
    o, lse = L.attention_forward(qkv_full[: rows.stop], heads)
    return o[rows], lse[:, rows]


def attention_rows(qkv_full, heads: int, rows) -> tuple:
    """Causal attention for selected query rows only (global token indices):
    query i of head n sees keys 0..i.  Returns O [len(rows), heads*d] and
    lse [heads, len(rows)].  One query at a time, for sampled checks at sizes
    where the full attention is too slow."""
    qkv_full = np.asarray(qkv_full, dtype=np.float64)
    d = qkv_full.shape[1] // (3 * heads)
    scale = 1.0 / math.sqrt(d)
    rows = list(rows)
    o = np.zeros((len(rows), heads * d))
    lse = np.zeros((heads, len(rows)))
    for n in range(heads):
        sq, sk, sv = L.head_slices(heads, d, n)
        for j, i in enumerate(rows):
            s = (qkv_full[i, sq] @ qkv_full[: i + 1, sk].T) * scale
            m = s.max()
            e = np.exp(s - m)
            z = e.sum()
            o[j, n * d:(n + 1) * d] = (e / z) @ qkv_full[: i + 1, sv]
            lse[n, j] = m + math.log(z)
    return o, lse


def rank_attention_backward(qkv_full, do_rank, heads: int, cp: int, rank: int) -> dict:
    """Gradients that flow from CP rank `rank`'s output gradient dO [C, heads*d]
    (its own rows only) back into the QKV of the sequence, split the way the
    ranks own them:

    * ``dq``: dQ of the rank's queries [C, heads*d] (heads in order), complete;
    * ``dkv[j]`` for j <= rank: the [C, 2*heads*d] dK and dV (per head
      [dK_n | dV_n]) of chunk j's keys from the rank's queries, the share the
      rank hands back to chunk j's owner (for j = rank, its own diagonal share).

    Definition: the causal attention backward over the whole sequence with dO
    zero outside the rank's rows; chunks after the rank receive nothing."""
    qkv_full = np.asarray(qkv_full, dtype=np.float64)
    rows = chunk_rows(qkv_full.shape[0], cp, rank)
    prefix = qkv_full[: rows.stop]
    d = prefix.shape[1] // (3 * heads)
    do_full = np.zeros((prefix.shape[0], heads * d))
    do_full[rows] = np.asarray(do_rank, dtype=np.float64)
    g = L.attention_backward(prefix, do_full, heads)
    dq = np.concatenate([g[rows, L.head_slices(heads, d, n)[0]] for n in range(heads)], axis=1)
    dkv = []
    for j in range(rank + 1):
        rj = chunk_rows(qkv_full.shape[0], cp, j)
        parts = []
        for n in range(heads):
            _, sk, sv = L.head_slices(heads, d, n)
            parts += [g[rj, sk], g[rj, sv]]
        dkv.append(np.concatenate(parts, axis=1))
    return dict(dq=dq, dkv=dkv)


def dq_rows(qkv_full, do_rows, heads: int, rows) -> np.ndarray:
    """dQ [len(rows), heads*d] of selected query rows (global indices) of causal
    attention, given their dO rows [len(rows), heads*d]: per head and query i
    over keys 0..i, P = softmax(q K^T * scale), D = dO_i . (P V),
    dS = P * (dO_i V^T - D), dq = dS K * scale.  A query's dQ depends only on
    its own dO row, so this is the rank backward's dq on those rows."""
    qkv_full = np.asarray(qkv_full, dtype=np.float64)
    do_rows = np.asarray(do_rows, dtype=np.float64)
    d = qkv_full.shape[1] // (3 * heads)
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((len(rows), heads * d))
    for n in range(heads):
        sq, sk, sv = L.head_slices(heads, d, n)
        for j, i in enumerate(rows):
            k, v = qkv_full[: i + 1, sk], qkv_full[: i + 1, sv]
            s = (qkv_full[i, sq] @ k.T) * scale
            p = np.exp(s - s.max())
            p /= p.sum()
            g = do_rows[j, n * d:(n + 1) * d]
            ds = p * (v @ g - g @ (p @ v))
            out[j, n * d:(n + 1) * d] = (ds @ k) * scale
    return out


def dkv_rows(qkv_full, do_rank, heads: int, cp: int, rank: int, key_rows, head_ids=None,
             block: int = 512) -> np.ndarray:
    """dK and dV of selected key rows (global indices, before the end of the
    rank's chunk) from CP rank `rank`'s queries, in the per-head [dK_n | dV_n]
    layout of ``rank_attention_backward``'s shares, for the heads ``head_ids``
    (default: all, in order): [len(key_rows), 2*len(head_ids)*d].

    The textbook attention backward restricted to those key columns: per head
    and block of the rank's queries i, P = softmax over keys j <= i of
    q_i k_j * scale, O = P V, D_i = dO_i . O_i; for each selected key k,
    dV_k = sum_i P_ik dO_i and dK_k = scale * sum_i P_ik (dO_i . v_k - D_i) q_i.
    For sampled checks at sizes where the whole backward is too slow."""
    qkv_full = np.asarray(qkv_full, dtype=np.float64)
    do_rank = np.asarray(do_rank, dtype=np.float64)
    rows = chunk_rows(qkv_full.shape[0], cp, rank)
    d = qkv_full.shape[1] // (3 * heads)
    scale = 1.0 / math.sqrt(d)
    keys = np.asarray(list(key_rows), dtype=np.int64)
    if keys.size and (keys.min() < 0 or keys.max() >= rows.stop):
        raise ValueError("key rows outside the keys the rank's queries see")
    head_ids = list(range(heads)) if head_ids is None else list(head_ids)
    out = np.zeros((len(keys), 2 * len(head_ids) * d))
    kv_end = rows.stop
    for hi, n in enumerate(head_ids):
        sq, sk, sv = L.head_slices(heads, d, n)
        K, V = qkv_full[:kv_end, sk], qkv_full[:kv_end, sv]
        for b0 in range(rows.start, rows.stop, block):
            b1 = min(b0 + block, rows.stop)
            q = qkv_full[b0:b1, sq]
            g = do_rank[b0 - rows.start:b1 - rows.start, n * d:(n + 1) * d]
            s = (q @ K.T) * scale
            # keys of the rank's own chunk are visible up to the query itself;
            # every earlier chunk's key is visible to all of its queries
            own = s[:, rows.start:]
            own[np.arange(b0, b1)[:, None] < np.arange(rows.start, kv_end)[None, :]] = -np.inf
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            p /= p.sum(axis=1, keepdims=True)
            D = np.sum(g * (p @ V), axis=1)
            pk = p[:, keys]                       # [queries, selected keys]
            ds = pk * (g @ V[keys].T - D[:, None])
            out[:, 2 * hi * d:(2 * hi + 1) * d] += (ds.T @ q) * scale
            out[:, (2 * hi + 1) * d:(2 * hi + 2) * d] += pk.T @ g
    return out
