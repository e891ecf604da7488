"""Pin: MoE routing and permutation against hand-worked cases and brute force."""
import json
import os

import numpy as np
import pytest

from oracle import moe as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_topk(row, k):
    """Repeatedly take the largest remaining logit; on a tie the lower id wins."""
    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best is None or v > row[best]:
                best = e
        chosen.append(best)
    return chosen


def _brute_permute(idx, experts, ep, rank):
    per = experts // ep
    lo = rank * per
    buckets = [[] for _ in range(per)]
    for t in range(idx.shape[0]):
        for s in range(idx.shape[1]):
            e = int(idx[t, s])
            if lo <= e < lo + per:
                buckets[e - lo].append((t, s))
    counts = [len(b) for b in buckets]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    flat = [a for b in buckets for a in b]
    return counts, offsets, [a[0] for a in flat], [a[1] for a in flat]


def test_routing_golden():
    g = json.load(open(os.path.join(GOLDEN, "routing.json")))
    logits = np.array(g["logits"], dtype=np.float32)
    idx, gates = M.route_topk(logits, g["k"])
    assert idx.tolist() == g["idx"]
    assert np.max(np.abs(gates - np.array(g["gates"]))) < 1e-15
    for r in range(g["ep"]):
        c, o, pt, ps = M.permute(idx, logits.shape[1], g["ep"], r)
        assert c.tolist() == g[f"rank{r}_counts"]
        assert o.tolist() == g[f"rank{r}_offsets"]
        assert pt.tolist() == g[f"rank{r}_perm_token"]
        assert ps.tolist() == g[f"rank{r}_perm_slot"]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_routing_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, E, k, ep = 40, 16, 4, 4
    # coarse values so that ties are common
    logits = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
    idx, gates = M.route_topk(logits, k)
    for t in range(T):
        assert idx[t].tolist() == _brute_topk(logits[t].tolist(), k)
        sel = logits[t, idx[t]].astype(np.float64)
        assert abs(gates[t].sum() - 1.0) < 1e-15
        assert np.all(np.diff(sel) <= 0)
    for r in range(ep):
        c, o, pt, ps = M.permute(idx, E, ep, r)
        bc, bo, bpt, bps = _brute_permute(idx, E, ep, r)
        assert c.tolist() == bc and o.tolist() == bo and pt.tolist() == bpt and ps.tolist() == bps


def _rank_key(v):
    """Larger is earlier: NaN below every number, -0 equal to +0."""
    return (0, 0.0) if v != v else (1, v + 0.0)


def _brute_topk_nonfinite(row, k):
    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e not in chosen and (best is None or _rank_key(v) > _rank_key(row[best])):
                best = e
        chosen.append(best)
    return chosen


def test_routing_nonfinite_hand_worked():
    """NaN ranks below -inf, -inf below every finite value, -0 ties +0 (lower
    id first): [NaN, -inf, 1, NaN, 0, -0] top-5 is 2, 4, 5, 1, 0."""
    nan, inf = float("nan"), float("inf")
    logits = np.array([[nan, -inf, 1.0, nan, 0.0, -0.0],
                       [3.0, inf, nan, -2.0, -inf, 0.5]], dtype=np.float32)
    idx, gates = M.route_topk(logits, 5)
    assert idx.tolist() == [[2, 4, 5, 1, 0], [1, 0, 5, 3, 4]]
    # a NaN selected in row 0; +inf minus itself in row 1: both rows' gates NaN
    assert np.all(np.isnan(gates))
    idx3, gates3 = M.route_topk(logits, 3)
    assert idx3.tolist() == [[2, 4, 5], [1, 0, 5]]
    assert np.all(np.isfinite(gates3[0])) and abs(gates3[0].sum() - 1.0) < 1e-15
    # exp(-inf) gates: -inf selected beside finite logits gets exactly 0
    idx4, gates4 = M.route_topk(np.array([[0.0, -inf, 1.0]], dtype=np.float32), 3)
    assert idx4.tolist() == [[2, 0, 1]] and gates4[0, 2] == 0.0


@pytest.mark.parametrize("seed", [0, 1])
def test_routing_nonfinite_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, E, k = 64, 12, 6
    pool = np.array([np.nan, -np.inf, np.inf, 0.0, -0.0, -1.0, 1.0, 2.0], dtype=np.float32)
    logits = pool[rng.integers(0, len(pool), size=(T, E))]
    idx, _ = M.route_topk(logits, k)
    for t in range(T):
        assert idx[t].tolist() == _brute_topk_nonfinite(logits[t].tolist(), k)
