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
