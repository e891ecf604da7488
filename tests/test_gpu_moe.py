"""Parity of one expert-parallel rank's MoE block on the GPU against the fp64
oracle: routing ids, counts, offsets, the permutation and its inverse, and the
gathered token rows are compared bit for bit; gates to fp32 rounding; every
floating-point output of the grouped GEMMs, the combine and the backward to
the bf16 tolerance."""
import numpy as np
import pytest

import synth
from oracle import layer as L
from oracle import moe as M
from tests.parity_util import assert_bf16, f64

MS = synth.MoeShape
CASES = {
    # (shape, rank, logit quantum or None)
    "small-ep2-rank0": (MS(tokens=200, hidden=128, ffn=256, experts=8, topk=2, ep=2), 0, None),
    "small-ep2-rank1": (MS(tokens=200, hidden=128, ffn=256, experts=8, topk=2, ep=2), 1, None),
    # 77 tokens, ffn 136: nothing is a multiple of a tile
    "ragged-ep4-rank3": (MS(tokens=77, hidden=64, ffn=136, experts=16, topk=4, ep=4), 3, None),
    # two local experts but k = 4: every token has at most two local slots
    "fewer-local-than-k": (MS(tokens=150, hidden=128, ffn=128, experts=8, topk=4, ep=4), 1, None),
    # logits on a 0.5 grid: many exact ties, broken toward the lower expert id
    "tied-logits": (MS(tokens=256, hidden=64, ffn=64, experts=32, topk=8, ep=2), 0, 0.5),
    # ~300 rows per expert: several row tiles per expert, ragged last tile
    "multi-tile-ep1": (MS(tokens=600, hidden=256, ffn=384, experts=4, topk=2, ep=1), 0, None),
    # 12 tokens over 16 local experts with steep loads: most experts get no rows
    "empty-experts": (MS(tokens=12, hidden=64, ffn=64, experts=64, topk=1, ep=4, zipf_s=2.0), 0, None),
    # the same tokens seen from rank 1: no local rows at all
    "no-local-rows": (MS(tokens=12, hidden=64, ffn=64, experts=64, topk=1, ep=4, zipf_s=2.0), 1, None),
    "one-token": (MS(tokens=1, hidden=64, ffn=64, experts=4, topk=2, ep=1), 0, None),
}


def _inputs(shape, rank, quantum, seed=0):
    logits = synth.moe_logits(shape, seed)
    if quantum:
        logits = (np.round(logits / quantum) * quantum).astype(np.float32)
    lo, hi = M.local_range(shape.experts, shape.ep, rank)
    w1 = np.stack([synth.moe_expert_weight(shape, "moe_w1", e, seed) for e in range(lo, hi)])
    w2 = np.stack([synth.moe_expert_weight(shape, "moe_w2", e, seed) for e in range(lo, hi)])
    return dict(logits=logits, x=synth.moe_tokens(shape, seed, "moe_x"), dy=synth.moe_tokens(shape, seed, "moe_dy"),
                w1=w1, w2=w2)


def _run(shape, rank, inp, flags=0, repeat_bwd=1):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    from megatron_tensor_transformer_layer_amd.moe import MoeRank
    r = MoeRank(shape.tokens, shape.hidden, shape.ffn, shape.experts, shape.topk, shape.ep, rank,
                bf16_dev(inp["w1"]), bf16_dev(inp["w2"]), flags=flags)
    logits = torch.from_numpy(inp["logits"]).cuda()
    r.route(logits)
    r.permute()
    r.forward(bf16_dev(inp["x"]))
    dy = bf16_dev(inp["dy"])
    for _ in range(repeat_bwd):
        r.backward(dy)
    torch.cuda.synchronize()
    return r


def _host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _slot_row_ref(ptok, pslot, tokens, k):
    ref = np.full((tokens, k), -1, dtype=np.int32)
    ref[ptok, pslot] = np.arange(len(ptok), dtype=np.int32)
    return ref


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(CASES))
def test_moe_rank_matches_oracle(mtl, case):
    shape, rank, quantum = CASES[case]
    print(f"case {case} {shape} rank={rank}", flush=True)
    inp = _inputs(shape, rank, quantum)
    r = _run(shape, rank, inp)
    x, w1, w2, dy = f64(inp["x"]), f64(inp["w1"]), f64(inp["w2"]), f64(inp["dy"])
    fwd = M.moe_forward(x, w1, w2, inp["logits"], shape.topk, shape.ep, rank)
    bwd = M.moe_backward(x, w1, w2, fwd, dy)
    n = int(fwd["offsets"][-1])

    # integer outputs: exact
    assert np.array_equal(_host(r.idx), fwd["idx"])
    assert np.array_equal(_host(r.counts), fwd["counts"])
    assert np.array_equal(_host(r.offsets), fwd["offsets"])
    assert np.array_equal(_host(r.perm_token)[:n], fwd["perm_token"])
    assert np.array_equal(_host(r.perm_slot)[:n], fwd["perm_slot"])
    assert np.array_equal(_host(r.slot_row),
                          _slot_row_ref(fwd["perm_token"], fwd["perm_slot"], shape.tokens, shape.topk))
    # the softmax of k fp32 logits, in fp32
    assert np.max(np.abs(_host(r.gates) - fwd["gates"])) <= 1e-6
    # the gather moves bf16 rows unchanged
    assert np.array_equal(f64(_host(r.xp)[:n]), fwd["xp"])

    assert_bf16("gz", f64(_host(r.gz)[:n]), L.gelu_grad(fwd["z"]))
    for key in ("a", "ye"):
        assert_bf16(key, f64(_host(getattr(r, key))[:n]), fwd[key])
    assert_bf16("y", f64(_host(r.y)), fwd["y"])
    assert_bf16("dx", f64(_host(r.dx)), bwd["dx"])
    assert_bf16("dgates", _host(r.dgates), bwd["dgates"])
    dw1, dw2 = _host(r.dw1), _host(r.dw2)
    assert_bf16("dw1", dw1, bwd["dw1"])
    assert_bf16("dw2", dw2, bwd["dw2"])
    # an expert with no rows has exactly zero weight gradients; slots whose
    # expert lives elsewhere have exactly zero gate gradients
    for e in np.flatnonzero(fwd["counts"] == 0):
        assert not dw1[e].any() and not dw2[e].any()
    assert not _host(r.dgates)[_slot_row_ref(fwd["perm_token"], fwd["perm_slot"], shape.tokens,
                                             shape.topk) < 0].any()


@pytest.mark.gpu
def test_moe_is_deterministic(mtl):
    shape, rank, q = CASES["multi-tile-ep1"]
    inp = _inputs(shape, rank, q, seed=3)
    a, b = _run(shape, rank, inp), _run(shape, rank, inp)
    n = int(_host(a.offsets)[-1])
    for key in ("idx", "gates", "offsets", "slot_row", "y", "dx", "dw1", "dw2", "dgates"):
        assert np.array_equal(_host(getattr(a, key)), _host(getattr(b, key))), key
    for key in ("perm_token", "perm_slot", "xp", "gz", "a", "ye"):  # rows past N are never written
        assert np.array_equal(_host(getattr(a, key))[:n], _host(getattr(b, key))[:n]), key


@pytest.mark.gpu
def test_moe_wgrad_accumulates(mtl):
    shape, rank, q = CASES["small-ep2-rank1"]
    inp = _inputs(shape, rank, q, seed=5)
    once = _run(shape, rank, inp)
    twice = _run(shape, rank, inp, flags=mtl.MTL_F_WGRAD_ACCUM, repeat_bwd=2)
    # the same products added to themselves: exactly twice the single result
    assert np.array_equal(_host(twice.dw1), 2 * _host(once.dw1))
    assert np.array_equal(_host(twice.dw2), 2 * _host(once.dw2))


@pytest.mark.gpu
@pytest.mark.parametrize("seed", [0, 1])
def test_route_nonfinite_logits_bit_exact(mtl, seed):
    """Rows holding NaN, +-inf and +-0 logits: the device picks the oracle's ids
    bit for bit (NaN below -inf, ties to the lower id) and its gates are NaN
    exactly where the oracle's are, equal to fp32 rounding elsewhere."""
    import torch
    from megatron_tensor_transformer_layer_amd import make_moe_cfg, mtl_moe_route
    rng = np.random.default_rng(seed)
    T, E, k = 300, 70, 8
    pool = np.array([np.nan, -np.inf, np.inf, 0.0, -0.0, -1.0, 1.0, 2.5], dtype=np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    mask = rng.random((T, E)) < 0.3
    logits[mask] = pool[rng.integers(0, len(pool), size=int(mask.sum()))]
    logits[0, :] = np.nan  # every logit NaN: ids 0..k-1
    logits[1, :] = -np.inf
    print(f"route nonfinite seed={seed} T={T} E={E} k={k}", flush=True)
    cfg = make_moe_cfg(T, 64, 64, E, k)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, k, dtype=torch.float32, device="cuda")
    mtl_moe_route(cfg, torch.from_numpy(logits).cuda(), idx, gates)
    torch.cuda.synchronize()
    ref_idx, ref_g = M.route_topk(logits, k)
    got_idx, got_g = idx.cpu().numpy(), gates.cpu().numpy()
    assert np.array_equal(got_idx, ref_idx)
    assert got_idx[0].tolist() == list(range(k)) and got_idx[1].tolist() == list(range(k))
    assert np.array_equal(np.isnan(got_g), np.isnan(ref_g))
    fin = ~np.isnan(ref_g)
    assert np.max(np.abs(got_g[fin] - ref_g[fin])) <= 1e-6
