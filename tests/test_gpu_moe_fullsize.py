"""Parity of the MoE block at the full workload size, in the launch configuration
bench.py times: rank 0 of 16 expert-parallel ranks, 256 experts, top-8,
hidden 7168, ffn 18432, 4096 tokens with Zipf(1.1) expert loads.

Routing (ids, gates, counts, offsets, permutation, inverse map) and the gather
are compared in full.  The grouped GEMMs are checked where the fp64 oracle can
afford them, on two experts: 0 (the hottest, ~3600 rows) and 15 (the coldest
local one).  Their weights come from the host generator; the other 14 local
experts get device-drawn weights that no check reads.

* Every token whose local slots all fall in experts {0, 15} (and the token
  with no local slot) is checked in full: its GeLU'(z), a, ye rows, its combined
  output y, its input gradient dx and its gate gradients.  Those tokens' rows
  form an exact sub-problem for the oracle.
* dW1[e][:, c] and dW2[e][c, :] for sampled ffn columns c of both experts:
  restricting the ffn dimension to those columns leaves these entries exact,
  so the oracle runs each expert with w1[:, c] and w2[c, :].
"""
import numpy as np
import pytest

import synth
from oracle import layer as L
from oracle import moe as M
from tests.parity_util import assert_bf16, f64

CHECKED = (0, 15)
FFN_COLS = [0, 1, 7, 8, 255, 256, 4095, 9000, 18431]


def _host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _sub_rows(fwd, tokens_sel, experts):
    """Rows (in oracle order: by expert, tokens ascending) of the selected
    tokens' assignments to the given local experts."""
    ptok, pslot, off = fwd["perm_token"], fwd["perm_slot"], fwd["offsets"]
    rows, offsets = [], [0]
    for e in experts:
        r = np.arange(off[e], off[e + 1])
        r = r[np.isin(ptok[r], tokens_sel)]
        rows.append(r)
        offsets.append(offsets[-1] + len(r))
    rows = np.concatenate(rows)
    return rows, np.array(offsets), ptok[rows], pslot[rows]


@pytest.mark.gpu
def test_moe_rank0_full_size(mtl):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    from megatron_tensor_transformer_layer_amd.moe import MoeRank

    shape = synth.MOE_WORKLOADS["moe-256e-top8-ep16"]
    rank, El = 0, shape.experts // shape.ep
    print(f"moe full size rank {rank}: {shape}", flush=True)
    logits = synth.moe_logits(shape)
    xb, dyb = synth.moe_tokens(shape, 0, "moe_x"), synth.moe_tokens(shape, 0, "moe_dy")
    host_w = {(n, e): synth.moe_expert_weight(shape, n, e) for n in ("moe_w1", "moe_w2") for e in CHECKED}

    def stack(name):
        return torch.stack([bf16_dev(host_w[(name, e)]) if e in CHECKED else
                            synth.moe_expert_weight_device(shape, name, e) for e in range(El)])

    r = MoeRank(shape.tokens, shape.hidden, shape.ffn, shape.experts, shape.topk, shape.ep, rank,
                stack("moe_w1"), stack("moe_w2"))
    r.step(torch.from_numpy(logits).cuda(), bf16_dev(xb), bf16_dev(dyb))
    torch.cuda.synchronize()
    print("device step done", flush=True)

    # ---- routing and gather, in full
    idx, gates = M.route_topk(logits, shape.topk)
    counts, offsets, ptok, pslot = M.permute(idx, shape.experts, shape.ep, rank)
    n = int(offsets[-1])
    assert np.array_equal(_host(r.idx), idx)
    assert np.max(np.abs(_host(r.gates) - gates)) <= 1e-6
    assert np.array_equal(_host(r.counts), counts)
    assert np.array_equal(_host(r.offsets), offsets)
    assert np.array_equal(_host(r.perm_token)[:n], ptok)
    assert np.array_equal(_host(r.perm_slot)[:n], pslot)
    slot_row = _host(r.slot_row)
    ref = np.full(idx.shape, -1, dtype=np.int32)
    ref[ptok, pslot] = np.arange(n, dtype=np.int32)
    assert np.array_equal(slot_row, ref)
    assert np.array_equal(_host(r.xp)[:n], xb[ptok])
    fwd_idx = dict(perm_token=ptok, perm_slot=pslot, offsets=offsets, gates=gates)

    x, dy = f64(xb), f64(dyb)
    w1 = {e: f64(host_w[("moe_w1", e)]) for e in CHECKED}
    w2 = {e: f64(host_w[("moe_w2", e)]) for e in CHECKED}

    # ---- tokens whose local experts are all checked: an exact sub-problem
    local = [set(int(e) for e in row if e < El) for row in idx]
    toks = np.array([t for t, s in enumerate(local) if s <= set(CHECKED)])
    assert len(toks) >= 5 and any(not s for s in local)
    rows, sub_off, sptok, spslot = _sub_rows(fwd_idx, toks, CHECKED)
    W1 = np.stack([w1[e] for e in CHECKED])
    W2 = np.stack([w2[e] for e in CHECKED])
    ef = M.expert_forward(x, W1, W2, sub_off, sptok)
    y = M.combine(ef["ye"], gates, sptok, spslot, shape.tokens)
    sub = dict(perm_token=sptok, perm_slot=spslot, offsets=sub_off, gates=gates, **ef)
    bwd = M.moe_backward(x, W1, W2, sub, dy)
    del W1, W2
    exp = dict(gz=L.gelu_grad(ef["z"]), a=ef["a"], ye=ef["ye"])
    for key in exp:
        assert_bf16(key, f64(_host(getattr(r, key)[torch.from_numpy(rows).cuda()])), exp[key])
    assert_bf16("y", f64(_host(r.y))[toks], y[toks])
    assert_bf16("dx", f64(_host(r.dx))[toks], bwd["dx"][toks])
    assert_bf16("dgates", _host(r.dgates)[toks], bwd["dgates"][toks])

    # ---- weight gradients of the checked experts on sampled ffn columns
    dw1, dw2 = r.dw1, r.dw2
    cols = np.array(FFN_COLS)
    for e in CHECKED:
        er, eoff, etok, eslot = _sub_rows(fwd_idx, np.arange(shape.tokens), [e])
        w1c, w2c = w1[e][:, cols][None], w2[e][cols, :][None]
        efc = M.expert_forward(x, w1c, w2c, eoff, etok)
        b = M.moe_backward(x, w1c, w2c, dict(perm_token=etok, perm_slot=eslot, offsets=eoff, gates=gates, **efc), dy)
        assert_bf16(f"dw1[{e}]", _host(dw1[e][:, torch.from_numpy(cols).cuda()]), b["dw1"][0])
        assert_bf16(f"dw2[{e}]", _host(dw2[e][torch.from_numpy(cols).cuda(), :]), b["dw2"][0])
