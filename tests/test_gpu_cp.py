"""Parity of mtl_cp_attn_fwd and mtl_cp_attn_bwd (one context-parallel rank's
causal attention share, forward and backward) with the fp64 oracle: every rank
of small sequences in full, and ranks of the 32768-token, CP 4 workload on
sampled query rows of every head plus, for dK and dV, identities that hold at
any size."""
import numpy as np
import pytest

import synth
from oracle import cp as CP
from tests.parity_util import assert_bf16, f64

LSE_ABS = 5e-3  # fp32 row log-sum-exp of bf16 inputs: far inside the bf16 bound, checked as well

SMALL = {
    "d128-cp4": synth.CpShape(seq=1024, heads=2, head_dim=128, cp=4),
    "d64-cp3": synth.CpShape(seq=768, heads=3, head_dim=64, cp=3),
    "d128-cp2-chunk64": synth.CpShape(seq=128, heads=1, head_dim=128, cp=2),
    "d128-cp1": synth.CpShape(seq=320, heads=2, head_dim=128, cp=1),
}


def _run(shape, rank, qkv_dev):
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_cp_attn_fwd, mtl_cp_attn_scratch_bytes
    C, H, d = shape.chunk, shape.heads, shape.head_dim
    ld = 3 * H * d
    chunks = [qkv_dev.data_ptr() + j * C * ld * 2 for j in range(shape.cp)]
    o = torch.empty(C, H * d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(H, C, dtype=torch.float32, device="cuda")
    nb = mtl_cp_attn_scratch_bytes(shape.cp, rank, C, H, d)
    scratch = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    mtl_cp_attn_fwd(shape.cp, rank, C, H, d, chunks, o, lse, scratch, nb)
    torch.cuda.synchronize()
    return o, lse


def _check_lse(name, got, ref):
    err = float(np.max(np.abs(got - ref)))
    assert err <= LSE_ABS, f"{name}: lse max|diff| {err:.3e}"


@pytest.mark.gpu
@pytest.mark.parametrize("case", sorted(SMALL))
def test_cp_attention_every_rank(mtl, case):
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev, host_f64
    shape = SMALL[case]
    print(f"cp attention {case} {shape}", flush=True)
    bits = synth.cp_qkv(shape, seed=3)
    qkv = bf16_dev(bits)
    full = f64(bits)
    for r in range(shape.cp):
        o, lse = _run(shape, r, qkv)
        o_ref, lse_ref = CP.rank_attention(full, shape.heads, shape.cp, r)
        assert_bf16(f"{case} rank {r} O", host_f64(o), o_ref)
        assert_bf16(f"{case} rank {r} lse", host_f64(lse), lse_ref)
        _check_lse(f"{case} rank {r}", host_f64(lse), lse_ref)


@pytest.mark.gpu
def test_cp_attention_deterministic(mtl):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    shape = SMALL["d128-cp4"]
    qkv = bf16_dev(synth.cp_qkv(shape, seed=4))
    o1, l1 = _run(shape, 3, qkv)
    o2, l2 = _run(shape, 3, qkv)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.gpu
@pytest.mark.parametrize("rank", [3, 1])
def test_cp_attention_fullsize_sampled(mtl, rank):
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev, host_f64
    shape = synth.CP_WORKLOADS["cp4-seq32k-7b-tp4"]
    print(f"cp attention full size rank {rank} {shape}", flush=True)
    bits = synth.cp_qkv(shape)
    o, lse = _run(shape, rank, bf16_dev(bits))
    o, lse = host_f64(o), host_f64(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    C = shape.chunk
    rng = np.random.default_rng(11 + rank)
    # chunk edges, 64-row block edges and random rows of the rank's chunk
    local = sorted(set([0, 1, 63, 64, 127, C // 2, C - 65, C - 64, C - 1] + rng.choice(C, 23, replace=False).tolist()))
    rows = [rank * C + i for i in local]
    o_ref, lse_ref = CP.attention_rows(f64(bits[: (rank + 1) * C]), shape.heads, rows)
    assert_bf16(f"rank {rank} O rows", o[local], o_ref)
    assert_bf16(f"rank {rank} lse rows", lse[:, local], lse_ref)
    _check_lse(f"rank {rank}", lse[:, local], lse_ref)


BWD = dict(SMALL, **{"d128-cp4-seq4096": synth.CpShape(seq=4096, heads=2, head_dim=128, cp=4)})


def _dout(shape, seed=5):
    return synth.cp_dout(shape, seed)


def _run_bwd(shape, rank, qkv_dev, o, lse, dout):
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_cp_attn_bwd, mtl_cp_attn_bwd_scratch_bytes
    C, H, d = shape.chunk, shape.heads, shape.head_dim
    ld = 3 * H * d
    chunks = [qkv_dev.data_ptr() + j * C * ld * 2 for j in range(shape.cp)]
    dqkv = torch.full((C, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    dkv = [torch.full((C, ld), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(rank)]
    nb = mtl_cp_attn_bwd_scratch_bytes(shape.cp, rank, C, H, d)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    mtl_cp_attn_bwd(shape.cp, rank, C, H, d, chunks, o, lse, dout, dqkv, dkv, scratch, nb)
    torch.cuda.synchronize()
    return dqkv, dkv


def _split(dqkv_host, heads, d):
    """head-interleaved [C, 3*heads*d] -> dq [C, heads*d], dkv [C, 2*heads*d] ([dK_n | dV_n] per head)"""
    dq = np.concatenate([dqkv_host[:, n * 3 * d:n * 3 * d + d] for n in range(heads)], axis=1)
    dkv = np.concatenate([dqkv_host[:, n * 3 * d + d:(n + 1) * 3 * d] for n in range(heads)], axis=1)
    return dq, dkv


@pytest.mark.gpu
@pytest.mark.parametrize("case", sorted(BWD))
def test_cp_attention_backward_every_rank(mtl, case):
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev, host_f64
    shape = BWD[case]
    H, d = shape.heads, shape.head_dim
    print(f"cp attention backward {case} {shape}", flush=True)
    bits = synth.cp_qkv(shape, seed=6)
    qkv = bf16_dev(bits)
    full = f64(bits)
    do_bits = _dout(shape)
    dout = bf16_dev(do_bits)
    for r in range(shape.cp):
        o, lse = _run(shape, r, qkv)
        dqkv, dkv = _run_bwd(shape, r, qkv, o, lse, dout)
        ref = CP.rank_attention_backward(full, f64(do_bits), H, shape.cp, r)
        dq, dkv_own = _split(host_f64(dqkv), H, d)
        assert_bf16(f"{case} rank {r} dQ", dq, ref["dq"])
        assert_bf16(f"{case} rank {r} own dK|dV", dkv_own, ref["dkv"][r])
        for j in range(r):
            got = host_f64(dkv[j])
            assert np.all(np.isnan(_split(got, H, d)[0])), "query columns of a peer share were written"
            assert_bf16(f"{case} rank {r} dK|dV share of chunk {j}", _split(got, H, d)[1], ref["dkv"][j])


@pytest.mark.gpu
def test_cp_attention_backward_deterministic(mtl):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    shape = SMALL["d128-cp4"]
    qkv = bf16_dev(synth.cp_qkv(shape, seed=7))
    dout = bf16_dev(_dout(shape, 8))
    o, lse = _run(shape, 3, qkv)
    a, pa = _run_bwd(shape, 3, qkv, o, lse, dout)
    b, pb = _run_bwd(shape, 3, qkv, o, lse, dout)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for x, y in zip(pa, pb):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.gpu
@pytest.mark.parametrize("rank", [3, 1])
def test_cp_attention_backward_fullsize(mtl, rank):
    """dQ on sampled query rows and dK/dV on sampled key rows of every chunk
    the rank sees (its own diagonal chunk and each earlier chunk's share),
    element-wise against the oracle; and, over every key, two identities of
    the exact gradient: summed over the keys, dV gives the column sums of dO
    (each query's probabilities sum to 1) and dK gives zero (each query's dS
    sums to 0)."""
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev, host_f64
    shape = synth.CP_WORKLOADS["cp4-seq32k-7b-tp4"]
    H, d, C = shape.heads, shape.head_dim, shape.chunk
    print(f"cp attention backward full size rank {rank} {shape}", flush=True)
    bits = synth.cp_qkv(shape)
    qkv = bf16_dev(bits)
    do_bits = _dout(shape, 9)
    o, lse = _run(shape, rank, qkv)
    dqkv, dkv = _run_bwd(shape, rank, qkv, o, lse, bf16_dev(do_bits))
    dq, own = _split(host_f64(dqkv), H, d)
    shares = [_split(host_f64(t), H, d)[1] for t in dkv] + [own]
    for x in shares + [dq]:
        assert np.all(np.isfinite(x))
    rng = np.random.default_rng(21 + rank)
    local = sorted(set([0, 63, 64, C // 2, C - 1] + rng.choice(C, 11, replace=False).tolist()))
    ref = CP.dq_rows(f64(bits[: (rank + 1) * C]), f64(do_bits)[local], H, [rank * C + i for i in local])
    assert_bf16(f"rank {rank} dQ rows", dq[local], ref)
    allkv = np.concatenate(shares, axis=0)  # every key row of chunks 0..rank
    keys = sorted(set([j * C + i for j in range(rank + 1) for i in (0, 1, 63, 64, C // 2, C - 1)]
                      + rng.choice((rank + 1) * C, 10, replace=False).tolist()))
    hs = [0, H - 1]  # two of the heads: the restricted backward still takes every query of the rank
    ref_kv = CP.dkv_rows(f64(bits), f64(do_bits), H, shape.cp, rank, keys, head_ids=hs)
    got_kv = np.concatenate([allkv[keys][:, 2 * n * d:(2 * n + 2) * d] for n in hs], axis=1)
    print(f"  dK|dV on {len(keys)} key rows of heads {hs}", flush=True)
    assert_bf16(f"rank {rank} dK|dV rows", got_kv, ref_kv)
    dsum = f64(do_bits).sum(axis=0)
    for n in range(H):
        dk = allkv[:, 2 * n * d:(2 * n + 1) * d]
        dv = allkv[:, (2 * n + 1) * d:(2 * n + 2) * d]
        assert_bf16(f"rank {rank} head {n} sum of dV", dv.sum(axis=0), dsum[n * d:(n + 1) * d])
        ksum = np.abs(dk.sum(axis=0)).max()
        assert ksum <= 1e-2 * np.abs(dk).sum(axis=0).max(), f"head {n}: |sum dK| {ksum:.3e}"
