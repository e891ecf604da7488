"""Parity of mtl_cp_attn_fwd (one context-parallel rank's causal attention
share) with the fp64 oracle: every rank of small sequences in full, and rank 3
of the 32768-token, CP 4 workload on sampled query rows of every head."""
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
