"""The seeded input generator: bf16 rounding and shard independence."""
import numpy as np
import pytest
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(51)
    v = (rng.standard_normal(100000) * np.exp2(rng.uniform(-40, 40, 100000))).astype(np.float32)
    ties = synth.bf16_bits_to_f32(rng.integers(0, 1 << 16, 1000).astype(np.uint16) & 0x7F7F)
    ties = (ties.view(np.uint32) | np.uint32(0x8000)).view(np.float32)  # exact halfway points
    v = np.concatenate([v, ties, -ties])
    mine = synth.bf16_round_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(mine), torch.from_numpy(v).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("tp", [2, 4])
def test_shards_concatenate_to_full(tp):
    shape = synth.LayerShape(hidden=64, heads=8, ffn=256, seq=16, micro_batch=1)
    for name, axis in [("w_qkv", 1), ("b_qkv", 0), ("w_o", 0), ("w1", 1), ("b1", 0), ("w2", 0)]:
        full = synth.layer_tensor(shape, name, seed=0)
        parts = [synth.layer_tensor(shape, name, seed=0, tp=tp, rank=r) for r in range(tp)]
        assert np.array_equal(np.concatenate(parts, axis=axis), full), name
    for name in ("x", "dy", "b_o", "b2"):
        assert np.array_equal(synth.layer_tensor(shape, name, tp=tp, rank=1), synth.layer_tensor(shape, name))


def test_shapes_and_distributions():
    shape = synth.LayerShape(hidden=128, heads=4, ffn=512, seq=64, micro_batch=2)
    d = synth.layer_inputs(shape)
    assert d["x"].shape == (128, 128) and d["w_qkv"].shape == (128, 384) and d["w2"].shape == (512, 128)
    x = synth.bf16_bits_to_f64(d["x"])
    w = synth.bf16_bits_to_f64(d["w1"])
    assert abs(x.std() - 1) < 0.05 and abs(w.std() - 0.02) < 0.002
    # values do not change between calls (seeded)
    assert np.array_equal(synth.layer_tensor(shape, "w1"), d["w1"])
    assert not np.array_equal(synth.layer_tensor(shape, "w1", seed=1), d["w1"])


def test_moe_logits_follow_zipf():
    shape = synth.MoeShape(tokens=4096, hidden=16, ffn=32, experts=256, topk=8, ep=16)
    logits = synth.moe_logits(shape)
    assert logits.dtype == np.float32 and logits.shape == (4096, 256)
    top = np.argsort(-logits, axis=1, kind="stable")[:, :8]
    loads = np.bincount((top // 16).reshape(-1), minlength=16)
    assert loads.sum() == 4096 * 8
    assert loads[0] == loads.max() and loads[0] > 4 * loads.mean()
