"""Pins of the fp8 layer oracle (the reference with quantised GEMM operands).

* With identity quantisers it must be the pinned plain sharded oracle, exactly:
  no product may be dropped, transposed or fed the wrong operand.
* With the gradient quantiser replaced by a doubling marker, every output must
  scale by the power of two that counts the gradient operands upstream of it:
  the E5M2 quantiser reaches exactly the gradient operands of the dgrad and
  wgrad products, and nothing else.
* Its forward matches an independent recomputation with library primitives:
  torch's float8_e4m3fn cast (after scaling and saturation) for the
  quantisation, torch's scaled_dot_product_attention and gelu.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import fp8 as Q
from oracle import fp8_layer as F
from oracle import shard as S
from tests.parity_util import f64, full_params

SHAPE = synth.LayerShape(hidden=32, heads=4, ffn=64, seq=9, micro_batch=1, tp=2)


def _inputs(seed=0):
    full = synth.layer_inputs(SHAPE, seed=seed)
    return full_params(full), f64(full["x"]), f64(full["dy"])


def _ident(x):
    return np.asarray(x, dtype=np.float64)


def _flat(out):
    yield "y", out["y"]
    yield "h", out["h"]
    yield "dh", out["dh"]
    yield "dx", out["dx"]
    for part in ("att", "mlp", "mlp_bwd", "attn_bwd"):
        for r, d in enumerate(out[part]):
            for k, v in d.items():
                yield f"{part}[{r}].{k}", v


def test_identity_quantisers_give_the_plain_oracle():
    p, x, g = _inputs()
    for residual in (False, True):
        a = F.sharded_layer(p, x, g, SHAPE.heads, SHAPE.tp, residual=residual, fq=_ident, gq=_ident)
        b = S.sharded_layer(p, x, g, SHAPE.heads, SHAPE.tp, residual=residual)
        for (ka, va), (kb, vb) in zip(_flat(a), _flat(b)):
            assert ka == kb
            np.testing.assert_allclose(va, vb, rtol=1e-12, atol=1e-14, err_msg=ka)


def test_gradient_quantiser_reaches_exactly_the_gradient_operands():
    p, x, g = _inputs(1)
    a = F.sharded_layer(p, x, g, SHAPE.heads, SHAPE.tp, fq=_ident, gq=lambda t: 2.0 * np.asarray(t))
    b = S.sharded_layer(p, x, g, SHAPE.heads, SHAPE.tp)
    # forward untouched
    for k in ("y", "h"):
        np.testing.assert_allclose(a[k], b[k], rtol=1e-12)
    # MLP: dz = 2 dz (dY doubled once); dW2 = 2x; dW1 and dh use doubled dz again: 4x
    for ra, rb in zip(a["mlp_bwd"], b["mlp_bwd"]):
        for k, m in (("dz", 2), ("dw2", 2), ("db1", 2), ("dw1", 4), ("dh_partial", 4), ("db2", 1)):
            np.testing.assert_allclose(ra[k], m * rb[k], rtol=1e-12, atol=1e-14, err_msg=k)
    # attention: dh arrives as 4 dh; do = 8 do; dqkv = 8 dqkv; dW_qkv and dx_partial 16x
    for ra, rb in zip(a["attn_bwd"], b["attn_bwd"]):
        for k, m in (("do", 8), ("dw_o", 8), ("db_o", 4), ("dqkv", 8), ("db_qkv", 8), ("dw_qkv", 16),
                     ("dx_partial", 16)):
            np.testing.assert_allclose(ra[k], m * rb[k], rtol=1e-11, atol=1e-14, err_msg=k)


def _torch_q4(x):
    """Scaled E4M3 quant-dequant through torch's float8_e4m3fn cast."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    amax = t.abs().max()
    s = torch.tensor(448.0, dtype=torch.float32) / amax if amax > 0 else torch.tensor(1.0)
    y = (t * s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64)
    return (y / s.double()).numpy()


def test_forward_matches_library_primitives():
    p, x, _ = _inputs(2)
    heads, tp = SHAPE.heads, SHAPE.tp
    lh, d = heads // tp, SHAPE.hidden // heads
    for r in range(tp):
        pr = S.shard_params(p, heads, tp, r)
        got_a = F.rank_attn_forward(pr, x, lh)
        qkv = _torch_q4(x) @ _torch_q4(pr["w_qkv"]) + pr["b_qkv"]
        np.testing.assert_allclose(got_a["qkv"], qkv, rtol=1e-12, atol=1e-14)
        t = torch.from_numpy(qkv).view(SHAPE.seq, lh, 3, d)
        q, k, v = (t[:, :, j].permute(1, 0, 2) for j in range(3))
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
        o = o.permute(1, 0, 2).reshape(SHAPE.seq, lh * d).numpy()
        np.testing.assert_allclose(got_a["o"], o, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(got_a["partial"], _torch_q4(got_a["o"]) @ _torch_q4(pr["w_o"]), rtol=1e-10,
                                   atol=1e-12)
        got_m = F.rank_mlp_forward(pr, x)
        z = _torch_q4(x) @ _torch_q4(pr["w1"]) + pr["b1"]
        a = torch.nn.functional.gelu(torch.from_numpy(z)).numpy()
        np.testing.assert_allclose(got_m["z"], z, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got_m["partial"], _torch_q4(a) @ _torch_q4(pr["w2"]), rtol=1e-10, atol=1e-12)


def test_recipe_moves_by_more_than_the_bf16_bound_under_last_bit_perturbations():
    """Why the fp8 layer is not compared element-wise with the quantised-operand
    reference: two runs of the recipe whose stored intermediates differ by a
    relative 2^-10 (about half a bf16 step, what a different fp32 summation
    order gives) quantise a few per cent of those intermediates to a code one
    step away, and the outputs behind them move by more than the bf16 bound."""
    from tests.parity_util import BF16_REL, f64, full_params
    shape = synth.LayerShape(hidden=512, heads=4, ffn=2048, seq=256, micro_batch=1, tp=1)
    full = synth.layer_inputs(shape, seed=0)
    p, x, g = full_params(full), f64(full["x"]), f64(full["dy"])
    rng = np.random.default_rng(5)
    bf = lambda t: synth.bf16_bits_to_f64(synth.bf16_round_bits(np.asarray(t, dtype=np.float64)))
    nz = lambda t: bf(np.asarray(t) * (1 + 2.0 ** -10 * rng.standard_normal(np.shape(t))))
    a = F.sharded_layer(p, x, g, shape.heads, 1, fq=lambda t: F.q4(bf(t)), gq=lambda t: F.q5(bf(t)))
    b = F.sharded_layer(p, x, g, shape.heads, 1, fq=lambda t: F.q4(nz(t)), gq=lambda t: F.q5(nz(t)))
    moved = {k: float(np.max(np.abs(a[k] - b[k])) / np.max(np.abs(a[k]))) for k in ("y", "dh", "dx")}
    print(moved)
    assert all(v > BF16_REL for v in moved.values()), moved
