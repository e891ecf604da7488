"""Parity of the MoE router on the GPU (mtl_moe_router_fwd, mtl_moe_route,
mtl_moe_router_bwd) against the fp64 router oracle.

The logits are compared with x . W_r to the bf16 tolerance; the routing is
then checked bit for bit (ids) and to fp32 rounding (gates) against the
oracle's top-k of the device's own fp32 logits, so that both sides take every
selection from the same values.  dlogits (gate backward plus load-balancing
gradient, fp32 arithmetic) and the loss value are compared tightly; the
load-balancing gradient alone (dgates = 0) gets its own check, since next to
the gate gradient it is orders of magnitude smaller.  dW_r and the router's dX
are bf16-operand products: bf16 tolerance.
"""
import numpy as np
import pytest

import synth
from oracle import moe as M
from oracle import router as R
from tests.parity_util import assert_bf16, f64

MS = synth.MoeShape
CASES = {
    # (shape, alpha)
    "small-a0.5": (MS(tokens=200, hidden=128, ffn=8, experts=32, topk=4, ep=1), 0.5),
    "ragged": (MS(tokens=77, hidden=64, ffn=8, experts=16, topk=3, ep=1), 0.001),
    "all-experts": (MS(tokens=64, hidden=64, ffn=8, experts=8, topk=8, ep=1), 0.1),
    "512-experts": (MS(tokens=50, hidden=96, ffn=8, experts=512, topk=8, ep=1), 0.01),
    "full-256e-top8": (MS(tokens=4096, hidden=7168, ffn=8, experts=256, topk=8, ep=16), 0.001),
}
TIGHT = 1e-4


def _tight(name, got, ref, floor=0.0):
    """max|diff| <= TIGHT * max|ref|, element-wise relaxed by `floor`."""
    scale = float(np.max(np.abs(ref)))
    bad = np.abs(got - ref) > TIGHT * scale + floor
    assert not bad.any(), f"{name}: {int(bad.sum())} elements off, max|diff| {np.max(np.abs(got - ref)):.3e}, " \
                          f"max|ref| {scale:.3e}"


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(CASES))
def test_router_matches_oracle(mtl, case):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    from megatron_tensor_transformer_layer_amd.moe import Router
    shape, alpha = CASES[case]
    T, E, k = shape.tokens, shape.experts, shape.topk
    print(f"router case {case} {shape} alpha={alpha}", flush=True)
    xb = synth.moe_tokens(shape, 0, "moe_x")
    wb = synth.router_weight(shape)
    dg = synth.gate_grads(shape)
    x, w = bf16_dev(xb), bf16_dev(wb)
    r = Router(T, shape.hidden, E, k, w, aux_coeff=alpha)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, k, dtype=torch.float32, device="cuda")
    logits = r.forward(x)
    mtl.mtl_moe_route(r.cfg, logits, idx, gates)
    dgates = torch.from_numpy(dg).cuda()
    r.backward(x, idx, gates, dgates)
    torch.cuda.synchronize()
    got = dict(logits=logits.cpu().numpy(), idx=idx.cpu().numpy(), gates=gates.cpu().numpy(),
               dlogits=r.dlogits.cpu().numpy().astype(np.float64), dw_r=r.dw_r.cpu().numpy().astype(np.float64),
               dx=f64(r.dx.cpu().view(torch.int16).numpy().view(np.uint16)), aux=float(r.aux_loss.item()))
    # the load-balancing gradient alone
    r.backward(x, idx, gates, torch.zeros_like(dgates))
    torch.cuda.synchronize()
    got_aux_grad = r.dlogits.cpu().numpy().astype(np.float64)

    X, W = f64(xb), f64(wb)
    assert_bf16("logits", got["logits"].astype(np.float64), R.router_forward(X, W))
    ref_idx, ref_gates = M.route_topk(got["logits"], k)
    assert np.array_equal(got["idx"], ref_idx)
    assert np.max(np.abs(got["gates"] - ref_gates)) <= 1e-6
    L = got["logits"].astype(np.float64)
    bw = R.router_backward(X, W, L, got["idx"], got["gates"], dg, alpha)
    _tight("dlogits", got["dlogits"], bw["dlogits"])
    # dL_aux/dl_te = coef p_te (c_e - q_t) cancels where c_e ~ q_t = sum_e p_te c_e (every count equal, as
    # with k = E, makes it exactly 0): allow fp32 rounding of the cancelling terms, coef p_te q_t
    coef = alpha * E / (T * T * k)
    p = R.softmax_rows(L)
    q = np.sum(p * R.expert_counts(got["idx"], E), axis=1, keepdims=True)
    _tight("load-balancing dlogits", got_aux_grad,
           R.router_backward(X, W, L, got["idx"], got["gates"], np.zeros_like(dg), alpha)["dlogits"],
           floor=1e-5 * coef * p * q)
    assert abs(got["aux"] - bw["aux"]) <= 1e-5 * abs(bw["aux"]), (got["aux"], bw["aux"])
    assert_bf16("dw_r", got["dw_r"], bw["dw_r"])
    assert_bf16("dx", got["dx"], bw["dx"])


@pytest.mark.gpu
def test_router_wgrad_accumulates(mtl):
    import torch
    from megatron_tensor_transformer_layer_amd import MTL_F_WGRAD_ACCUM
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    from megatron_tensor_transformer_layer_amd.moe import Router
    shape = MS(tokens=77, hidden=64, ffn=8, experts=16, topk=3, ep=1)
    x, w = bf16_dev(synth.moe_tokens(shape, 0, "moe_x")), bf16_dev(synth.router_weight(shape))
    idx = torch.empty(shape.tokens, shape.topk, dtype=torch.int32, device="cuda")
    gates = torch.empty(shape.tokens, shape.topk, dtype=torch.float32, device="cuda")
    dgates = torch.from_numpy(synth.gate_grads(shape)).cuda()
    outs = []
    for flags in (0, MTL_F_WGRAD_ACCUM):
        r = Router(shape.tokens, shape.hidden, shape.experts, shape.topk, w, flags=flags)
        mtl.mtl_moe_route(r.cfg, r.forward(x), idx, gates)
        r.backward(x, idx, gates, dgates)
        r.backward(x, idx, gates, dgates)
        torch.cuda.synchronize()
        outs.append(r.dw_r.cpu().numpy())
    assert np.array_equal(outs[1], 2 * outs[0])
