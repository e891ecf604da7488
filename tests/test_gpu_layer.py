"""Parity of the whole tensor-parallel layer step on the GPU against the fp64
oracle of the unsharded layer: all t rank shards run on one device through the
C ABI, the four reductions add their partials, and every output (Y, dX, H, dH,
the concatenated QKV/O/A and GeLU'(Z), every weight and bias gradient) must match the
oracle to the bf16 tolerance."""
import numpy as np
import pytest

import synth
from oracle import layer as L
from tests.parity_util import assert_bf16, f64, full_params

CASES = {
    # the GPT-2-small layer split over TP=2 (both shards on one device)
    "gpt2-small-tp2": (synth.WORKLOADS["gpt2-small-tp2"], False),
    # ragged: 77 tokens (not a multiple of any tile), d = 64
    "ragged-d64-tp2": (synth.LayerShape(hidden=128, heads=2, ffn=256, seq=77, micro_batch=1, tp=2), False),
    # ragged, d = 128, two micro-batch elements, ffn/t = 264
    "ragged-d128-mb2-tp2": (synth.LayerShape(hidden=256, heads=2, ffn=528, seq=200, micro_batch=2, tp=2), False),
    # TP=4 with residual connections
    "tp4-residual": (synth.LayerShape(hidden=512, heads=8, ffn=1024, seq=130, micro_batch=1, tp=4), True),
    # TP=1: the plain layer; single token
    "tp1-one-token": (synth.LayerShape(hidden=128, heads=2, ffn=256, seq=1, micro_batch=1, tp=1), False),
}


def _run(shape, residual, seed=0):
    from megatron_tensor_transformer_layer_amd.layer import run_sharded_layer
    full = synth.layer_inputs(shape, seed=seed)
    shards = [synth.layer_inputs(shape, seed=seed, tp=shape.tp, rank=r) for r in range(shape.tp)]
    got = run_sharded_layer(shape, shape.tp, shards, full["x"], full["b_o"], full["b2"], full["dy"], residual)
    return full, got


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(CASES))
def test_layer_matches_oracle(mtl, case):
    shape, residual = CASES[case]
    print(f"case {case} {shape} residual={residual}", flush=True)
    full, got = _run(shape, residual)
    p = full_params(full)
    x, g = f64(full["x"]), f64(full["dy"])
    fwd = L.layer_forward(p, x, shape.heads, shape.micro_batch, residual)
    bwd = L.layer_backward(p, x, fwd, g, shape.heads, shape.micro_batch, residual)
    for k in ("qkv", "o", "lse", "h", "a", "y"):
        assert_bf16(k, got[k], fwd[k])
    assert_bf16("gz", got["gz"], L.gelu_grad(fwd["z"]))
    assert_bf16("dh", got["dh"], bwd["dh"])
    for k in ("dx", "dw_qkv", "db_qkv", "dw_o", "db_o", "dw1", "db1", "dw2", "db2"):
        assert_bf16(k, got[k], bwd[k])
    for r in range(shape.tp):  # every rank computes the same row-parallel bias gradients
        assert np.array_equal(got["db_o_all"][r], got["db_o"])
        assert np.array_equal(got["db2_all"][r], got["db2"])


@pytest.mark.gpu
def test_layer_is_deterministic(mtl):
    shape = CASES["ragged-d128-mb2-tp2"][0]
    _, a = _run(shape, False)
    _, b = _run(shape, False)
    for k in a:
        if isinstance(a[k], list):
            continue
        assert np.array_equal(a[k], b[k]), k
