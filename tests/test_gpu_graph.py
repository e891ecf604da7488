"""The whole small layer captured into a HIP graph: every replay gives the eager
step's outputs bit for bit, with the program's own eager work and
synchronisations between the replays (the step's kernels are deterministic,
and none of its calls records a memset into the graph)."""
import numpy as np
import pytest

import synth


def _snapshot(outs):
    return {k: v.clone() for k, v in outs.items()}


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["gpt2-small-tp2", "ragged-tp2-fp8", "ragged-tp2-fp8-kept", "gpt2-small-tp2-concurrent"])
def test_graph_replays_match_eager_step(mtl, case):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import AllShardsStep
    if case.startswith("gpt2-small-tp2"):
        shape, prec = synth.WORKLOADS["gpt2-small-tp2"], mtl.MTL_PREC_BF16
    else:
        shape, prec = synth.LayerShape(hidden=256, heads=2, ffn=544, seq=208, micro_batch=1, tp=2), \
            mtl.MTL_PREC_FP8_HYBRID
    print(f"graph case {case} {shape}", flush=True)
    full = synth.layer_inputs(shape, seed=0)
    shards = [synth.layer_inputs(shape, seed=0, tp=shape.tp, rank=r) for r in range(shape.tp)]
    flags = mtl.MTL_F_FP8_KEEP_CODES if case.endswith("kept") else 0
    step = AllShardsStep(shape, shape.tp, shards, full["x"], full["dy"], full["b_o"], full["b2"], precision=prec,
                         concurrent=case.endswith("concurrent"), flags=flags)
    step()
    torch.cuda.synchronize()
    eager = _snapshot(step.outputs())
    if step.streams is not None:  # the concurrent step equals the shards run one after the other
        serial = AllShardsStep(shape, shape.tp, shards, full["x"], full["dy"], full["b_o"], full["b2"],
                               precision=prec)
        serial()
        torch.cuda.synchronize()
        assert all(torch.equal(serial.outputs()[k], eager[k]) for k in eager)
        del serial

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    g = torch.Generator(device="cuda").manual_seed(3)
    for rep in range(3):
        for v in step.outputs().values():  # poison every output between replays
            v.copy_(torch.full_like(v, float("nan")))
        a = torch.randn(512, 512, device="cuda", generator=g)
        _ = (a @ a).sum().item()  # unrelated eager work, then a synchronisation
        graph.replay()
        torch.cuda.synchronize()
        got = step.outputs()
        bad = [k for k in eager if not torch.equal(got[k], eager[k])]
        assert not bad, f"replay {rep}: {bad}"
    # the eager step still runs after the graph and agrees
    step()
    torch.cuda.synchronize()
    assert all(torch.equal(step.outputs()[k], eager[k]) for k in eager)
    assert np.isfinite(step.outputs()["y"].float().cpu().numpy()).all()
