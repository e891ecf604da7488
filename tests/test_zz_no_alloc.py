"""mtl_mlp_bwd_noalloc (scratch in a device array held by the library) against
mtl_mlp_bwd (scratch from the caller) on the same inputs: every output
bit-identical (the same kernels in the same order), on calls in a row whose
sizes shrink, so that each later call finds the earlier call's contents in
the array."""
import numpy as np
import pytest

import synth

CASES = [
    # the 96-layer-GPT-shaped TP=8 rank: the largest MLP backward of the workloads (35 MiB of scratch)
    ("gpt96l-tp8", synth.WORKLOADS["gpt96l-tp8"], 0),
    # ragged and smaller
    ("ragged-tp2", synth.LayerShape(hidden=256, heads=2, ffn=544, seq=208, micro_batch=1, tp=2), 0),
    # fp8 codes fit at this size
    ("ragged-tp2-fp8", synth.LayerShape(hidden=256, heads=2, ffn=544, seq=208, micro_batch=1, tp=2), 1),
]


@pytest.mark.gpu
def test_noalloc_mlp_backward_matches_mlp_backward(mtl):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev, dims_of
    for name, shape, prec in CASES:
        print(f"noalloc case {name} {shape} precision={prec}", flush=True)
        t, r = shape.tp, 0
        cfg = mtl.make_cfg(shape.hidden, shape.heads, shape.ffn, shape.seq, shape.micro_batch, t, r, prec)
        D = dims_of(shape.hidden, shape.heads, shape.ffn, shape.seq, shape.micro_batch, t)
        inp = synth.layer_inputs(shape, tp=t, rank=r)
        w1, w2, dy = bf16_dev(inp["w1"]), bf16_dev(inp["w2"]), bf16_dev(inp["dy"])
        h = bf16_dev(synth.layer_tensor(shape, "h"))
        g = torch.Generator(device="cuda").manual_seed(11)
        gz = (torch.rand(D.S, D.f_l, device="cuda", generator=g) * 1.2 - 0.1).to(torch.bfloat16)
        a = torch.randn(D.S, D.f_l, device="cuda", generator=g).to(torch.bfloat16)

        def outputs():
            return dict(dh=torch.empty(D.S, D.h, dtype=torch.bfloat16, device="cuda"),
                        dw1=torch.empty(D.h, D.f_l, device="cuda"), db1=torch.empty(D.f_l, device="cuda"),
                        dw2=torch.empty(D.f_l, D.h, device="cuda"), db2=torch.empty(D.h, device="cuda"))

        ref, got = outputs(), outputs()
        scratch = torch.empty(mtl.mtl_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
        mtl.mtl_mlp_bwd(cfg, dy, h, gz, a, w1, w2, ref["dh"], ref["dw1"], ref["db1"], ref["dw2"], ref["db2"], scratch)
        mtl.mtl_mlp_bwd_noalloc(cfg, dy, h, gz, a, w1, w2, got["dh"], got["dw1"], got["db1"], got["dw2"], got["db2"])
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"{name}: {k} differs"
        assert np.isfinite(got["dw1"].cpu().numpy()).all()
        del scratch, ref, got, w1, w2, dy, h, gz, a
        torch.cuda.empty_cache()


@pytest.mark.gpu
def test_noalloc_refuses_what_does_not_fit(mtl):
    """A configuration whose MLP backward needs more than the array is refused
    with MTL_E_WORKSPACE before any launch (the pointers are never used)."""
    import ctypes
    cfg = mtl.make_cfg(4096, 32, 32768, 4096, 1, 4, 0)
    P = 1 << 20
    st = mtl.lib().mtl_mlp_bwd_noalloc(ctypes.byref(cfg), *([P] * 11), None)
    assert st == mtl.MTL_E_WORKSPACE
