"""Throughput of one tensor-parallel rank's transformer-layer training step on one MI355X.

A step is the rank's whole share of the layer's forward and backward pass:
column-parallel QKV projection, causal attention over its heads, row-parallel
output projection, the all-reduce stand-in, column-parallel fc1 with GeLU,
row-parallel fc2, all-reduce stand-in; then the backward of all of it (dgrad
and wgrad of every linear, bias gradients, attention backward) with its two
all-reduce stand-ins.  Each all-reduce stands in as its two halves on one GPU:
the rank's reduce-scatter share (rows [rank*S/t, (rank+1)*S/t) summed over its
own partial and t-1 resident peer partials) and the all-gather of the peers'
t-1 reduced shares into its full buffer.

Prints one JSON line.  Default workload: rank 0 of a 96-layer-GPT-shaped layer
at TP=8 (hidden 8192, 64 heads, ffn 32768, seq 4096, micro-batch 1, bf16);
--workload 7b-tp4 is rank 0 of a 7B-class layer at TP=4; --workload
gpt2-small-tp2 is the whole GPT-2-small layer (both TP=2 shards and the four
full reductions) replayed as one HIP graph.  Besides the K timed steps, the
line carries a window of steps timed per launch group with HIP events inside
the library (mtl_prof_*: the whole-step GEMM rate, the attention rate, the
HBM rate of the memory-bound kernels) and three windows of at least 20 steps
(each window's mean, the worst window, P50/P95 over their steps).

With --workload moe-256e-top8-ep16 the step is one expert-parallel rank's MoE
expert block instead (route, permute, grouped expert GEMMs, combine, backward);
with --workload cp4-seq32k-7b-tp4 it is one context-parallel rank's causal
attention share, forward and backward (by default the last of 4 ranks of a
32768-token sequence: its own chunk causally and the three earlier chunks in
full); with --workload mxfp4-gemm-7b-tp4 (or mxfp6-gemm-7b-tp4) it is the
rank's fc1 GEMM in MXFP4 (MXFP6): both operands quantised, then the
block-scaled MFMA GEMM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA
PEAK_FP4_TFLOPS = 10066.3  # MI355X dense fp4 / fp6 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt96l-tp8")
    ap.add_argument("--rank", type=int, default=None,
                    help="the rank whose share runs (default 0; for a CP workload the last, busiest rank)")
    ap.add_argument("--precision", choices=("bf16", "fp8", "mxfp4"), default="bf16",
                    help="fp8: the linears' GEMMs on per-tensor scaled E4M3/E5M2 codes (--fp8-format hybrid); "
                         "mxfp4: on MXFP4 codes blocked along each product's contraction")
    ap.add_argument("--sp", action="store_true",
                    help="sequence parallel: X, H, dY, dH arrive as row shares and are gathered in place "
                         "(mtl_allgather_rows) before each column-parallel linear")
    ap.add_argument("--router", action="store_true",
                    help="with an MoE workload: time the router alone (linear, top-k routing, gate and "
                         "load-balancing backward, dW_r and dX) over all tokens")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seq", type=int, default=4096)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (for scaling HBM byte counters)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="time the MFMA-only kernel (the 256x256-tile GEMM's MFMA stream of a 4096^3 product with "
                         "every operand in registers) in bf16 and fp8 on N(0,1) operands, and exit")
    ap.add_argument("--copy-rate", action="store_true",
                    help="time the plain copy at 64 MiB, 256 MiB and 1 GiB (the practical HBM ceiling) and exit")
    return ap.parse_args()


HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(HERE, "megatron_tensor_transformer_layer_amd", "csrc", "gemm.hip")
COPY_BYTES = 64 << 20  # one 32 Mi-element bf16 tensor read and written


def gemm_source_hash() -> str:
    import hashlib
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def calibrate_copy():
    """A plain copy of COPY_BYTES/2 bytes through the library (mtl_reduce with a
    single partial, no bias, no residual): reads and writes exactly that many bytes."""
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_reduce
    n = COPY_BYTES // 2 // 2
    rows, cols = n // 4096, 4096
    src = torch.randn(rows, cols, device="cuda").to(torch.bfloat16)
    dst = torch.empty_like(src)
    for _ in range(3):
        mtl_reduce([src], None, None, dst, rows, cols)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    print(json.dumps({"copy_kernel": "reduce_partials_kernel (t=1)", "bytes_read": rows * cols * 2,
                      "bytes_written": rows * cols * 2, "launches": 3}), flush=True)


def copy_rate():
    """The rate the plain copy of calibrate_copy reaches, read + written bytes
    over the launch time (HIP events, 20 launches), at 64 MiB, 256 MiB and
    1 GiB: the practical HBM ceiling of the streaming kernels."""
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_reduce
    cols = 4096
    for mib in (64, 256, 1024):
        rows = (mib << 20) // 2 // cols
        src = torch.randn(rows, cols, device="cuda").to(torch.bfloat16)
        dst = torch.empty_like(src)
        for _ in range(3):
            mtl_reduce([src], None, None, dst, rows, cols)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for _ in range(reps):
            mtl_reduce([src], None, None, dst, rows, cols)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        print(json.dumps({"copy_mib": mib, "us_per_launch": round(us, 2),
                          "gb_per_s": round(2 * rows * cols * 2 / us / 1e3, 1)}), flush=True)
        del src, dst


def mfma_ceiling():
    """The matrix cores' own rate: mtl_mfma_ceiling issuing the MFMAs of a
    4096x4096x4096 product in 256x256 tiles (256 workgroups of 4 waves) with
    every operand in registers, on N(0,1) bf16 values, on their E4M3 codes and
    on their MXFP4 codes; HIP events around 20 launches after 3 untimed ones."""
    import torch
    from megatron_tensor_transformer_layer_amd import (MTL_CEILING_DATA_BYTES, mtl_mfma_ceiling,
                                                       mtl_mxfp4_quantize)
    g = torch.Generator(device="cuda").manual_seed(0)
    wgs = 256
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    for kind, name, iters, per_iter, peak in ((0, "bf16", 128, 1 << 20, PEAK_BF16_TFLOPS),
                                               (1, "fp8", 64, 2 << 20, PEAK_FP8_TFLOPS),
                                               (2, "mxfp4", 64, 2 << 20, PEAK_FP4_TFLOPS)):
        n = MTL_CEILING_DATA_BYTES // 2 if kind == 0 else MTL_CEILING_DATA_BYTES * (2 if kind == 2 else 1)
        vals = torch.randn(n, device="cuda", generator=g)
        if kind == 2:
            data = torch.empty(MTL_CEILING_DATA_BYTES, dtype=torch.uint8, device="cuda")
            scales = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
            mtl_mxfp4_quantize(vals.to(torch.bfloat16), 1024, n // 1024, data, scales)
        else:
            data = vals.to(torch.bfloat16) if kind == 0 else vals.to(torch.float8_e4m3fn)
        for _ in range(3):
            mtl_mfma_ceiling(data, kind, wgs, iters, out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for _ in range(reps):
            mtl_mfma_ceiling(data, kind, wgs, iters, out)
        e1.record()
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        us = e0.elapsed_time(e1) * 1e3 / reps
        flop = wgs * 4 * iters * per_iter
        print(json.dumps({"mfma_ceiling": name, "flop_per_launch": flop, "workgroups": wgs, "iters": iters,
                          "us_per_launch": round(us, 2), "tflops": round(flop / us / 1e6, 1),
                          "frac_of_peak": round(flop / us / 1e6 / peak, 4), "peak": peak}), flush=True)


def cpu_baseline(shape, rank, sample_seq, precision="bf16"):
    """The oracle (fp64 numpy, as it stands) on a bounded sample: the same rank's
    forward + backward over the first sample_seq tokens (for fp8 and mxfp4, the
    reference with quantised GEMM operands)."""
    import synth
    from oracle import layer as L
    from oracle import shard as S
    if precision == "fp8":
        from oracle import fp8_layer as S  # noqa: F811 -- same rank functions, quantised operands
    elif precision == "mxfp4":
        from oracle import mx_layer as S  # noqa: F811

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    sub = synth.LayerShape(hidden=shape.hidden, heads=shape.heads, ffn=shape.ffn, seq=sample_seq,
                           micro_batch=1, tp=shape.tp)
    inp = synth.layer_inputs(sub, tp=shape.tp, rank=rank)
    f = {k: synth.bf16_bits_to_f64(v) for k, v in inp.items()}
    hh = synth.bf16_bits_to_f64(synth.layer_tensor(sub, "h"))
    dh = synth.bf16_bits_to_f64(synth.layer_tensor(sub, "dh"))
    lh = shape.heads // shape.tp
    t0 = time.perf_counter()
    att = S.rank_attn_forward(f, f["x"], lh)
    mlp = S.rank_mlp_forward(f, hh)
    S.rank_mlp_backward(f, f["dy"], hh, mlp["z"], mlp["a"])
    S.rank_attn_backward(f, dh, f["x"], att["qkv"], lh)
    dt = time.perf_counter() - t0
    flops = L.layer_flops(shape.hidden, shape.heads, shape.ffn, sample_seq, 1, shape.tp)["total"]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"rank {rank} shard forward+backward on the first {sample_seq} of {shape.seq} tokens "
                      f"(fp64 numpy{'' if precision == 'bf16' else ', ' + precision + ' quant-dequant operands'}), "
                      f"{dt:.2f} s"}


def moe_cpu_baseline(shape, rank, sample_tokens, sample_ffn):
    """The MoE oracle (fp64 numpy, as it stands) on a bounded sample of the
    workload: the first sample_tokens tokens, routed as in the full run, with
    every expert's ffn width cut to sample_ffn."""
    import synth
    from oracle import moe as M

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    sub = synth.MoeShape(tokens=sample_tokens, hidden=shape.hidden, ffn=sample_ffn, experts=shape.experts,
                         topk=shape.topk, ep=shape.ep, zipf_s=shape.zipf_s)
    lo, hi = M.local_range(shape.experts, shape.ep, rank)
    w1 = np.stack([synth.bf16_bits_to_f64(synth.moe_expert_weight(sub, "moe_w1", e)) for e in range(lo, hi)])
    w2 = np.stack([synth.bf16_bits_to_f64(synth.moe_expert_weight(sub, "moe_w2", e)) for e in range(lo, hi)])
    logits = synth.moe_logits(shape)[:sample_tokens]
    x = synth.bf16_bits_to_f64(synth.moe_tokens(sub, 0, "moe_x"))
    dy = synth.bf16_bits_to_f64(synth.moe_tokens(sub, 0, "moe_dy"))
    t0 = time.perf_counter()
    fwd = M.moe_forward(x, w1, w2, logits, shape.topk, shape.ep, rank)
    M.moe_backward(x, w1, w2, fwd, dy)
    dt = time.perf_counter() - t0
    flops = M.moe_flops(fwd["counts"], shape.hidden, sample_ffn)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"EP rank {rank} expert block forward+backward on the first {sample_tokens} of {shape.tokens} "
                      f"tokens ({int(fwd['offsets'][-1])} local assignments) with ffn cut to {sample_ffn} "
                      f"(fp64 numpy), {dt:.2f} s"}


def router_cpu_baseline(shape, sample_tokens, alpha):
    """The router oracle (fp64 numpy) on the first sample_tokens tokens."""
    import synth
    from oracle import moe as M
    from oracle import router as R
    x = synth.bf16_bits_to_f64(synth.moe_tokens(shape, 0, "moe_x"))[:sample_tokens]
    w = synth.bf16_bits_to_f64(synth.router_weight(shape))
    dg = synth.gate_grads(shape)[:sample_tokens].astype(np.float64)
    t0 = time.perf_counter()
    logits = R.router_forward(x, w)
    idx, gates = M.route_topk(logits, shape.topk)
    R.router_backward(x, w, logits, idx, gates, dg, alpha)
    dt = time.perf_counter() - t0
    fl = 6.0 * sample_tokens * shape.hidden * shape.experts
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"router forward+backward on the first {sample_tokens} of {shape.tokens} tokens "
                      f"(fp64 numpy), {dt:.2f} s"}


def router_main(args):
    """The MoE router over all tokens: logits = x W_r, top-k routing, the gate
    and load-balancing backward into the logits, dW_r and the router's dX."""
    import torch
    import synth
    from megatron_tensor_transformer_layer_amd import mtl_moe_route
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    from megatron_tensor_transformer_layer_amd.moe import Router

    shape = synth.MOE_WORKLOADS[args.workload]
    T, E, k, alpha = shape.tokens, shape.experts, shape.topk, 0.001
    x = bf16_dev(synth.moe_tokens(shape, 0, "moe_x"))
    ro = Router(T, shape.hidden, E, k, bf16_dev(synth.router_weight(shape)), aux_coeff=alpha)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, k, dtype=torch.float32, device="cuda")
    dgates = torch.from_numpy(synth.gate_grads(shape)).cuda()

    def step():
        mtl_moe_route(ro.cfg, ro.forward(x), idx, gates)
        ro.backward(x, idx, gates, dgates)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    fl = 6.0 * T * shape.hidden * E  # the three router products, 2*T*h*E FLOP each
    out = {
        "metric": "TFLOP/s of the MoE router fwd+bwd (bf16 GEMMs) and % of MI355X MFMA peak",
        "value": round(fl / (ms / 1e3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1) tokens, N(0,0.02) router weight, N(0,1) gate gradients)",
        "config": {"workload": f"{args.workload} router: {T} tokens, hidden {shape.hidden}, {E} experts, "
                               f"top-{k}, load-balancing coefficient {alpha}",
                   "global_batch": 1, "seq_len": T, "parallelism": "router-replicated-1gpu"},
        "pct_of_peak": round(100 * fl / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "flop_per_step": fl,
        "roofline": None,
        "cpu_baseline": None if args.no_cpu_baseline else router_cpu_baseline(shape, 1024, alpha),
    }
    print(json.dumps(out), flush=True)


def cp_flops(chunk, heads, d, rank):
    """Algorithmic FLOP of CP rank `rank`'s causal attention forward: QK^T and
    PV over the causal triangle of its own chunk (C(C+1)/2 scores) and over
    every score of the `rank` earlier chunks, 2 products x 2 FLOP per score and
    dimension."""
    return float(heads) * (2.0 * chunk * (chunk + 1) * d + rank * 4.0 * chunk * chunk * d)


def cp_cpu_baseline(shape, rank, sample_seq, sample_heads):
    """The CP oracle (fp64 numpy, as it stands) on a bounded sample of the
    workload: the same rank of the same CP degree over a sequence of sample_seq
    tokens with sample_heads heads, forward and backward."""
    import synth
    from oracle import cp as CP
    sub = synth.CpShape(seq=sample_seq, heads=sample_heads, head_dim=shape.head_dim, cp=shape.cp)
    full = synth.bf16_bits_to_f64(synth.cp_qkv(sub))
    do = synth.bf16_bits_to_f64(synth.cp_dout(sub))
    t0 = time.perf_counter()
    CP.rank_attention(full, sub.heads, sub.cp, rank)
    CP.rank_attention_backward(full, do, sub.heads, sub.cp, rank)
    dt = time.perf_counter() - t0
    fl = 3.0 * cp_flops(sub.chunk, sub.heads, sub.head_dim, rank)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"rank {rank} of CP {sub.cp} over a {sample_seq}-token sequence (chunks of {sub.chunk}), "
                      f"{sample_heads} of {shape.heads} heads, forward+backward (fp64 numpy), {dt:.2f} s"}


def cp_main(args):
    """One context-parallel rank's causal attention share, forward and backward
    (mtl_cp_attn_fwd, mtl_cp_attn_bwd): its chunk's queries against its own
    chunk (causal) and every earlier chunk, merged by log-sum-exp; then dQ of
    its queries and the dK/dV shares of every chunk up to its own."""
    import torch
    import synth
    from megatron_tensor_transformer_layer_amd import (mtl_cp_attn_bwd, mtl_cp_attn_bwd_scratch_bytes,
                                                       mtl_cp_attn_fwd, mtl_cp_attn_scratch_bytes)
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev

    shape = synth.CP_WORKLOADS[args.workload]
    C, H, d, cp = shape.chunk, shape.heads, shape.head_dim, shape.cp
    r = cp - 1 if args.rank is None else args.rank
    bits = synth.cp_qkv(shape)
    qkv = bf16_dev(bits)
    dout = bf16_dev(synth.cp_dout(shape))
    ld = 3 * H * d
    chunks = [qkv.data_ptr() + j * C * ld * 2 for j in range(cp)]
    o = torch.empty(C, H * d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(H, C, dtype=torch.float32, device="cuda")
    dqkv = torch.empty(C, ld, dtype=torch.bfloat16, device="cuda")
    dkv = [torch.empty(C, ld, dtype=torch.bfloat16, device="cuda") for _ in range(r)]
    nf = mtl_cp_attn_scratch_bytes(cp, r, C, H, d)
    nbw = mtl_cp_attn_bwd_scratch_bytes(cp, r, C, H, d)
    scratch = torch.empty(max(nf, nbw, 1), dtype=torch.uint8, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = []

    def step(record=False):
        e = [ev(), ev(), ev()] if record else None
        if record:
            e[0].record()
        mtl_cp_attn_fwd(cp, r, C, H, d, chunks, o, lse, scratch, nf)
        if record:
            e[1].record()
        mtl_cp_attn_bwd(cp, r, C, H, d, chunks, o, lse, dout, dqkv, dkv, scratch, nbw)
        if record:
            e[2].record()
            marks.append(e)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    fwd_ms = float(np.mean([m[0].elapsed_time(m[1]) for m in marks]))
    bwd_ms = float(np.mean([m[1].elapsed_time(m[2]) for m in marks]))
    ffl = cp_flops(C, H, d, r)
    fl = 3.0 * ffl  # the backward counts twice the forward
    achieved = 2.0 * ffl / (bwd_ms / 1e3) / 1e12
    out = {
        "metric": "TFLOP/s of one CP rank's causal attention share fwd+bwd (bf16) and % of MI355X MFMA peak",
        "value": round(fl / (ms / 1e3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": f"synthetic (QKV N(0,{synth.CP_QKV_STD:.2f}), the spread of a projection of N(0,1) activations; "
                f"dO N(0,1))",
        "config": {"workload": f"{args.workload}: CP rank {r} of {cp}, sequence {shape.seq} in chunks of {C}, "
                               f"{H} heads of {d}; its chunk causal + {r} earlier chunks, log-sum-exp merge; "
                               f"backward to dQ and the dK/dV shares of chunks 0..{r}",
                   "global_batch": 1, "seq_len": shape.seq, "parallelism": f"cp{cp}-rank{r}-of-1gpu"},
        "pct_of_peak": round(100 * fl / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "flop_per_step": fl,
        "roofline": {"bound": "mfma",
                     "kernel": "attn_bwd_kernel<128> (causal and unmasked variants) with the D and dQ-sum "
                               "launches: the whole mtl_cp_attn_bwd call (2x the forward FLOP), timed with HIP "
                               "events on its stream",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "bwd_call_us": round(bwd_ms * 1e3, 1), "fwd_call_us": round(fwd_ms * 1e3, 1),
                     "fwd_tflops": round(ffl / (fwd_ms / 1e3) / 1e12, 1)},
        "cpu_baseline": None if args.no_cpu_baseline else cp_cpu_baseline(shape, r, 8192, 8),
    }
    print(json.dumps(out), flush=True)


def mx_cpu_baseline(shape, sample_rows):
    """The MX oracle (fp64, as it stands) on a bounded sample: quantise
    sample_rows rows of A and of B and multiply them (sample_rows^2 outputs)."""
    import synth
    from oracle import mxfp4 as MX
    a = synth.bf16_bits_to_f64(synth.mx_operand(shape.M, shape.K, "mx_a", 1.0)[:sample_rows])
    b = synth.bf16_bits_to_f64(synth.mx_operand(shape.N, shape.K, "mx_b", synth.WEIGHT_STD)[:sample_rows])
    t0 = time.perf_counter()
    ca, sa = MX.quantize(a, shape.elem)
    cb, sb = MX.quantize(b, shape.elem)
    MX.gemm(ca, sa, cb, sb, shape.elem)
    dt = time.perf_counter() - t0
    fl = 2.0 * sample_rows * sample_rows * shape.K
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"quantise {sample_rows} rows of A and of B and multiply them ({sample_rows}x{sample_rows}x"
                      f"{shape.K}, fp64), {dt:.2f} s"}


def mx_main(args):
    """One GEMM of the 7B-class rank in MXFP4 or MXFP6: quantise the activations
    and the weight in the GEMM's byte order (mtl_mx_quantize_ordered) and
    multiply them on the block-scaled MFMA (mtl_mx_gemm_ordered)."""
    import torch
    import synth
    import megatron_tensor_transformer_layer_amd as mtl
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev

    shape = synth.MX_WORKLOADS[args.workload]
    fp6 = shape.elem == "e2m3"
    name = "MXFP6" if fp6 else "MXFP4"
    elem = mtl.MTL_MX_E2M3 if fp6 else mtl.MTL_MX_E2M1
    quant = lambda x, r, k, q, s_: mtl.mtl_mx_quantize_ordered(elem, x, r, k, q, s_, mtl.MTL_MX_ORDER_GEMM)
    gemm = lambda *g: mtl.mtl_mx_gemm_ordered(elem, *g, mtl.MTL_MX_ORDER_GEMM)
    M, N, K = shape.M, shape.N, shape.K
    cb_cols = K * 3 // 4 if fp6 else K // 2
    a = bf16_dev(synth.mx_operand(M, K, "mx_a", 1.0))
    b = bf16_dev(synth.mx_operand(N, K, "mx_b", synth.WEIGHT_STD))
    ca = torch.empty(M, cb_cols, dtype=torch.uint8, device="cuda")
    sa = torch.empty(M, K // 32, dtype=torch.uint8, device="cuda")
    cb = torch.empty(N, cb_cols, dtype=torch.uint8, device="cuda")
    sb = torch.empty(N, K // 32, dtype=torch.uint8, device="cuda")
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = []

    def step(record=False):
        quant(a, M, K, ca, sa)
        quant(b, N, K, cb, sb)
        if record:
            e0, e1 = ev(), ev()
            e0.record()
        gemm(M, N, K, ca, sa, cb, sb, c)
        if record:
            e1.record()
            marks.append((e0, e1))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    gemm_ms = float(np.mean([x.elapsed_time(y) for x, y in marks]))
    fl = 2.0 * M * N * K
    achieved = fl / (gemm_ms / 1e3) / 1e12
    out = {
        "metric": f"TFLOP/s of one {name} GEMM of the TP-rank layer (quantisation included) and % of MI355X MFMA peak",
        "value": round(fl / (ms / 1e3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": name.lower(),
        "data": "synthetic (N(0,1) activations, N(0,0.02) weight, bf16 before quantisation)",
        "config": {"workload": f"{args.workload}: fc1 forward of the 7B-class TP=4 rank, {M}x{N}x{K}, both "
                               f"operands quantised to {name} each step, bf16 output",
                   "global_batch": 1, "seq_len": M, "parallelism": "tp4-rank0-of-1gpu"},
        "pct_of_peak": round(100 * fl / (ms / 1e3) / 1e12 / PEAK_FP4_TFLOPS, 2),
        "flop_per_step": fl,
        "roofline": {"bound": "mfma", "kernel": f"gemm_bf16_kernel in its {name} mode (operands in the GEMM's byte "
                               "order, 256x256 tiles), HIP events on its stream",
                     "achieved": round(achieved, 1), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP4_TFLOPS, 4), "traffic": None,
                     "gemm_launch_us": round(gemm_ms * 1e3, 1)},
        "cpu_baseline": None if args.no_cpu_baseline else mx_cpu_baseline(shape, 64),
    }
    print(json.dumps(out), flush=True)


def moe_group_rates(groups, n, h, f, el, tokens, k):
    """Rates of the MoE launch groups from the rank's row count n (the library
    records only their times): 2*n*h*f FLOP per grouped GEMM, and the bytes
    each one must move -- its activations, its expert weights (bf16, read) or
    weight gradients (fp32, written, for every local expert)."""
    w = 2.0 * el * h * f  # one expert weight tensor of the rank, bf16
    by = {"moe_gather": 2.0 * n * h * 2, "moe_combine": 2.0 * (n * h + tokens * h) + 4.0 * tokens * k,
          "moe_combine_bwd": 2.0 * (tokens * h + 2 * n * h) + 4.0 * tokens * k * 2,
          "moe_scatter": 2.0 * (n * h + tokens * h),
          "moe_fc1_fwd": 2.0 * (n * h + 2 * n * f) + w, "moe_fc2_fwd": 2.0 * (n * f + n * h) + w,
          "moe_fc2_dgrad": 2.0 * (n * h + 2 * n * f) + w, "moe_fc2_wgrad": 2.0 * (n * f + n * h) + 2 * w,
          "moe_fc1_wgrad": 2.0 * (n * h + n * f) + 2 * w, "moe_fc1_dgrad": 2.0 * (n * f + n * h) + w}
    out = {}
    for name, v in groups.items():
        us = v["ms"] * 1e3 / max(v["launches"], 1)
        fl = 2.0 * n * h * f if v["kind"] == "gemm" else 0.0
        b = by.get(name, 0.0)
        out[name] = {"kind": v["kind"], "us": round(us, 1), "flop": fl, "bytes": b,
                     "tflops": round(fl / (us / 1e6) / 1e12, 1) if fl else None,
                     "gb_per_s": round(b / (us / 1e6) / 1e9, 1), "frac_of_hbm_peak": round(b / (us / 1e6) / 1e9 /
                                                                                         PEAK_HBM_GBS, 4)}
    return out


def moe_main(args):
    """One EP rank's MoE expert block: route, permute, grouped fc1+GeLU, fc2,
    combine, and the backward (combine', grouped dgrad and wgrad, dX scatter)."""
    if args.router:
        router_main(args)
        return
    import torch
    import synth
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    from megatron_tensor_transformer_layer_amd.moe import MoeRank
    from oracle.moe import moe_flops  # FLOP count only (closed form)

    shape = synth.MOE_WORKLOADS[args.workload]
    r, El = args.rank or 0, shape.experts // shape.ep
    lo = r * El
    w1 = torch.stack([synth.moe_expert_weight_device(shape, "moe_w1", lo + e) for e in range(El)])
    w2 = torch.stack([synth.moe_expert_weight_device(shape, "moe_w2", lo + e) for e in range(El)])
    st = MoeRank(shape.tokens, shape.hidden, shape.ffn, shape.experts, shape.topk, shape.ep, r, w1, w2)
    logits = torch.from_numpy(synth.moe_logits(shape)).cuda()
    x = bf16_dev(synth.moe_tokens(shape, 0, "moe_x"))
    dy = bf16_dev(synth.moe_tokens(shape, 0, "moe_dy"))
    st.step(logits, x, dy)
    torch.cuda.synchronize()
    counts = st.counts.cpu().numpy()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    fwd_ev = []

    def step(record=False):
        st.route(logits)
        st.permute()
        if record:
            e0, e1 = ev(), ev()
            e0.record()
        st.forward(x)
        if record:
            e1.record()
            fwd_ev.append((e0, e1))
        st.backward(dy)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall / args.steps * 1e3
    fl = moe_flops(counts, shape.hidden, shape.ffn)
    n = int(counts.sum())
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b in fwd_ev]))
    groups, _ = prof_window(step, 2)
    moe_groups = moe_group_rates(groups, n, shape.hidden, shape.ffn, El, shape.tokens, shape.topk)
    # the roofline kernel: the grouped GEMM launch that takes the most time; it is
    # bound by HBM when its FLOP per byte moved lies below the ridge point
    # (peak FLOP/s over peak bytes/s), else by the matrix cores
    dom = max((k for k, v in moe_groups.items() if v["kind"] == "gemm"), key=lambda k: moe_groups[k]["us"])
    dg = moe_groups[dom]
    hbm = dg["flop"] / dg["bytes"] < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm:
        roof = {"bound": "hbm", "achieved": dg["gb_per_s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dg["gb_per_s"] / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": dg["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dg["tflops"] / PEAK_BF16_TFLOPS, 4)}
    roof.update(kernel=f"{dom}: gemm_bf16_kernel grouped over the rank's experts (256x256 tiles), HIP events around "
                       "the launch", traffic=None, launch_us=dg["us"], flop_per_launch=dg["flop"],
                bytes_per_launch=dg["bytes"], flop_per_byte=round(dg["flop"] / dg["bytes"], 1))
    out = {
        "metric": "TFLOP/s per EP-rank MoE expert block fwd+bwd (bf16) and % of MI355X MFMA peak",
        "value": round(fl / (ms / 1e3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (Zipf(%.1f) router logits, N(0,1) tokens, N(0,0.02) expert weights)" % shape.zipf_s,
        "config": {"workload": f"{args.workload}: EP rank {r} of {shape.ep}, {El} of {shape.experts} experts, "
                               f"top-{shape.topk}, hidden {shape.hidden}, ffn {shape.ffn}, {shape.tokens} tokens; "
                               f"{n} local assignments, per-expert rows {counts.min()}..{counts.max()}",
                   "global_batch": 1, "seq_len": shape.tokens, "parallelism": f"ep{shape.ep}-rank{r}-of-1gpu"},
        "pct_of_peak": round(100 * fl / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "flop_per_step": fl,
        "roofline": roof,
        "forward_ms": round(fwd_ms, 4),
        "launch_groups": moe_groups,
        "gemm_tflops": round(sum(v["flop"] for v in moe_groups.values()) /
                             (sum(v["us"] for v in moe_groups.values() if v["kind"] == "gemm") / 1e6) / 1e12, 1),
        "slowest_expert_rows": int(counts.max()),
        "per_expert_rows": [int(c) for c in counts],
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = moe_cpu_baseline(shape, r, 512, shape.ffn // 16)
    print(json.dumps(out), flush=True)


def prof_window(run_step, n_steps):
    """Run n_steps steps with the library's launch timing on (mtl_prof_*) and
    return the per-step mean of each launch group, keyed by name, with its kind,
    algorithmic FLOP and bytes, plus the per-step totals by kind."""
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_prof_record, mtl_prof_start, mtl_prof_stop
    torch.cuda.synchronize()
    mtl_prof_start()
    for _ in range(n_steps):
        run_step()
    n = mtl_prof_stop()
    torch.cuda.synchronize()
    groups, kinds = {}, {}
    for i in range(n):
        r = mtl_prof_record(i)
        g = groups.setdefault(r["name"], dict(kind=r["kind"], flop=0.0, bytes=0.0, ms=0.0, launches=0))
        g["flop"] += r["flop"]
        g["bytes"] += r["bytes"]
        g["ms"] += r["ms"]
        g["launches"] += 1
        k = kinds.setdefault(r["kind"], dict(flop=0.0, bytes=0.0, ms=0.0, launches=0))
        for f in ("flop", "bytes", "ms"):
            k[f] += r[f]
        k["launches"] += 1
    for d in list(groups.values()) + list(kinds.values()):
        for f in ("flop", "bytes", "ms"):
            d[f] /= n_steps
        d["launches"] /= n_steps
    return groups, kinds


def windows(run_step, n_windows, per_window):
    """n_windows windows of per_window steps, each step bracketed by HIP events:
    the mean step time of each window and the P50/P95 over every step."""
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)
    means, all_ms = [], []
    for _ in range(n_windows):
        marks = [(ev(), ev()) for _ in range(per_window)]
        for a, b in marks:
            a.record()
            run_step()
            b.record()
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in marks]
        means.append(float(np.mean(ms)))
        all_ms += ms
    return dict(n_windows=n_windows, steps_per_window=per_window,
                window_mean_ms=[round(m, 4) for m in means], worst_window_ms=round(max(means), 4),
                step_ms_p50=round(float(np.percentile(all_ms, 50)), 4),
                step_ms_p95=round(float(np.percentile(all_ms, 95)), 4))


def timed_steps(run_step, steps, warmup):
    """W untimed steps, then exactly K steps between two synchronisations; the
    mean wall-clock milliseconds per step."""
    import torch
    for _ in range(warmup):
        run_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run_step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def breakdown(groups, kinds, peak):
    """The graded GEMM number (sum of GEMM FLOP over the sum of GEMM launch
    times), the rate of each launch group, and the HBM rate of the memory-bound
    kinds."""
    g = kinds.get("gemm", dict(flop=0.0, ms=0.0))
    a = kinds.get("attention", dict(flop=0.0, ms=0.0))
    out = {
        "gemm_tflops": round(g["flop"] / (g["ms"] / 1e3) / 1e12, 1) if g["ms"] else None,
        "gemm_frac_of_peak": round(g["flop"] / (g["ms"] / 1e3) / 1e12 / peak, 4) if g["ms"] else None,
        "gemm_us_per_step": round(g["ms"] * 1e3, 1),
        "attention_tflops": round(a["flop"] / (a["ms"] / 1e3) / 1e12, 1) if a["ms"] else None,
        "attention_frac_of_bf16_peak": round(a["flop"] / (a["ms"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if a["ms"] else None,
        "attention_us_per_step": round(a["ms"] * 1e3, 1),
        "memory_bound": {k: {"us_per_step": round(v["ms"] * 1e3, 1), "launch_groups": v["launches"],
                             "gb_per_s": round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1),
                             "frac_of_hbm_peak": round(v["bytes"] / (v["ms"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
                         for k, v in kinds.items() if k not in ("gemm", "attention") and v["ms"] > 0},
        "groups": {n: {"kind": v["kind"], "us": round(v["ms"] * 1e3 / max(v["launches"], 1), 1),
                       "launches": v["launches"],
                       **({"tflops": round(v["flop"] / (v["ms"] / 1e3) / 1e12, 1)} if v["flop"] else
                          {"gb_per_s": round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1)})}
                   for n, v in groups.items()},
    }
    return out


# The kernel of each GEMM launch group on the 256x256 backward pairs, as the
# profiler names it (for the roofline's rocprofv3 cross-check).
GROUP_KERNEL = {
    "fc2_bwd": "gemm_pair_kernel: fp32 wgrad dW2 = A^T dY (256x256 tiles) with dZ = (dY W2^T) * GeLU'(z) "
               "(256x256 tiles), one launch",
    "fc1_bwd": "gemm_pair_kernel: fp32 wgrad dW1 = H^T dZ (256x256 tiles) with dH = dZ W1^T (256x256 tiles), one "
               "launch",
    "qkv_bwd": "the QKV projection's wgrad and dgrad (one gemm_pair_kernel launch where both take 256x256 tiles)",
    "fc1_fwd": "gemm_bf16_kernel<256,256> with the bias + GeLU epilogue (8 waves)",
    "fc2_fwd": "gemm_bf16_kernel<256,256>, bf16 output",
    "qkv_fwd": "gemm_bf16_kernel with the bias epilogue",
    "proj_fwd": "gemm_bf16_kernel, bf16 output",
    "proj_bwd": "the output projection's wgrad and dgrad",
}


def traffic_file(workload, group, precision):
    # each precision has its own kernels and counters: bf16 files carry no suffix
    return os.path.join(HERE, "profiles",
                        f"gemm_{group}{'' if precision == 'bf16' else '_' + precision}_{workload}_traffic.txt")


def stored_traffic(workload, group, precision):
    """Counter-derived HBM bytes per launch of a GEMM launch group, from the
    committed rocprofv3 summary; None when there is none or when gemm.hip has
    changed since the counters were taken."""
    path = traffic_file(workload, group, precision)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def all_shards_cpu_baseline(shape):
    """The oracle (fp64 numpy, as it stands) on the whole small layer: every
    shard's forward and backward plus the four reductions."""
    import synth
    from oracle import layer as L
    from oracle import shard as S
    full = synth.layer_inputs(shape, seed=0)
    p = {k: synth.bf16_bits_to_f64(full[k]) for k in ("w_qkv", "b_qkv", "w_o", "b_o", "w1", "b1", "w2", "b2")}
    x, g = synth.bf16_bits_to_f64(full["x"]), synth.bf16_bits_to_f64(full["dy"])
    reps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 10.0:
        S.sharded_layer(p, x, g, shape.heads, shape.tp)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    fl = L.layer_flops(shape.hidden, shape.heads, shape.ffn, shape.seq, shape.micro_batch, 1)["total"]
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(cpu_cores()), "kind": "oracle",
            "sample": f"the whole layer as {shape.tp} shards plus the four reductions (fp64 numpy), {reps} runs, "
                      f"{dt * 1e3:.1f} ms each"}


def all_shards_main(args, shape):
    """The whole small layer on one GPU: every TP shard's forward and backward
    plus the four full reductions standing in for the all-reduces, timed as
    one step.  At this size a launch is a few microseconds of work on a
    fraction of the chip, so the shards run side by side, each on a stream of
    its own, and the step is captured in a HIP graph (replayed K times); the
    line also gives the step launched eagerly, with the shards concurrent and
    one after the other."""
    import torch
    import synth
    from megatron_tensor_transformer_layer_amd.layer import AllShardsStep
    from oracle.layer import layer_flops  # FLOP count only (closed form)

    t = shape.tp
    full = synth.layer_inputs(shape, seed=0)
    shards = [synth.layer_inputs(shape, seed=0, tp=t, rank=r) for r in range(t)]
    serial = AllShardsStep(shape, t, shards, full["x"], full["dy"], full["b_o"], full["b2"])
    eager_serial_ms = timed_steps(serial, args.steps, args.warmup)
    groups, kinds = prof_window(serial, 5)  # per-group times with the shards one after the other
    del serial
    # the product form: each shard on its own stream, the step captured as one graph
    step = AllShardsStep(shape, t, shards, full["x"], full["dy"], full["b_o"], full["b2"], concurrent=True)
    eager_ms = timed_steps(step, args.steps, args.warmup)
    # capture one step on a side stream (torch makes it current inside the context)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    graph_ms = timed_steps(graph.replay, args.steps, args.warmup)
    win = windows(graph.replay, 3, max(20, args.steps))
    fl = layer_flops(shape.hidden, shape.heads, shape.ffn, shape.seq, shape.micro_batch, 1)
    bd = breakdown(groups, kinds, PEAK_BF16_TFLOPS)
    launches = sum(v["launches"] for v in kinds.values())
    out = {
        "metric": "TFLOP/s per TP-shard layer fwd+bwd (bf16) and % of MI355X MFMA peak",
        "value": round(fl["total"] / (graph_ms / 1e3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(graph_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": f"{args.workload}: the whole layer, all {t} TP shards and the four full reductions "
                               f"on one GPU, hidden {shape.hidden}, heads {shape.heads}, ffn {shape.ffn}, "
                               f"seq {shape.seq}, micro-batch {shape.micro_batch}; the shards on concurrent streams, "
                               f"the step replayed as one HIP graph",
                   "global_batch": shape.micro_batch, "seq_len": shape.seq,
                   "parallelism": f"tp{t}-all-shards-1gpu"},
        "pct_of_peak": round(100 * fl["total"] / (graph_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "flop_per_step": fl["total"],
        "eager_serial_ms_per_step": round(eager_serial_ms, 4),
        "eager_concurrent_ms_per_step": round(eager_ms, 4),
        "graph_concurrent_ms_per_step": round(graph_ms, 4),
        "launch_groups_per_step": launches,
        **win,
        **{k: v for k, v in bd.items() if k != "groups"},
        "roofline": {"bound": "mfma", "kernel": "every GEMM launch of the step (HIP events, eager launches, shards "
                                                "one after the other)",
                     "achieved": bd["gemm_tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": bd["gemm_frac_of_peak"], "traffic": None},
        "cpu_baseline": None if args.no_cpu_baseline else all_shards_cpu_baseline(shape),
    }
    print(json.dumps(out), flush=True)


def dense_main(args):
    """One TP rank's layer step (the rank's shard plus its share of the four
    all-reduces), forward and backward.  Each all-reduce stands in as its two
    halves on one GPU: the rank's reduce-scatter share (its S/t rows summed
    over its own and t-1 resident peer partials) and the all-gather of the
    other t-1 reduced shares into the rank's full buffer (mtl_allgather_rows
    over resident peer buffers).  With --sp (sequence parallelism) the gathers
    move to the inputs of the column-parallel linears (X, H, dY, dH) and Y, dX
    stay row-sharded: four reduce-scatters and four gathers either way."""
    import torch
    import synth
    from megatron_tensor_transformer_layer_amd import (MTL_PREC_BF16, MTL_PREC_FP8_HYBRID, mtl_allgather_rows,
                                                       mtl_reduce)
    from megatron_tensor_transformer_layer_amd.layer import RankState, bf16_dev, empty_bf16
    from oracle.layer import layer_flops  # FLOP count only (closed form)

    shape = synth.WORKLOADS[args.workload]
    t, r = shape.tp, args.rank or 0
    if t > 1 and shape.seq * shape.micro_batch % t:
        raise SystemExit("the reduce-scatter shares need S % t == 0")
    inp = synth.layer_inputs(shape, tp=t, rank=r)
    fp8, mx = args.precision == "fp8", args.precision == "mxfp4"
    from megatron_tensor_transformer_layer_amd import MTL_PREC_MXFP4
    from megatron_tensor_transformer_layer_amd import MTL_F_KEEP_CODES
    # fp8 / MXFP4: the forward's codes of the operands the backward needs are kept for it
    st = RankState(shape, t, r, inp, flags=MTL_F_KEEP_CODES if (fp8 or mx) else 0,
                   precision={"bf16": MTL_PREC_BF16, "fp8": MTL_PREC_FP8_HYBRID,
                              "mxfp4": MTL_PREC_MXFP4}[args.precision])
    D = st.D
    x = bf16_dev(inp["x"])
    dy = bf16_dev(inp["dy"])
    b_o = bf16_dev(inp["b_o"])
    b2 = bf16_dev(inp["b2"])
    g = torch.Generator(device="cuda").manual_seed(1234)
    rnd = lambda: torch.randn(D.S, D.h, device="cuda", generator=g).to(torch.bfloat16)
    # partial sums the other t-1 ranks would contribute to this rank's reduce-scatter share
    peers = {k: [rnd() for _ in range(t - 1)] for k in ("attn", "mlp", "dh", "dx")}
    # the peers' full-size buffers whose own (reduced or input) shares the gathers copy
    gat = ("x", "h", "dy", "dh") if args.sp else ("h", "y", "dh", "dx")
    gpeers = {k: [rnd() for _ in range(t - 1)] for k in gat}
    h, y, dh, dx = (empty_bf16(D.S, D.h) for _ in range(4))
    r0, r1 = r * D.S // t, (r + 1) * D.S // t

    def gather(key, buf):
        if key in gat and t > 1:
            mtl_allgather_rows(gpeers[key][:r] + [buf] + gpeers[key][r:], buf, D.S, D.h, r)

    def step():
        gather("x", x)
        st.attn_fwd(x)
        mtl_reduce([st.p_attn] + peers["attn"], b_o, None, h, D.S, D.h, r0, r1)
        gather("h", h)
        st.mlp_fwd(h)
        mtl_reduce([st.p_mlp] + peers["mlp"], b2, None, y, D.S, D.h, r0, r1)
        gather("y", y)
        gather("dy", dy)
        st.mlp_bwd(dy, h)
        mtl_reduce([st.p_dh] + peers["dh"], None, None, dh, D.S, D.h, r0, r1)
        gather("dh", dh)
        st.attn_bwd(dh, x)
        mtl_reduce([st.p_dx] + peers["dx"], None, None, dx, D.S, D.h, r0, r1)
        gather("dx", dx)

    ms = timed_steps(step, args.steps, args.warmup)
    groups, kinds = prof_window(step, 5)
    win = windows(step, 3, max(20, args.steps))

    fl = layer_flops(shape.hidden, shape.heads, shape.ffn, shape.seq, shape.micro_batch, t)
    peak = PEAK_FP8_TFLOPS if fp8 else (PEAK_FP4_TFLOPS if mx else PEAK_BF16_TFLOPS)
    bd = breakdown(groups, kinds, peak)
    # the roofline kernel: the GEMM launch group that takes the most time per step
    dom = max((n for n, v in groups.items() if v["kind"] == "gemm"), key=lambda n: groups[n]["ms"])
    dg = groups[dom]
    per_launch_ms = dg["ms"] / dg["launches"]
    achieved = dg["flop"] / dg["launches"] / (per_launch_ms / 1e3) / 1e12
    out = {
        "metric": ("TFLOP/s per TP-shard layer fwd+bwd (fp8 hybrid GEMMs) and % of MI355X MFMA peak" if fp8 else
                   "TFLOP/s per TP-shard layer fwd+bwd (MXFP4 GEMMs) and % of MI355X MFMA peak" if mx else
                   "TFLOP/s per TP-shard layer fwd+bwd (bf16) and % of MI355X MFMA peak"),
        "value": round(fl["total"] / (ms / 1e3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.precision,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": f"{args.workload}: rank {r} of TP={t}, hidden {shape.hidden}, heads {shape.heads} "
                               f"({shape.heads // t} local), ffn {shape.ffn} ({shape.ffn // t} local), "
                               f"seq {shape.seq}, micro-batch {shape.micro_batch}"
                               + (", fp8 hybrid (E4M3 activations/weights, E5M2 gradients, per-tensor current "
                                  "scaling; attention bf16)" if fp8 else "")
                               + (", MXFP4 GEMMs (E2M1 in blocks of 32 along each product's contraction, E8M0 "
                                  "scales; attention bf16)" if mx else "")
                               + (", sequence parallel (reduce-scatter shares, in-place all-gathers of X, H, dY, dH)"
                                  if args.sp else ", each all-reduce as the rank's reduce-scatter share plus the "
                                                  "all-gather of the peers' shares"),
                   "global_batch": shape.micro_batch, "seq_len": shape.seq,
                   "parallelism": f"tp{t}{'-sp' if args.sp else ''}-rank{r}-of-1gpu"},
        "pct_of_peak": round(100 * fl["total"] / (ms / 1e3) / 1e12 / peak, 2),
        "pct_of_bf16_peak": round(100 * fl["total"] / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "flop_per_step": fl["total"],
        **win,
        **{k: v for k, v in bd.items() if k != "groups"},
        "launch_groups": bd["groups"],
        "roofline": {"bound": "mfma", "kernel": (f"{dom}: {GROUP_KERNEL.get(dom, dom)}" if args.precision == "bf16"
                                                 else f"{dom}: the {args.precision} GEMM launch group of that name"),
                     "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": stored_traffic(args.workload, dom, args.precision),
                     "flop_per_launch": dg["flop"] / dg["launches"],
                     "launch_us": round(per_launch_ms * 1e3, 2)},
        "cpu_baseline": None,
    }
    if fp8 or mx:
        q = kinds.get("quantize", dict(ms=0.0))
        out["quantize_us_per_step"] = round(q["ms"] * 1e3, 1)
        g8 = kinds.get("gemm")
        out["gemm_frac_of_bf16_peak"] = round(g8["flop"] / (g8["ms"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    if fp8 or mx:
        # The same step for the micro-batches after the first of a step with
        # gradient accumulation: the weights' codes stay those the first
        # micro-batch's forward kept (MTL_F_REUSE_WEIGHTS).  value and
        # ms_per_step above quantise the weights in every step.
        from megatron_tensor_transformer_layer_amd import MTL_F_REUSE_WEIGHTS
        st.cfg.flags = MTL_F_KEEP_CODES | MTL_F_REUSE_WEIGHTS
        ms_r = timed_steps(step, args.steps, args.warmup)
        _, kinds_r = prof_window(step, 5)
        st.cfg.flags = MTL_F_KEEP_CODES
        out["reused_weight_codes"] = {
            "ms_per_step": round(ms_r, 4), "value": round(fl["total"] / (ms_r / 1e3) / 1e12, 2),
            "quantize_us_per_step": round(kinds_r.get("quantize", dict(ms=0.0))["ms"] * 1e3, 1),
            "note": "micro-batches after the first of a gradient-accumulation step: the forward takes the "
                    "weights' codes kept by the first micro-batch's forward (MTL_F_REUSE_WEIGHTS)"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, r, min(args.cpu_sample_seq, shape.seq), args.precision)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (collectives are replaced by an "
              "on-device reduce); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.copy_rate:
        copy_rate()
        return
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    import torch
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.workload in synth.MOE_WORKLOADS:
        moe_main(args)
        return
    if args.workload in synth.CP_WORKLOADS:
        cp_main(args)
        return
    if args.workload in synth.MX_WORKLOADS:
        mx_main(args)
        return
    shape = synth.WORKLOADS[args.workload]
    if args.workload == "gpt2-small-tp2":
        all_shards_main(args, shape)
        return
    dense_main(args)


if __name__ == "__main__":
    main()
