"""Write ``fp8_layer_7b_tp4.npz``: the oracle's values for the whole fp8 layer
at the 7B-class TP=4 size (hidden 4096, 32 heads, ffn 16384, seq 4096,
micro-batch 1, all four shards), on sampled rows, with whole-tensor statistics.

Calls only ``oracle/`` (and ``synth`` for the seeded inputs).  Two references:

* ``ref``: the plain fp64 layer on the unquantised bf16 inputs (the reference
  the fp8 tolerance is stated against);
* ``recipe``: the same layer with every GEMM operand quantised per tensor
  (E4M3 forward operands, E5M2 gradient operands, current amax scaling), each
  quantisation taking the bf16 value the device stores, in exact arithmetic.

Stored per output: the sampled rows of ``ref`` (whole vectors for the bias
gradients), and, over the whole tensor and over the sampled rows, max|ref|,
RMS(ref), max|recipe - ref| and RMS(recipe - ref).  The full computation takes
about 15 minutes on 8 cores and ~20 GB of memory, which is why its result is
stored rather than recomputed by the GPU test.

Usage: python tests/golden/make_fp8_layer_7b_tp4.py
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import fp8_layer as F8  # noqa: E402
from oracle import layer as L  # noqa: E402

OUT = os.path.join(HERE, "fp8_layer_7b_tp4.npz")
WORKLOAD = "7b-tp4"

# Sampled rows: first and last tokens, tile edges and a spread in between
# (activations [S, h]); input features spread over the whole range for the
# weight gradients [in, out], across every rank's slice for dw2 [ffn, h].
ACT_ROWS = [0, 1, 63, 64, 1000, 2047, 3333, 4095]
H_ROWS = [0, 1, 127, 128, 2049, 3000, 4094, 4095]
F_ROWS = [0, 1, 4095, 4096, 8200, 12287, 12288, 16383]
SAMPLES = {"y": ACT_ROWS, "h": ACT_ROWS, "dh": ACT_ROWS, "dx": ACT_ROWS,
           "dw_qkv": H_ROWS, "dw_o": H_ROWS, "dw1": H_ROWS, "dw2": F_ROWS}
BIASES = ("db_qkv", "db_o", "db1", "db2")


def _bf16(t):
    return synth.bf16_bits_to_f64(synth.bf16_round_bits(np.asarray(t, dtype=np.float64)))


def _q4(t):
    return F8.q4(_bf16(t))


def _q5(t):
    return F8.q5(_bf16(t))


def _rms(t):
    return float(np.sqrt(np.mean(np.square(t))))


def main():
    shape = synth.WORKLOADS[WORKLOAD]
    t0 = time.time()
    full = synth.layer_inputs(shape, seed=0)
    f = lambda k: synth.bf16_bits_to_f64(full[k])
    p = {k: f(k) for k in ("w_qkv", "b_qkv", "w_o", "b_o", "w1", "b1", "w2", "b2")}
    x, g = f("x"), f("dy")
    print(f"inputs drawn {time.time() - t0:.0f} s", flush=True)

    fwd = L.layer_forward(p, x, shape.heads, shape.micro_batch)
    bwd = L.layer_backward(p, x, fwd, g, shape.heads, shape.micro_batch)
    ref = {"y": fwd["y"], "h": fwd["h"], **{k: bwd[k] for k in ("dh", "dx", "dw_qkv", "db_qkv", "dw_o", "db_o",
                                                                  "dw1", "db1", "dw2", "db2")}}
    del fwd, bwd
    print(f"plain layer {time.time() - t0:.0f} s", flush=True)

    q = F8.sharded_layer(p, x, g, shape.heads, shape.tp, shape.micro_batch, fq=_q4, gq=_q5)
    cat = lambda part, key, axis: np.concatenate([d[key] for d in q[part]], axis=axis)
    recipe = dict(y=q["y"], h=q["h"], dh=q["dh"], dx=q["dx"], dw_qkv=cat("attn_bwd", "dw_qkv", 1),
                  db_qkv=cat("attn_bwd", "db_qkv", 0), dw_o=cat("attn_bwd", "dw_o", 0),
                  db_o=q["attn_bwd"][0]["db_o"], dw1=cat("mlp_bwd", "dw1", 1), db1=cat("mlp_bwd", "db1", 0),
                  dw2=cat("mlp_bwd", "dw2", 0), db2=q["mlp_bwd"][0]["db2"])
    del q
    print(f"fp8 recipe {time.time() - t0:.0f} s", flush=True)

    out = {"workload": np.array(WORKLOAD), "seed": np.array(0)}
    for k, r in ref.items():
        d = recipe[k] - r
        if k in BIASES:
            out[f"{k}/ref"] = r.astype(np.float32)
            rs, ds = r, d
        else:
            rows = np.array(SAMPLES[k])
            out[f"{k}/rows"] = rows
            out[f"{k}/ref"] = r[rows].astype(np.float32)
            rs, ds = r[rows], d[rows]
        out[f"{k}/stats"] = np.array([
            np.max(np.abs(r)), _rms(r), np.max(np.abs(d)), _rms(d),      # whole tensor
            np.max(np.abs(rs)), _rms(rs), np.max(np.abs(ds)), _rms(ds),  # sampled rows
        ])
        print(f"  {k:7s} recipe max|q-ref|/max|ref| {np.max(np.abs(d)) / np.max(np.abs(r)):.4f}  "
              f"rms ratio {_rms(d) / _rms(r):.4f}", flush=True)
    np.savez_compressed(OUT, **out)
    print(f"wrote {OUT} ({os.path.getsize(OUT) / 1e6:.2f} MB) in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
