"""The oracle: a plain, slow fp64 CPU implementation of one transformer layer's
training step, of its tensor-parallel sharded view, of one context-parallel
rank's share of causal attention, of the MoE expert block and its router
(linear, gate backward, load-balancing loss), of fp8 quantisation and the
layer with fp8 GEMM operands, and of MXFP4 quantisation, GEMMs on MXFP4
operands and the layer with MXFP4 GEMM operands.

TEST INFRASTRUCTURE ONLY.  Nothing in the library path imports, calls or links
this package; only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP path.

Sources (pages as cited throughout):
  [tutorial]  cf-1.com/news/5344657 -- a Megatron beginner tutorial:
              section 2.2 (tensor parallelism: QKV split by output columns,
              first MLP layer by columns, second by rows; divisibility of
              hidden size and heads by the TP degree), section 4.2 (12 heads /
              TP 2 = 6 per card).
  [guide]     ai.lansai.wang/82226 -- Megatron Core vs Megatron-LM guide:
              "integer checks first" section; the semantic-alignment table
              (compare parameters regrouped by logical parameter, forward
              outputs and gradients).
  [site]      navi2ai.com/sites/1106 -- Megatron-Core 0.17 summary: deploy
              step 6 (MoE: 256 experts, top-8 router, EP 16, hidden 7168, ffn
              18432, ``--fp8-format hybrid``).
The pages name the pieces but print no formulas; where they leave a step open
the oracle takes the plain textbook definition (scaled dot-product causal
attention, exact erf GeLU, softmax gates over the selected experts, OCP fp8
encodings) -- each reading is listed in the module that uses it.
"""
from . import layer, shard, moe, fp8, router, cp, mxfp4  # noqa: F401
from . import fp8_layer, mx_layer  # noqa: F401
