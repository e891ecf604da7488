"""Device buffers and the call sequence of one expert-parallel rank's MoE block.

Plumbing only: allocates torch device tensors and passes their addresses to
the C entry points (see ``__init__``) in the order a training step needs them.
No arithmetic of the block happens here.
"""
from __future__ import annotations

import torch

from . import (MTL_PREC_BF16, make_moe_cfg, mtl_moe_bwd, mtl_moe_fwd, mtl_moe_permute, mtl_moe_route,
               mtl_moe_router_bwd, mtl_moe_router_fwd, mtl_moe_router_sizes, mtl_moe_sizes)

DEV = "cuda"


class MoeRank:
    """Routing tables, saved activations, outputs, gradients and scratch of one
    EP rank.  ``w1`` [E/ep, h, f] and ``w2`` [E/ep, f, h] are bf16 device tensors."""

    def __init__(self, tokens, hidden, ffn, experts, topk, ep, rank, w1, w2, flags=0, device=DEV):
        self.cfg = make_moe_cfg(tokens, hidden, ffn, experts, topk, ep, rank, MTL_PREC_BF16, flags)
        self.max_rows, self.scratch_bytes = mtl_moe_sizes(self.cfg)
        T, h, f, k, El, N = tokens, hidden, ffn, topk, experts // ep, self.max_rows
        i32 = dict(dtype=torch.int32, device=device)
        bf = dict(dtype=torch.bfloat16, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.w1, self.w2 = w1, w2
        self.idx = torch.empty(T, k, **i32)
        self.gates = torch.empty(T, k, **f32)
        self.counts = torch.empty(El, **i32)
        self.offsets = torch.empty(El + 1, **i32)
        self.perm_token = torch.empty(N, **i32)
        self.perm_slot = torch.empty(N, **i32)
        self.slot_row = torch.empty(T, k, **i32)
        self.xp = torch.empty(N, h, **bf)
        self.gz = torch.empty(N, f, **bf)  # GeLU'(z)
        self.a = torch.empty(N, f, **bf)
        self.ye = torch.empty(N, h, **bf)
        self.y = torch.empty(T, h, **bf)
        self.dx = torch.empty(T, h, **bf)
        self.dw1 = torch.zeros(El, h, f, **f32)
        self.dw2 = torch.zeros(El, f, h, **f32)
        self.dgates = torch.empty(T, k, **f32)
        self.scratch = torch.empty(self.scratch_bytes, dtype=torch.uint8, device=device)

    def route(self, logits):
        mtl_moe_route(self.cfg, logits, self.idx, self.gates)

    def permute(self):
        mtl_moe_permute(self.cfg, self.idx, self.counts, self.offsets, self.perm_token, self.perm_slot,
                        self.slot_row)

    def forward(self, x):
        mtl_moe_fwd(self.cfg, x, self.offsets, self.perm_token, self.slot_row, self.gates, self.w1, self.w2,
                    self.xp, self.gz, self.a, self.ye, self.y)

    def backward(self, dy):
        mtl_moe_bwd(self.cfg, dy, self.offsets, self.perm_token, self.perm_slot, self.slot_row, self.gates,
                    self.xp, self.gz, self.a, self.ye, self.w1, self.w2, self.dx, self.dw1, self.dw2, self.dgates,
                    self.scratch)

    def step(self, logits, x, dy):
        self.route(logits)
        self.permute()
        self.forward(x)
        self.backward(dy)


class Router:
    """The MoE router's linear and its backward (replicated on every EP rank):
    logits, the gate/logit gradients, the load-balancing loss, dW_r and the
    router's share of dX.  ``w_r`` [h, E] is a bf16 device tensor."""

    def __init__(self, tokens, hidden, experts, topk, w_r, aux_coeff=0.001, ep=1, rank=0, flags=0, device=DEV):
        # the router calls do not read ffn; 8 passes the configuration check
        self.cfg = make_moe_cfg(tokens, hidden, 8, experts, topk, ep, rank, MTL_PREC_BF16, flags)
        self.scratch_bytes = mtl_moe_router_sizes(self.cfg)
        f32 = dict(dtype=torch.float32, device=device)
        self.w_r, self.aux_coeff = w_r, aux_coeff
        self.logits = torch.empty(tokens, experts, **f32)
        self.dlogits = torch.empty(tokens, experts, **f32)
        self.dw_r = torch.zeros(hidden, experts, **f32)
        self.dx = torch.empty(tokens, hidden, dtype=torch.bfloat16, device=device)
        self.aux_loss = torch.zeros(1, **f32)
        self.scratch = torch.empty(self.scratch_bytes, dtype=torch.uint8, device=device)

    def forward(self, x):
        mtl_moe_router_fwd(self.cfg, x, self.w_r, self.logits)
        return self.logits

    def backward(self, x, idx, gates, dgates):
        mtl_moe_router_bwd(self.cfg, x, self.w_r, self.logits, idx, gates, dgates, self.aux_coeff, self.aux_loss,
                           self.dlogits, self.dw_r, self.dx, self.scratch)
