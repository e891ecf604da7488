"""Device buffers and the call sequence of a tensor-parallel layer step.

Plumbing only: allocates torch device tensors, passes their addresses to the
C entry points (see ``__init__``) in the order a training step needs them, and
converts bf16 bit patterns to and from host arrays.  No arithmetic of the layer
happens here.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (MTL_PREC_BF16, make_cfg, mtl_allgather_rows, mtl_attn_bwd, mtl_attn_fwd, mtl_mlp_bwd, mtl_mlp_fwd,
               mtl_reduce, mtl_workspace_bytes)

DEV = "cuda"


def bf16_dev(bits: np.ndarray, device=DEV) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> bfloat16 device tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def empty_bf16(*shape, device=DEV):
    return torch.empty(*shape, dtype=torch.bfloat16, device=device)


def zeros_f32(*shape, device=DEV):
    return torch.zeros(*shape, dtype=torch.float32, device=device)


@dataclass
class Dims:
    S: int
    h: int
    heads_l: int
    d: int
    f_l: int

    @property
    def qkv_l(self):
        return 3 * self.heads_l * self.d

    @property
    def o_l(self):
        return self.heads_l * self.d


def dims_of(hidden, heads, ffn, seq, micro_batch, tp) -> Dims:
    return Dims(S=seq * micro_batch, h=hidden, heads_l=heads // tp, d=hidden // heads, f_l=ffn // tp)


class RankState:
    """All device buffers of one TP rank: shard weights, saved activations,
    partial outputs, gradients and scratch."""

    def __init__(self, shape, tp: int, rank: int, shard: dict, flags: int = 0, device=DEV,
                 precision: int = MTL_PREC_BF16):
        self.cfg = make_cfg(shape.hidden, shape.heads, shape.ffn, shape.seq, shape.micro_batch, tp, rank,
                            precision, flags)
        D = self.D = dims_of(shape.hidden, shape.heads, shape.ffn, shape.seq, shape.micro_batch, tp)
        self.w = {k: bf16_dev(shard[k], device) for k in ("w_qkv", "b_qkv", "w_o", "w1", "b1", "w2")}
        self.qkv = empty_bf16(D.S, D.qkv_l, device=device)
        self.o = empty_bf16(D.S, D.o_l, device=device)
        self.lse = torch.empty(D.heads_l, D.S, dtype=torch.float32, device=device)
        self.gz = empty_bf16(D.S, D.f_l, device=device)  # GeLU'(z)
        self.a = empty_bf16(D.S, D.f_l, device=device)
        self.p_attn = empty_bf16(D.S, D.h, device=device)
        self.p_mlp = empty_bf16(D.S, D.h, device=device)
        self.p_dh = empty_bf16(D.S, D.h, device=device)
        self.p_dx = empty_bf16(D.S, D.h, device=device)
        self.dw_qkv = zeros_f32(D.h, D.qkv_l, device=device)
        self.db_qkv = zeros_f32(D.qkv_l, device=device)
        self.dw_o = zeros_f32(D.o_l, D.h, device=device)
        self.db_o = zeros_f32(D.h, device=device)
        self.dw1 = zeros_f32(D.h, D.f_l, device=device)
        self.db1 = zeros_f32(D.f_l, device=device)
        self.dw2 = zeros_f32(D.f_l, D.h, device=device)
        self.db2 = zeros_f32(D.h, device=device)
        self.scratch_bytes = mtl_workspace_bytes(self.cfg)
        self.scratch = torch.empty(self.scratch_bytes, dtype=torch.uint8, device=device)

    def attn_fwd(self, x):
        mtl_attn_fwd(self.cfg, x, self.w["w_qkv"], self.w["b_qkv"], self.w["w_o"], self.qkv, self.o, self.lse,
                     self.p_attn, self.scratch)

    def mlp_fwd(self, h):
        mtl_mlp_fwd(self.cfg, h, self.w["w1"], self.w["b1"], self.w["w2"], self.gz, self.a, self.p_mlp,
                    self.scratch)

    def mlp_bwd(self, dy, h, want_db2=True):
        mtl_mlp_bwd(self.cfg, dy, h, self.gz, self.a, self.w["w1"], self.w["w2"], self.p_dh, self.dw1, self.db1,
                    self.dw2, self.db2 if want_db2 else None, self.scratch)

    def attn_bwd(self, dh, x, want_db_o=True):
        mtl_attn_bwd(self.cfg, dh, x, self.qkv, self.o, self.lse, self.w["w_qkv"], self.w["w_o"], self.p_dx,
                     self.dw_qkv, self.db_qkv, self.dw_o, self.db_o if want_db_o else None, self.scratch)


def run_sharded_layer(shape, tp: int, shards: list, x_bits, b_o_bits, b2_bits, dy_bits, residual: bool = False,
                      precision: int = MTL_PREC_BF16, device=DEV, sp: bool = False, flags: int = 0) -> dict:
    """Run the whole layer as tp rank shards plus the four full reductions on
    one device; returns host fp64 copies of every output.  With sp, the
    sequence-parallel form: every rank holds full-size buffers of X, H, dY, dH
    with only its own row share filled, reduces only its share of each sum and
    gathers the peers' shares in place (mtl_allgather_rows) before the next
    column-parallel linear; Y and dX stay row-sharded."""
    ranks = [RankState(shape, tp, r, shards[r], flags=flags, device=device, precision=precision) for r in range(tp)]
    D = ranks[0].D
    if sp:
        return _run_sp(ranks, tp, D, x_bits, b_o_bits, b2_bits, dy_bits, residual, device)
    x = bf16_dev(x_bits, device)
    b_o = bf16_dev(b_o_bits, device)
    b2 = bf16_dev(b2_bits, device)
    dy = bf16_dev(dy_bits, device)
    h = empty_bf16(D.S, D.h, device=device)
    y = empty_bf16(D.S, D.h, device=device)
    dh = empty_bf16(D.S, D.h, device=device)
    dx = empty_bf16(D.S, D.h, device=device)
    for r in ranks:
        r.attn_fwd(x)
    mtl_reduce([r.p_attn for r in ranks], b_o, x if residual else None, h, D.S, D.h)
    for r in ranks:
        r.mlp_fwd(h)
    mtl_reduce([r.p_mlp for r in ranks], b2, h if residual else None, y, D.S, D.h)
    for r in ranks:
        r.mlp_bwd(dy, h)
    mtl_reduce([r.p_dh for r in ranks], None, dy if residual else None, dh, D.S, D.h)
    for r in ranks:
        r.attn_bwd(dh, x)
    mtl_reduce([r.p_dx for r in ranks], None, dh if residual else None, dx, D.S, D.h)
    torch.cuda.synchronize()
    return _outputs(ranks, host_f64(y), host_f64(h), host_f64(dh), host_f64(dx))


def _outputs(ranks, y, h, dh, dx) -> dict:
    cat = lambda key, axis: np.concatenate([host_f64(getattr(r, key)) for r in ranks], axis=axis)
    return dict(
        y=y, h=h, dh=dh, dx=dx,
        qkv=cat("qkv", 1), o=cat("o", 1), lse=cat("lse", 0), gz=cat("gz", 1), a=cat("a", 1),
        dw_qkv=cat("dw_qkv", 1), db_qkv=cat("db_qkv", 0), dw_o=cat("dw_o", 0), dw1=cat("dw1", 1),
        db1=cat("db1", 0), dw2=cat("dw2", 0),
        db_o=host_f64(ranks[0].db_o), db2=host_f64(ranks[0].db2),
        db_o_all=[host_f64(r.db_o) for r in ranks], db2_all=[host_f64(r.db2) for r in ranks],
    )


def _run_sp(ranks, tp, D, x_bits, b_o_bits, b2_bits, dy_bits, residual, device) -> dict:
    S, H = D.S, D.h
    share = [(i * S // tp, (i + 1) * S // tp) for i in range(tp)]
    full = lambda: [torch.zeros(S, H, dtype=torch.bfloat16, device=device) for _ in range(tp)]

    def gather(bufs):
        for i in range(tp):
            mtl_allgather_rows(bufs, bufs[i], S, H, i)

    def scattered(bits):  # each rank starts with only its own rows of the tensor
        src = bf16_dev(bits, device)
        bufs = full()
        for i, (r0, r1) in enumerate(share):
            bufs[i][r0:r1] = src[r0:r1]
        return bufs

    def reduce_scatter(partials, bias, residuals, out):
        for i, (r0, r1) in enumerate(share):
            mtl_reduce(partials, bias, residuals[i] if residual else None, out[i], S, H, r0, r1)

    b_o, b2 = bf16_dev(b_o_bits, device), bf16_dev(b2_bits, device)
    xs = scattered(x_bits)
    gather(xs)
    for i, r in enumerate(ranks):
        r.attn_fwd(xs[i])
    hs = full()
    reduce_scatter([r.p_attn for r in ranks], b_o, xs, hs)
    gather(hs)
    for i, r in enumerate(ranks):
        r.mlp_fwd(hs[i])
    ys = full()
    reduce_scatter([r.p_mlp for r in ranks], b2, hs, ys)
    dys = scattered(dy_bits)
    gather(dys)
    for i, r in enumerate(ranks):
        r.mlp_bwd(dys[i], hs[i])
    dhs = full()
    reduce_scatter([r.p_dh for r in ranks], None, dys, dhs)
    gather(dhs)
    for i, r in enumerate(ranks):
        r.attn_bwd(dhs[i], xs[i])
    dxs = full()
    reduce_scatter([r.p_dx for r in ranks], None, dhs, dxs)
    torch.cuda.synchronize()
    rows = lambda bufs: np.concatenate([host_f64(bufs[i][r0:r1]) for i, (r0, r1) in enumerate(share)], axis=0)
    out = _outputs(ranks, rows(ys), host_f64(hs[0]), host_f64(dhs[0]), rows(dxs))
    out["gathered"] = {k: [host_f64(b) for b in v] for k, v in (("x", xs), ("h", hs), ("dy", dys), ("dh", dhs))}
    return out


class AllShardsStep:
    """The whole layer on one device as one callable step: every TP rank's
    forward and backward plus the four full reductions, on fixed buffers (so the
    step can be captured into a HIP graph and replayed).  shards: per-rank
    inputs; x, dy, b_o, b2: bf16 bit patterns of the full tensors.  With
    concurrent, each rank's calls go to a stream of its own (forked from and
    joined back into the current stream around every phase), so the shards'
    small launches run side by side instead of one after the other."""

    def __init__(self, shape, tp: int, shards: list, x_bits, dy_bits, b_o_bits, b2_bits, device=DEV,
                 precision: int = MTL_PREC_BF16, concurrent: bool = False, flags: int = 0):
        self.ranks = [RankState(shape, tp, r, shards[r], flags=flags, device=device, precision=precision)
                      for r in range(tp)]
        D = self.D = self.ranks[0].D
        self.x, self.dy = bf16_dev(x_bits, device), bf16_dev(dy_bits, device)
        self.b_o, self.b2 = bf16_dev(b_o_bits, device), bf16_dev(b2_bits, device)
        self.h, self.y, self.dh, self.dx = (empty_bf16(D.S, D.h, device=device) for _ in range(4))
        self.streams = [torch.cuda.Stream(device=device) for _ in range(tp)] if concurrent else None

    def _per_rank(self, fn):
        if self.streams is None:
            for r in self.ranks:
                fn(r)
            return
        main = torch.cuda.current_stream()
        for r, s in zip(self.ranks, self.streams):
            s.wait_stream(main)
            with torch.cuda.stream(s):
                fn(r)
        for s in self.streams:
            main.wait_stream(s)

    def __call__(self):
        rk, D = self.ranks, self.D
        self._per_rank(lambda r: r.attn_fwd(self.x))
        mtl_reduce([r.p_attn for r in rk], self.b_o, None, self.h, D.S, D.h)
        self._per_rank(lambda r: r.mlp_fwd(self.h))
        mtl_reduce([r.p_mlp for r in rk], self.b2, None, self.y, D.S, D.h)
        self._per_rank(lambda r: r.mlp_bwd(self.dy, self.h, want_db2=r is rk[0]))
        mtl_reduce([r.p_dh for r in rk], None, None, self.dh, D.S, D.h)
        self._per_rank(lambda r: r.attn_bwd(self.dh, self.x, want_db_o=r is rk[0]))
        mtl_reduce([r.p_dx for r in rk], None, None, self.dx, D.S, D.h)

    def outputs(self) -> dict:
        """The step's device outputs (views of the step's own buffers)."""
        out = dict(h=self.h, y=self.y, dh=self.dh, dx=self.dx)
        for i, r in enumerate(self.ranks):
            for k in ("qkv", "o", "lse", "gz", "a", "dw_qkv", "db_qkv", "dw_o", "dw1", "db1", "dw2"):
                out[f"{k}{i}"] = getattr(r, k)
        out["db_o"], out["db2"] = self.ranks[0].db_o, self.ranks[0].db2
        return out
