"""Python binding of libmtl.so -- argument marshalling only.

Every function here has the name of the C entry point it calls (include/mtl.h
documents each one).  Tensor arguments may be torch tensors (their
``data_ptr()`` is passed) or integer device addresses; ``stream`` defaults to
torch's current stream on the current device.  A non-OK status raises
``MtlError``.  Every step of the computation runs in the library's HIP kernels;
there is no fallback path: if libmtl.so is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmtl.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mtl.h")

MTL_OK, MTL_E_NULL, MTL_E_DIVISIBILITY, MTL_E_RANK, MTL_E_SHAPE = 0, 1, 2, 3, 4
MTL_E_ALIGN, MTL_E_WORKSPACE, MTL_E_UNSUPPORTED, MTL_E_HIP = 5, 6, 7, 8
MTL_PREC_BF16, MTL_PREC_FP8_HYBRID, MTL_PREC_MXFP4 = 0, 1, 2
MTL_MX_E2M1, MTL_MX_E2M3 = 0, 1
MTL_MX_ORDER_PLAIN, MTL_MX_ORDER_GEMM = 0, 1
MTL_FP8_E4M3, MTL_FP8_E5M2 = 0, 1
MTL_FP8_AMAX_SCRATCH = 4096
MTL_CP_MAX = 64
MTL_F_RESIDUAL, MTL_F_WGRAD_ACCUM, MTL_F_KEEP_CODES, MTL_F_REUSE_WEIGHTS = 1, 2, 4, 8
MTL_F_FP8_KEEP_CODES, MTL_F_FP8_REUSE_WEIGHTS = MTL_F_KEEP_CODES, MTL_F_REUSE_WEIGHTS  # earlier names
MTL_PROF_MAX = 2048
MTL_NOALLOC_SCRATCH_BYTES = 48 << 20
MTL_CEILING_DATA_BYTES = 1 << 20
MTL_PROF_KINDS = ("gemm", "attention", "reduce", "colsum", "quantize", "gather")


class MtlError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_text(status)})")


class LayerCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("hidden", "heads", "ffn", "seq", "micro_batch", "tp", "rank", "precision", "flags")]


class MoeCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("tokens", "hidden", "ffn", "experts", "topk", "ep", "rank", "precision", "flags")]


_P = ctypes.c_void_p
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_CFG = ctypes.POINTER(LayerCfg)
_MCFG = ctypes.POINTER(MoeCfg)
_SIGS = {
    "mtl_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "mtl_validate": (ctypes.c_int, [_CFG]),
    "mtl_workspace_bytes": (ctypes.c_int, [_CFG, ctypes.POINTER(_SZ)]),
    "mtl_attn_fwd": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mtl_reduce": (ctypes.c_int, [_I32, ctypes.POINTER(_P), _P, _P, _P, _I64, _I64, _I64, _I64, _P]),
    "mtl_allgather_rows": (ctypes.c_int, [_I32, _I32, ctypes.POINTER(_P), _P, _I64, _I64, _P]),
    "mtl_cp_attn_scratch_bytes": (ctypes.c_int, [_I32, _I32, _I64, _I32, _I32, ctypes.POINTER(_SZ)]),
    "mtl_cp_attn_fwd": (ctypes.c_int, [_I32, _I32, _I64, _I32, _I32, ctypes.POINTER(_P), _P, _P, _P, _SZ, _P]),
    "mtl_mxfp4_quantize": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "mtl_mxfp4_gemm": (ctypes.c_int, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _I64, _P]),
    "mtl_mxfp4_quantize_t": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "mtl_mxfp6_quantize": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "mtl_mxfp6_gemm": (ctypes.c_int, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _I64, _P]),
    "mtl_mx_quantize_ordered": (ctypes.c_int, [_I32, _P, _I64, _I64, _P, _P, _I32, _P]),
    "mtl_mx_gemm_ordered": (ctypes.c_int, [_I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I64, _I32, _P]),
    "mtl_cp_attn_bwd_scratch_bytes": (ctypes.c_int, [_I32, _I32, _I64, _I32, _I32, ctypes.POINTER(_SZ)]),
    "mtl_cp_attn_bwd": (ctypes.c_int, [_I32, _I32, _I64, _I32, _I32, ctypes.POINTER(_P), _P, _P, _P, _P,
                                       ctypes.POINTER(_P), _P, _SZ, _P]),
    "mtl_mlp_fwd": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mtl_mlp_bwd": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mtl_attn_bwd": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mtl_fp8_amax": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _SZ, _P]),
    "mtl_fp8_cast": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P, _P]),
    "mtl_fp8_quantize": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P, _P, _SZ, _P]),
    "mtl_fp8_gemm": (ctypes.c_int, [_I64, _I64, _I64, _P, _I32, _P, _P, _I32, _P, _P, _P, _I64, _P]),
    "mtl_moe_validate": (ctypes.c_int, [_MCFG]),
    "mtl_moe_router_fwd": (ctypes.c_int, [_MCFG, _P, _P, _P, _P]),
    "mtl_moe_router_sizes": (ctypes.c_int, [_MCFG, ctypes.POINTER(_SZ)]),
    "mtl_moe_router_bwd": (ctypes.c_int, [_MCFG, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P, _SZ,
                                          _P]),
    "mtl_moe_sizes": (ctypes.c_int, [_MCFG, ctypes.POINTER(_I64), ctypes.POINTER(_SZ)]),
    "mtl_moe_route": (ctypes.c_int, [_MCFG, _P, _P, _P, _P]),
    "mtl_moe_permute": (ctypes.c_int, [_MCFG, _P, _P, _P, _P, _P, _P, _P]),
    "mtl_moe_fwd": (ctypes.c_int, [_MCFG] + [_P] * 13),
    "mtl_moe_bwd": (ctypes.c_int, [_MCFG] + [_P] * 17 + [_SZ, _P]),
    "mtl_attn_bwd_scratch_layout": (ctypes.c_int, [_CFG, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "mtl_mlp_bwd_noalloc": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "mtl_mfma_ceiling": (ctypes.c_int, [_P, _SZ, _I32, _I64, _I64, _P, _P]),
    "mtl_prof_start": (ctypes.c_int, []),
    "mtl_prof_stop": (ctypes.c_int, [ctypes.POINTER(_I32)]),
    "mtl_prof_record": (ctypes.c_int, [_I32, ctypes.POINTER(_I32), ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_float),
                                       ctypes.POINTER(ctypes.c_char_p)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmtl.so (built in-tree by ``megatron_tensor_transformer_layer_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m megatron_tensor_transformer_layer_amd.build")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_text(status: int) -> str:
    try:
        return lib().mtl_status_str(status).decode()
    except Exception:  # pragma: no cover - library missing
        return "?"


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != MTL_OK:
        raise MtlError(status, where)


def make_cfg(hidden, heads, ffn, seq, micro_batch=1, tp=1, rank=0, precision=MTL_PREC_BF16, flags=0) -> LayerCfg:
    return LayerCfg(hidden, heads, ffn, seq, micro_batch, tp, rank, precision, flags)


def mtl_validate(cfg: LayerCfg) -> int:
    """Returns the status code (does not raise)."""
    return lib().mtl_validate(ctypes.byref(cfg))


def mtl_workspace_bytes(cfg: LayerCfg) -> int:
    n = _SZ(0)
    _check(lib().mtl_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)), "mtl_workspace_bytes")
    return n.value


def _nbytes(scratch, scratch_bytes):
    if scratch_bytes is not None:
        return scratch_bytes
    return 0 if scratch is None or isinstance(scratch, int) else scratch.numel() * scratch.element_size()


def mtl_attn_fwd(cfg, x, w_qkv, b_qkv, w_o, qkv, o, lse, partial, scratch=None, scratch_bytes=None, stream=None):
    _check(lib().mtl_attn_fwd(ctypes.byref(cfg), _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_o), _ptr(qkv), _ptr(o),
                              _ptr(lse), _ptr(partial), _ptr(scratch), _nbytes(scratch, scratch_bytes),
                              _stream(stream)), "mtl_attn_fwd")


def mtl_reduce(partials, bias, residual, out, rows, cols, row_begin=0, row_end=None, stream=None):
    t = len(partials)
    arr = (_P * t)(*[_ptr(p) for p in partials])
    _check(lib().mtl_reduce(t, arr, _ptr(bias), _ptr(residual), _ptr(out), rows, cols, row_begin,
                            rows if row_end is None else row_end, _stream(stream)), "mtl_reduce")


def mtl_allgather_rows(bufs, out, rows, cols, rank, stream=None):
    t = len(bufs)
    arr = (_P * t)(*[_ptr(b) for b in bufs])
    _check(lib().mtl_allgather_rows(t, rank, arr, _ptr(out), rows, cols, _stream(stream)), "mtl_allgather_rows")


def mtl_cp_attn_scratch_bytes(cp, rank, chunk, heads, head_dim) -> int:
    n = _SZ(0)
    _check(lib().mtl_cp_attn_scratch_bytes(cp, rank, chunk, heads, head_dim, ctypes.byref(n)),
           "mtl_cp_attn_scratch_bytes")
    return int(n.value)


def mtl_cp_attn_fwd(cp, rank, chunk, heads, head_dim, qkv_chunks, o, lse, scratch=None, scratch_bytes=None,
                    stream=None):
    arr = (_P * len(qkv_chunks))(*[_ptr(c) for c in qkv_chunks])
    _check(lib().mtl_cp_attn_fwd(cp, rank, chunk, heads, head_dim, arr, _ptr(o), _ptr(lse), _ptr(scratch),
                                 _nbytes(scratch, scratch_bytes), _stream(stream)), "mtl_cp_attn_fwd")


def mtl_cp_attn_bwd_scratch_bytes(cp, rank, chunk, heads, head_dim) -> int:
    n = _SZ(0)
    _check(lib().mtl_cp_attn_bwd_scratch_bytes(cp, rank, chunk, heads, head_dim, ctypes.byref(n)),
           "mtl_cp_attn_bwd_scratch_bytes")
    return int(n.value)


def mtl_cp_attn_bwd(cp, rank, chunk, heads, head_dim, qkv_chunks, o, lse, dout, dqkv, dkv_chunks, scratch,
                    scratch_bytes=None, stream=None):
    arr = (_P * len(qkv_chunks))(*[_ptr(c) for c in qkv_chunks])
    dkv = (_P * max(len(dkv_chunks), 1))(*[_ptr(c) for c in dkv_chunks])
    _check(lib().mtl_cp_attn_bwd(cp, rank, chunk, heads, head_dim, arr, _ptr(o), _ptr(lse), _ptr(dout), _ptr(dqkv),
                                 dkv, _ptr(scratch), _nbytes(scratch, scratch_bytes), _stream(stream)),
           "mtl_cp_attn_bwd")


def mtl_mxfp4_quantize(x, rows, cols, codes, scales, stream=None):
    _check(lib().mtl_mxfp4_quantize(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)),
           "mtl_mxfp4_quantize")


def mtl_mxfp4_quantize_t(x, rows, cols, codes, scales, stream=None):
    _check(lib().mtl_mxfp4_quantize_t(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)),
           "mtl_mxfp4_quantize_t")


def mtl_mxfp4_gemm(M, N, K, a_codes, a_scales, b_codes, b_scales, c, ldc=None, stream=None):
    _check(lib().mtl_mxfp4_gemm(M, N, K, _ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), _ptr(c),
                                N if ldc is None else ldc, _stream(stream)), "mtl_mxfp4_gemm")


def mtl_mxfp6_quantize(x, rows, cols, codes, scales, stream=None):
    _check(lib().mtl_mxfp6_quantize(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)),
           "mtl_mxfp6_quantize")


def mtl_mxfp6_gemm(M, N, K, a_codes, a_scales, b_codes, b_scales, c, ldc=None, stream=None):
    _check(lib().mtl_mxfp6_gemm(M, N, K, _ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), _ptr(c),
                                N if ldc is None else ldc, _stream(stream)), "mtl_mxfp6_gemm")


def mtl_mx_quantize_ordered(elem, x, rows, cols, codes, scales, order, stream=None):
    _check(lib().mtl_mx_quantize_ordered(elem, _ptr(x), rows, cols, _ptr(codes), _ptr(scales), order,
                                         _stream(stream)), "mtl_mx_quantize_ordered")


def mtl_mx_gemm_ordered(elem, M, N, K, a_codes, a_scales, b_codes, b_scales, c, order, ldc=None, stream=None):
    _check(lib().mtl_mx_gemm_ordered(elem, M, N, K, _ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales),
                                     _ptr(c), N if ldc is None else ldc, order, _stream(stream)),
           "mtl_mx_gemm_ordered")


def mtl_mlp_fwd(cfg, h, w1, b1, w2, gz, a, partial, scratch=None, scratch_bytes=None, stream=None):
    _check(lib().mtl_mlp_fwd(ctypes.byref(cfg), _ptr(h), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(gz), _ptr(a),
                             _ptr(partial), _ptr(scratch), _nbytes(scratch, scratch_bytes), _stream(stream)),
           "mtl_mlp_fwd")


def mtl_mlp_bwd(cfg, dy, h, gz, a, w1, w2, dh_partial, dw1, db1, dw2, db2, scratch, scratch_bytes=None, stream=None):
    nbytes = scratch.numel() * scratch.element_size() if scratch_bytes is None else scratch_bytes
    _check(lib().mtl_mlp_bwd(ctypes.byref(cfg), _ptr(dy), _ptr(h), _ptr(gz), _ptr(a), _ptr(w1), _ptr(w2),
                             _ptr(dh_partial), _ptr(dw1), _ptr(db1), _ptr(dw2), _ptr(db2), _ptr(scratch), nbytes,
                             _stream(stream)), "mtl_mlp_bwd")


def mtl_attn_bwd_scratch_layout(cfg):
    """(do_offset, dqkv_offset): byte offsets of dO and dQKV in mtl_attn_bwd's scratch."""
    a, b = _SZ(0), _SZ(0)
    _check(lib().mtl_attn_bwd_scratch_layout(ctypes.byref(cfg), ctypes.byref(a), ctypes.byref(b)),
           "mtl_attn_bwd_scratch_layout")
    return a.value, b.value


def mtl_mlp_bwd_noalloc(cfg, dy, h, gz, a, w1, w2, dh_partial, dw1, db1, dw2, db2, stream=None):
    _check(lib().mtl_mlp_bwd_noalloc(ctypes.byref(cfg), _ptr(dy), _ptr(h), _ptr(gz), _ptr(a), _ptr(w1), _ptr(w2),
                                     _ptr(dh_partial), _ptr(dw1), _ptr(db1), _ptr(dw2), _ptr(db2), _stream(stream)),
           "mtl_mlp_bwd_noalloc")


def mtl_attn_bwd(cfg, dh, x, qkv, o, lse, w_qkv, w_o, dx_partial, dw_qkv, db_qkv, dw_o, db_o, scratch,
                 scratch_bytes=None, stream=None):
    nbytes = scratch.numel() * scratch.element_size() if scratch_bytes is None else scratch_bytes
    _check(lib().mtl_attn_bwd(ctypes.byref(cfg), _ptr(dh), _ptr(x), _ptr(qkv), _ptr(o), _ptr(lse), _ptr(w_qkv),
                              _ptr(w_o), _ptr(dx_partial), _ptr(dw_qkv), _ptr(db_qkv), _ptr(dw_o), _ptr(db_o),
                              _ptr(scratch), nbytes, _stream(stream)), "mtl_attn_bwd")


def make_moe_cfg(tokens, hidden, ffn, experts, topk, ep=1, rank=0, precision=MTL_PREC_BF16, flags=0) -> MoeCfg:
    return MoeCfg(tokens, hidden, ffn, experts, topk, ep, rank, precision, flags)


def mtl_moe_validate(cfg: MoeCfg) -> int:
    """Returns the status code (does not raise)."""
    return lib().mtl_moe_validate(ctypes.byref(cfg))


def mtl_moe_sizes(cfg: MoeCfg):
    """Returns (max_rows, scratch_bytes)."""
    rows, n = _I64(0), _SZ(0)
    _check(lib().mtl_moe_sizes(ctypes.byref(cfg), ctypes.byref(rows), ctypes.byref(n)), "mtl_moe_sizes")
    return rows.value, n.value


def mtl_moe_router_fwd(cfg, x, w_r, logits, stream=None):
    _check(lib().mtl_moe_router_fwd(ctypes.byref(cfg), _ptr(x), _ptr(w_r), _ptr(logits), _stream(stream)),
           "mtl_moe_router_fwd")


def mtl_moe_router_sizes(cfg) -> int:
    n = _SZ(0)
    _check(lib().mtl_moe_router_sizes(ctypes.byref(cfg), ctypes.byref(n)), "mtl_moe_router_sizes")
    return int(n.value)


def mtl_moe_router_bwd(cfg, x, w_r, logits, topk_idx, gates, dgates, aux_coeff, aux_loss, dlogits, dw_r, dx,
                       scratch, scratch_bytes=None, stream=None):
    _check(lib().mtl_moe_router_bwd(ctypes.byref(cfg), _ptr(x), _ptr(w_r), _ptr(logits), _ptr(topk_idx), _ptr(gates),
                                    _ptr(dgates), float(aux_coeff), _ptr(aux_loss), _ptr(dlogits), _ptr(dw_r),
                                    _ptr(dx), _ptr(scratch), _nbytes(scratch, scratch_bytes), _stream(stream)),
           "mtl_moe_router_bwd")


def mtl_moe_route(cfg, logits, topk_idx, gates, stream=None):
    _check(lib().mtl_moe_route(ctypes.byref(cfg), _ptr(logits), _ptr(topk_idx), _ptr(gates), _stream(stream)),
           "mtl_moe_route")


def mtl_moe_permute(cfg, topk_idx, counts, offsets, perm_token, perm_slot, slot_row, stream=None):
    _check(lib().mtl_moe_permute(ctypes.byref(cfg), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm_token),
                                 _ptr(perm_slot), _ptr(slot_row), _stream(stream)), "mtl_moe_permute")


def mtl_moe_fwd(cfg, x, offsets, perm_token, slot_row, gates, w1, w2, xp, gz, a, ye, y_partial, stream=None):
    _check(lib().mtl_moe_fwd(ctypes.byref(cfg), _ptr(x), _ptr(offsets), _ptr(perm_token), _ptr(slot_row),
                             _ptr(gates), _ptr(w1), _ptr(w2), _ptr(xp), _ptr(gz), _ptr(a), _ptr(ye), _ptr(y_partial),
                             _stream(stream)), "mtl_moe_fwd")


def mtl_moe_bwd(cfg, dy, offsets, perm_token, perm_slot, slot_row, gates, xp, gz, a, ye, w1, w2, dx_partial, dw1,
                dw2, dgates, scratch, scratch_bytes=None, stream=None):
    nbytes = scratch.numel() * scratch.element_size() if scratch_bytes is None else scratch_bytes
    _check(lib().mtl_moe_bwd(ctypes.byref(cfg), _ptr(dy), _ptr(offsets), _ptr(perm_token), _ptr(perm_slot),
                             _ptr(slot_row), _ptr(gates), _ptr(xp), _ptr(gz), _ptr(a), _ptr(ye), _ptr(w1), _ptr(w2),
                             _ptr(dx_partial), _ptr(dw1), _ptr(dw2), _ptr(dgates), _ptr(scratch), nbytes,
                             _stream(stream)), "mtl_moe_bwd")


def mtl_fp8_amax(x, n, fmt, rec, scratch, scratch_bytes=None, stream=None):
    _check(lib().mtl_fp8_amax(_ptr(x), n, fmt, _ptr(rec), _ptr(scratch), _nbytes(scratch, scratch_bytes),
                              _stream(stream)), "mtl_fp8_amax")


def mtl_fp8_cast(x, rows, cols, fmt, rec, out, out_t=None, stream=None):
    _check(lib().mtl_fp8_cast(_ptr(x), rows, cols, fmt, _ptr(rec), _ptr(out), _ptr(out_t), _stream(stream)),
           "mtl_fp8_cast")


def mtl_fp8_quantize(x, rows, cols, fmt, rec, out, out_t, scratch, scratch_bytes=None, stream=None):
    _check(lib().mtl_fp8_quantize(_ptr(x), rows, cols, fmt, _ptr(rec), _ptr(out), _ptr(out_t), _ptr(scratch),
                                  _nbytes(scratch, scratch_bytes), _stream(stream)), "mtl_fp8_quantize")


def mtl_prof_start():
    _check(lib().mtl_prof_start(), "mtl_prof_start")


def mtl_prof_stop() -> int:
    n = _I32(0)
    _check(lib().mtl_prof_stop(ctypes.byref(n)), "mtl_prof_stop")
    return n.value


def mtl_prof_record(i: int) -> dict:
    """Launch group i of the last recording: kind, name, algorithmic flop and
    bytes, and the milliseconds between its two HIP events."""
    kind, flop, nbytes, ms, name = _I32(0), ctypes.c_double(0), ctypes.c_double(0), ctypes.c_float(0), \
        ctypes.c_char_p()
    _check(lib().mtl_prof_record(i, ctypes.byref(kind), ctypes.byref(flop), ctypes.byref(nbytes), ctypes.byref(ms),
                                 ctypes.byref(name)), "mtl_prof_record")
    return dict(kind=MTL_PROF_KINDS[kind.value], name=name.value.decode(), flop=flop.value, bytes=nbytes.value,
                ms=ms.value)


def mtl_mfma_ceiling(data, kind, workgroups, iters, out, data_bytes=None, stream=None):
    _check(lib().mtl_mfma_ceiling(_ptr(data), _nbytes(data, data_bytes), kind, workgroups, iters, _ptr(out),
                                  _stream(stream)), "mtl_mfma_ceiling")


def mtl_fp8_gemm(M, N, K, a, fmt_a, a_rec, b, fmt_b, b_rec, bias, c, ldc=None, stream=None):
    _check(lib().mtl_fp8_gemm(M, N, K, _ptr(a), fmt_a, _ptr(a_rec), _ptr(b), fmt_b, _ptr(b_rec), _ptr(bias), _ptr(c),
                              N if ldc is None else ldc, _stream(stream)), "mtl_fp8_gemm")
