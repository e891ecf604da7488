"""The C-ABI library on a host without a GPU: it loads, exports every entry
point the header declares, and its host-side validation returns the documented
status codes before any launch."""
import ctypes
import json
import os
import re

import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _declared(header):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mtl_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(mtl):
    names = _declared(mtl.HEADER)
    assert "mtl_attn_fwd" in names and "mtl_reduce" in names
    lib = mtl.lib()
    for n in names:
        assert hasattr(lib, n), n
    # every declared entry point has a Python binding of the same name
    for n in names:
        if n not in ("mtl_status_str",):
            assert hasattr(mtl, n), n


def test_validate_divisibility_cases_from_the_pages(mtl):
    cases = json.load(open(os.path.join(GOLDEN, "divisibility.json")))
    for c in cases["dense"]:
        d = c["hidden"] // c["heads"] if c["hidden"] % c["heads"] == 0 else 0
        cfg = mtl.make_cfg(c["hidden"], c["heads"], c["ffn"], 512, 1, c["tp"], 0)
        st = mtl.mtl_validate(cfg)
        if not c["ok"]:
            assert st == mtl.MTL_E_DIVISIBILITY, c
        elif d in (64, 128):
            assert st == mtl.MTL_OK, c
        else:  # legal split, head size outside what the kernels are built for
            assert st == mtl.MTL_E_SHAPE, c


def test_validate_codes(mtl):
    ok = dict(hidden=4096, heads=32, ffn=16384, seq=4096, micro_batch=1, tp=4, rank=0)
    assert mtl.mtl_validate(mtl.make_cfg(**ok)) == mtl.MTL_OK
    bad = [
        (dict(rank=4), mtl.MTL_E_RANK), (dict(rank=-1), mtl.MTL_E_RANK),
        (dict(ffn=16382), mtl.MTL_E_DIVISIBILITY), (dict(heads=30), mtl.MTL_E_DIVISIBILITY),
        (dict(seq=0), mtl.MTL_E_SHAPE), (dict(hidden=0), mtl.MTL_E_SHAPE),
        (dict(hidden=3072, heads=32), mtl.MTL_E_SHAPE),  # d = 96
        (dict(ffn=4 * 1028), mtl.MTL_E_SHAPE),  # ffn/tp = 1028, not a multiple of 8
    ]
    for change, want in bad:
        assert mtl.mtl_validate(mtl.make_cfg(**{**ok, **change})) == want, change
    c = mtl.make_cfg(**ok)
    c.precision = 7
    assert mtl.mtl_validate(c) == mtl.MTL_E_UNSUPPORTED
    c = mtl.make_cfg(**ok)
    c.flags = 64
    assert mtl.mtl_validate(c) == mtl.MTL_E_UNSUPPORTED
    assert mtl.lib().mtl_validate(None) == mtl.MTL_E_NULL


def test_workspace_bytes(mtl):
    cfg = mtl.make_cfg(4096, 32, 16384, 4096, 1, 4, 0)
    n = mtl.mtl_workspace_bytes(cfg)
    S, f_l, qkv_l = 4096, 4096, 3072
    assert n >= S * f_l * 2 and n >= S * qkv_l * 2
    assert n < 1 << 30
    with pytest.raises(mtl.MtlError) as e:
        mtl.mtl_workspace_bytes(mtl.make_cfg(4096, 32, 16384, 4096, 1, 4, 9))
    assert e.value.status == mtl.MTL_E_RANK


def test_errors_before_launch(mtl):
    """NULL, misaligned and too-small-scratch arguments are refused on the host:
    nothing touches the (fake, never dereferenced) addresses."""
    cfg = mtl.make_cfg(256, 2, 512, 64, 1, 2, 0)
    P = 1 << 20  # a fake, aligned address
    lib = mtl.lib()
    st = lib.mtl_attn_fwd(ctypes.byref(cfg), None, P, P, P, P, P, P, P, None, 0, None)
    assert st == mtl.MTL_E_NULL
    st = lib.mtl_attn_fwd(ctypes.byref(cfg), P + 2, P, P, P, P, P, P, P, None, 0, None)
    assert st == mtl.MTL_E_ALIGN
    st = lib.mtl_mlp_bwd(ctypes.byref(cfg), P, P, P, P, P, P, P, P, P, P, None, P, 16, None)
    assert st == mtl.MTL_E_WORKSPACE
    st = lib.mtl_attn_bwd(ctypes.byref(cfg), P, P, P, P, P, P, P, P, P, P, P, None, P, 16, None)
    assert st == mtl.MTL_E_WORKSPACE
    arr = (ctypes.c_void_p * 2)(P, P)
    assert lib.mtl_reduce(2, arr, None, None, P, 64, 12, 0, 64, None) == mtl.MTL_E_SHAPE  # cols % 8
    assert lib.mtl_reduce(2, arr, None, None, P, 64, 16, 0, 65, None) == mtl.MTL_E_SHAPE
    assert lib.mtl_reduce(0, arr, None, None, P, 64, 16, 0, 64, None) == mtl.MTL_E_SHAPE
    assert lib.mtl_reduce(2, arr, None, None, P, 64, 16, 0, 64, None) == mtl.MTL_E_UNSUPPORTED  # out aliases
    assert lib.mtl_reduce(2, None, None, None, P, 64, 16, 0, 64, None) == mtl.MTL_E_NULL
    Q = P + (1 << 16)
    bufs = (ctypes.c_void_p * 2)(P, Q)
    assert lib.mtl_allgather_rows(2, 0, bufs, P, 63, 16, None) == mtl.MTL_E_SHAPE  # rows % t
    assert lib.mtl_allgather_rows(2, 0, bufs, P, 64, 12, None) == mtl.MTL_E_SHAPE  # cols % 8
    assert lib.mtl_allgather_rows(2, 2, bufs, P, 64, 16, None) == mtl.MTL_E_RANK
    assert lib.mtl_allgather_rows(2, -1, bufs, P, 64, 16, None) == mtl.MTL_E_RANK
    assert lib.mtl_allgather_rows(2, 1, bufs, P, 64, 16, None) == mtl.MTL_E_UNSUPPORTED  # a peer buffer is out
    assert lib.mtl_allgather_rows(2, 0, None, P, 64, 16, None) == mtl.MTL_E_NULL
    assert lib.mtl_allgather_rows(2, 0, (ctypes.c_void_p * 2)(P, None), Q, 64, 16, None) == mtl.MTL_E_NULL
    assert lib.mtl_allgather_rows(2, 0, (ctypes.c_void_p * 2)(P, Q + 8), P, 64, 16, None) == mtl.MTL_E_ALIGN


def test_status_strings(mtl):
    for s in range(9):
        assert mtl.status_text(s) not in ("", "unknown status")


def test_moe_validate_codes(mtl):
    cases = json.load(open(os.path.join(GOLDEN, "divisibility.json")))
    for c in cases["moe"]:
        cfg = mtl.make_moe_cfg(4096, 7168, 18432, c["experts"], c["topk"], c["ep"], 0)
        st = mtl.mtl_moe_validate(cfg)
        assert st == (mtl.MTL_OK if c["ok"] else mtl.MTL_E_DIVISIBILITY), c
    ok = dict(tokens=4096, hidden=7168, ffn=18432, experts=256, topk=8, ep=16, rank=0)
    assert mtl.mtl_moe_validate(mtl.make_moe_cfg(**ok)) == mtl.MTL_OK
    bad = [
        (dict(rank=16), mtl.MTL_E_RANK), (dict(rank=-1), mtl.MTL_E_RANK),
        (dict(experts=250), mtl.MTL_E_DIVISIBILITY),
        (dict(tokens=0), mtl.MTL_E_SHAPE), (dict(topk=0), mtl.MTL_E_SHAPE),
        (dict(hidden=7170), mtl.MTL_E_SHAPE), (dict(ffn=18436), mtl.MTL_E_SHAPE),
        (dict(experts=2048, ep=16), mtl.MTL_E_SHAPE),  # more experts than the router kernel holds
        (dict(experts=4, ep=1, topk=5), mtl.MTL_E_SHAPE),  # k > E
        (dict(tokens=1 << 20), mtl.MTL_E_SHAPE),  # grouped rows x 18432 past 4 GiB
    ]
    for change, want in bad:
        assert mtl.mtl_moe_validate(mtl.make_moe_cfg(**{**ok, **change})) == want, change
    c = mtl.make_moe_cfg(**ok)
    c.precision = mtl.MTL_PREC_FP8_HYBRID
    assert mtl.mtl_moe_validate(c) == mtl.MTL_E_UNSUPPORTED
    assert mtl.lib().mtl_moe_validate(None) == mtl.MTL_E_NULL


def test_moe_sizes(mtl):
    # N_max = T * min(k, E/ep): every one of a token's k slots can be local
    rows, scratch = mtl.mtl_moe_sizes(mtl.make_moe_cfg(4096, 7168, 18432, 256, 8, 16, 0))
    assert rows == 4096 * 8
    assert scratch >= rows * (7168 + 18432) * 2
    # fewer local experts than k bounds the rows by T * E/ep
    rows, _ = mtl.mtl_moe_sizes(mtl.make_moe_cfg(100, 64, 128, 8, 4, 4, 1))
    assert rows == 100 * 2


def test_moe_errors_before_launch(mtl):
    cfg = mtl.make_moe_cfg(64, 128, 256, 8, 2, 2, 0)
    P = 1 << 20
    lib = mtl.lib()
    assert lib.mtl_moe_route(ctypes.byref(cfg), P, None, P, None) == mtl.MTL_E_NULL
    assert lib.mtl_moe_permute(ctypes.byref(cfg), P, P, P, P, P + 4, P, None) == mtl.MTL_E_ALIGN
    args = [P] * 12
    args[3] = None
    assert lib.mtl_moe_fwd(ctypes.byref(cfg), *args, None) == mtl.MTL_E_NULL
    assert lib.mtl_moe_bwd(ctypes.byref(cfg), *([P] * 17), 16, None) == mtl.MTL_E_WORKSPACE


def test_fp8_validate_and_errors_before_launch(mtl):
    ok = dict(hidden=4096, heads=32, ffn=16384, seq=4096, micro_batch=1, tp=4, rank=0,
              precision=mtl.MTL_PREC_FP8_HYBRID)
    assert mtl.mtl_validate(mtl.make_cfg(**ok)) == mtl.MTL_OK
    # fp8 GEMMs contract over 16-byte code chunks
    assert mtl.mtl_validate(mtl.make_cfg(**{**ok, "seq": 4088})) == mtl.MTL_E_SHAPE
    assert mtl.mtl_validate(mtl.make_cfg(**{**ok, "ffn": 4 * 4104})) == mtl.MTL_E_SHAPE
    assert mtl.mtl_validate(mtl.make_cfg(**{**ok, "seq": 4088, "precision": mtl.MTL_PREC_BF16})) == mtl.MTL_OK
    # fp8 needs scratch in the forward calls too, for the operands' codes
    n8 = mtl.mtl_workspace_bytes(mtl.make_cfg(**ok))
    n16 = mtl.mtl_workspace_bytes(mtl.make_cfg(**{**ok, "precision": mtl.MTL_PREC_BF16}))
    assert n8 > n16
    cfg = mtl.make_cfg(**ok)
    P = 1 << 20
    lib = mtl.lib()
    assert lib.mtl_attn_fwd(ctypes.byref(cfg), P, P, P, P, P, P, P, P, None, 0, None) == mtl.MTL_E_NULL
    assert lib.mtl_attn_fwd(ctypes.byref(cfg), P, P, P, P, P, P, P, P, P, 64, None) == mtl.MTL_E_WORKSPACE
    assert lib.mtl_mlp_fwd(ctypes.byref(cfg), P, P, P, P, P, P, P, P, 64, None) == mtl.MTL_E_WORKSPACE
    assert lib.mtl_mlp_bwd(ctypes.byref(cfg), P, P, P, P, P, P, P, P, P, P, None, P, n16, None) == \
        mtl.MTL_E_WORKSPACE
    # the standalone amax / cast calls
    assert lib.mtl_fp8_amax(P, 1024, 0, P, P, 64, None) == mtl.MTL_E_WORKSPACE
    assert lib.mtl_fp8_amax(P, 0, 0, P, P, mtl.MTL_FP8_AMAX_SCRATCH, None) == mtl.MTL_E_SHAPE
    assert lib.mtl_fp8_amax(P, 1024, 2, P, P, mtl.MTL_FP8_AMAX_SCRATCH, None) == mtl.MTL_E_UNSUPPORTED
    assert lib.mtl_fp8_cast(P, 64, 12, 0, P, P, None, None) == mtl.MTL_E_SHAPE  # cols % 8
    assert lib.mtl_fp8_cast(P, 40, 16, 0, P, None, P, None) == mtl.MTL_E_SHAPE  # transposed needs rows % 16
    assert lib.mtl_fp8_cast(P, 64, 16, 0, P, None, None, None) == mtl.MTL_E_NULL
    assert lib.mtl_fp8_cast(P, 64, 16, 0, P, P + 8, None, None) == mtl.MTL_E_ALIGN
    S = mtl.MTL_FP8_AMAX_SCRATCH
    assert lib.mtl_fp8_quantize(P, 64, 16, 0, P, P, None, P, 64, None) == mtl.MTL_E_WORKSPACE
    assert lib.mtl_fp8_quantize(P, 64, 12, 0, P, P, None, P, S, None) == mtl.MTL_E_SHAPE
    assert lib.mtl_fp8_quantize(P, 40, 16, 0, P, None, P, P, S, None) == mtl.MTL_E_SHAPE
    assert lib.mtl_fp8_quantize(P, 64, 16, 0, P, None, None, P, S, None) == mtl.MTL_E_NULL
    assert lib.mtl_fp8_quantize(P, 64, 16, 0, P, P, None, None, S, None) == mtl.MTL_E_NULL
    assert lib.mtl_fp8_quantize(P, 64, 16, 3, P, P, None, P, S, None) == mtl.MTL_E_UNSUPPORTED


def test_router_validation_before_any_launch(mtl):
    """The router calls check their configuration, pointers, coefficient and
    workspace on the host (fake, never dereferenced addresses)."""
    P = 1 << 20
    lib = mtl.lib()
    cfg = mtl.make_moe_cfg(64, 128, 8, 32, 4)
    n = mtl.mtl_moe_router_sizes(cfg)
    assert n > 0
    assert lib.mtl_moe_router_fwd(ctypes.byref(cfg), P, P, None, None) == mtl.MTL_E_NULL
    assert lib.mtl_moe_router_fwd(ctypes.byref(cfg), P, P + 4, P, None) == mtl.MTL_E_ALIGN
    bad = mtl.make_moe_cfg(64, 128, 8, 12, 4)  # experts % 8
    assert lib.mtl_moe_router_fwd(ctypes.byref(bad), P, P, P, None) == mtl.MTL_E_SHAPE
    args = [P, P, P, P, P, P]
    for coeff in (-1.0, float("nan"), float("inf")):
        assert lib.mtl_moe_router_bwd(ctypes.byref(cfg), *args, coeff, None, P, P, P, P, n, None) == mtl.MTL_E_SHAPE
    assert lib.mtl_moe_router_bwd(ctypes.byref(cfg), *args, 0.001, None, P, P, P, P, n - 1, None) == \
        mtl.MTL_E_WORKSPACE
    assert lib.mtl_moe_router_bwd(ctypes.byref(cfg), *args, 0.001, None, P, P, None, P, n, None) == mtl.MTL_E_NULL


def test_cp_attention_validation_before_any_launch(mtl):
    """mtl_cp_attn_fwd / _scratch_bytes refuse bad shapes, ranks, pointers and
    scratch on the host; the fake addresses are never dereferenced."""
    lib = mtl.lib()
    P = 1 << 20
    n = ctypes.c_size_t(0)
    sb = lambda *a: lib.mtl_cp_attn_scratch_bytes(*a, ctypes.byref(n))
    assert sb(4, 0, 256, 2, 128) == mtl.MTL_OK and n.value == 0  # rank 0 merges nothing
    assert sb(4, 3, 256, 2, 128) == mtl.MTL_OK
    # four partials: O_j [256, 2*128] bf16 and L_j [2, 256] fp32 each, 256-byte aligned
    assert n.value == 4 * (256 * 256 * 2 + 2 * 256 * 4)
    assert sb(4, 4, 256, 2, 128) == mtl.MTL_E_RANK
    assert sb(4, -1, 256, 2, 128) == mtl.MTL_E_RANK
    assert sb(0, 0, 256, 2, 128) == mtl.MTL_E_SHAPE
    assert sb(mtl.MTL_CP_MAX + 1, 0, 256, 2, 128) == mtl.MTL_E_SHAPE
    assert sb(4, 1, 200, 2, 128) == mtl.MTL_E_SHAPE  # chunk % 64
    assert sb(4, 1, 256, 2, 96) == mtl.MTL_E_SHAPE  # head_dim 64 or 128
    assert sb(4, 1, 256, 0, 128) == mtl.MTL_E_SHAPE
    assert sb(4, 1, 1 << 22, 64, 128) == mtl.MTL_E_SHAPE  # past 32-bit buffer offsets
    # (chunk + 64) * 3 * heads * head_dim * 2 = 3 * 2^69 wraps to 0 in 64 bits: still refused
    assert sb(4, 1, (1 << 31) - 64, 1 << 30, 128) == mtl.MTL_E_SHAPE
    assert sb(4, 1, 64, (1 << 31) - 1, 128) == mtl.MTL_E_SHAPE
    assert lib.mtl_cp_attn_scratch_bytes(4, 1, 256, 2, 128, None) == mtl.MTL_E_NULL

    chunks = (ctypes.c_void_p * 4)(P, P + 4096, None, None)  # only entries 0..rank are read
    need = 2 * (256 * 256 * 2 + 2 * 256 * 4)
    fwd = lambda rank, ch, o, lse, scr, nb: lib.mtl_cp_attn_fwd(4, rank, 256, 2, 128, ch, o, lse, scr, nb, None)
    assert fwd(1, chunks, P, P, P, need - 1) == mtl.MTL_E_WORKSPACE
    assert fwd(1, chunks, P, P, None, need) == mtl.MTL_E_NULL
    assert fwd(2, chunks, P, P, P, 10 * need) == mtl.MTL_E_NULL  # chunk 2 missing
    assert fwd(1, None, P, P, P, need) == mtl.MTL_E_NULL
    assert fwd(1, chunks, None, P, P, need) == mtl.MTL_E_NULL
    assert fwd(1, chunks, P + 8, P, P, need) == mtl.MTL_E_ALIGN
    assert fwd(1, (ctypes.c_void_p * 2)(P, P + 2), P, P, P, need) == mtl.MTL_E_ALIGN
    assert fwd(4, chunks, P, P, P, need) == mtl.MTL_E_RANK


def test_cp_attention_backward_validation_before_any_launch(mtl):
    lib = mtl.lib()
    P = 1 << 20
    n = ctypes.c_size_t(0)
    assert lib.mtl_cp_attn_bwd_scratch_bytes(4, 0, 256, 2, 128, ctypes.byref(n)) == mtl.MTL_OK
    assert n.value == 2 * 256 * 4  # D only
    assert lib.mtl_cp_attn_bwd_scratch_bytes(4, 2, 256, 2, 128, ctypes.byref(n)) == mtl.MTL_OK
    assert n.value == 2 * 256 * 4 + 2 * 256 * 256 * 2  # D and two dQ partials
    assert lib.mtl_cp_attn_bwd_scratch_bytes(4, 4, 256, 2, 128, ctypes.byref(n)) == mtl.MTL_E_RANK
    assert lib.mtl_cp_attn_bwd_scratch_bytes(4, 1, 100, 2, 128, ctypes.byref(n)) == mtl.MTL_E_SHAPE
    need = 2 * 256 * 4 + 256 * 256 * 2
    qkv = (ctypes.c_void_p * 2)(P, P + 4096)
    dkv = (ctypes.c_void_p * 1)(P + 8192)
    bwd = lambda rank, q, o, lse, do, dqkv, dk, scr, nb: lib.mtl_cp_attn_bwd(4, rank, 256, 2, 128, q, o, lse, do,
                                                                             dqkv, dk, scr, nb, None)
    assert bwd(1, qkv, P, P, P, P, dkv, P, need - 1) == mtl.MTL_E_WORKSPACE
    assert bwd(1, qkv, P, P, P, P, None, P, need) == mtl.MTL_E_NULL
    assert bwd(1, qkv, P, P, None, P, dkv, P, need) == mtl.MTL_E_NULL
    assert bwd(1, qkv, P, P, P, P, (ctypes.c_void_p * 1)(None), P, need) == mtl.MTL_E_NULL
    assert bwd(1, qkv, P, P, P, P + 8192, dkv, P, need) == mtl.MTL_E_UNSUPPORTED  # a peer share is dqkv
    assert bwd(1, qkv, P, P, P, P + 2, dkv, P, need) == mtl.MTL_E_ALIGN
    assert bwd(1, qkv, P, P, P, P, dkv, None, need) == mtl.MTL_E_NULL
    assert bwd(5, qkv, P, P, P, P, dkv, P, need) == mtl.MTL_E_RANK


def test_mxfp4_validation_before_any_launch(mtl):
    lib = mtl.lib()
    P = 1 << 20
    assert lib.mtl_mxfp4_quantize(None, 4, 64, P, P, None) == mtl.MTL_E_NULL
    assert lib.mtl_mxfp4_quantize(P, 4, 48, P, P, None) == mtl.MTL_E_SHAPE  # cols % 32
    assert lib.mtl_mxfp4_quantize(P, 0, 64, P, P, None) == mtl.MTL_E_SHAPE
    assert lib.mtl_mxfp4_quantize(P, 4, 64, P + 4, P, None) == mtl.MTL_E_ALIGN
    g = lambda M, N, K, c, ldc: lib.mtl_mxfp4_gemm(M, N, K, P, P, P, P, c, ldc, None)
    assert g(128, 128, 256, None, 128) == mtl.MTL_E_NULL
    assert g(100, 128, 256, P, 128) == mtl.MTL_E_SHAPE  # M % 128
    assert g(128, 192, 256, P, 192) == mtl.MTL_E_SHAPE  # N % 128
    assert g(128, 128, 320, P, 128) == mtl.MTL_E_SHAPE  # K % 256
    assert g(128, 128, 256, P, 64) == mtl.MTL_E_SHAPE  # ldc < N
    assert g(128, 128, 256, P + 8, 128) == mtl.MTL_E_ALIGN


def test_mxfp6_validation_before_any_launch(mtl):
    lib = mtl.lib()
    P = 1 << 20
    assert lib.mtl_mxfp6_quantize(P, 4, 48, P, P, None) == mtl.MTL_E_SHAPE  # cols % 32
    assert lib.mtl_mxfp6_quantize(P, 4, 64, None, P, None) == mtl.MTL_E_NULL
    g = lambda M, N, K: lib.mtl_mxfp6_gemm(M, N, K, P, P, P, P, P, N, None)
    assert g(128, 128, 192) == mtl.MTL_E_SHAPE  # K % 128
    assert g(64, 128, 128) == mtl.MTL_E_SHAPE
    assert lib.mtl_mxfp6_gemm(128, 128, 128, P, P, P + 4, P, P, 128, None) == mtl.MTL_E_ALIGN


def test_mx_ordered_validation_before_any_launch(mtl):
    lib = mtl.lib()
    P = 1 << 20
    E4, E6, PL, GO = mtl.MTL_MX_E2M1, mtl.MTL_MX_E2M3, mtl.MTL_MX_ORDER_PLAIN, mtl.MTL_MX_ORDER_GEMM
    q = lambda e, x, r, c, o: lib.mtl_mx_quantize_ordered(e, x, r, c, P, P, o, None)
    assert q(E4, None, 32, 256, GO) == mtl.MTL_E_NULL
    assert q(2, P, 32, 256, GO) == mtl.MTL_E_UNSUPPORTED  # element format
    assert q(E6, P, 32, 256, 2) == mtl.MTL_E_UNSUPPORTED  # order
    assert q(E4, P, 48, 256, GO) == mtl.MTL_E_SHAPE  # rows % 32 in GEMM order
    assert q(E6, P, 32, 384, GO) == mtl.MTL_E_SHAPE  # cols % 256 in GEMM order
    assert q(E4, P, 4, 48, PL) == mtl.MTL_E_SHAPE  # cols % 32
    assert q(E4, P + 4, 32, 256, GO) == mtl.MTL_E_ALIGN
    g = lambda e, M, N, K, o, c=P, ldc=None: lib.mtl_mx_gemm_ordered(e, M, N, K, P, P, P, P, c, N if ldc is None
                                                                     else ldc, o, None)
    assert g(E4, 64, 64, 256, GO, c=None) == mtl.MTL_E_NULL
    assert g(3, 64, 64, 256, GO) == mtl.MTL_E_UNSUPPORTED
    assert g(E4, 64, 64, 256, 5) == mtl.MTL_E_UNSUPPORTED
    assert g(E4, 48, 64, 256, GO) == mtl.MTL_E_SHAPE  # M % 32
    assert g(E6, 64, 80, 256, GO) == mtl.MTL_E_SHAPE  # N % 32
    assert g(E6, 64, 64, 384, GO) == mtl.MTL_E_SHAPE  # K % 256
    assert g(E4, 64, 128, 256, PL) == mtl.MTL_E_SHAPE  # plain: M % 128
    assert g(E6, 128, 128, 192, PL) == mtl.MTL_E_SHAPE  # plain MXFP6: K % 128
    assert g(E4, 64, 64, 256, GO, ldc=32) == mtl.MTL_E_SHAPE  # ldc < N
    assert g(E4, 64, 64, 256, GO, c=P + 8) == mtl.MTL_E_ALIGN


def test_launch_timing_host_side(mtl):
    """The launch-timing calls on a host without a GPU: start reports the
    missing device, stop and record validate their arguments."""
    lib = mtl.lib()
    n = ctypes.c_int32(-1)
    assert lib.mtl_prof_start() == mtl.MTL_E_HIP
    assert lib.mtl_prof_stop(None) == mtl.MTL_E_NULL
    assert lib.mtl_prof_stop(ctypes.byref(n)) == mtl.MTL_OK and n.value == 0
    k, f, b, ms, name = ctypes.c_int32(), ctypes.c_double(), ctypes.c_double(), ctypes.c_float(), ctypes.c_char_p()
    refs = [ctypes.byref(v) for v in (k, f, b, ms, name)]
    assert lib.mtl_prof_record(0, *refs) == mtl.MTL_E_SHAPE
    assert lib.mtl_prof_record(-1, *refs) == mtl.MTL_E_SHAPE
    assert lib.mtl_prof_record(0, None, *refs[1:]) == mtl.MTL_E_NULL


def test_noalloc_mlp_backward_host_side(mtl):
    """mtl_mlp_bwd_noalloc refuses, before any HIP call, a configuration whose
    MLP backward needs more scratch than its array holds, and a bad
    configuration; a configuration that fits reaches the device lookup, which
    fails without a GPU.  The fake addresses are never dereferenced."""
    lib = mtl.lib()
    P = 1 << 20
    args = [P] * 11 + [None]
    call = lambda cfg: lib.mtl_mlp_bwd_noalloc(ctypes.byref(cfg), *args)
    # dz alone: 2 * 4096 * 8192 bytes = 64 MiB > 48 MiB
    assert call(mtl.make_cfg(4096, 32, 32768, 4096, 1, 4, 0)) == mtl.MTL_E_WORKSPACE
    # fp8 codes at the 7B-class TP=4 shape do not fit either
    assert call(mtl.make_cfg(4096, 32, 16384, 4096, 1, 4, 0, mtl.MTL_PREC_FP8_HYBRID)) == mtl.MTL_E_WORKSPACE
    assert call(mtl.make_cfg(768, 12, 3072, 512, 1, 5, 0)) == mtl.MTL_E_DIVISIBILITY
    # the 96-layer GPT TP=8 rank fits (35 MiB)
    assert call(mtl.make_cfg(8192, 64, 32768, 4096, 1, 8, 0)) == mtl.MTL_E_HIP
    # kept codes would be read from a scratch the forward never wrote
    for prec in (mtl.MTL_PREC_FP8_HYBRID, mtl.MTL_PREC_MXFP4):
        assert call(mtl.make_cfg(1024, 8, 4096, 512, 1, 2, 0, prec, mtl.MTL_F_KEEP_CODES)) == mtl.MTL_E_UNSUPPORTED


def test_attn_bwd_scratch_layout(mtl):
    """dO sits at the start of mtl_attn_bwd's scratch and dQKV after it, at the
    next 256-byte boundary; both fit in the size mtl_workspace_bytes reports."""
    for hidden, heads, ffn, seq, tp in ((4096, 32, 16384, 4096, 4), (768, 12, 3072, 500, 2)):
        cfg = mtl.make_cfg(hidden, heads, ffn, seq, 1, tp, 0)
        off_do, off_dqkv = mtl.mtl_attn_bwd_scratch_layout(cfg)
        o_l, qkv_l = hidden // tp, 3 * hidden // tp
        assert off_do == 0
        assert off_dqkv == (seq * o_l * 2 + 255) // 256 * 256
        assert off_dqkv + seq * qkv_l * 2 <= mtl.mtl_workspace_bytes(cfg)
    with pytest.raises(mtl.MtlError):
        mtl.mtl_attn_bwd_scratch_layout(mtl.make_cfg(768, 12, 3072, 512, 1, 5, 0))


def test_fp8_gemm_validation_before_any_launch(mtl):
    lib = mtl.lib()
    P = 1 << 20
    g = lambda M, N, K, fa, fb, bias, c, ldc: lib.mtl_fp8_gemm(M, N, K, P, fa, P, P, fb, P, bias, c, ldc, None)
    E4, E5 = mtl.MTL_FP8_E4M3, mtl.MTL_FP8_E5M2
    assert g(256, 256, 100, E4, E4, None, P, 256) == mtl.MTL_E_SHAPE  # K % 16
    assert g(256, 256, 128, E4, E4, None, P, 200) == mtl.MTL_E_SHAPE  # ldc < N
    assert g(256, 256, 128, E4, E4, None, P, 260) == mtl.MTL_E_SHAPE  # ldc % 8
    assert g(0, 256, 128, E4, E4, None, P, 256) == mtl.MTL_E_SHAPE
    assert g(256, 256, 128, E5, E5, None, P, 256) == mtl.MTL_E_UNSUPPORTED  # not a pair of the recipe
    assert g(256, 256, 128, E5, E4, P, P, 256) == mtl.MTL_E_UNSUPPORTED  # bias on a dgrad
    assert g(256, 256, 128, E4, E4, P + 2, P, 256) == mtl.MTL_E_ALIGN
    assert g(256, 256, 128, E4, E4, None, None, 256) == mtl.MTL_E_NULL
    assert g(1 << 20, 256, 1 << 13, E4, E4, None, P, 256) == mtl.MTL_E_SHAPE  # A past 4 GiB


def test_fp8_keep_codes_flag(mtl):
    """MTL_F_KEEP_CODES (earlier name MTL_F_FP8_KEEP_CODES) is for fp8 and
    MXFP4; in fp8 its kept region adds the transposed codes (1 byte per
    element) and records of x, o, h and a, and both orientations of the four
    weights' codes, to the scratch size; in MXFP4 the column-blocked codes and
    scales of x, o, h, a and both blockings of the weights."""
    base = mtl.make_cfg(768, 12, 3072, 512, 1, 2, 0, mtl.MTL_PREC_FP8_HYBRID)
    kept = mtl.make_cfg(768, 12, 3072, 512, 1, 2, 0, mtl.MTL_PREC_FP8_HYBRID, mtl.MTL_F_FP8_KEEP_CODES)
    assert mtl.mtl_validate(kept) == mtl.MTL_OK
    S, h, o_l, f_l, qkv_l = 512, 768, 384, 1536, 1152
    up = lambda n: (n + 255) // 256 * 256
    # x, o, h, a transposed; w_qkv, w_o, w1, w2 in both orientations; 8 records
    extra = 8 * 256 + up(S * h) * 2 + up(S * o_l) + up(S * f_l) + 2 * (up(h * qkv_l) + up(o_l * h) + 2 * up(h * f_l))
    assert mtl.mtl_workspace_bytes(kept) == mtl.mtl_workspace_bytes(base) + extra
    bad = mtl.make_cfg(768, 12, 3072, 512, 1, 2, 0, mtl.MTL_PREC_BF16, mtl.MTL_F_FP8_KEEP_CODES)
    assert mtl.mtl_validate(bad) == mtl.MTL_E_UNSUPPORTED
    # MXFP4 keeps the column-blocked codes of x, o, h, a and both blockings of the weights (codes + scales in
    # 17/32 byte per element)
    mb = mtl.make_cfg(1024, 8, 4096, 512, 1, 2, 0, mtl.MTL_PREC_MXFP4)
    mk = mtl.make_cfg(1024, 8, 4096, 512, 1, 2, 0, mtl.MTL_PREC_MXFP4, mtl.MTL_F_KEEP_CODES)
    assert mtl.mtl_validate(mk) == mtl.MTL_OK
    S, h, o_l, f_l, qkv_l = 512, 1024, 512, 2048, 1536
    mx = lambda r, k: up(r * k // 2) + up(r * k // 32)
    extra_mx = (mx(h, S) + mx(o_l, S) + mx(h, S) + mx(f_l, S) + 2 * (mx(h, qkv_l) + mx(o_l, h) + mx(h, f_l) +
                                                                    mx(f_l, h)))
    assert mtl.mtl_workspace_bytes(mk) == mtl.mtl_workspace_bytes(mb) + extra_mx
    # reusing the weights' kept codes needs the kept region, and adds no scratch
    reuse = mtl.make_cfg(768, 12, 3072, 512, 1, 2, 0, mtl.MTL_PREC_FP8_HYBRID,
                         mtl.MTL_F_FP8_KEEP_CODES | mtl.MTL_F_FP8_REUSE_WEIGHTS)
    assert mtl.mtl_validate(reuse) == mtl.MTL_OK
    assert mtl.mtl_workspace_bytes(reuse) == mtl.mtl_workspace_bytes(kept)
    for prec, flags in ((mtl.MTL_PREC_FP8_HYBRID, mtl.MTL_F_FP8_REUSE_WEIGHTS),
                        (mtl.MTL_PREC_BF16, mtl.MTL_F_FP8_KEEP_CODES | mtl.MTL_F_FP8_REUSE_WEIGHTS)):
        assert mtl.mtl_validate(mtl.make_cfg(768, 12, 3072, 512, 1, 2, 0, prec, flags)) == mtl.MTL_E_UNSUPPORTED


def test_mfma_ceiling_argument_checks(mtl):
    """mtl_mfma_ceiling refuses bad arguments before any HIP call."""
    import ctypes
    f = mtl.lib().mtl_mfma_ceiling
    fake = ctypes.c_void_p(1 << 20)
    assert f(None, 1 << 20, 0, 256, 1, fake, None) == mtl.MTL_E_NULL
    assert f(ctypes.c_void_p((1 << 20) + 8), 1 << 20, 0, 256, 1, fake, None) == mtl.MTL_E_ALIGN
    assert f(fake, 1 << 20, 3, 256, 1, fake, None) == mtl.MTL_E_UNSUPPORTED
    assert f(fake, 1 << 20, -1, 256, 1, fake, None) == mtl.MTL_E_UNSUPPORTED
    assert f(fake, (1 << 20) - 16, 0, 256, 1, fake, None) == mtl.MTL_E_SHAPE
    assert f(fake, 1 << 20, 0, 0, 1, fake, None) == mtl.MTL_E_SHAPE
    assert f(fake, 1 << 20, 1, 256, 0, fake, None) == mtl.MTL_E_SHAPE
