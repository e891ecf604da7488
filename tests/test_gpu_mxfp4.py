"""Parity of mtl_mxfp4_quantize / mtl_mxfp6_quantize (bit-exact codes and
scales) and mtl_mxfp4_gemm / mtl_mxfp6_gemm with the fp64 MX oracle: every
finite bf16 value, special blocks (ties, saturation, zeros, tiny and huge
magnitudes), a GEMM spanning several tiles and K slabs, and on sampled rows
and columns (tile edges among them) the 4096 x 4096 x 4096 GEMM and products
that take each of the GEMM's tile shapes."""
import numpy as np
import pytest

import synth
from oracle import mxfp4 as MX
from tests.parity_util import assert_bf16, f64


def _quant_dev(bits):
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_mxfp4_quantize
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    rows, cols = bits.shape
    x = bf16_dev(bits)
    codes = torch.empty(rows, cols // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device="cuda")
    mtl_mxfp4_quantize(x, rows, cols, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((b >> 7) & 0xFF) != 0xFF
    return b[finite]


def _special_blocks():
    rows = []
    for k in (-126, -40, -1, 0, 3, 100, 125):
        for mids in ([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], [6.0, 7.0, 7.9, 5.5, 0.2, 0.1, 4.5]):
            blk = np.zeros(32)
            blk[0] = 6.0
            blk[1:1 + len(mids)] = mids
            blk[16:16 + len(mids)] = -np.array(mids)
            rows.append(blk * 2.0 ** k)
    rows.append(np.zeros(32))
    z = np.zeros(32)
    z[5] = -0.0
    rows.append(z)
    rows.append(np.full(32, 2.0 ** -133))  # bf16 subnormals
    rows.append(np.full(32, 3.0e38))
    return synth.bf16_round_bits(np.array(rows))


@pytest.mark.gpu
@pytest.mark.parametrize("layout", ["sorted", "shuffled", "special"])
def test_mxfp4_quantize_bit_exact(mtl, layout):
    if layout == "special":
        bits = _special_blocks()
    else:
        vals = _all_finite_bf16()
        vals = vals[: (len(vals) // 256) * 256]
        if layout == "shuffled":
            vals = np.random.default_rng(1).permutation(vals)
        bits = vals.reshape(-1, 256)
    print(f"mxfp4 quantize {layout} {bits.shape}", flush=True)
    codes, scales = _quant_dev(bits)
    ref_codes, ref_scales = MX.quantize(f64(bits))
    assert np.array_equal(scales.cpu().numpy(), ref_scales)
    assert np.array_equal(codes.cpu().numpy(), MX.pack(ref_codes))


def _gemm_dev(a_bits, b_bits):
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_mxfp4_gemm
    ca, sa = _quant_dev(a_bits)
    cb, sb = _quant_dev(b_bits)
    M, K = a_bits.shape
    N = b_bits.shape[0]
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    mtl_mxfp4_gemm(M, N, K, ca, sa, cb, sb, c)
    torch.cuda.synchronize()
    return c, (ca, sa, cb, sb)


def _close(name, got, ref):
    assert_bf16(name, got, ref)
    # products of scaled E2M1 values are exact and summed in fp32: only the bf16 output rounding remains
    rel = np.abs(got - ref) / (np.abs(ref) + 1e-3 * np.abs(ref).max())
    assert rel.max() <= 2.0 ** -7, f"{name}: max relative error {rel.max():.3e}"


@pytest.mark.gpu
def test_mxfp4_gemm_tiles_and_slabs(mtl):
    from megatron_tensor_transformer_layer_amd.layer import host_f64
    M, N, K = 256, 384, 768
    print(f"mxfp4 gemm {M}x{N}x{K}", flush=True)
    a = synth.mx_operand(M, K, "mx_a", 1.0, seed=2)
    b = synth.mx_operand(N, K, "mx_b", synth.WEIGHT_STD, seed=2)
    c, _ = _gemm_dev(a, b)
    ca, sa = MX.quantize(f64(a))
    cb, sb = MX.quantize(f64(b))
    _close("C", host_f64(c), MX.gemm(ca, sa, cb, sb))


# (M, N, K): the full-size workload (256 x 256 tiles), a product taking
# 256 x 192 tiles (fewer than 240 tiles of 256 x 256, N % 192 == 0) and one
# filling exactly 240 tiles of 256 x 256
GEMM_SHAPES = {
    "full-4096": (synth.MX_WORKLOADS["mxfp4-gemm-7b-tp4"].M, synth.MX_WORKLOADS["mxfp4-gemm-7b-tp4"].N,
                  synth.MX_WORKLOADS["mxfp4-gemm-7b-tp4"].K),
    "tiles-256x192": (2048, 6144, 1024),
    "tiles-256x256-240": (4096, 3840, 768),
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(GEMM_SHAPES))
def test_mxfp4_gemm_fullsize_sampled(mtl, case):
    from megatron_tensor_transformer_layer_amd.layer import host_f64
    M, N, K = GEMM_SHAPES[case]
    print(f"mxfp4 gemm {case} {M}x{N}x{K}", flush=True)
    a = synth.mx_operand(M, K, "mx_a", 1.0)
    b = synth.mx_operand(N, K, "mx_b", synth.WEIGHT_STD)
    c, (ca_d, sa_d, cb_d, sb_d) = _gemm_dev(a, b)
    rng = np.random.default_rng(5)
    edges = [0, 31, 32, 127, 128, 191, 192, 255, 256]  # fragment, 128-, 192- and 256-tile boundaries
    rm = sorted(set([e for e in edges if e < M] + [M - 1] + rng.choice(M, 8, replace=False).tolist()))
    rn = sorted(set([e for e in edges if e < N] + [N - 1] + rng.choice(N, 8, replace=False).tolist()))
    ca, sa = MX.quantize(f64(a[rm]))
    cb, sb = MX.quantize(f64(b[rn]))
    assert np.array_equal(ca_d.cpu().numpy()[rm], MX.pack(ca)) and np.array_equal(sa_d.cpu().numpy()[rm], sa)
    assert np.array_equal(cb_d.cpu().numpy()[rn], MX.pack(cb)) and np.array_equal(sb_d.cpu().numpy()[rn], sb)
    got = host_f64(c)[np.ix_(rm, rn)]
    assert np.all(np.isfinite(host_f64(c)))
    _close("C sampled", got, MX.gemm(ca, sa, cb, sb))


# ---------------------------------------------------------------- MXFP6
def _quant6_dev(bits):
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_mxfp6_quantize
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    rows, cols = bits.shape
    codes = torch.empty(rows, cols * 3 // 4, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device="cuda")
    mtl_mxfp6_quantize(bf16_dev(bits), rows, cols, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def _special6():
    rows = []
    mids = [0.0625, 0.1875, 0.9375, 1.0625, 1.9375, 3.875, 7.75, 7.7, 5.25, 5.26, 0.05, 2.125, 6.75]
    for k in (-126, -40, -1, 0, 3, 100, 125):
        blk = np.zeros(32)
        blk[0] = 7.5
        blk[1:1 + len(mids)] = mids
        blk[16:16 + len(mids)] = -np.array(mids)
        rows.append(blk * 2.0 ** k)
    rows.append(np.zeros(32))
    rows.append(np.full(32, 2.0 ** -133))
    rows.append(np.full(32, 3.0e38))
    return synth.bf16_round_bits(np.array(rows))


@pytest.mark.gpu
@pytest.mark.parametrize("layout", ["sorted", "shuffled", "special"])
def test_mxfp6_quantize_bit_exact(mtl, layout):
    if layout == "special":
        bits = _special6()
    else:
        vals = _all_finite_bf16()
        vals = vals[: (len(vals) // 256) * 256]
        if layout == "shuffled":
            vals = np.random.default_rng(2).permutation(vals)
        bits = vals.reshape(-1, 256)
    print(f"mxfp6 quantize {layout} {bits.shape}", flush=True)
    codes, scales = _quant6_dev(bits)
    ref_codes, ref_scales = MX.quantize(f64(bits), "e2m3")
    assert np.array_equal(scales.cpu().numpy(), ref_scales)
    assert np.array_equal(codes.cpu().numpy(), MX.pack6(ref_codes))


def _gemm6_dev(a_bits, b_bits):
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_mxfp6_gemm
    ca, sa = _quant6_dev(a_bits)
    cb, sb = _quant6_dev(b_bits)
    M, K = a_bits.shape
    N = b_bits.shape[0]
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    mtl_mxfp6_gemm(M, N, K, ca, sa, cb, sb, c)
    torch.cuda.synchronize()
    return c, (ca, sa, cb, sb)


@pytest.mark.gpu
def test_mxfp6_gemm_tiles_and_slabs(mtl):
    from megatron_tensor_transformer_layer_amd.layer import host_f64
    M, N, K = 256, 384, 640
    print(f"mxfp6 gemm {M}x{N}x{K}", flush=True)
    a = synth.mx_operand(M, K, "mx_a", 1.0, seed=3)
    b = synth.mx_operand(N, K, "mx_b", synth.WEIGHT_STD, seed=3)
    c, _ = _gemm6_dev(a, b)
    ca, sa = MX.quantize(f64(a), "e2m3")
    cb, sb = MX.quantize(f64(b), "e2m3")
    _close("C", host_f64(c), MX.gemm(ca, sa, cb, sb, "e2m3"))


@pytest.mark.gpu
def test_mxfp6_gemm_fullsize_sampled(mtl):
    from megatron_tensor_transformer_layer_amd.layer import host_f64
    shape = synth.MX_WORKLOADS["mxfp4-gemm-7b-tp4"]
    M, N, K = shape.M, shape.N, shape.K
    print(f"mxfp6 gemm full size {M}x{N}x{K}", flush=True)
    a = synth.mx_operand(M, K, "mx_a", 1.0)
    b = synth.mx_operand(N, K, "mx_b", synth.WEIGHT_STD)
    c, (ca_d, sa_d, cb_d, sb_d) = _gemm6_dev(a, b)
    rng = np.random.default_rng(6)
    rm = sorted(set([0, 127, 128, M - 1] + rng.choice(M, 6, replace=False).tolist()))
    rn = sorted(set([0, 127, 128, N - 1] + rng.choice(N, 6, replace=False).tolist()))
    ca, sa = MX.quantize(f64(a[rm]), "e2m3")
    cb, sb = MX.quantize(f64(b[rn]), "e2m3")
    assert np.array_equal(ca_d.cpu().numpy()[rm], MX.pack6(ca)) and np.array_equal(sa_d.cpu().numpy()[rm], sa)
    assert np.array_equal(cb_d.cpu().numpy()[rn], MX.pack6(cb)) and np.array_equal(sb_d.cpu().numpy()[rn], sb)
    assert np.all(np.isfinite(host_f64(c)))
    _close("C sampled", host_f64(c)[np.ix_(rm, rn)], MX.gemm(ca, sa, cb, sb, "e2m3"))
