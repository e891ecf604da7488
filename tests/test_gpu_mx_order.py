"""The MX quantisers and GEMMs in the GEMM's byte order (mtl_mx_quantize_ordered,
mtl_mx_gemm_ordered with MTL_MX_ORDER_GEMM).

* Layout: the GEMM-order codes and scales are exactly the plain ones moved as
  the header describes (the permutation is rebuilt here in numpy from that
  description), and the plain ones are the oracle's (bit-exact).
* Products: MXFP4 and MXFP6 GEMMs on GEMM-order operands against the fp64
  product of the oracle's dequantised codes, in full on a product spanning
  several tiles and slabs, and on sampled rows and columns (tile edges among
  them) at the 4096 x 4096 x 4096 workload and at shapes taking each tile
  shape.
"""
import numpy as np
import pytest

import synth
from oracle import mxfp4 as MX
from tests.parity_util import assert_bf16, f64

ELEMS = {"mxfp4": "e2m1", "mxfp6": "e2m3"}


def scales_to_gemm_order(plain):
    """[rows, cols/32] -> bytes in GEMM order: group (r // 32) * (cols // 256) +
    q // 8 of 256 bytes, block q % 8 of row r at 4 * (r % 32 + 32 * (q % 2)) + (q % 8) // 2."""
    rows, nb = plain.shape
    r, q = np.meshgrid(np.arange(rows), np.arange(nb), indexing="ij")
    qq = q % 8
    idx = ((r // 32) * (nb // 8) + q // 8) * 256 + 4 * (r % 32 + 32 * (qq % 2)) + qq // 2
    out = np.zeros(rows * nb, dtype=np.uint8)
    out[idx.ravel()] = plain.ravel()
    return out


def codes6_to_gemm_order(plain):
    """[rows, cols*3/4] MXFP6 codes -> GEMM order: per 128-element span (96
    bytes) the four blocks' first 16 bytes, then the last 8 bytes of blocks 0
    and 1, then of blocks 2 and 3, the two 8-byte halves swapped in rows with
    (row // 16) odd."""
    rows, nbytes = plain.shape
    out = np.zeros_like(plain)
    blocks = plain.reshape(rows, nbytes // 24, 24)
    for r in range(rows):
        swap = (r // 16) % 2
        for q in range(blocks.shape[1]):
            base, b = (q // 4) * 96, q % 4
            out[r, base + 16 * b:base + 16 * b + 16] = blocks[r, q, :16]
            t = base + 64 + (b // 2) * 16 + 8 * ((b % 2) ^ swap)
            out[r, t:t + 8] = blocks[r, q, 16:]
    return out


def _quant(mtl, elem, bits, order):
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_mx_quantize_ordered
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    rows, cols = bits.shape
    cb = cols * 3 // 4 if elem == "mxfp6" else cols // 2
    codes = torch.empty(rows, cb, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device="cuda")
    e = mtl.MTL_MX_E2M3 if elem == "mxfp6" else mtl.MTL_MX_E2M1
    mtl_mx_quantize_ordered(e, bf16_dev(bits), rows, cols, codes, scales, order)
    torch.cuda.synchronize()
    return codes, scales


@pytest.mark.gpu
@pytest.mark.parametrize("elem", list(ELEMS))
def test_gemm_order_is_the_plain_order_moved(mtl, elem):
    rows, cols = 96, 768
    print(f"{elem} order layout {rows}x{cols}", flush=True)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((rows, cols)) * np.exp(rng.standard_normal((rows, 1)) * 3)
    bits = synth.bf16_round_bits(x)
    cp, sp = _quant(mtl, elem, bits, mtl.MTL_MX_ORDER_PLAIN)
    cg, sg = _quant(mtl, elem, bits, mtl.MTL_MX_ORDER_GEMM)
    cp, sp, cg, sg = (t.cpu().numpy() for t in (cp, sp, cg, sg))
    ref_c, ref_s = MX.quantize(f64(bits), ELEMS[elem])
    assert np.array_equal(sp, ref_s)
    assert np.array_equal(cp, MX.pack6(ref_c) if elem == "mxfp6" else MX.pack(ref_c))
    assert np.array_equal(sg.ravel(), scales_to_gemm_order(sp))
    assert np.array_equal(cg, codes6_to_gemm_order(cp) if elem == "mxfp6" else cp)


# (M, N, K); the sampled ones at full size, the first compared in full
SHAPES = {
    "tiles-and-slabs": (256, 384, 768),
    "full-4096": (4096, 4096, 4096),
    "tiles-256x192": (2048, 6144, 1024),
    "tiles-256x256-240": (4096, 3840, 768),
    "ragged-mn-32": (480, 800, 512),
}


@pytest.mark.gpu
@pytest.mark.parametrize("elem", list(ELEMS))
@pytest.mark.parametrize("case", list(SHAPES))
def test_gemm_order_product(mtl, elem, case):
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_mx_gemm_ordered
    from megatron_tensor_transformer_layer_amd.layer import host_f64
    M, N, K = SHAPES[case]
    print(f"{elem} gemm-order product {case} {M}x{N}x{K}", flush=True)
    a = synth.mx_operand(M, K, "mx_a", 1.0, seed=4)
    b = synth.mx_operand(N, K, "mx_b", synth.WEIGHT_STD, seed=4)
    ca, sa = _quant(mtl, elem, a, mtl.MTL_MX_ORDER_GEMM)
    cb, sb = _quant(mtl, elem, b, mtl.MTL_MX_ORDER_GEMM)
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    e = mtl.MTL_MX_E2M3 if elem == "mxfp6" else mtl.MTL_MX_E2M1
    mtl_mx_gemm_ordered(e, M, N, K, ca, sa, cb, sb, c, mtl.MTL_MX_ORDER_GEMM)
    torch.cuda.synchronize()
    got = host_f64(c)
    assert np.all(np.isfinite(got))
    if case == "tiles-and-slabs" or case == "ragged-mn-32":
        rm, rn = np.arange(M), np.arange(N)
    else:
        rng = np.random.default_rng(7)
        edges = [0, 31, 32, 127, 128, 191, 192, 255, 256]
        rm = np.array(sorted(set([e_ for e_ in edges if e_ < M] + [M - 1] + rng.choice(M, 8, replace=False).tolist())))
        rn = np.array(sorted(set([e_ for e_ in edges if e_ < N] + [N - 1] + rng.choice(N, 8, replace=False).tolist())))
    qa, qsa = MX.quantize(f64(a[rm]), ELEMS[elem])
    qb, qsb = MX.quantize(f64(b[rn]), ELEMS[elem])
    ref = MX.gemm(qa, qsa, qb, qsb, ELEMS[elem])
    assert_bf16("C", got[np.ix_(rm, rn)], ref)
    rel = np.abs(got[np.ix_(rm, rn)] - ref) / (np.abs(ref) + 1e-3 * np.abs(ref).max())
    assert rel.max() <= 2.0 ** -7, f"max relative error {rel.max():.3e}"
