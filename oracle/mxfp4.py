"""fp64 oracle of MXFP4 and MXFP6 quantisation and of GEMMs on such operands.

Test infrastructure only (see the package docstring).

The site summary ([site] navi2ai.com/sites/1106, its precision list and deploy
step 7, `--fp4-format nvfp4` on Blackwell) names 4-bit floating-point
training and gives no format details.  The reading taken here is AMD's
native counterpart, the OCP Microscaling (MX) format MXFP4, as the OCP MX
specification v1.0 defines it:

* element type FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit, no
  infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
* blocks of 32 consecutive elements along the reduction (K) dimension share
  one scale X = 2^e stored as E8M0 (biased exponent e + 127);
* e = floor(log2(max |v|)) - 2 (2 is the largest exponent of E2M1), clamped to
  E8M0's lowest exponent -127 (an all-zero block gets -127);
* each element is v / X rounded to the nearest E2M1 value, ties to the even
  code (mantissa bit 0), magnitudes past 6 saturating to 6; the sign bit
  follows the sign of v, zero included.

MXFP6 is the same with FP6 E2M3 elements (sign, 2 exponent bits of bias 1,
3 mantissa bits; largest magnitude 7.5, largest exponent 2, so the same scale
rule).  Finite inputs only.  FP4 codes pack two per byte, the even element in
the low nibble; FP6 codes pack four per three bytes, element j of a block at
bits 6j .. 6j+5 of the block's 24 bytes read as one little-endian number.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 32
EMAX_ELEM = 2
E8M0_BIAS = 127
SCALE_EXP_MIN = -127


def small_float_value(code: int, ebits: int, mbits: int, bias: int) -> float:
    """Value of a sign / exponent / mantissa code with no infinities or NaN
    (exponent field 0: subnormal)."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        mag = m / 2.0 ** mbits * 2.0 ** (1 - bias)
    else:
        mag = (1.0 + m / 2.0 ** mbits) * 2.0 ** (e - bias)
    return -mag if s else mag


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code from its fields."""
    return small_float_value(code, 2, 1, 1)


def e2m3_value(code: int) -> float:
    """Value of a 6-bit E2M3 code from its fields."""
    return small_float_value(code, 2, 3, 1)


E2M1_MAGNITUDES = np.array([e2m1_value(c) for c in range(8)])
E2M3_MAGNITUDES = np.array([e2m3_value(c) for c in range(32)])


def _round(y: float, mags) -> int:
    """Code of the value nearest to y among the magnitudes (ties to the even
    code, saturating at the largest), with the sign bit above them."""
    if not math.isfinite(y):
        raise ValueError("finite inputs only")
    dist = np.abs(mags - abs(y))
    best = np.flatnonzero(dist == dist.min())
    code = int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])
    return code | (len(mags) if math.copysign(1.0, y) < 0 else 0)


def round_e2m1(y: float) -> int:
    """Code of the E2M1 value nearest to y (ties to the even code, saturating)."""
    return _round(y, E2M1_MAGNITUDES)


def round_e2m3(y: float) -> int:
    """Code of the E2M3 value nearest to y (ties to the even code, saturating)."""
    return _round(y, E2M3_MAGNITUDES)


def block_scale_exp(block) -> int:
    amax = float(np.max(np.abs(block)))
    if amax == 0.0:
        return SCALE_EXP_MIN
    return max(math.floor(math.log2(amax)) - EMAX_ELEM, SCALE_EXP_MIN)


def quantize(x, elem: str = "e2m1"):
    """x [rows, cols] (cols % 32 == 0) -> (codes uint8 [rows, cols] one code per
    element, scales uint8 [rows, cols/32] E8M0); elem "e2m1" (MXFP4) or
    "e2m3" (MXFP6), both with largest exponent 2."""
    rnd = {"e2m1": round_e2m1, "e2m3": round_e2m3}[elem]
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, cols // BLOCK), dtype=np.uint8)
    for r in range(rows):
        for b in range(cols // BLOCK):
            blk = x[r, b * BLOCK:(b + 1) * BLOCK]
            e = block_scale_exp(blk)
            scales[r, b] = e + E8M0_BIAS
            for i, v in enumerate(blk):
                codes[r, b * BLOCK + i] = rnd(math.ldexp(v, -e))
    return codes, scales


def pack(codes):
    """One code per element -> two per byte (element 2i in the low nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.zeros((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def pack6(codes):
    """One 6-bit code per element -> 24 bytes per block of 32: element j at bits
    6j .. 6j+5 of the block read as a little-endian number."""
    c = np.asarray(codes, dtype=np.uint8)
    rows, cols = c.shape
    out = np.zeros((rows, cols // 32 * 24), dtype=np.uint8)
    for r in range(rows):
        for b in range(cols // 32):
            v = 0
            for j in range(32):
                v |= int(c[r, 32 * b + j]) << (6 * j)
            out[r, 24 * b:24 * b + 24] = np.frombuffer(v.to_bytes(24, "little"), dtype=np.uint8)
    return out


def quantize_fast(x, elem: str = "e2m1"):
    """The codes and scales of ``quantize`` computed on whole arrays, for the
    sizes where its element loop is too slow (pinned to it element for element).
    floor(log2 amax) is the exponent frexp returns minus one; the nearest
    magnitude is chosen by distance with ties to the even code; the sign bit
    follows the sign of the value, zero included."""
    mags = {"e2m1": E2M1_MAGNITUDES, "e2m3": E2M3_MAGNITUDES}[elem]
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("finite inputs only")
    blocks = x.reshape(rows, cols // BLOCK, BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    _, fe = np.frexp(amax)
    e = np.where(amax > 0, fe - 1 - EMAX_ELEM, SCALE_EXP_MIN)
    e = np.maximum(e, SCALE_EXP_MIN)
    y = np.ldexp(blocks, -e[:, :, None])
    dist = np.abs(mags[None, None, None, :] - np.abs(y)[..., None])
    nearest = dist == dist.min(axis=-1, keepdims=True)
    even = (np.arange(len(mags)) % 2 == 0)
    code = np.argmax(nearest * np.where(even, 2, 1), axis=-1)  # an even code wins a tie
    code = code | np.where(np.signbit(y), len(mags), 0)
    return code.reshape(rows, cols).astype(np.uint8), (e + E8M0_BIAS).astype(np.uint8)


def dequantize(codes, scales, elem: str = "e2m1"):
    """Values X * element(code) [rows, cols] in fp64 (codes one per element)."""
    c = np.asarray(codes, dtype=np.int64)
    table = [e2m1_value(k) for k in range(16)] if elem == "e2m1" else [e2m3_value(k) for k in range(64)]
    vals = np.array(table)[c]
    e = np.asarray(scales, dtype=np.int64) - E8M0_BIAS
    return vals * np.repeat(np.ldexp(1.0, e), BLOCK, axis=1)


def gemm(a_codes, a_scales, b_codes, b_scales, elem: str = "e2m1"):
    """C [M, N] = A B^T of two MX operands, both K-contiguous ([M, K] and
    [N, K], one code per element), in fp64."""
    return dequantize(a_codes, a_scales, elem) @ dequantize(b_codes, b_scales, elem).T
