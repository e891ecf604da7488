"""Oracle of fp8 per-tensor scaled quantisation (the ``--fp8-format hybrid`` recipe).

Test infrastructure only (see the package docstring).

The site summary's MoE deploy step passes ``--fp8-format hybrid`` and its
mixed-precision section lists FP8 among the training precisions; it gives no
encoding or scaling rule.  Readings:

* "hybrid" = E4M3 for forward tensors (activations, weights), E5M2 for gradients;
* the encodings are the OCP 8-bit formats: E4M3FN (bias 7, 3 mantissa bits, no
  infinities, largest finite 448) and E5M2 (bias 15, 2 mantissa bits,
  largest finite 57344);
* current per-tensor scaling: amax = max|x| over the tensor, scale s =
  fmt_max / amax (s = 1 when amax = 0), code = round-to-nearest-even of x*s onto
  the format's grid, saturated to +-fmt_max; NaN stays NaN;
* s and x*s are computed in fp32 -- the precision the device uses -- so the codes
  are one well-defined integer per element.  Dequantisation multiplies the code's
  value by 1/s.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Fp8Format:
    name: str
    exp_bits: int
    man_bits: int
    bias: int
    max_finite: float
    has_inf: bool

    @property
    def emin(self) -> int:  # exponent of the smallest normal
        return 1 - self.bias


E4M3 = Fp8Format("e4m3", 4, 3, 7, 448.0, False)
E5M2 = Fp8Format("e5m2", 5, 2, 15, 57344.0, True)


def round_to_grid(y, fmt: Fp8Format):
    """Round fp64 values (exact fp32 values) to the format's grid, nearest-even,
    then saturate to +-max_finite.  NaN passes through."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, e = np.frexp(np.where(a > 0, a, 1.0))  # a = m * 2^e, 0.5 <= m < 1
    expo = np.maximum(e - 1, fmt.emin)
    ulp = np.ldexp(1.0, expo - fmt.man_bits)
    q = np.rint(a / ulp) * ulp
    q = np.minimum(q, fmt.max_finite)
    out = np.copysign(q, y)
    return np.where(np.isnan(y), np.nan, out)


def encode(q, fmt: Fp8Format):
    """Bit patterns (uint8) of values already on the grid (output of round_to_grid)."""
    q = np.asarray(q, dtype=np.float64)
    nan = np.isnan(q)
    a = np.abs(np.where(nan, 0.0, q))
    sign = (np.signbit(q) & ~nan).astype(np.uint8) << 7
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    expo = e - 1
    normal = (a > 0) & (expo >= fmt.emin)
    efield = np.where(normal, expo + fmt.bias, 0)
    mant = np.where(normal, a / np.ldexp(1.0, expo) - 1.0, a / np.ldexp(1.0, fmt.emin))
    mfield = np.rint(mant * (1 << fmt.man_bits)).astype(np.int64)
    code = sign | ((efield.astype(np.int64) << fmt.man_bits) | mfield).astype(np.uint8)
    nan_code = 0x7F if not fmt.has_inf else 0x7F  # all-ones exponent, nonzero mantissa
    return np.where(nan, np.uint8(nan_code), code).astype(np.uint8)


def decode(codes, fmt: Fp8Format):
    """fp64 values of fp8 bit patterns."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    efield = (c >> fmt.man_bits) & ((1 << fmt.exp_bits) - 1)
    mfield = c & ((1 << fmt.man_bits) - 1)
    emax_field = (1 << fmt.exp_bits) - 1
    frac = mfield / float(1 << fmt.man_bits)
    val = np.where(efield == 0, np.ldexp(frac, fmt.emin), np.ldexp(1.0 + frac, efield - fmt.bias))
    if fmt.has_inf:
        special = efield == emax_field
        val = np.where(special & (mfield == 0), np.inf, np.where(special, np.nan, val))
    else:
        val = np.where((efield == emax_field) & (mfield == (1 << fmt.man_bits) - 1), np.nan, val)
    return sign * val


def amax(x) -> np.float32:
    """max |x| over the tensor, as fp32 (x holds bf16 or fp32 values: exact)."""
    return np.float32(np.max(np.abs(np.asarray(x, dtype=np.float64))))


def scale_for(a: np.float32, fmt: Fp8Format) -> np.float32:
    """s = fmt_max / amax in fp32 (correctly rounded division); 1 when amax is 0."""
    a = np.float32(a)
    if a == 0 or not np.isfinite(a):
        return np.float32(1.0)
    return np.float32(np.float32(fmt.max_finite) / a)


def quantize(x, fmt: Fp8Format, s: np.float32 | None = None):
    """Per-tensor scaled quantisation.  Returns (codes uint8, s fp32, scale_inv fp32)
    where scale_inv = 1/s in fp32."""
    x32 = np.asarray(x, dtype=np.float32)
    if s is None:
        s = scale_for(amax(x32), fmt)
    y = (x32 * np.float32(s)).astype(np.float32)  # one fp32 rounding
    codes = encode(round_to_grid(y.astype(np.float64), fmt), fmt)
    return codes, np.float32(s), np.float32(np.float32(1.0) / np.float32(s))


def quant_dequant(x, fmt: Fp8Format):
    """fp64 value the fp8 GEMM sees for x: decode(code) * (1/s) with 1/s exact in fp64."""
    codes, s, _ = quantize(x, fmt)
    return decode(codes, fmt) / np.float64(s)
