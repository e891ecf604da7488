"""Pin: the fp8 oracle against the OCP format definitions (closed-form code
points) and against torch CPU's float8_e4m3fn / float8_e5m2 casts (an
independent library implementation of round-to-nearest-even) after explicit
saturation."""
import numpy as np
import pytest
import torch

from oracle import fp8 as Q
import synth


@pytest.mark.parametrize("fmt,tdt", [(Q.E4M3, torch.float8_e4m3fn), (Q.E5M2, torch.float8_e5m2)])
def test_round_matches_torch_cast(fmt, tdt):
    rng = np.random.default_rng(41)
    # every bf16 bit pattern (finite ones) plus random fp32 values over the whole range
    bits = np.arange(65536, dtype=np.uint16)
    a = synth.bf16_bits_to_f32(bits)
    b = (rng.standard_normal(200000) * np.exp2(rng.uniform(-30, 20, 200000))).astype(np.float32)
    v = np.concatenate([a, b])
    v = v[np.isfinite(v)]
    mine = Q.round_to_grid(v.astype(np.float64), fmt)
    clamped = np.clip(v, -fmt.max_finite, fmt.max_finite)
    ref = torch.from_numpy(clamped).to(tdt).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)
    # codes: encode(round) must be the same bit pattern as torch's
    codes = Q.encode(mine, fmt)
    tcodes = torch.from_numpy(clamped).to(tdt).view(torch.uint8).numpy()
    # +-0: torch keeps the sign of zero, so do we
    assert np.array_equal(codes, tcodes)
    assert np.array_equal(Q.decode(codes, fmt), mine)


def test_closed_form_code_points():
    E4, E5 = Q.E4M3, Q.E5M2
    enc = lambda x, f: int(Q.encode(Q.round_to_grid(np.array([x]), f), f)[0])
    assert enc(1.0, E4) == 0x38 and enc(1.0, E5) == 0x3C
    assert enc(448.0, E4) == 0x7E and enc(-448.0, E4) == 0xFE
    assert enc(1e6, E4) == 0x7E  # saturates, never NaN
    assert enc(57344.0, E5) == 0x7B and enc(1e9, E5) == 0x7B
    assert enc(2.0 ** -9, E4) == 0x01 and enc(2.0 ** -16, E5) == 0x01
    assert enc(0.5 * 2.0 ** -9, E4) == 0x00  # tie -> even (zero)
    assert enc(1.5 * 2.0 ** -9, E4) == 0x02  # tie between 1 and 2 ulps -> even
    assert enc(1.0625, E4) == 0x38  # tie between 1.0 and 1.125 -> even mantissa
    assert enc(1.1875, E4) == 0x3A  # tie between 1.125 and 1.25 -> even (1.25)
    assert Q.decode(np.array([0x7F], dtype=np.uint8), E4)[0] != Q.decode(np.array([0x7F], dtype=np.uint8), E4)[0]
    assert np.isinf(Q.decode(np.array([0x7C], dtype=np.uint8), E5)[0])
    assert Q.decode(np.array([0x7E], dtype=np.uint8), E4)[0] == 448.0
    assert np.isnan(Q.round_to_grid(np.array([np.nan]), E4)[0])


def test_scaled_quantize_uses_fp32_scale():
    x = np.array([0.0, 1.0, -3.5, 0.001, 2.75], dtype=np.float32)
    codes, s, sinv = Q.quantize(x, Q.E4M3)
    assert s == np.float32(448.0) / np.float32(3.5) == np.float32(128.0)
    assert int(codes[2]) == 0xFE  # -3.5 * 128 = -448
    assert Q.quantize(np.zeros(4, np.float32), Q.E4M3)[1] == 1.0
    # the largest |x| always lands on +-max_finite
    rng = np.random.default_rng(42)
    y = rng.standard_normal(1000).astype(np.float32)
    c, s, _ = Q.quantize(y, Q.E5M2)
    assert np.max(np.abs(Q.decode(c, Q.E5M2))) == 57344.0
    # quant-dequant error is within half an fp8 ulp of the scaled value
    qd = Q.quant_dequant(y, Q.E4M3)
    assert np.max(np.abs(qd - y) / np.maximum(np.abs(y), 2.0 ** -6 / 448 * np.max(np.abs(y)))) <= 2.0 ** -4 + 1e-12
