"""Pins of the MXFP4 oracle (oracle/mxfp4.py) against the OCP MX v1.0 format
definitions: the E2M1 value table, exact round trips of representable blocks,
saturation, ties to even, the scale rule, packing, and a GEMM on lossless
inputs against the plain product."""
import math

import numpy as np
import pytest

from oracle import mxfp4 as MX

# The OCP MX specification's E2M1 magnitudes, codes 0..7.
SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_matches_the_spec():
    assert [MX.e2m1_value(c) for c in range(8)] == SPEC_E2M1
    assert [MX.e2m1_value(c + 8) for c in range(8)] == [-v for v in SPEC_E2M1]


def test_representable_blocks_round_trip_exactly():
    rng = np.random.default_rng(1)
    for k in (-20, -3, 0, 5, 60):
        vals = rng.choice(SPEC_E2M1, 32) * rng.choice([-1, 1], 32)
        vals[7] = 6.0  # amax 6 * 2^k gives the scale 2^k
        x = (vals * 2.0 ** k)[None, :]
        codes, scales = MX.quantize(x)
        assert scales[0, 0] == k + 127
        assert np.array_equal(MX.dequantize(codes, scales), x)


def test_scale_rule_and_saturation():
    # amax 7 (floor(log2 7) = 2): scale 2^0, 7 saturates to 6
    x = np.zeros((1, 32))
    x[0, 0], x[0, 1] = 7.0, -7.9
    codes, scales = MX.quantize(x)
    assert scales[0, 0] == 127
    assert codes[0, 0] == 7 and codes[0, 1] == 15
    # amax 8 (floor(log2 8) = 3): scale 2^1, 8 -> 4 exactly
    x[0, 0] = 8.0
    codes, scales = MX.quantize(x)
    assert scales[0, 0] == 128 and MX.dequantize(codes, scales)[0, 0] == 8.0
    # all-zero block: the lowest E8M0 exponent, code 0 (negative zero keeps its sign)
    z = np.zeros((1, 32))
    z[0, 3] = -0.0
    codes, scales = MX.quantize(z)
    assert scales[0, 0] == 0 and codes[0, 0] == 0 and codes[0, 3] == 8
    # a tiny block clamps at 2^-127
    t = np.full((1, 32), 2.0 ** -130)
    codes, scales = MX.quantize(t)
    assert scales[0, 0] == 0 and MX.dequantize(codes, scales)[0, 0] == 0.0


@pytest.mark.parametrize("mid,want", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)])
def test_ties_go_to_the_even_code(mid, want):
    x = np.zeros((1, 32))
    x[0, 0], x[0, 1] = 6.0, mid  # scale 2^0
    codes, _ = MX.quantize(x)
    assert codes[0, 1] == want
    x[0, 1] = -mid
    codes, _ = MX.quantize(x)
    assert codes[0, 1] == want | 8


def test_nearest_value_within_half_a_step():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 64)) * 3.0
    codes, scales = MX.quantize(x)
    d = MX.dequantize(codes, scales)
    for r in range(4):
        for b in range(2):
            e = int(scales[r, b]) - 127
            blk, q = x[r, 32 * b:32 * b + 32], d[r, 32 * b:32 * b + 32]
            y = blk / 2.0 ** e
            # spacing of the E2M1 grid around |y|: 0.5 below 2, 1 below 4, 2 up to 6
            step = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
            ok = np.abs(y) <= 6
            assert np.all(np.abs(q / 2.0 ** e - y)[ok] <= step[ok] / 2 + 1e-12)
            assert np.all(np.abs(q[~ok]) == 6 * 2.0 ** e)


def test_pack_unpack():
    c = np.arange(32, dtype=np.uint8).reshape(2, 16) % 16
    p = MX.pack(c)
    assert p.shape == (2, 8) and p[0, 0] == (0 | (1 << 4))
    assert np.array_equal(MX.unpack(p), c)


def test_gemm_of_lossless_operands_is_the_plain_product():
    rng = np.random.default_rng(3)
    M, N, K = 5, 7, 96
    a = rng.choice(SPEC_E2M1, (M, K)) * rng.choice([-1, 1], (M, K))
    b = rng.choice(SPEC_E2M1, (N, K)) * rng.choice([-1, 1], (N, K))
    a[:, ::32] = 6.0
    b[:, ::32] = -6.0
    a *= 2.0 ** np.arange(M)[:, None]
    b *= 2.0 ** -np.arange(N)[:, None]
    ca, sa = MX.quantize(a)
    cb, sb = MX.quantize(b)
    assert np.array_equal(MX.gemm(ca, sa, cb, sb), a @ b.T)


# ---------------------------------------------------------------- MXFP6 (E2M3)
# The OCP MX specification's E2M3 magnitudes: subnormals k/8, then 1..1.875,
# 2..3.75, 4..7.5 in steps of 1/8, 1/4, 1/2.
SPEC_E2M3 = [k / 8 for k in range(8)] + [1 + k / 8 for k in range(8)] + [2 + k / 4 for k in range(8)] + \
    [4 + k / 2 for k in range(8)]


def test_e2m3_table_matches_the_spec():
    assert [MX.e2m3_value(c) for c in range(32)] == SPEC_E2M3
    assert MX.e2m3_value(32 + 31) == -7.5


def test_e2m3_rounding_ties_and_saturation():
    x = np.zeros((1, 32))
    x[0, 0] = 7.5  # floor(log2 7.5) = 2: scale 2^0
    probes = {1: (0.0625, 0), 2: (0.1875, 2), 3: (0.9375, 8), 4: (1.0625, 8), 5: (1.9375, 16), 6: (3.875, 24),
              7: (7.75, 31), 8: (7.7, 31), 9: (5.25, 26), 10: (5.26, 27)}
    for col, (v, _) in probes.items():
        x[0, col] = v
    codes, scales = MX.quantize(x, "e2m3")
    assert scales[0, 0] == 127
    for col, (v, want) in probes.items():
        assert codes[0, col] == want, (v, codes[0, col], want)
    x[0, 1:] = -x[0, 1:]
    codes, _ = MX.quantize(x, "e2m3")
    assert codes[0, 3] == 8 | 32


def test_e2m3_round_trip_and_pack6():
    rng = np.random.default_rng(4)
    vals = rng.choice(SPEC_E2M3, (3, 64)) * rng.choice([-1, 1], (3, 64))
    vals[:, 0] = vals[:, 32] = 7.5
    x = vals * 2.0 ** np.array([[-5], [0], [9]])
    codes, scales = MX.quantize(x, "e2m3")
    assert np.array_equal(MX.dequantize(codes, scales, "e2m3"), x)
    p = MX.pack6(codes)
    assert p.shape == (3, 48)
    # element j of a block at bits 6j..6j+5 of its 24 little-endian bytes
    v = int.from_bytes(bytes(p[1, 24:48]), "little")
    assert [(v >> (6 * j)) & 63 for j in range(32)] == codes[1, 32:64].tolist()


def test_pack6_hand_worked_bytes():
    """pack6 against bytes worked out by hand from the FP6 operand layout of the
    block-scaled MFMA (code j in bits 6j..6j+5 of a lane's 6 dwords)."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack6.json")))
    for case in g["cases"]:
        codes = np.array([case["codes"]], dtype=np.uint8)
        assert MX.pack6(codes)[0].tolist() == case["bytes"], case["note"]
    # two blocks in one row: each packs on its own
    both = np.array([g["cases"][0]["codes"] + g["cases"][1]["codes"]], dtype=np.uint8)
    assert MX.pack6(both)[0].tolist() == g["cases"][0]["bytes"] + g["cases"][1]["bytes"]
