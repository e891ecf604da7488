"""Pins of the MXFP4 layer oracle (oracle/mx_layer.py) and of the vectorised
MX quantiser it uses."""
import numpy as np
import pytest

import synth
from oracle import mx_layer as X
from oracle import mxfp4 as MX
from oracle import shard as S
from tests.parity_util import f64, full_params


@pytest.mark.parametrize("elem", ["e2m1", "e2m3"])
def test_quantize_fast_equals_the_element_loop(elem):
    """On bf16 values of every kind -- Gaussian blocks at several scales,
    powers of two and their neighbours, every tie, zeros and -0, saturating
    blocks -- the vectorised quantiser gives the loop's codes and scales."""
    rng = np.random.default_rng(3)
    rows = [synth.bf16_bits_to_f64(synth.bf16_round_bits(rng.standard_normal(64) * s)) for s in
            (1e-30, 1e-5, 0.02, 1.0, 7.0, 3e4)]
    pw = 2.0 ** np.arange(-20, 12)
    rows += [np.concatenate([pw, -pw]), np.concatenate([pw * (1 - 2 ** -8), pw * (1 + 2 ** -7)])]
    mags = MX.E2M1_MAGNITUDES if elem == "e2m1" else MX.E2M3_MAGNITUDES
    mids = (mags[1:] + mags[:-1]) / 2  # every tie at scale 1 (block max 6 or 7.5 pins the scale to 2^0)
    tie = np.zeros(64)
    tie[0] = mags[-1]
    tie[1:1 + len(mids)] = mids[:31]
    tie[40] = -0.0
    rows += [tie, np.zeros(64), np.full(64, -0.0)]
    x = np.stack(rows)
    c1, s1 = MX.quantize(x, elem)
    c2, s2 = MX.quantize_fast(x, elem)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1, c2)


def test_identity_quantiser_gives_the_plain_layer():
    shape = synth.LayerShape(hidden=256, heads=2, ffn=512, seq=64, micro_batch=1, tp=2)
    full = synth.layer_inputs(shape, seed=0)
    p, x, g = full_params(full), f64(full["x"]), f64(full["dy"])
    a = X.sharded_layer(p, x, g, shape.heads, shape.tp, q=lambda t: np.asarray(t, dtype=np.float64))
    b = S.sharded_layer(p, x, g, shape.heads, shape.tp)
    for k in ("y", "dh", "dx"):
        assert np.array_equal(a[k], b[k]), k
    for part in ("mlp_bwd", "attn_bwd"):
        for ra, rb in zip(a[part], b[part]):
            for k in ra:
                if k in rb:
                    assert np.array_equal(ra[k], rb[k]), (part, k)


def test_product_quantises_along_the_contraction_hand_worked():
    """One 32-element block along K: a = (8, 1, 0.3, 0, ...) has amax 8, so its
    scale is 2^(3-2) = 2 and a/2 = (4, 0.5, 0.15) rounds to (4, 0.5, 0): the
    quantised a is (8, 1, 0); b = (1, 1, 1, 0, ...) is exact (scale 2^-2, codes
    4 = 1/0.25).  a . b = 9 (the exact product is 9.3)."""
    a = np.zeros((1, 32))
    a[0, :3] = [8.0, 1.0, 0.3]
    b = np.zeros((32, 1))
    b[:3, 0] = 1.0
    assert X.mm(a, b)[0, 0] == 9.0
    # Along the contraction, not the other axis: in A [32, 32] row 1 holds 8 at
    # k = 0 and 0.3 at k = 1 (one K block, scale 2: 0.3 -> 0), while column 1
    # of A holds only the 0.3 (as an M block it would keep 0.25).  B picks k = 1.
    A = np.zeros((32, 32))
    A[1, 0], A[1, 1], A[0, 1] = 8.0, 0.3, 0.0
    B = np.zeros((32, 32))
    B[1, 0] = 1.0
    C = X.mm(A, B)
    assert C[1, 0] == 0.0
    # and B is blocked down its columns: a K block of B with 6 at k = 0 and 0.2
    # at k = 1 turns the 0.2 into 0 (scale 2^0: 0.2 -> 0), so A = e_1 sees 0
    A2 = np.zeros((32, 32))
    A2[0, 1] = 1.0
    B2 = np.zeros((32, 32))
    B2[0, 0], B2[1, 0] = 6.0, 0.2
    assert X.mm(A2, B2)[0, 0] == 0.0
