"""Tolerance checks of the device results against the oracle.

bf16 path: max|diff| <= 2e-2 * max|ref| + 1e-3, per output tensor (each
activation, each weight and bias gradient), written here and nowhere else."""
import numpy as np

import synth

BF16_REL, BF16_ABS = 2e-2, 1e-3
FP8_REL = 8e-2


def within_bf16(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    bound = BF16_REL * float(np.max(np.abs(ref))) + BF16_ABS if ref.size else BF16_ABS
    return err, bound


def assert_bf16(name, got, ref):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err, bound = within_bf16(got, ref)
    assert err <= bound, f"{name}: max|diff| {err:.4e} > bound {bound:.4e}"
    return err, bound


def f64(bits):
    return synth.bf16_bits_to_f64(bits)


def full_params(full):
    return {k: f64(full[k]) for k in ("w_qkv", "b_qkv", "w_o", "b_o", "w1", "b1", "w2", "b2")}
