"""Small fp64 parameter sets for the oracle's CPU pins (no bf16 rounding needed)."""
import numpy as np


def tiny_params(h, f, seed=0, scale=0.5):
    rng = np.random.default_rng(seed)
    return dict(
        w_qkv=rng.standard_normal((h, 3 * h)) * scale, b_qkv=rng.standard_normal(3 * h) * scale,
        w_o=rng.standard_normal((h, h)) * scale, b_o=rng.standard_normal(h) * scale,
        w1=rng.standard_normal((h, f)) * scale, b1=rng.standard_normal(f) * scale,
        w2=rng.standard_normal((f, h)) * scale, b2=rng.standard_normal(h) * scale,
    )


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))
