"""fp8 path on the GPU.

* amax and the scaled cast (E4M3 / E5M2), separately and as the one-call
  quantisation, are bit-exact against the oracle:
  the scale record {amax, s, 1/s} and every code, on tensors that reach every
  code point and every rounding tie (all bf16 values within the format's range
  at scale 1), on Gaussian tensors (s not a power of two), on zeros, and on
  tensors holding inf and NaN; the transposed copy is the transpose.
* The whole tensor-parallel layer in fp8 (all shards on one device) against
  the plain fp64 layer on the unquantised inputs, the reference the fp8
  tolerance is stated against, in two parts per output:
  - the stated bound, max|diff| <= 8e-2 * max|ref|, wherever the recipe itself
    (the same layer with quantised GEMM operands, in exact arithmetic) meets
    it; where the recipe does not, no implementation of it can, and the test
    reports the miss instead;
  - the device's error is the recipe's error: RMS(got - ref) <= 1.05 *
    RMS(recipe - ref) + 2e-3 * RMS(ref).  Both are realisations of the same
    quantisation noise (the device's intermediates differ from the exact ones
    in their last bf16 bit, which moves a few codes by one step and so changes
    the realisation, not its size), so their RMS agree to within sampling
    noise; a wrong scale, format or operand multiplies it.
  An element-wise comparison with the quantised-operand reference is not a
  test of the kernels beyond the first quantised intermediate: a relative
  perturbation of 2^-10 in the stored intermediates alone moves that reference
  by 0.04-0.09 * max|ref| on Y, dH and dX of a 256-token layer of hidden 512
  (test_oracle_fp8_layer.py), more than the bf16 bound.  The kernels are
  instead checked on identical codes, GEMM by GEMM, below and in the full-size
  tests.
"""
import os

import numpy as np
import pytest

import synth
from oracle import fp8 as Q
from oracle import fp8_layer as F8
from oracle import layer as L
from tests.parity_util import BF16_ABS, BF16_REL, FP8_REL, assert_bf16, f64, full_params

FMT = {0: Q.E4M3, 1: Q.E5M2}


def _bits_within(limit):
    """Every finite bf16 bit pattern with |value| <= limit (both signs)."""
    bits = np.arange(65536, dtype=np.uint16)
    v = synth.bf16_bits_to_f64(bits)
    return bits[np.isfinite(v) & (np.abs(v) <= limit)]


def _cast_case(name):
    rng = np.random.default_rng(7)
    if name == "grid-e4m3":
        return _bits_within(448.0), 0
    if name == "grid-e5m2":
        return _bits_within(57344.0), 1
    if name in ("gauss-e4m3", "gauss-e5m2"):
        return synth.bf16_round_bits(rng.standard_normal(4096 * 48) * 3.7), int(name.endswith("e5m2"))
    if name == "zeros":
        return np.zeros(4096, np.uint16), 0
    if name == "inf-nan":
        b = synth.bf16_round_bits(rng.standard_normal(4096))
        b[17], b[1000], b[2001] = 0x7F80, 0xFF80, 0x7FC1  # +inf, -inf, NaN
        return b, 1
    if name in ("saturate-e4m3", "saturate-e5m2"):
        # an infinity makes amax unusable, so s = 1 and finite values beyond the
        # format's maximum reach the saturation: just above it, at the rounding
        # midpoint to the next (absent) step, far beyond, both signs; NaN and -0
        fmt = int(name.endswith("e5m2"))
        mx = 448.0 if fmt == 0 else 57344.0
        over = np.array([mx, mx * 1.0078125, mx * 1.03125, mx * 1.0625, mx * 1.07, 2 * mx, 1e30])
        b = synth.bf16_round_bits(rng.standard_normal(4096) * mx / 4)
        b[:7] = synth.bf16_round_bits(over)
        b[7:14] = synth.bf16_round_bits(-over)
        b[14], b[15], b[16], b[17] = 0x7F80, 0xFF80, 0x7FC1, 0x8000  # +inf, -inf, NaN, -0
        return b, fmt
    raise KeyError(name)


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["grid-e4m3", "grid-e5m2", "gauss-e4m3", "gauss-e5m2", "zeros", "inf-nan",
                                  "saturate-e4m3", "saturate-e5m2"])
def test_amax_and_cast_bit_exact(mtl, case):
    import torch
    from megatron_tensor_transformer_layer_amd.layer import bf16_dev
    bits, fmt = _cast_case(case)
    cols = 64
    n = (len(bits) + 16 * cols - 1) // (16 * cols) * 16 * cols
    bits = np.concatenate([bits, np.zeros(n - len(bits), np.uint16)])  # pad with zeros: amax unchanged
    rows = n // cols
    print(f"cast case {case}: {rows} x {cols}, format {fmt}", flush=True)
    x = bf16_dev(bits.reshape(rows, cols))
    rec = torch.zeros(4, dtype=torch.float32, device="cuda")
    ws = torch.empty(mtl.MTL_FP8_AMAX_SCRATCH, dtype=torch.uint8, device="cuda")
    out = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    out_t = torch.empty(cols, rows, dtype=torch.uint8, device="cuda")
    mtl.mtl_fp8_amax(x, rows * cols, fmt, rec, ws)
    mtl.mtl_fp8_cast(x, rows, cols, fmt, rec, out, out_t)
    torch.cuda.synchronize()
    got_rec = rec.cpu().numpy()
    vals = synth.bf16_bits_to_f32(bits)
    with np.errstate(invalid="ignore"):
        amax = Q.amax(vals)
    codes, s, sinv = Q.quantize(vals, FMT[fmt])
    if np.isnan(amax):
        assert np.isnan(got_rec[0])
    else:
        assert got_rec[0].tobytes() == np.float32(amax).tobytes()
    assert got_rec[1].tobytes() == np.float32(s).tobytes()
    assert got_rec[2].tobytes() == np.float32(sinv).tobytes()
    got = out.cpu().numpy()
    assert np.array_equal(got.reshape(-1), codes), np.flatnonzero(got.reshape(-1) != codes)[:10]
    assert np.array_equal(out_t.cpu().numpy(), got.T)
    # the one-call quantisation (the cast finishing the amax) gives the same bits
    rec2 = torch.zeros(4, dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out)
    out2_t = torch.empty_like(out_t)
    mtl.mtl_fp8_quantize(x, rows, cols, fmt, rec2, out2, out2_t, ws)
    torch.cuda.synchronize()
    assert rec2.cpu().numpy()[:3].tobytes() == got_rec[:3].tobytes()
    assert torch.equal(out2, out) and torch.equal(out2_t, out_t)


FP8_CASES = {
    "gpt2-small-tp2": (synth.WORKLOADS["gpt2-small-tp2"], False),
    # TP=4 with residual connections, 144 tokens (9 row tiles of 16), d = 64
    "tp4-residual": (synth.LayerShape(hidden=512, heads=8, ffn=1024, seq=144, micro_batch=1, tp=4), True),
    # d = 128, two micro-batch elements, ffn/t = 272
    "d128-mb2-tp2": (synth.LayerShape(hidden=256, heads=2, ffn=544, seq=96, micro_batch=2, tp=2), False),
}


def _bf16(t):
    """The bf16 value the device stores for t (round to nearest even)."""
    return synth.bf16_bits_to_f64(synth.bf16_round_bits(np.asarray(t, dtype=np.float64)))


# The reference with quantised operands, taking each quantisation decision from
# the bf16 value the device holds (inputs are bf16 already, so this only
# touches the intermediates A, O, H, dZ, dH, dQKV).
def _q4(t):
    return F8.q4(_bf16(t))


def _q5(t):
    return F8.q5(_bf16(t))


def _rms(t):
    return float(np.sqrt(np.mean(np.square(t))))


def fp8_two_part_check(name, got, ref, recipe_err_max, recipe_rms, ref_max, ref_rms):
    """The two-part fp8 check of one output (see the module docstring);
    returns (bad, line): bad is a reason string or None, line the table row."""
    err = float(np.max(np.abs(got - ref)))
    rms = _rms(got - ref)
    recipe_meets = recipe_err_max <= FP8_REL * ref_max
    line = (f"  {name:8s} device max|diff|/max|ref| {err / ref_max:.4f}  recipe {recipe_err_max / ref_max:.4f}  "
            f"(8e-2: {'met' if err <= FP8_REL * ref_max else 'MISSED'}; recipe {'meets' if recipe_meets else 'misses'})"
            f"  rms/rms(ref) device {rms / ref_rms:.4f} recipe {recipe_rms / ref_rms:.4f}")
    if not np.all(np.isfinite(got)):
        return "non-finite", line
    if recipe_meets and err > FP8_REL * ref_max:
        return f"max|diff| {err / ref_max:.4f} > 8e-2 where the recipe meets it", line
    if rms > 1.05 * recipe_rms + 2e-3 * ref_rms:
        return f"rms {rms / ref_rms:.4f} above the recipe's {recipe_rms / ref_rms:.4f}", line
    return None, line


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(FP8_CASES))
def test_fp8_layer_error_is_the_recipe_error(mtl, case):
    """The whole layer in fp8 against the plain fp64 layer on the unquantised
    inputs, by the two-part check of the module docstring."""
    from megatron_tensor_transformer_layer_amd.layer import run_sharded_layer
    shape, residual = FP8_CASES[case]
    print(f"fp8 case {case} {shape} residual={residual}", flush=True)
    full = synth.layer_inputs(shape, seed=0)
    shards = [synth.layer_inputs(shape, seed=0, tp=shape.tp, rank=r) for r in range(shape.tp)]
    got = run_sharded_layer(shape, shape.tp, shards, full["x"], full["b_o"], full["b2"], full["dy"], residual,
                            precision=mtl.MTL_PREC_FP8_HYBRID)
    p = full_params(full)
    x, g = f64(full["x"]), f64(full["dy"])
    fwd = L.layer_forward(p, x, shape.heads, shape.micro_batch, residual)
    bwd = L.layer_backward(p, x, fwd, g, shape.heads, shape.micro_batch, residual)
    ref_i = {**{k: fwd[k] for k in ("qkv", "h", "a", "y")}, "gz": L.gelu_grad(fwd["z"]), "dh": bwd["dh"],
             **{k: bwd[k] for k in ("dx", "dw_qkv", "db_qkv", "dw_o", "db_o", "dw1", "db1", "dw2", "db2")}}
    q = F8.sharded_layer(p, x, g, shape.heads, shape.tp, shape.micro_batch, residual, fq=_q4, gq=_q5)
    cat = lambda part, key, axis: np.concatenate([d[key] for d in q[part]], axis=axis)
    ref_q = dict(y=q["y"], h=q["h"], dh=q["dh"], dx=q["dx"], qkv=cat("att", "qkv", 1), gz=L.gelu_grad(cat("mlp", "z", 1)),
                 a=cat("mlp", "a", 1), dw_qkv=cat("attn_bwd", "dw_qkv", 1), db_qkv=cat("attn_bwd", "db_qkv", 0),
                 dw_o=cat("attn_bwd", "dw_o", 0), dw1=cat("mlp_bwd", "dw1", 1), db1=cat("mlp_bwd", "db1", 0),
                 dw2=cat("mlp_bwd", "dw2", 0), db_o=q["attn_bwd"][0]["db_o"], db2=q["mlp_bwd"][0]["db2"])
    bad = []
    for k, ref in ref_i.items():
        d = ref_q[k] - ref
        why, line = fp8_two_part_check(k, got[k], ref, float(np.max(np.abs(d))), _rms(d),
                                       float(np.max(np.abs(ref))), _rms(ref))
        print(line)
        if why:
            bad.append(f"{k}: {why}")
    assert not bad, bad


@pytest.mark.gpu
def test_fp8_gemms_on_identical_codes(mtl):
    """Every fp8 GEMM kind whose operands are call inputs -- so the device and
    the reference quantise the same bf16 values to the same codes (the cast is
    bit-exact) -- within the bf16 bound of the quantised-operand reference:
    fwd E4M3 x E4M3 with bias (qkv) and with bias + GeLU (GeLU'(z), a); dgrad E5M2 x
    E4M3 with GeLU' (through db1 = colsum(dz)); wgrad E4M3^T x E5M2 (dw2,
    dw_o).  Each call gets independent inputs, as in a real step."""
    import torch
    from megatron_tensor_transformer_layer_amd.layer import RankState, bf16_dev, host_f64
    shape = synth.WORKLOADS["gpt2-small-tp2"]
    t, r = shape.tp, 1
    f_l, o_l = shape.ffn // t, shape.hidden // t
    inp = synth.layer_inputs(shape, tp=t, rank=r)
    hb, dhb = synth.layer_tensor(shape, "h"), synth.layer_tensor(shape, "dh")
    # independent saved activations for the backward calls: Z ~ N(0, 4), A, O ~ N(0, 1)
    zb = synth.bf16_round_bits(np.tile(f64(synth.layer_tensor(shape, "dh", seed=3)), (1, 2))[:, :f_l] * 2.0)
    ab = np.tile(synth.layer_tensor(shape, "h", seed=4), (1, 2))[:, :f_l].copy()
    ob = synth.layer_tensor(shape, "x", seed=6)[:, :o_l].copy()
    st = RankState(shape, t, r, inp, precision=mtl.MTL_PREC_FP8_HYBRID)
    x, dy, h, dh = bf16_dev(inp["x"]), bf16_dev(inp["dy"]), bf16_dev(hb), bf16_dev(dhb)
    st.attn_fwd(x)
    st.mlp_fwd(h)
    torch.cuda.synchronize()
    got = dict(qkv=host_f64(st.qkv), gz=host_f64(st.gz), a=host_f64(st.a))
    st.gz.copy_(bf16_dev(synth.bf16_round_bits(L.gelu_grad(f64(zb)))))  # the saved GeLU'(z) of an independent z
    st.a.copy_(bf16_dev(ab))
    st.o.copy_(bf16_dev(ob))
    st.mlp_bwd(dy, h)
    st.attn_bwd(dh, x)
    torch.cuda.synchronize()
    got.update(db1=host_f64(st.db1), dw2=host_f64(st.dw2), dw_o=host_f64(st.dw_o), db_o=host_f64(st.db_o))

    pr = {k: f64(inp[k]) for k in ("w_qkv", "b_qkv", "w_o", "w1", "b1", "w2")}
    X, DY, H, DH, Z, A, O = (f64(v) for v in (inp["x"], inp["dy"], hb, dhb, zb, ab, ob))
    fa = F8.rank_attn_forward(pr, X, shape.heads // t)
    fm = F8.rank_mlp_forward(pr, H)
    mb = F8.rank_mlp_backward(pr, DY, H, Z, A)
    ref = dict(qkv=fa["qkv"], gz=L.gelu_grad(fm["z"]), a=fm["a"], db1=mb["db1"], dw2=mb["dw2"],
               dw_o=F8.q4(O).T @ F8.q5(DH), db_o=DH.sum(axis=0))
    for k in ref:
        assert_bf16(k, got[k], ref[k])


GOLDEN_7B = os.path.join(os.path.dirname(__file__), "golden", "fp8_layer_7b_tp4.npz")


@pytest.mark.gpu
def test_fp8_layer_full_size_7b_tp4(mtl):
    """The fp8 variant of the 7B-class TP=4 layer at full size (hidden 4096,
    32 heads, ffn 16384, seq 4096; all four shards and the four reductions on
    one GPU, the step bench.py --workload 7b-tp4 --precision fp8 times one
    shard of) against the stored fp64 reference on the unquantised inputs
    (tests/golden/make_fp8_layer_7b_tp4.py, which calls only the oracle): the
    two-part check of the module docstring on sampled rows of every output and
    the whole bias gradients, the 8e-2 bound taken against each output's
    whole-tensor max|ref|, the RMS against the recipe's RMS on the same rows."""
    import torch
    from megatron_tensor_transformer_layer_amd.layer import AllShardsStep, host_f64
    gold = np.load(GOLDEN_7B)
    shape = synth.WORKLOADS[str(gold["workload"])]
    print(f"fp8 full-size layer {shape}", flush=True)
    full = synth.layer_inputs(shape, seed=int(gold["seed"]))
    shards = [synth.layer_inputs(shape, seed=int(gold["seed"]), tp=shape.tp, rank=r) for r in range(shape.tp)]
    print("inputs drawn", flush=True)
    step = AllShardsStep(shape, shape.tp, shards, full["x"], full["dy"], full["b_o"], full["b2"],
                         precision=mtl.MTL_PREC_FP8_HYBRID)
    step()
    torch.cuda.synchronize()
    rk = step.ranks
    cat = lambda key, dim: torch.cat([getattr(r, key) for r in rk], dim=dim)
    dev = dict(y=step.y, h=step.h, dh=step.dh, dx=step.dx, dw_qkv=cat("dw_qkv", 1), dw_o=cat("dw_o", 0),
               dw1=cat("dw1", 1), dw2=cat("dw2", 0), db_qkv=cat("db_qkv", 0), db1=cat("db1", 0),
               db_o=rk[0].db_o, db2=rk[0].db2)
    bad = []
    for k, t in dev.items():
        ref = gold[f"{k}/ref"].astype(np.float64)
        got = host_f64(t[torch.from_numpy(gold[f"{k}/rows"]).cuda()] if f"{k}/rows" in gold else t)
        st = gold[f"{k}/stats"]  # whole tensor: max|ref|, rms ref, max|q-ref|, rms(q-ref); then on the samples
        ref_max, recipe_max = float(st[0]), float(st[2])
        why, line = fp8_two_part_check(k, got, ref, recipe_max, float(st[7]), ref_max, float(st[5]))
        print(line, flush=True)
        if why:
            bad.append(f"{k}: {why}")
    assert not bad, bad


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["gpt2-small-tp2", "d128-mb2-tp2"])
def test_fp8_kept_codes_are_bit_identical(mtl, case):
    """With MTL_F_FP8_KEEP_CODES the backward takes the transposed codes of x,
    o, h and a that the forward wrote instead of quantising them again: every
    output equals the layer without the flag bit for bit."""
    from megatron_tensor_transformer_layer_amd.layer import run_sharded_layer
    shape, residual = FP8_CASES[case]
    print(f"fp8 kept codes {case} {shape}", flush=True)
    full = synth.layer_inputs(shape, seed=0)
    shards = [synth.layer_inputs(shape, seed=0, tp=shape.tp, rank=r) for r in range(shape.tp)]
    run = lambda flags: run_sharded_layer(shape, shape.tp, shards, full["x"], full["b_o"], full["b2"], full["dy"],
                                          residual, precision=mtl.MTL_PREC_FP8_HYBRID, flags=flags)
    a, b = run(0), run(mtl.MTL_F_FP8_KEEP_CODES)
    for k, v in a.items():
        if isinstance(v, np.ndarray):
            assert np.array_equal(v, b[k]), k


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["gpt2-small-tp2", "d128-mb2-tp2"])
def test_fp8_reused_weight_codes(mtl, case):
    """MTL_F_FP8_REUSE_WEIGHTS: a rank step after a step without the flag gives
    the first step's outputs bit for bit, and it reads no bf16 weight: with the
    weights overwritten (a second micro-batch may not do that, but the call
    must not notice) the outputs are still those of the first step."""
    import torch
    from megatron_tensor_transformer_layer_amd.layer import RankState, bf16_dev
    shape, _ = FP8_CASES[case]
    t, r = shape.tp, shape.tp - 1
    print(f"fp8 reused weight codes {case} {shape}", flush=True)
    inp = synth.layer_inputs(shape, tp=t, rank=r)
    keep = mtl.MTL_F_FP8_KEEP_CODES
    st = RankState(shape, t, r, inp, flags=keep, precision=mtl.MTL_PREC_FP8_HYBRID)
    x, dy = bf16_dev(inp["x"]), bf16_dev(inp["dy"])
    h, dh = bf16_dev(synth.layer_tensor(shape, "h")), bf16_dev(synth.layer_tensor(shape, "dh"))
    names = ("qkv", "o", "lse", "gz", "a", "p_attn", "p_mlp", "p_dh", "p_dx", "dw_qkv", "db_qkv", "dw_o", "db_o",
             "dw1", "db1", "dw2", "db2")

    def step():
        st.attn_fwd(x)
        st.mlp_fwd(h)
        st.mlp_bwd(dy, h)
        st.attn_bwd(dh, x)
        torch.cuda.synchronize()
        return {k: getattr(st, k).clone() for k in names}

    first = step()
    st.cfg.flags = keep | mtl.MTL_F_FP8_REUSE_WEIGHTS
    again = step()
    bad = [k for k in names if not torch.equal(first[k], again[k])]
    assert not bad, f"reused codes differ: {bad}"
    for k in ("w_qkv", "w_o", "w1", "w2"):
        st.w[k].mul_(-3.0)
    ignored = step()
    bad = [k for k in names if not torch.equal(first[k], ignored[k])]
    assert not bad, f"bf16 weights were read: {bad}"


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["gpt2-small-tp2", "d128-mb2-tp2"])
def test_fp8_producer_amax_equals_the_amax_pass(mtl, case):
    """The amax of O (from the attention kernel) and of A (from the fc1
    epilogue), which the fp8 forward takes from the kernels that produced them,
    is the one mtl_fp8_amax finds over the stored tensor: the kept records
    (MTL_F_FP8_KEEP_CODES) equal mtl_fp8_amax's records bit for bit."""
    import torch
    from megatron_tensor_transformer_layer_amd import mtl_fp8_amax, MTL_FP8_AMAX_SCRATCH
    from megatron_tensor_transformer_layer_amd.layer import RankState, bf16_dev
    shape, _ = FP8_CASES[case]
    t, r = shape.tp, shape.tp - 1
    print(f"fp8 producer amax {case} {shape}", flush=True)
    inp = synth.layer_inputs(shape, tp=t, rank=r)
    st = RankState(shape, t, r, inp, flags=mtl.MTL_F_FP8_KEEP_CODES, precision=mtl.MTL_PREC_FP8_HYBRID)
    x, h = bf16_dev(inp["x"]), bf16_dev(synth.layer_tensor(shape, "h"))
    st.attn_fwd(x)
    st.mlp_fwd(h)
    torch.cuda.synchronize()
    S, hd, o_l, f_l = shape.seq * shape.micro_batch, shape.hidden, shape.hidden // t, shape.ffn // t
    up = lambda n: (n + 255) // 256 * 256
    # kept region: x_t, o_t, h_t, a_t, each a 256-byte record then its codes
    off_o = 256 + up(S * hd)
    off_a = off_o + 256 + up(S * o_l) + 256 + up(S * hd)
    scratch = torch.empty(MTL_FP8_AMAX_SCRATCH, dtype=torch.uint8, device="cuda")
    for name, off, ten in (("o", off_o, st.o), ("a", off_a, st.a)):
        kept = st.scratch[off:off + 12].view(torch.float32).clone()
        rec = torch.zeros(4, dtype=torch.float32, device="cuda")
        mtl_fp8_amax(ten, ten.numel(), mtl.MTL_FP8_E4M3, rec, scratch)
        torch.cuda.synchronize()
        assert torch.equal(kept[:3], rec[:3]), (name, kept.tolist(), rec.tolist())
        assert kept[0].item() == ten.float().abs().max().item(), name
