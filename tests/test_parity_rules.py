"""The GPU-vs-oracle comparison rules themselves (host only, no GPU).

The parity tests trust ``parity.compare``; these tests pin it: a result that differs from
the oracle only by pre-quant noise inside the tolerance (and is then quantized by the
same rule) passes, and each kind of planted mistake -- a pre-quant error above the
tolerance, a code or exponent that does not follow from the f32 output, an exponent off
the fp64 oracle outside the rounding band -- fails.  ``tie_aware_tolerance`` is pinned
against a direct fp64 evaluation of the two-term-q scores it models, and against its
closed forms (equal rows, q = 0).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from prefill_token_amd import inputs

from parity import compare, run_oracle, tie_aware_tolerance


@pytest.fixture(scope="module")
def case():
    inp = inputs.make("decode_sq64", seed=404, s_q=3)
    return inp, run_oracle(inp)


def fake_gpu(o, noise, rng):
    """o plus noise of at most ``noise`` times each block's amax, in f32, quantized by the
    oracle's rule (so check (i) holds by construction)."""
    blk = o.reshape(*o.shape[:-1], -1, 32)
    amax = np.abs(blk).max(-1, keepdims=True)
    g = (blk + noise * amax * rng.uniform(-1, 1, blk.shape)).reshape(o.shape).astype(np.float32)
    codes, scales = oracle.quantize_blocks(g.astype(np.float64))
    return dict(f32=g, codes=codes, scales=scales)


def test_noise_inside_tolerance_passes(case):
    inp, ref = case
    rng = np.random.default_rng(1)
    st = compare(fake_gpu(ref["o"], 0.004, rng), ref)
    assert st["prequant_max_rel_block"] <= 0.004 * 1.0001
    st = compare(fake_gpu(ref["o"], 0.0, rng), ref)  # f32 rounding only
    assert st["codes_within_1_ordinal_step"] == 1.0


def test_prequant_error_above_tolerance_fails(case):
    inp, ref = case
    g = fake_gpu(ref["o"], 0.0, np.random.default_rng(2))
    blk_amax = np.abs(ref["o"][1, 7, 64:96]).max()
    g["f32"][1, 7, 70] += np.float32(0.02 * blk_amax)
    g["codes"], g["scales"] = oracle.quantize_blocks(g["f32"].astype(np.float64))
    with pytest.raises(AssertionError, match="pre-quant"):
        compare(g, ref)


def test_code_not_from_f32_fails(case):
    inp, ref = case
    g = fake_gpu(ref["o"], 0.0, np.random.default_rng(3))
    c = g["codes"][0, 3, 10]
    g["codes"][0, 3, 10] = (c & 0x80) | min((c & 0x7F) + 2, 0x7E)
    with pytest.raises(AssertionError, match="codes differ"):
        compare(g, ref)


def test_exponent_not_from_f32_fails(case):
    inp, ref = case
    g = fake_gpu(ref["o"], 0.0, np.random.default_rng(4))
    g["scales"][2, 5, 3] += 1
    with pytest.raises(AssertionError, match="exponents differ"):
        compare(g, ref)


def test_exponent_off_outside_band_fails_without_f32(case):
    inp, ref = case
    g = fake_gpu(ref["o"], 0.0, np.random.default_rng(5))
    # choose a block whose amax is far from a power of two times 448
    a = np.abs(ref["o"].reshape(3, 64, 16, 32)).max(-1)
    frac = np.abs(np.log2(a / 448.0) - np.round(np.log2(a / 448.0)))
    t, h, b = np.unravel_index(np.argmax(frac), frac.shape)
    g["scales"][t, h, b] += 1
    g["f32"] = None
    with pytest.raises(AssertionError, match="band rule"):
        compare(g, ref, check_f32=False)


def test_extra_tolerance_widens_only_its_head(case):
    inp, ref = case
    g = fake_gpu(ref["o"], 0.0, np.random.default_rng(6))
    blk_amax = np.abs(ref["o"][1, 7, 64:96]).max()
    g["f32"][1, 7, 70] += np.float32(0.05 * blk_amax)
    g["codes"], g["scales"] = oracle.quantize_blocks(g["f32"].astype(np.float64))
    extra = np.zeros((3, 64))
    extra[1, 7] = 0.05 * blk_amax
    compare(g, ref, extra=extra)
    extra[1, 7] = 0.0
    extra[1, 8] = 0.05 * blk_amax
    with pytest.raises(AssertionError):
        compare(g, ref, extra=extra)


def _two_term_output(inp):
    """fp64 attention with the two-term E4M3 q' the kernel uses (the model the tolerance
    bounds), before inverse RoPE is applied; then inverse RoPE."""
    s_q, h, d = inp["q"].shape
    c = inp["sm_scale"] / math.log(2.0)
    v_all = oracle.mx_decode(inp["kv_pool"], inp["kv_scales"])
    out = np.zeros((s_q, h, d))
    for t in range(s_q):
        L = min(int(inp["topk_length"][t]), inp["topk"])
        row = inp["indices"][t, :max(L, 0)]
        v = v_all[row[row >= 0]]
        x = inputs.bf16_values(inp["q"][t]).astype(np.float64)
        y = np.stack([oracle.rope(r, inp["rope_dim"], float(inp["positions"][t]), inp["theta"])
                      for r in (oracle.rmsnorm(xr, np.asarray(inp["norm_w"], np.float64), inp["eps"]) for xr in x)]) * c
        yb = y.reshape(h, d // 32, 32)
        e1 = oracle.ue8m0_exponent(np.abs(yb).max(-1)).astype(np.int64)
        S1 = np.ldexp(1.0, e1 - 127)[..., None]
        t1 = oracle.e4m3_decode(oracle.e4m3_encode(yb / S1)) * S1
        S2 = np.ldexp(1.0, np.maximum(e1 - 4, 0) - 127)[..., None]
        t2 = oracle.e4m3_decode(oracle.e4m3_encode((yb - t1) / S2)) * S2
        s = (t1 + t2).reshape(h, d) @ v.T
        w = np.exp2(s - s.max(1, keepdims=True))
        w /= w.sum(1, keepdims=True)
        u = w @ v
        out[t] = np.stack([oracle.rope(r, inp["rope_dim"], float(inp["positions"][t]), inp["theta"], -1) for r in u])
    return out


def test_tie_aware_tolerance_bounds_the_two_term_model():
    # sharp softmax: scores 16x the natural scale, so many heads are near one-hot and some
    # have near-tied top rows
    inp = inputs.make("decode_sq64", seed=405, s_q=2)
    inp["sm_scale"] *= 16.0
    ref = run_oracle(inp)
    E = tie_aware_tolerance(inp)
    model = _two_term_output(inp)
    err = np.abs(model - ref["o"]).max(-1)
    assert (err <= E * 1.0001 + 1e-12).all()
    assert E.max() > 0


def test_tie_aware_tolerance_closed_forms():
    inp = inputs.make("decode_sq64", seed=406, s_q=2)
    inp["kv_pool"][:] = inp["kv_pool"][3]  # every row the same: the output cannot move
    inp["kv_scales"][:] = inp["kv_scales"][3]
    vmax = np.abs(oracle.mx_decode(inp["kv_pool"][3:4], inp["kv_scales"][3:4])).max()
    assert np.all(tie_aware_tolerance(inp) <= 1e-12 * vmax)  # zero up to the rounding of sum_j w_j
    inp = inputs.make("decode_sq64", seed=407, s_q=2)
    inp["q"][:] = 0  # q = 0: exact scores (all zero), no score error
    assert np.all(tie_aware_tolerance(inp, slack=0.0) == 0.0)
