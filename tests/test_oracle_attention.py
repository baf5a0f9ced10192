"""Pins for the oracle's whole step (norm -> RoPE -> sparse attention -> inverse RoPE -> FP8).

The sparse step is pinned against an independent formulation: dense attention over the
whole pool through torch's scaled_dot_product_attention in fp64 on the CPU, with an
additive bias log(multiplicity) per pool row (-inf for rows the token does not read);
the query path uses torch's rms_norm and a complex-number rotation, the rows use
torch's float8_e4m3fn decode.  Invariants from the definition: sentinel entries
contribute nothing, the order of entries does not matter, entries at or beyond
topk_length are never read (even when they point at rows that decode to NaN), and a
duplicated entry weighs twice.  Closed forms: one valid row, all rows equal, q = 0,
empty row, rope_dim = 0.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from prefill_token_amd import inputs

SM_EPS = 1e-6
THETA = 10000.0


def small_case(seed, kv_format, s_q=3, h=8, d=128, r=32, n_rows=96, topk=40, p_sent=0.1, distinct=True):
    rng = np.random.default_rng(seed)
    q = inputs.bf16_bits(rng.standard_normal((s_q, h, d)).astype(np.float32))
    norm_w = inputs.bf16_values(inputs.bf16_bits(rng.normal(1, 0.1, d).astype(np.float32))).astype(np.float64)
    if kv_format == inputs.KV_BF16:
        pool = inputs.bf16_bits(rng.standard_normal((n_rows, d)).astype(np.float32))
        scales = None
    else:
        pool, scales = inputs.mx_pool(rng.standard_normal((n_rows, d)).astype(np.float32))
    idx = np.empty((s_q, topk), dtype=np.int32)
    for t in range(s_q):
        idx[t] = rng.choice(n_rows, size=topk, replace=not distinct)
    idx[rng.random((s_q, topk)) < p_sent] = -1
    return dict(q=q, kv_pool=pool, kv_scales=scales, indices=idx,
                topk_length=np.full(s_q, topk, dtype=np.int32),
                positions=rng.integers(0, 32768, s_q).astype(np.int32), norm_w=norm_w,
                sm_scale=1.0 / math.sqrt(d), rope_dim=r, kv_format=kv_format)


def run_oracle(orc, c):
    return orc.sparse_mla(c["q"], c["kv_pool"], c["kv_scales"], c["indices"], c["topk_length"],
                          c["positions"], c["norm_w"], sm_scale=c["sm_scale"], eps=SM_EPS, theta=THETA,
                          rope_dim=c["rope_dim"], kv_format=c["kv_format"])


def dense_rows(c):
    """All pool rows decoded with library casts: [n, d] float64."""
    if c["kv_format"] == inputs.KV_BF16:
        t = torch.from_numpy(c["kv_pool"].view(np.int16).copy()).view(torch.bfloat16)
        return t.double().numpy()
    codes = torch.from_numpy(c["kv_pool"].copy()).view(torch.float8_e4m3fn).double().numpy()
    sc = np.repeat(c["kv_scales"].astype(np.int64) - 127, 32, axis=1)
    return np.ldexp(codes, sc)


def complex_rope(y, r, pos, direction):
    d = y.shape[-1]
    o0, half = d - r, r // 2
    if r == 0:
        return y.copy()
    i = np.arange(half)
    ang = direction * pos * THETA ** (-(2.0 * i) / r)
    z = (y[..., o0:o0 + half] + 1j * y[..., o0 + half:]) * np.exp(1j * ang)
    out = y.copy()
    out[..., o0:o0 + half] = z.real
    out[..., o0 + half:] = z.imag
    return out


def brute_force(c):
    """Dense masked attention through torch SDPA in fp64 (independent of the oracle)."""
    q = torch.from_numpy(c["q"].view(np.int16).copy()).view(torch.bfloat16).double()
    s_q, h, d = q.shape
    V = torch.from_numpy(dense_rows(c))
    n = V.shape[0]
    out = np.zeros((s_q, h, d))
    for t in range(s_q):
        y = F.rms_norm(q[t], (d,), weight=torch.from_numpy(c["norm_w"]), eps=SM_EPS).numpy()
        y = complex_rope(y, c["rope_dim"], float(c["positions"][t]), +1)
        L = min(int(c["topk_length"][t]), c["indices"].shape[1])
        ids = c["indices"][t, :L]
        ids = ids[ids >= 0]
        if ids.size == 0:
            continue
        count = np.bincount(ids, minlength=n).astype(np.float64)
        with np.errstate(divide="ignore"):
            bias = np.log(count)
        o = F.scaled_dot_product_attention(
            torch.from_numpy(y)[None, :, None, :], V[None, None].expand(1, h, n, d),
            V[None, None].expand(1, h, n, d), attn_mask=torch.from_numpy(bias)[None, None, None, :],
            scale=c["sm_scale"])[0, :, 0, :].numpy()
        out[t] = complex_rope(o, c["rope_dim"], float(c["positions"][t]), -1)
    return out


def assert_close_rows(a, b, tol):
    den = np.maximum(np.abs(b).max(axis=-1, keepdims=True), 1e-300)
    err = (np.abs(a - b) / den).max()
    assert err <= tol, err


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("kv_format", [inputs.KV_BF16, inputs.KV_E4M3_UE8M0])
def test_matches_dense_sdpa(oracle_mod, seed, kv_format):
    c = small_case(seed, kv_format)
    o, codes, scales = run_oracle(oracle_mod, c)
    ref = brute_force(c)
    assert_close_rows(o, ref, 1e-12)
    # quantizer consistency with the library cast on the oracle's own fp64 output
    S = np.ldexp(1.0, scales.astype(np.int64) - 127)
    amax = np.abs(o.reshape(*o.shape[:-1], -1, 32)).max(-1)
    assert (448 * S >= amax).all() and ((amax == 0) | (224 * S < amax)).all()


def test_matches_dense_sdpa_d512_fp8(oracle_mod):
    c = small_case(5, inputs.KV_E4M3_UE8M0, s_q=2, h=4, d=512, r=64, n_rows=700, topk=640)
    o, _, _ = run_oracle(oracle_mod, c)
    # angles reach ~3e4 rad here, where fp64 rounding of the angle itself is ~4e-12 rad
    assert_close_rows(o, brute_force(c), 1e-11)


def test_duplicates_weigh_twice(oracle_mod):
    c = small_case(3, inputs.KV_BF16, n_rows=20, topk=40, distinct=False, p_sent=0.0)
    assert any(len(set(r.tolist())) < len(r) for r in c["indices"])
    o, _, _ = run_oracle(oracle_mod, c)
    assert_close_rows(o, brute_force(c), 1e-12)


def test_sentinel_equals_deletion(oracle_mod):
    c = small_case(4, inputs.KV_E4M3_UE8M0, p_sent=0.3)
    o, codes, scales = run_oracle(oracle_mod, c)
    # compact every row: drop the -1 entries, shorten topk_length, pad with stale ids
    c2 = dict(c)
    idx2 = np.full_like(c["indices"], 5)
    L2 = np.zeros(c["indices"].shape[0], dtype=np.int32)
    for t, row in enumerate(c["indices"]):
        keep = row[row >= 0]
        idx2[t, : keep.size] = keep
        L2[t] = keep.size
    c2["indices"], c2["topk_length"] = idx2, L2
    o2, codes2, scales2 = run_oracle(oracle_mod, c2)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13 * np.abs(o).max())


def test_permutation_invariance(oracle_mod):
    c = small_case(6, inputs.KV_E4M3_UE8M0)
    o, _, _ = run_oracle(oracle_mod, c)
    rng = np.random.default_rng(9)
    c2 = dict(c)
    c2["indices"] = np.stack([rng.permutation(r) for r in c["indices"]])
    o2, _, _ = run_oracle(oracle_mod, c2)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12 * np.abs(o).max())


def test_truncation_never_reads_beyond_length(oracle_mod):
    c = small_case(7, inputs.KV_E4M3_UE8M0, p_sent=0.0)
    L = 17
    # rows 0..4 decode to NaN (code 0x7F); point the tail of every row at them
    pool = c["kv_pool"].copy()
    pool[:5, :] = 0x7F
    c_short = dict(c, kv_pool=pool)
    idx = c["indices"].copy()
    idx = np.where(idx < 5, idx + 5, idx)  # keep the prefix away from the NaN rows
    c_short["indices"] = idx[:, :L].copy()
    c_short["topk_length"] = np.full(idx.shape[0], L, dtype=np.int32)
    c_stale = dict(c_short)
    stale = idx.copy()
    stale[:, L:] = np.arange(stale.shape[1] - L)[None, :] % 5
    c_stale["indices"] = stale
    c_stale["topk_length"] = np.full(idx.shape[0], L, dtype=np.int32)
    o1, k1, s1 = run_oracle(oracle_mod, c_short)
    o2, k2, s2 = run_oracle(oracle_mod, c_stale)
    assert np.isfinite(o2).all()
    assert np.array_equal(o1, o2) and np.array_equal(k1, k2) and np.array_equal(s1, s2)


def test_single_row_closed_form(oracle_mod):
    c = small_case(8, inputs.KV_E4M3_UE8M0, s_q=2, p_sent=0.0)
    c["indices"][:, 1:] = -1
    o, _, _ = run_oracle(oracle_mod, c)
    V = dense_rows(c)
    for t in range(2):
        want = complex_rope(V[c["indices"][t, 0]], c["rope_dim"], float(c["positions"][t]), -1)
        for hh in range(o.shape[1]):
            np.testing.assert_allclose(o[t, hh], want, rtol=0, atol=1e-13 * np.abs(want).max())


def test_zero_query_is_uniform_mean(oracle_mod):
    c = small_case(10, inputs.KV_BF16, s_q=2)
    c["q"] = np.zeros_like(c["q"])
    o, _, _ = run_oracle(oracle_mod, c)
    V = dense_rows(c)
    for t in range(2):
        ids = c["indices"][t][c["indices"][t] >= 0]
        want = complex_rope(V[ids].mean(axis=0), c["rope_dim"], float(c["positions"][t]), -1)
        np.testing.assert_allclose(o[t], np.broadcast_to(want, o[t].shape), rtol=0, atol=1e-12)


def test_all_rows_equal(oracle_mod):
    c = small_case(12, inputs.KV_BF16, s_q=2)
    c["kv_pool"] = np.broadcast_to(c["kv_pool"][7], c["kv_pool"].shape).copy()
    o, _, _ = run_oracle(oracle_mod, c)
    v = dense_rows(c)[0]
    for t in range(2):
        want = complex_rope(v, c["rope_dim"], float(c["positions"][t]), -1)
        np.testing.assert_allclose(o[t], np.broadcast_to(want, o[t].shape), rtol=0, atol=1e-12)


def test_empty_rows_give_zero(oracle_mod):
    c = small_case(13, inputs.KV_E4M3_UE8M0, s_q=3)
    c["indices"][0, :] = -1          # all sentinels
    c["topk_length"][1] = 0          # nothing read
    c["topk_length"][2] = 1          # one entry, itself a sentinel
    c["indices"][2, 0] = -1
    o, codes, scales = run_oracle(oracle_mod, c)
    assert (o == 0).all() and (codes & 0x7F == 0).all() and (scales == 0).all()


def test_rope_dim_zero_is_plain_mqa(oracle_mod):
    c = small_case(14, inputs.KV_E4M3_UE8M0, r=0)
    o, _, _ = run_oracle(oracle_mod, c)
    assert_close_rows(o, brute_force(c), 1e-12)


def test_topk_length_beyond_row_is_capped(oracle_mod):
    c = small_case(15, inputs.KV_BF16)
    o, _, _ = run_oracle(oracle_mod, c)
    c2 = dict(c, topk_length=np.full(c["q"].shape[0], 10_000, dtype=np.int32))
    o2, _, _ = run_oracle(oracle_mod, c2)
    assert np.array_equal(o, o2)


def test_index_out_of_range_is_an_error(oracle_mod):
    c = small_case(16, inputs.KV_BF16)
    c["indices"][1, 3] = c["kv_pool"].shape[0]
    with pytest.raises(ValueError):
        run_oracle(oracle_mod, c)
    c["indices"][1, 3] = -2
    with pytest.raises(ValueError):
        run_oracle(oracle_mod, c)
    # beyond topk_length the content is ignored
    c["topk_length"][1] = 3
    run_oracle(oracle_mod, c)
