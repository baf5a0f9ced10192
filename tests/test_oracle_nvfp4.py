"""Pins for the oracle's two-pool step over the nvfp4_ds_mla cache (E4M3 + UE8M0 SWA rows,
NVFP4 compressed rows) [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose: fp8 528 B
SWA rows + fp4 288 B compressed rows].

- E2M1 decode, exhaustive over all 16 codes, through torch's E4M3 cast: every E2M1 value
  is an E4M3 value, code (s, e, m) with e >= 1 being E4M3 code (s, e + 6, m << 2) and the
  subnormal 0.5 being E4M3 0x30 -- an independent derivation through a library routine
  (a wrong bias, mantissa weight or sign fails it).
- NVFP4 row decode: value = e2m1(nibble) * e4m3(scale of its 16 elements), element 2i in
  the low nibble of byte i; checked element by element against torch's E4M3 cast of the
  scale and the pinned E2M1 table, and by the round trip of the stand-in producer
  (every decoded value within half an E2M1 step of the latent at its block's scale).
- The whole two-pool step against dense fp64 SDPA (torch) over both pools' decoded rows,
  with entries j < swa_entries naming SWA rows and later entries compressed rows.
- Equivalence with the one-pool step when the compressed rows are also representable in
  the E4M3 + UE8M0 format: the two-pool oracle must equal the one-pool oracle on the
  concatenated pool bit for bit (the segment mapping is the only difference).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from prefill_token_amd import inputs

from test_oracle_attention import complex_rope

SM_EPS = 1e-6
THETA = 10000.0


def test_e2m1_decode_exhaustive_through_e4m3():
    mapped = []
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e >= 1:
            code = (s << 7) | ((e + 6) << 3) | (m << 2)
        else:
            code = (s << 7) | (0x30 if m else 0x00)
        mapped.append(code)
    lib = torch.tensor(mapped, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert np.array_equal(got, lib)
    assert got[7] == 6.0 and got[1] == 0.5  # OCP E2M1: max normal 6, min subnormal 0.5
    assert np.all(np.diff(got[:8]) > 0) and np.array_equal(got[8:], -got[:8])


def test_nvfp4_row_decode_elementwise():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 256, (3, 64), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (3, 8), dtype=np.uint8)  # E4M3 codes without NaN
    got = oracle.nvfp4_decode(codes, scales)
    lut = oracle.e2m1_decode(np.arange(16, dtype=np.uint8))
    sc = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).double().numpy()
    for r in range(3):
        for i in range(128):
            byte = codes[r, i // 2]
            nib = byte & 15 if i % 2 == 0 else byte >> 4
            assert got[r, i] == lut[nib] * sc[r, i // 16]


def test_producer_round_trip():
    lat = np.random.default_rng(12).standard_normal((16, 512)).astype(np.float32)
    c, s = inputs.nvfp4_pool(lat)
    dec = oracle.nvfp4_decode(c, s)
    sc = np.repeat(torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).double().numpy(), 16, axis=1)
    x = np.abs(lat.astype(np.float64)) / np.where(sc > 0, sc, 1)
    # E2M1 step at |x|: 0.5 below 2, 1 in [2, 4), 2 above; clipped at 6
    step = np.where(x < 2, 0.5, np.where(x < 4, 1.0, 2.0))
    err = np.abs(dec - lat) / np.where(sc > 0, sc, 1)
    assert (err <= step / 2 + 1e-12 + np.maximum(x - 6.0, 0)).all()


def ds_case(seed, s_q=3, h=4, d=512, r=64, n_swa=150, n_cmp=200, swa_entries=64, topk=192, p_sent=0.1):
    rng = np.random.default_rng(seed)
    q = inputs.bf16_bits(rng.standard_normal((s_q, h, d)).astype(np.float32))
    norm_w = inputs.bf16_values(inputs.bf16_bits(rng.normal(1, 0.1, d).astype(np.float32))).astype(np.float64)
    sw, ss = inputs.mx_pool(rng.standard_normal((n_swa, d)).astype(np.float32))
    cc, cs = inputs.nvfp4_pool(rng.standard_normal((n_cmp, d)).astype(np.float32))
    idx = np.empty((s_q, topk), dtype=np.int32)
    for t in range(s_q):
        idx[t, :swa_entries] = rng.choice(n_swa, swa_entries, replace=False)
        idx[t, swa_entries:] = rng.choice(n_cmp, topk - swa_entries, replace=False)
    idx[rng.random((s_q, topk)) < p_sent] = -1
    L = np.array([topk, topk - 5, swa_entries + 3][:s_q], dtype=np.int32)
    return dict(q=q, swa_codes=sw, swa_scales=ss, cmp_codes=cc, cmp_scales=cs, indices=idx, topk_length=L,
                positions=rng.integers(0, 32768, s_q).astype(np.int32), norm_w=norm_w,
                sm_scale=1.0 / math.sqrt(d), rope_dim=r, swa_entries=swa_entries)


def run_ds(c):
    return oracle.sparse_mla_ds_nvfp4(c["q"], c["swa_codes"], c["swa_scales"], c["cmp_codes"], c["cmp_scales"],
                                      c["indices"], c["topk_length"], c["positions"], c["norm_w"],
                                      swa_entries=c["swa_entries"], sm_scale=c["sm_scale"], eps=SM_EPS, theta=THETA,
                                      rope_dim=c["rope_dim"])


@pytest.mark.parametrize("seed", [0, 1])
def test_two_pool_step_matches_dense_sdpa(seed):
    c = ds_case(seed)
    o, _, _ = run_ds(c)
    # dense rows: SWA rows (library E4M3 cast times 2^(e-127)), then compressed rows
    sw = torch.from_numpy(c["swa_codes"].copy()).view(torch.float8_e4m3fn).double().numpy()
    sw = np.ldexp(sw, np.repeat(c["swa_scales"].astype(np.int64) - 127, 32, axis=1))
    V = torch.from_numpy(np.concatenate([sw, oracle.nvfp4_decode(c["cmp_codes"], c["cmp_scales"])]))
    n_swa = c["swa_codes"].shape[0]
    n = V.shape[0]
    q = torch.from_numpy(c["q"].view(np.int16).copy()).view(torch.bfloat16).double()
    s_q, h, d = q.shape
    for t in range(s_q):
        y = F.rms_norm(q[t], (d,), weight=torch.from_numpy(c["norm_w"]), eps=SM_EPS).numpy()
        y = complex_rope(y, c["rope_dim"], float(c["positions"][t]), +1)
        L = min(int(c["topk_length"][t]), c["indices"].shape[1])
        ids = c["indices"][t, :L].astype(np.int64)
        cols = np.arange(L)
        glob = np.where(cols < c["swa_entries"], ids, n_swa + ids)[ids >= 0]
        with np.errstate(divide="ignore"):
            bias = np.log(np.bincount(glob, minlength=n).astype(np.float64))
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(y)[None, :, None, :], V[None, None].expand(1, h, n, d), V[None, None].expand(1, h, n, d),
            attn_mask=torch.from_numpy(bias)[None, None, None, :], scale=c["sm_scale"])[0, :, 0, :].numpy()
        ref = complex_rope(ref, c["rope_dim"], float(c["positions"][t]), -1)
        den = np.abs(ref).max(axis=-1, keepdims=True)
        assert (np.abs(o[t] - ref) / den).max() <= 1e-11


def test_two_pool_equals_one_pool_when_rows_coincide():
    c = ds_case(3)
    # compressed rows whose scales are powers of two (E4M3 mantissa 0, exponent 1..14): each
    # value e2m1 * 2^k is an E4M3 value times a power of two, so an E4M3 + UE8M0 pool holds
    # the same numbers
    rng = np.random.default_rng(4)
    n_cmp, d = c["cmp_codes"].shape[0], 512
    c["cmp_scales"] = (rng.integers(4, 10, (n_cmp, d // 16)) << 3).astype(np.uint8)
    vals = oracle.nvfp4_decode(c["cmp_codes"], c["cmp_scales"])
    blk = np.abs(vals.reshape(n_cmp, d // 32, 32)).max(-1)
    e = np.where(blk > 0, np.ceil(np.log2(np.maximum(blk, 1e-300) / 448.0)) + 127, 0).astype(np.int64)
    e = np.maximum(e, 0)
    codes = torch.from_numpy(vals / np.repeat(np.ldexp(1.0, e - 127), 32, axis=1)).to(torch.float8_e4m3fn)
    back = codes.double().numpy() * np.repeat(np.ldexp(1.0, e - 127), 32, axis=1)
    assert np.array_equal(back, vals)  # exactly representable
    pool = np.concatenate([c["swa_codes"], codes.view(torch.uint8).numpy()])
    scales = np.concatenate([c["swa_scales"], e.astype(np.uint8)])
    idx = c["indices"].copy()
    seg = idx[:, c["swa_entries"]:]
    idx[:, c["swa_entries"]:] = np.where(seg >= 0, seg + c["swa_codes"].shape[0], -1)
    one = oracle.sparse_mla(c["q"], pool, scales, idx, c["topk_length"], c["positions"], c["norm_w"],
                            sm_scale=c["sm_scale"], eps=SM_EPS, theta=THETA, rope_dim=c["rope_dim"])
    two = run_ds(c)
    for a, b in zip(one, two):
        assert np.array_equal(a, b)


def test_index_bounds_follow_the_segment():
    c = ds_case(5)
    c["indices"][0, 0] = c["swa_codes"].shape[0] - 1      # last SWA row: fine
    c["indices"][0, c["swa_entries"]] = c["cmp_codes"].shape[0] - 1  # last compressed row: fine
    run_ds(c)
    c["indices"][0, c["swa_entries"]] = c["cmp_codes"].shape[0]  # past the compressed pool
    with pytest.raises(ValueError):
        run_ds(c)
