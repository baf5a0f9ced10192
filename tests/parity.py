"""Helpers shared by the GPU parity tests: run the library and the oracle on the same
seeded inputs and compare them by the rules below.

Comparison rules (GPU vs the fp64 oracle):
  pre-quant  max_i |g_i - r_i| / A_ref(block(i)) <= 1e-2, A_ref = the oracle's block amax;
             a block whose oracle output is all zero (empty row) must be exactly zero.
  scales (i) the oracle's own quantizer applied to the GPU's f32 output reproduces the
             GPU's scales and codes bit for bit (codes up to the sign of zero): the GPU
             takes the same integer decision on the same f32 values.
  scales (ii) against the fp64 oracle the exponents are equal, except in "band" blocks
             where A_ref lies within the block's measured pre-quant error of a power of
             two times 448; there a difference of one is allowed (and counted).
  dequant    where the exponents agree, every dequantized value is within one E4M3 step
             of the block (the code step at the block's amax) of the oracle's dequantized
             value; in band blocks, within one step at the coarser of the two scales.
  codes      where the exponents agree, each code is within one step of the oracle's code
             in sign-magnitude order wherever the two pre-quant values differ by less than
             one code step at the smaller of the two magnitudes (round-to-nearest-even of
             two values closer than one grid step lands on the same or adjacent grid
             points).  Elsewhere a 1e-2 block-relative pre-quant difference can move a
             small element's code by several steps (the step at |o| = A/32 is A/256), so
             the code rule cannot be asked of them; their share is reported.

An optional per-(token, head) tolerance ``extra`` (output units) widens the pre-quant and
dequant bounds of that head; ``tie_aware_tolerance`` derives it from the sensitivity of
the softmax to the kernel's score error, for regimes where near-tied scores make the
output depend on that error (see there).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from prefill_token_amd import inputs

PREQUANT_TOL = 1e-2


def to_device(inp: dict, device="cuda"):
    t = {}
    t["q"] = torch.from_numpy(inp["q"].view(np.int16)).to(device).view(torch.bfloat16)
    if inp["kv_format"] == inputs.KV_BF16:
        t["kv_pool"] = torch.from_numpy(inp["kv_pool"].view(np.int16)).to(device).view(torch.bfloat16)
        t["kv_scales"] = None
    else:
        t["kv_pool"] = torch.from_numpy(inp["kv_pool"]).to(device)
        t["kv_scales"] = torch.from_numpy(inp["kv_scales"]).to(device)
    for k in ("indices", "topk_length", "positions"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.int32)).to(device)
    t["norm_w"] = torch.from_numpy(np.ascontiguousarray(inp["norm_w"], dtype=np.float32)).to(device)
    return t


def run_gpu(inp: dict, *, num_splits: int = 0, with_f32: bool = True, device="cuda", dev_inputs=None,
            workspace=None):
    from prefill_token_amd import sparse_mla_fwd

    t = dev_inputs if dev_inputs is not None else to_device(inp, device)
    s_q, h, d = inp["q"].shape
    # outputs start as values the step never writes (scale byte 255, f32 NaN), so a token
    # the kernels skipped cannot pass for a computed one
    out_fp8 = torch.full((s_q, h, d), 0xFF, dtype=torch.uint8, device=device)
    out_sc = torch.full((s_q, h, d // 32), 0xFF, dtype=torch.uint8, device=device)
    out_f32 = torch.full((s_q, h, d), float("nan"), dtype=torch.float32, device=device) if with_f32 else None
    sparse_mla_fwd(t["q"], t["kv_pool"], t["kv_scales"], t["indices"], t["topk_length"], t["positions"],
                   t["norm_w"], out_fp8, out_sc, sm_scale=inp["sm_scale"], rope_dim=inp["rope_dim"],
                   eps=inp["eps"], theta=inp["theta"], out_f32=out_f32, num_splits=num_splits,
                   workspace=workspace)
    torch.cuda.synchronize()
    return dict(codes=out_fp8.cpu().numpy(), scales=out_sc.cpu().numpy(),
                f32=None if out_f32 is None else out_f32.cpu().numpy())


def run_oracle(inp: dict):
    kvs = None if inp["kv_format"] == inputs.KV_BF16 else inp["kv_scales"]
    o, codes, scales = oracle.sparse_mla(inp["q"], inp["kv_pool"], kvs, inp["indices"], inp["topk_length"],
                                         inp["positions"], inp["norm_w"], sm_scale=inp["sm_scale"],
                                         eps=inp["eps"], theta=inp["theta"], rope_dim=inp["rope_dim"],
                                         kv_format=inp["kv_format"])
    return dict(o=o, codes=codes, scales=scales)


def run_gpu_ds(inp: dict, num_splits: int = 0, with_f32: bool = True, device="cuda"):
    """The step over the two-pool nvfp4_ds_mla cache on the GPU (sparse_mla_fwd_ds_nvfp4)."""
    from prefill_token_amd import sparse_mla_fwd_ds_nvfp4

    dev = device
    s_q, h, d = inp["q"].shape
    q = torch.from_numpy(inp["q"].view(np.int16)).to(dev).view(torch.bfloat16)
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
         for k in ("swa_codes", "swa_scales", "cmp_codes", "cmp_scales")}
    for k in ("indices", "topk_length", "positions"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.int32)).to(dev)
    w = torch.from_numpy(np.ascontiguousarray(inp["norm_w"], dtype=np.float32)).to(dev)
    out_fp8 = torch.full((s_q, h, d), 0xFF, dtype=torch.uint8, device=dev)
    out_sc = torch.full((s_q, h, d // 32), 0xFF, dtype=torch.uint8, device=dev)
    out_f32 = torch.full((s_q, h, d), float("nan"), dtype=torch.float32, device=dev) if with_f32 else None
    sparse_mla_fwd_ds_nvfp4(q, t["swa_codes"], t["swa_scales"], t["cmp_codes"], t["cmp_scales"], t["indices"],
                            t["topk_length"], t["positions"], w, out_fp8, out_sc, swa_entries=inp["swa_entries"],
                            sm_scale=inp["sm_scale"], rope_dim=inp["rope_dim"], eps=inp["eps"], theta=inp["theta"],
                            out_f32=out_f32, num_splits=num_splits)
    torch.cuda.synchronize()
    return dict(codes=out_fp8.cpu().numpy(), scales=out_sc.cpu().numpy(),
                f32=None if out_f32 is None else out_f32.cpu().numpy())


def run_oracle_ds(inp: dict):
    """The oracle's two-pool step on the same arrays."""
    o, codes, scales = oracle.sparse_mla_ds_nvfp4(
        inp["q"], inp["swa_codes"], inp["swa_scales"], inp["cmp_codes"], inp["cmp_scales"], inp["indices"],
        inp["topk_length"], inp["positions"], inp["norm_w"], swa_entries=inp["swa_entries"], sm_scale=inp["sm_scale"],
        eps=inp["eps"], theta=inp["theta"], rope_dim=inp["rope_dim"])
    return dict(o=o, codes=codes, scales=scales)


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def dequant(codes, scales):
    v = e4m3_values(codes)
    s = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    return v * s


def block_step(amax_ref, scales):
    """E4M3 step at the block's amax, in output units (the block's ulp)."""
    S = np.ldexp(1.0, scales.astype(np.int64) - 127)
    x = np.where(amax_ref > 0, amax_ref / S, 1.0)
    ex = np.floor(np.log2(np.maximum(x, 2.0 ** -9)))
    return np.ldexp(1.0, (np.maximum(ex, -6) - 3).astype(np.int64)) * S


def same_code(a, b):
    return (a == b) | (((a & 0x7F) == 0) & ((b & 0x7F) == 0))


def e4m3_step(mag):
    """E4M3 grid step at magnitude ``mag`` (in units of the block scale)."""
    mag = np.asarray(mag, dtype=np.float64)
    ex = np.floor(np.log2(np.maximum(mag, 2.0 ** -12)))
    return np.ldexp(1.0, (np.maximum(ex, -6) - 3).astype(np.int64))


def compare(gpu: dict, ref: dict, *, check_f32: bool = True, extra=None):
    """Assert the comparison rules; return a stats dict.  ``extra``: optional array of the
    shape of o without its last axis, an additional absolute tolerance per (token, head)."""
    o = ref["o"]
    d = o.shape[-1]
    blk = o.reshape(*o.shape[:-1], d // 32, 32)
    a_ref = np.abs(blk).max(axis=-1)
    ext = np.zeros(a_ref.shape) if extra is None else np.repeat(np.asarray(extra, np.float64)[..., None],
                                                                 d // 32, axis=-1)
    stats = {}
    err = None
    if check_f32 and gpu.get("f32") is not None:
        g = gpu["f32"].astype(np.float64)
        gb = g.reshape(blk.shape)
        err = np.abs(gb - blk).max(axis=-1)
        zero = a_ref == 0
        assert (err[zero] == 0).all(), "nonzero output where the oracle's block is all zero"
        rel = np.where(zero, 0.0, np.maximum(err - ext, 0.0) / np.maximum(a_ref, 1e-300))
        stats["prequant_max_rel_block"] = float(rel.max())
        if extra is not None:
            stats["prequant_max_rel_block_plain"] = float(np.where(zero, 0.0, err / np.maximum(a_ref, 1e-300)).max())
        row_amax = np.abs(o).max(axis=-1, keepdims=True)
        stats["prequant_max_rel_row"] = float((np.abs(g - o) / np.maximum(row_amax, 1e-300)).max())
        assert rel.max() <= PREQUANT_TOL, f"pre-quant block-relative error {rel.max():.3e} > {PREQUANT_TOL}"
        # (i) the oracle's quantizer on the GPU's own f32 output
        c_i, s_i = oracle.quantize_blocks(g)
        assert np.array_equal(s_i, gpu["scales"]), "UE8M0 exponents differ from the oracle rule on GPU f32"
        assert same_code(c_i, gpu["codes"]).all(), "E4M3 codes differ from the oracle rule on GPU f32"
        band_tol = err
    else:
        band_tol = None
    # (ii) exponents against the fp64 oracle
    eg = gpu["scales"].astype(np.int64)
    er = ref["scales"].astype(np.int64)
    diff = eg - er
    if band_tol is None:
        band_tol = PREQUANT_TOL * a_ref + ext
    with np.errstate(divide="ignore"):
        k = np.round(np.log2(np.maximum(a_ref, 1e-300) / 448.0))
    near = np.abs(a_ref - 448.0 * np.exp2(k)) <= band_tol * 1.0001 + 1e-300
    ok = (diff == 0) | ((np.abs(diff) == 1) & near)
    if extra is not None:
        # heads with a tie-aware tolerance: the exponent of any amax within the measured
        # (or allowed) pre-quant error of the oracle's
        lo = oracle.ue8m0_exponent(np.maximum(a_ref - band_tol * 1.0001, 0.0)).astype(np.int64)
        hi = oracle.ue8m0_exponent(a_ref + band_tol * 1.0001).astype(np.int64)
        ok |= (ext > 0) & (eg >= lo) & (eg <= hi)
    assert ok.all(), f"{int((~ok).sum())} blocks with exponents off the fp64 oracle beyond the band rule"
    stats["band_blocks"] = int((diff != 0).sum())
    stats["blocks"] = int(diff.size)
    # dequantized values
    dg = dequant(gpu["codes"], gpu["scales"]).reshape(blk.shape)
    dr = dequant(ref["codes"], ref["scales"]).reshape(blk.shape)
    step = block_step(a_ref, np.maximum(gpu["scales"], ref["scales"]))
    dq_err = np.abs(dg - dr).max(axis=-1)
    okd = dq_err <= step * 1.0000001 + 2.0 * ext
    assert okd.all(), f"{int((~okd).sum())} blocks with dequantized values more than one block step apart"
    stats["dequant_max_steps"] = float((dq_err / step).max())
    same = diff == 0
    cd = np.abs(ordinal(gpu["codes"]) - ordinal(ref["codes"])).reshape(blk.shape)
    stats["codes_within_1_ordinal_step"] = float((cd[same] <= 1).mean()) if same.any() else 1.0
    if err is not None:
        # per-code rule where the two pre-quant values are closer than one code step
        S = np.ldexp(1.0, ref["scales"].astype(np.int64) - 127)[..., None]
        gb = gpu["f32"].astype(np.float64).reshape(blk.shape)
        close = np.abs(gb - blk) / S < e4m3_step(np.minimum(np.abs(gb), np.abs(blk)) / S)
        sel = close & same[..., None]
        bad = sel & (cd > 1)
        assert not bad.any(), f"{int(bad.sum())} codes more than one step from the oracle's where the pre-quant " \
                              f"values are within one step"
        stats["codes_checked_per_code"] = float(sel.mean())
    return stats


def ordinal(codes):
    c = codes.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def tie_aware_tolerance(inp: dict, *, slack: float = 2.0 ** -12):
    """Extra pre-quant tolerance per (token, head) from the softmax's sensitivity to the
    kernel's score error (E4M3 + UE8M0 pools).

    The kernel computes the scores from q' held as two E4M3 terms with UE8M0 block scales
    (the first at the block's own scale, the second at 2^-4 of it, for the residual), times
    the exact E4M3 rows.  Let delta_j bound |s'_j - s_j| for row j in log2 units: the
    difference between the scores of that two-term q' (rebuilt here from the oracle's fp64
    q' with torch's E4M3 cast) and the exact scores, plus ``slack`` * sum_i |q'_i v_ji| for
    the kernel's f32 evaluation of q' (a rare different rounding of one code).  With
    weights w_j = softmax(s)_j, the perturbed weights satisfy |w'_j - w_j| <= min(1, w_j (2^(2
    delta) - 1)), delta = max_j delta_j, and since the weight changes sum to zero

        |o'_i - o_i| <= sum_j min(1, w_j (2^(2 delta) - 1)) |v_ji - u_i|,   u = sum_j w_j v_j.

    Inverse RoPE mixes element i with its rotary partner, so the bound is taken over both
    (a factor 2 on the per-head maximum).  Where the softmax is one-hot with a clear winner
    the bound is ~0 (the check stays strict); where the top scores are tied within delta it
    admits any mix of the tied rows.  Returns an array [s_q, h]."""
    import math

    s_q, h, d = inp["q"].shape
    c = inp["sm_scale"] / math.log(2.0)
    L = np.minimum(inp["topk_length"], inp["topk"])
    v_all = oracle.mx_decode(inp["kv_pool"], inp["kv_scales"])
    out = np.zeros((s_q, h))
    w_norm = np.asarray(inp["norm_w"], np.float64)
    for t in range(s_q):
        row = inp["indices"][t, :max(L[t], 0)]
        ids = row[row >= 0]
        if ids.size == 0:
            continue
        v = v_all[ids]                                            # [J, d]
        x = inputs.bf16_values(inp["q"][t]).astype(np.float64)   # [h, d]
        y = np.stack([oracle.rope(r, inp["rope_dim"], float(inp["positions"][t]), inp["theta"])
                      for r in (oracle.rmsnorm(xr, w_norm, inp["eps"]) for xr in x)])
        y2 = y * c                                                # log2 units
        # two-term E4M3 representation of y2 with UE8M0 block scales
        yb = y2.reshape(h, d // 32, 32)
        e1 = oracle.ue8m0_exponent(np.abs(yb).max(-1)).astype(np.int64)
        S1 = np.ldexp(1.0, e1 - 127)[..., None]
        t1 = torch.from_numpy(yb / S1).to(torch.float8_e4m3fn).double().numpy() * S1
        S2 = np.ldexp(1.0, np.maximum(e1 - 4, 0) - 127)[..., None]
        t2 = torch.from_numpy((yb - t1) / S2).to(torch.float8_e4m3fn).double().numpy() * S2
        yq = (t1 + t2).reshape(h, d)
        s_exact = y2 @ v.T                                        # [h, J]
        delta = np.abs(yq @ v.T - s_exact) + slack * (np.abs(y2) @ np.abs(v).T)
        dmax = delta.max(axis=1)
        # |w'_j - w_j| <= min(1, w_j (2^(2 delta) - 1)), evaluated in log2 so that huge
        # scores (one-hot weights, huge delta) give 0 * inf nowhere
        lw = s_exact - s_exact.max(axis=1, keepdims=True)
        lw -= np.log2(np.exp2(lw).sum(axis=1, keepdims=True))
        x2 = 2.0 * dmax * math.log(2.0)
        with np.errstate(divide="ignore"):  # delta = 0 gives -inf: no weight moves
            lf = np.where(x2 < 600.0, np.log2(np.expm1(np.minimum(x2, 600.0))), 2.0 * dmax)
        dw = np.minimum(1.0, np.exp2(np.minimum(lw + lf[:, None], 0.0)))
        wgt = np.exp2(lw)
        u = wgt @ v                                               # [h, d]
        spread = np.stack([(dw[k][:, None] * np.abs(v - u[k][None, :])).sum(0).max() for k in range(h)])
        out[t] = 2.0 * spread
    return out
