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


def compare(gpu: dict, ref: dict, *, check_f32: bool = True):
    """Assert the comparison rules; return a stats dict."""
    o = ref["o"]
    d = o.shape[-1]
    blk = o.reshape(*o.shape[:-1], d // 32, 32)
    a_ref = np.abs(blk).max(axis=-1)
    stats = {}
    if check_f32 and gpu.get("f32") is not None:
        g = gpu["f32"].astype(np.float64)
        gb = g.reshape(blk.shape)
        err = np.abs(gb - blk).max(axis=-1)
        zero = a_ref == 0
        assert (err[zero] == 0).all(), "nonzero output where the oracle's block is all zero"
        rel = np.where(zero, 0.0, err / np.maximum(a_ref, 1e-300))
        stats["prequant_max_rel_block"] = float(rel.max())
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
        band_tol = PREQUANT_TOL * a_ref
    with np.errstate(divide="ignore"):
        k = np.round(np.log2(np.maximum(a_ref, 1e-300) / 448.0))
    near = np.abs(a_ref - 448.0 * np.exp2(k)) <= band_tol * 1.0001 + 1e-300
    ok = (diff == 0) | ((np.abs(diff) == 1) & near)
    assert ok.all(), f"{int((~ok).sum())} blocks with exponents off the fp64 oracle beyond the band rule"
    stats["band_blocks"] = int((diff != 0).sum())
    stats["blocks"] = int(diff.size)
    # dequantized values
    dg = dequant(gpu["codes"], gpu["scales"]).reshape(blk.shape)
    dr = dequant(ref["codes"], ref["scales"]).reshape(blk.shape)
    step = block_step(a_ref, np.maximum(gpu["scales"], ref["scales"]))
    dq_err = np.abs(dg - dr).max(axis=-1)
    okd = dq_err <= step * 1.0000001
    assert okd.all(), f"{int((~okd).sum())} blocks with dequantized values more than one block step apart"
    stats["dequant_max_steps"] = float((dq_err / step).max())
    same = diff == 0
    cd = np.abs(ordinal(gpu["codes"]) - ordinal(ref["codes"])).reshape(blk.shape)
    stats["codes_within_1_ordinal_step"] = float((cd[same] <= 1).mean()) if same.any() else 1.0
    return stats


def ordinal(codes):
    c = codes.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)
