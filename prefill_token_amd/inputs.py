"""Seeded synthetic inputs for the sparse-MLA step (shared by the tests, the oracle and the bench).

This module holds no arithmetic of the step itself: it only draws random numbers and
lays them out.  The KV pool producer (the KV-insert step, which sits before the path)
is stood in for by the OCP MX v1.0 scale rule -- X = 2^(floor(log2 amax) - 8), E4M3
elements saturated to +-448 -- with the E4M3 and bf16 roundings done by torch's
library casts.  Neither the oracle nor the GPU library imports anything from here
except through the arrays it returns.

Workloads (shapes and distributions from the pages' kernel benchmark,
[vLLM #56344 "Deepseek V41 Attention MegaKernel", Performance]: h_q = 64, topk 128
SWA + 512 compressed, fp8_ds_mla KV rows of 512 E4M3 bytes + UE8M0 scales):

  index  name             s_q   pools (SWA + compressed)     row
  0      tiny             4     bf16 [256, 128]              48 distinct ids, 10 % -> -1
  1      decode_sq1       1     8192 + 2048  fp8             128 SWA before pos + 512 comp, 10 % -> -1
  2      decode_sq64      64    8192 + 2048  fp8             as decode_sq1
  3      decode_sq1024    1024  65536 + 16384 fp8            as decode_sq1, L ~ U[64, 640], tail -> -1
  4      prefill_sq2123   2123  8192 + 16384 fp8             causal 128 window incl. pos + 512 comp
  5      decode_sq256     256   8192 + 2048  fp8             as decode_sq1 (the pages' s_q = 256 row)
  6      prefill_sq184    184   8192 + 16384 fp8             as prefill_sq2123 (the pages' 184 row)

Generation order per workload (numpy PCG64, seed 20260000 + index): positions, norm_w,
q, pool latents, then per token the index row (compressed ids drawn without
replacement, then the sentinel mask), then topk_length.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

KV_E4M3_UE8M0 = 0
KV_BF16 = 1
KV_DS_NVFP4 = 2  # two pools: E4M3 + UE8M0 SWA rows, NVFP4 (E2M1 + E4M3 per 16) compressed rows

SEED_BASE = 20260000


@dataclass
class Workload:
    name: str
    index: int
    s_q: int
    h: int
    d: int
    rope_dim: int
    topk: int
    n_swa: int
    n_comp: int
    kv_format: int
    kind: str  # "tiny", "decode", "decode_ragged", "prefill"
    sentinel_p: float
    description: str

    @property
    def n_rows(self) -> int:
        return self.n_swa + self.n_comp


WORKLOADS: List[Workload] = [
    Workload("tiny", 0, 4, 8, 128, 32, 48, 256, 0, KV_BF16, "tiny", 0.1,
             "tiny: s_q=4, h_q=8, d=128 (32 rotary), bf16 pool [256,128], 48 ids/token, 10% -1"),
    Workload("decode_sq1", 1, 1, 64, 512, 64, 640, 8192, 2048, KV_E4M3_UE8M0, "decode", 0.1,
             "decode s_q=1, h_q=64, d=512 (64 rotary), topk 128 SWA + 512 compressed, fp8 pools 8192+2048"),
    Workload("decode_sq64", 2, 64, 64, 512, 64, 640, 8192, 2048, KV_E4M3_UE8M0, "decode", 0.1,
             "decode s_q=64, h_q=64, d=512 (64 rotary), topk 128 SWA + 512 compressed, fp8 pools 8192+2048"),
    Workload("decode_sq1024", 3, 1024, 64, 512, 64, 640, 65536, 16384, KV_E4M3_UE8M0, "decode_ragged", 0.0,
             "decode s_q=1024, h_q=64, d=512 (64 rotary), topk_length ~ U[64,640], fp8 pools 65536+16384"),
    Workload("prefill_sq2123", 4, 2123, 64, 512, 64, 640, 8192, 16384, KV_E4M3_UE8M0, "prefill", 0.0,
             "prefill s_q=2123 contiguous positions, h_q=64, d=512 (64 rotary), topk 640, fp8 pools 8192+16384"),
    Workload("decode_sq256", 5, 256, 64, 512, 64, 640, 8192, 2048, KV_E4M3_UE8M0, "decode", 0.1,
             "decode s_q=256, h_q=64, d=512 (64 rotary), topk 128 SWA + 512 compressed, fp8 pools 8192+2048"),
    Workload("prefill_sq184", 6, 184, 64, 512, 64, 640, 8192, 16384, KV_E4M3_UE8M0, "prefill", 0.0,
             "prefill s_q=184 contiguous positions, h_q=64, d=512 (64 rotary), topk 640, fp8 pools 8192+16384"),
]
BY_NAME: Dict[str, Workload] = {w.name: w for w in WORKLOADS}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (torch's RNE cast) and return the bit patterns (u16)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (a reinterpretation, exact)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def mx_pool(latents: np.ndarray):
    """Stand-in KV producer: OCP MX scale per 32-block, E4M3 codes by torch's cast.

    Returns ``(codes u8 [n, d], scales u8 [n, d/32])``.
    """
    n, d = latents.shape
    blocks = latents.reshape(n, d // 32, 32).astype(np.float32)
    amax = np.abs(blocks).max(axis=2)
    _, k = np.frexp(amax)  # amax = f * 2^k, f in [0.5, 1)
    X = np.where(amax > 0, k - 1 - 8, -127).astype(np.int32)
    X = np.clip(X, -127, 127)
    scaled = blocks / np.exp2(X.astype(np.float32))[..., None]
    scaled = np.clip(scaled, -448.0, 448.0)
    codes = torch.from_numpy(np.ascontiguousarray(scaled.reshape(n, d))).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).numpy().copy(), (X + 127).astype(np.uint8)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def nvfp4_pool(latents: np.ndarray):
    """Stand-in producer of NVFP4 rows: per 16 elements an E4M3 scale amax / 6 (torch's RNE
    cast), E2M1 codes round-to-nearest-even of x / scale on the grid 0 .. 6 (clipped at 6),
    element 2i in the low nibble of byte i.  Returns ``(codes u8 [n, d/2], scales u8 [n, d/16])``."""
    n, d = latents.shape
    blk = latents.reshape(n, d // 16, 16).astype(np.float64)
    amax = np.abs(blk).max(axis=2)
    sc = torch.from_numpy(amax / 6.0).to(torch.float8_e4m3fn)
    sc_codes = sc.view(torch.uint8).numpy().copy()
    sv = sc.double().numpy()
    x = np.where(sv[..., None] > 0, np.abs(blk) / np.where(sv > 0, sv, 1.0)[..., None], 0.0)
    x = np.minimum(x, 6.0)
    dist = np.abs(x[..., None] - E2M1_GRID)
    mag = np.argmin(dist, axis=-1)  # the lower code on a tie ...
    tie = np.isclose(np.take_along_axis(dist, np.minimum(mag + 1, 7)[..., None], -1)[..., 0],
                     np.take_along_axis(dist, mag[..., None], -1)[..., 0], rtol=0, atol=0) & (mag < 7)
    mag = np.where(tie & (mag % 2 == 1), mag + 1, mag)  # ... unless it is odd: ties to even
    code = (mag | np.where(blk < 0, 8, 0)).astype(np.uint8).reshape(n, d)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc_codes.reshape(n, d // 16)


def make_ds_nvfp4(name: str = "decode_sq64", seed: Optional[int] = None, s_q: Optional[int] = None) -> dict:
    """A workload over the two-pool nvfp4_ds_mla cache: the recipe of workload ``name``
    (positions, q, norm_w, window and compressed entries, sentinels, lengths) with the
    compressed rows in an NVFP4 pool of their own (``nvfp4_pool`` of N(0, 1) latents) and
    index entries 128 .. 639 naming rows of that pool (0 .. n_comp - 1) instead of rows
    n_swa + c of one concatenated pool.  Seed 20265000 + the workload's index unless
    ``seed`` is given."""
    w = BY_NAME[name]
    base = make(name, seed=(SEED_BASE + 5000 + w.index) if seed is None else seed, s_q=s_q)
    rng = np.random.Generator(np.random.PCG64((SEED_BASE + 5500 + w.index) if seed is None else seed + 1))
    lat = rng.standard_normal(size=(w.n_comp, w.d), dtype=np.float32)
    cmp_codes, cmp_scales = nvfp4_pool(lat)
    idx = base["indices"].copy()
    seg = idx[:, 128:]
    idx[:, 128:] = np.where(seg >= 0, seg - w.n_swa, -1)
    out = dict(base)
    out.update(name=name + "_nvfp4", description=base["description"] + ", compressed rows NVFP4 (288 B)",
               kv_format=KV_DS_NVFP4, swa_codes=base["kv_pool"][:w.n_swa].copy(),
               swa_scales=base["kv_scales"][:w.n_swa].copy(), cmp_codes=cmp_codes, cmp_scales=cmp_scales,
               indices=idx, swa_entries=128, n_swa_rows=w.n_swa, n_cmp_rows=w.n_comp)
    for k in ("kv_pool", "kv_scales"):
        out.pop(k)
    return out


def _rng(index: int, seed: Optional[int]) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(SEED_BASE + index if seed is None else seed))


def make(workload, seed: Optional[int] = None, s_q: Optional[int] = None) -> dict:
    """Build the arrays of one workload.

    ``workload`` is a name or an index; ``seed`` overrides the default seed; ``s_q``
    overrides the token count (same recipe, fewer or more tokens).
    """
    w = BY_NAME[workload] if isinstance(workload, str) else WORKLOADS[workload]
    rng = _rng(w.index, seed)
    S = w.s_q if s_q is None else int(s_q)
    h, d = w.h, w.d

    # positions
    if w.kind == "prefill":
        off = int(rng.integers(0, 30000))
        positions = (off + np.arange(S)).astype(np.int32)
    else:
        positions = rng.integers(0, 32768, size=S).astype(np.int32)
    # norm weight ~ N(1, 0.1), held in fp32 at bf16-representable values
    norm_w = bf16_values(bf16_bits(rng.normal(1.0, 0.1, size=d).astype(np.float32)))
    # queries ~ N(0, 1) in bf16
    q = bf16_bits(rng.standard_normal(size=(S, h, d), dtype=np.float32))
    # pool
    if w.kv_format == KV_BF16:
        kv_pool = bf16_bits(rng.standard_normal(size=(w.n_rows, d), dtype=np.float32))
        kv_scales = None
    else:
        lat = rng.standard_normal(size=(w.n_rows, d), dtype=np.float32)
        kv_pool, kv_scales = mx_pool(lat)
        del lat
    # index rows
    topk = w.topk
    indices = np.full((S, topk), -1, dtype=np.int32)
    if w.kind == "tiny":
        for t in range(S):
            indices[t] = rng.choice(w.n_rows, size=topk, replace=False)
        mask = rng.random(size=(S, topk)) < w.sentinel_p
        indices[mask] = -1
        topk_length = np.full(S, topk, dtype=np.int32)
    else:
        n_win = 128
        n_cmp = topk - n_win
        if w.kind == "prefill":
            win = positions[:, None] - (n_win - 1) + np.arange(n_win)[None, :]  # p-127 .. p
        else:
            win = positions[:, None] - n_win + np.arange(n_win)[None, :]  # p-128 .. p-1
        indices[:, :n_win] = np.where(win >= 0, np.mod(win, w.n_swa), -1)
        for t in range(S):
            indices[t, n_win:] = w.n_swa + rng.choice(w.n_comp, size=n_cmp, replace=False)
        if w.sentinel_p > 0:
            mask = rng.random(size=(S, topk)) < w.sentinel_p
            indices[mask] = -1
        if w.kind == "decode_ragged":
            topk_length = rng.integers(64, topk + 1, size=S).astype(np.int32)
            cols = np.arange(topk)[None, :]
            indices[cols >= topk_length[:, None]] = -1
        else:
            topk_length = np.full(S, topk, dtype=np.int32)
    return dict(
        name=w.name, description=w.description, s_q=S, h=h, d=d, rope_dim=w.rope_dim, topk=topk,
        n_rows=w.n_rows, n_swa=w.n_swa, kv_format=w.kv_format,
        sm_scale=1.0 / math.sqrt(d), eps=1e-6, theta=10000.0,
        q=q, kv_pool=kv_pool, kv_scales=kv_scales, indices=indices,
        topk_length=topk_length, positions=positions, norm_w=norm_w.astype(np.float32),
    )


# KV insert workloads (the pool-row producer before the step): the tokens of the
# decode / prefill workloads above, written into pools of the same sizes.
#   name                    n     pools (SWA + compressed)   positions
INSERT_WORKLOADS = {
    "insert_decode_sq1": (1, 8192, 2048, "decode"),
    "insert_decode_sq64": (64, 8192, 2048, "decode"),
    "insert_prefill_sq2123": (2123, 8192, 16384, "prefill"),
}


def make_insert(name: str, seed: Optional[int] = None, n: Optional[int] = None) -> dict:
    """Inputs of one KV-insert workload: kv latents ~ N(0, 1) in bf16, a norm weight
    ~ N(1, 0.1), positions (decode: uniform in [0, 32768) on distinct window rows;
    prefill: contiguous from a random offset below 30000), and a pool of random bytes
    (its rows are only overwritten, never decoded).  Seed 20261000 + the workload's
    position in ``INSERT_WORKLOADS`` unless ``seed`` is given."""
    names = list(INSERT_WORKLOADS)
    n0, n_swa, n_comp, kind = INSERT_WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + 1000 + names.index(name) if seed is None else seed))
    N = n0 if n is None else int(n)
    d = 512
    if kind == "prefill":
        positions = (int(rng.integers(0, 30000)) + np.arange(N)).astype(np.int32)
    else:
        rows = rng.choice(n_swa, size=N, replace=False)
        positions = (rows + n_swa * rng.integers(0, 32768 // n_swa, size=N)).astype(np.int32)
    norm_w = bf16_values(bf16_bits(rng.normal(1.0, 0.1, size=d).astype(np.float32)))
    kv = bf16_bits(rng.standard_normal(size=(N, d), dtype=np.float32))
    pool = rng.integers(0, 256, size=(n_swa + n_comp, d), dtype=np.uint8)
    scales = rng.integers(100, 140, size=(n_swa + n_comp, d // 32), dtype=np.uint8)
    return dict(name=name, n=N, d=d, rope_dim=64, n_swa=n_swa, n_rows=n_swa + n_comp,
                eps=1e-6, theta=10000.0, kv=kv, positions=positions, norm_w=norm_w.astype(np.float32),
                kv_pool=pool, kv_scales=scales)


# Index-row builder workloads: the positions of the attention workloads above, one row of
# candidate logits per token over the compressed pool (2048 or 16384 rows), keep 512.
#   name                  n     candidates   window / self   valid candidates
INDEX_WORKLOADS = {
    "index_decode_sq1": (1, 2048, "decode"),
    "index_decode_sq64": (64, 2048, "decode"),
    "index_decode_sq1024": (1024, 16384, "decode_ragged"),
    "index_prefill_sq2123": (2123, 16384, "prefill"),
}


def make_index(name: str, seed: Optional[int] = None, n: Optional[int] = None) -> dict:
    """Inputs of one index-row-builder workload.  Logits are N(0, 1) rounded to multiples
    of 1/8 in bf16 (few distinct values, as indexer logits have, so the k-th value is
    usually tied).  Valid candidates: all (decode), uniform in [256, n_cand]
    (decode_ragged), one per 4 positions up to the token (prefill, a compression ratio of
    4).  Window 128 rows before the token (decode) or ending at it (prefill), 8192-row
    ring, compressed rows after it.  Seed 20262000 + the workload's position."""
    names = list(INDEX_WORKLOADS)
    n0, n_cand, kind = INDEX_WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + 2000 + names.index(name) if seed is None else seed))
    N = n0 if n is None else int(n)
    if kind == "prefill":
        positions = (int(rng.integers(0, 30000)) + np.arange(N)).astype(np.int32)
    else:
        positions = rng.integers(0, 32768, size=N).astype(np.int32)
    logits = bf16_bits((np.round(rng.standard_normal((N, n_cand)) * 8) / 8).astype(np.float32))
    if kind == "prefill":
        n_valid = np.minimum((positions.astype(np.int64) + 1) // 4, n_cand).astype(np.int32)
    elif kind == "decode_ragged":
        n_valid = rng.integers(256, n_cand + 1, size=N).astype(np.int32)
    else:
        n_valid = np.full(N, n_cand, dtype=np.int32)
    return dict(name=name, n=N, n_cand=n_cand, positions=positions, logits=logits, n_valid=n_valid, topk=640,
                window=128, self_in_window=kind == "prefill", n_swa=8192, cmp_base=8192, k_cmp=512)


# Output-projection (wo_a) workloads: the attention output of the decode / prefill token
# counts in its E4M3 + UE8M0 form, projected per head (one head per group) to 128 outputs.
#   name                  tokens  heads  heads per group  outputs per group
WO_A_WORKLOADS = {
    "wo_a_decode_sq1": (1, 64, 1, 128),
    "wo_a_decode_sq64": (64, 64, 1, 128),
    "wo_a_prefill_sq2123": (2123, 64, 1, 128),
}


def make_wo_a(name: str, seed: Optional[int] = None, n: Optional[int] = None, heads_per_group: Optional[int] = None,
              d_out: Optional[int] = None) -> dict:
    """Inputs of one wo_a workload: the attention output ~ N(0, 0.05) (the spread of a
    softmax-weighted mean of N(0, 1) rows) and the weight ~ N(0, 1 / sqrt(hg * 512)), both
    as E4M3 codes with one UE8M0 scale per 32 values (the generator's MX rule,
    ``mx_pool``).  Seed 20263000 + the workload's position unless ``seed`` is given."""
    names = list(WO_A_WORKLOADS)
    n0, h, hg0, dout0 = WO_A_WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + 3000 + names.index(name) if seed is None else seed))
    N = n0 if n is None else int(n)
    hg = hg0 if heads_per_group is None else int(heads_per_group)
    dout = dout0 if d_out is None else int(d_out)
    d = 512
    G = h // hg
    x, xs = mx_pool((rng.standard_normal((N * h, d), dtype=np.float32) * np.float32(0.05)))
    w, ws = mx_pool(rng.standard_normal((G * dout, hg * d), dtype=np.float32) / np.float32(np.sqrt(hg * d)))
    return dict(name=name, n=N, h=h, d=d, heads_per_group=hg, d_out=dout,
                x=x.reshape(N, h, d), x_scales=xs.reshape(N, h, d // 32),
                w=w.reshape(G, dout, hg * d), w_scales=ws.reshape(G, dout, hg * d // 32))


def take_tokens(inp: dict, tokens) -> dict:
    """The same inputs restricted to a subset of tokens (the pool is shared)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    out = dict(inp)
    for k in ("q", "indices", "topk_length", "positions"):
        out[k] = np.ascontiguousarray(inp[k][tokens])
    out["s_q"] = int(tokens.size)
    return out


def valid_rows(inp: dict) -> np.ndarray:
    """Number of entries each token actually reads (j < topk_length and id >= 0)."""
    L = np.minimum(inp["topk_length"], inp["topk"])
    cols = np.arange(inp["topk"])[None, :]
    return ((cols < L[:, None]) & (inp["indices"] >= 0)).sum(axis=1)
