"""fp64 CPU oracle of the fused sparse-MLA attention step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product library never does, and the two share no code:
this wrapper loads ``liboracle.so`` built from ``sparse_mla_oracle.c`` by plain gcc.

The functions mirror the steps of the C file (each cites its passage there):
``bf16_decode``, ``e4m3_decode``, ``e4m3_encode``, ``ue8m0_exponent``,
``quantize_blocks``, ``rmsnorm``, ``rope``, the whole step ``sparse_mla`` (and over the
two-pool nvfp4_ds_mla cache, ``sparse_mla_ds_nvfp4`` with ``e2m1_decode`` /
``nvfp4_decode``), and the two
steps before it: the pool-row producer ``kv_insert`` and the index-row builder
``build_index`` (plain numpy, below), and the step after it, the output projection
``wo_a`` (plain numpy).

Parity pins: every function here is checked in ``tests/test_oracle_*.py`` against
library routines (torch's CPU float8_e4m3fn cast, torch SDPA and rms_norm in fp64,
the rotate-half routine of ``transformers``), closed forms and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sparse_mla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

KV_E4M3_UE8M0 = 0
KV_BF16 = 1


def build(verbose: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (fp64, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-fno-fast-math",
           "-ffp-contract=off", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    lib.oracle_bf16_decode.restype = ctypes.c_double
    lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_ue8m0_exponent.restype = ctypes.c_int
    lib.oracle_ue8m0_exponent.argtypes = [ctypes.c_double]
    lib.oracle_quantize_blocks.restype = None
    lib.oracle_quantize_blocks.argtypes = [P, ctypes.c_int64, P, P]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_rmsnorm.argtypes = [P, P, ctypes.c_int, ctypes.c_double, P]
    lib.oracle_rope.restype = None
    lib.oracle_rope.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_int]
    lib.oracle_sparse_mla.restype = ctypes.c_int
    lib.oracle_sparse_mla.argtypes = [P, P, P, P, P, P, P,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                      ctypes.c_double, P, P, P]
    lib.oracle_kv_insert.restype = ctypes.c_int
    lib.oracle_kv_insert.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int64, ctypes.c_double, ctypes.c_double, P, P]
    lib.oracle_e2m1_decode.restype = ctypes.c_double
    lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_sparse_mla_ds_nvfp4.restype = ctypes.c_int
    lib.oracle_sparse_mla_ds_nvfp4.argtypes = [P, P, P, P, P, P, P, P, P,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                               ctypes.c_double, ctypes.c_double, P, P, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def bf16_decode(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.oracle_bf16_decode(int(x)) for x in b.ravel()], dtype=np.float64).reshape(b.shape)


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e4m3_decode(int(x)) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3_encode(x) -> np.ndarray:
    lib = _load()
    v = np.asarray(x, dtype=np.float64)
    return np.array([lib.oracle_e4m3_encode(float(z)) for z in v.ravel()], dtype=np.uint8).reshape(v.shape)


def e2m1_decode(codes) -> np.ndarray:
    """OCP E2M1 (FP4) codes (low 4 bits) -> exact fp64 values."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e2m1_decode(int(x)) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def nvfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Rows of the NVFP4 pool decoded exactly: ``codes`` u8 [..., d/2] (element 2i in the low
    nibble of byte i), ``scales`` u8 [..., d/16] E4M3: value = e2m1(code) * e4m3(scale)."""
    c = np.asarray(codes, dtype=np.uint8)
    nib = np.stack([c & 15, c >> 4], axis=-1).reshape(*c.shape[:-1], 2 * c.shape[-1])
    lut = e2m1_decode(np.arange(16, dtype=np.uint8))
    sc = e4m3_decode(np.asarray(scales, dtype=np.uint8))
    return lut[nib] * np.repeat(sc, 16, axis=-1)


def ue8m0_exponent(amax) -> np.ndarray:
    lib = _load()
    v = np.asarray(amax, dtype=np.float64)
    return np.array([lib.oracle_ue8m0_exponent(float(z)) for z in v.ravel()], dtype=np.int32).reshape(v.shape)


def quantize_blocks(o: np.ndarray):
    """Block-32 UE8M0 + E4M3 quantization of ``o`` (last dim a multiple of 32).

    Returns ``(codes u8 like o, scales u8 [..., d/32])``.
    """
    lib = _load()
    o = np.ascontiguousarray(o, dtype=np.float64)
    assert o.shape[-1] % 32 == 0
    codes = np.empty(o.shape, dtype=np.uint8)
    scales = np.empty(o.shape[:-1] + (o.shape[-1] // 32,), dtype=np.uint8)
    lib.oracle_quantize_blocks(_ptr(o), o.size, _ptr(codes), _ptr(scales))
    return codes, scales


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    y = np.empty_like(x)
    lib.oracle_rmsnorm(_ptr(x), _ptr(w), x.shape[-1], float(eps), _ptr(y))
    return y


def rope(y: np.ndarray, rope_dim: int, pos: float, theta: float, direction: int = 1) -> np.ndarray:
    """Rotate-half RoPE on the last ``rope_dim`` entries of a 1-D vector (copy)."""
    lib = _load()
    out = np.ascontiguousarray(y, dtype=np.float64).copy()
    lib.oracle_rope(_ptr(out), out.shape[-1], int(rope_dim), float(pos), float(theta), int(direction))
    return out


def sparse_mla(q_bits: np.ndarray, kv_pool: np.ndarray, kv_scales: Optional[np.ndarray],
               indices: np.ndarray, topk_length: np.ndarray, positions: np.ndarray,
               norm_w: np.ndarray, *, sm_scale: float, eps: float, theta: float, rope_dim: int,
               kv_format: int = KV_E4M3_UE8M0):
    """The whole step for ``s_q`` tokens.

    ``q_bits`` u16 [s_q, h, d] (bf16 bits); ``kv_pool`` u8 [n, d] (E4M3 codes) or u16
    [n, d] (bf16 bits); ``kv_scales`` u8 [n, d/32] or None; ``indices`` i32 [s_q, topk];
    ``topk_length`` / ``positions`` i32 [s_q]; ``norm_w`` [d].

    Returns ``(o f64 [s_q, h, d], codes u8 [s_q, h, d], scales u8 [s_q, h, d/32])``.
    Raises ``ValueError`` on an argument or index error.
    """
    lib = _load()
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    s_q, h, d = q_bits.shape
    kv_pool = np.ascontiguousarray(kv_pool)
    n_rows = kv_pool.shape[0]
    if kv_format == KV_E4M3_UE8M0:
        assert kv_pool.dtype == np.uint8
        kv_scales = np.ascontiguousarray(kv_scales, dtype=np.uint8)
    else:
        assert kv_pool.dtype == np.uint16
        kv_scales = None
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    topk = indices.shape[1] if indices.ndim == 2 else 0
    topk_length = np.ascontiguousarray(topk_length, dtype=np.int32)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    norm_w = np.ascontiguousarray(norm_w, dtype=np.float64)
    o = np.zeros((s_q, h, d), dtype=np.float64)
    codes = np.zeros((s_q, h, d), dtype=np.uint8)
    scales = np.zeros((s_q, h, d // 32), dtype=np.uint8)
    rc = lib.oracle_sparse_mla(_ptr(q_bits), _ptr(kv_pool), _ptr(kv_scales), _ptr(indices),
                               _ptr(topk_length), _ptr(positions), _ptr(norm_w),
                               s_q, h, d, int(rope_dim), topk, n_rows, int(kv_format),
                               float(sm_scale), float(eps), float(theta),
                               _ptr(o), _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_sparse_mla failed with code {rc}")
    return o, codes, scales


def sparse_mla_ds_nvfp4(q_bits: np.ndarray, swa_codes: np.ndarray, swa_scales: np.ndarray, cmp_codes: np.ndarray,
                        cmp_scales: np.ndarray, indices: np.ndarray, topk_length: np.ndarray,
                        positions: np.ndarray, norm_w: np.ndarray, *, swa_entries: int, sm_scale: float,
                        eps: float, theta: float, rope_dim: int):
    """The step over the two-pool nvfp4_ds_mla cache: entries j < ``swa_entries`` of each index
    row name rows of the E4M3 + UE8M0 pool (``swa_codes`` u8 [n_swa, d], ``swa_scales`` u8
    [n_swa, d/32]), the later entries rows of the NVFP4 pool (``cmp_codes`` u8 [n_cmp, d/2],
    ``cmp_scales`` u8 [n_cmp, d/16]).  Returns ``(o, codes, scales)`` as ``sparse_mla``."""
    lib = _load()
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    s_q, h, d = q_bits.shape
    sw = np.ascontiguousarray(swa_codes, dtype=np.uint8)
    ss = np.ascontiguousarray(swa_scales, dtype=np.uint8)
    cc = np.ascontiguousarray(cmp_codes, dtype=np.uint8)
    cs = np.ascontiguousarray(cmp_scales, dtype=np.uint8)
    assert sw.shape[1] == d and ss.shape == (sw.shape[0], d // 32)
    assert cc.shape[1] == d // 2 and cs.shape == (cc.shape[0], d // 16)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    topk = indices.shape[1] if indices.ndim == 2 else 0
    topk_length = np.ascontiguousarray(topk_length, dtype=np.int32)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    norm_w = np.ascontiguousarray(norm_w, dtype=np.float64)
    o = np.zeros((s_q, h, d), dtype=np.float64)
    codes = np.zeros((s_q, h, d), dtype=np.uint8)
    scales = np.zeros((s_q, h, d // 32), dtype=np.uint8)
    rc = lib.oracle_sparse_mla_ds_nvfp4(_ptr(q_bits), _ptr(sw), _ptr(ss), _ptr(cc), _ptr(cs), _ptr(indices),
                                        _ptr(topk_length), _ptr(positions), _ptr(norm_w), s_q, h, d,
                                        int(rope_dim), topk, int(swa_entries), sw.shape[0], cc.shape[0],
                                        float(sm_scale), float(eps), float(theta), _ptr(o), _ptr(codes),
                                        _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_sparse_mla_ds_nvfp4 failed with code {rc}")
    return o, codes, scales


def kv_insert(kv_bits: np.ndarray, positions: np.ndarray, norm_w: np.ndarray, kv_pool: np.ndarray,
              kv_scales: np.ndarray, *, n_swa: int, eps: float, theta: float, rope_dim: int):
    """KV insert into copies of the pool: rows ``positions mod n_swa`` get the E4M3 codes and
    UE8M0 exponents of RoPE(RMSNorm(kv)); negative positions are skipped.

    ``kv_bits`` u16 [n, d]; ``kv_pool`` u8 [n_rows, d]; ``kv_scales`` u8 [n_rows, d/32].
    Returns ``(kv_pool, kv_scales)`` (new arrays).  Raises ``ValueError`` on bad arguments.
    """
    lib = _load()
    kv_bits = np.ascontiguousarray(kv_bits, dtype=np.uint16)
    n, d = kv_bits.shape
    pool = np.ascontiguousarray(kv_pool, dtype=np.uint8).copy()
    sc = np.ascontiguousarray(kv_scales, dtype=np.uint8).copy()
    assert pool.shape[1] == d and sc.shape == (pool.shape[0], d // 32)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    norm_w = np.ascontiguousarray(norm_w, dtype=np.float64)
    rc = lib.oracle_kv_insert(_ptr(kv_bits), _ptr(positions), _ptr(norm_w), n, d, int(rope_dim), int(n_swa),
                              pool.shape[0], float(eps), float(theta), _ptr(pool), _ptr(sc))
    if rc != 0:
        raise ValueError(f"oracle_kv_insert failed with code {rc}")
    return pool, sc


def mx_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E4M3 codes with one UE8M0 exponent per 32 consecutive values along the last axis,
    decoded exactly to fp64: ``e4m3(code) * 2^(scale - 127)``."""
    v = e4m3_decode(codes)
    sc = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    return v * np.repeat(sc, 32, axis=-1)


def wo_a(x_codes: np.ndarray, x_scales: np.ndarray, w_codes: np.ndarray, w_scales: np.ndarray,
         heads_per_group: int = 1) -> np.ndarray:
    """The consumer of the step's FP8 output: the per-group output projection (wo_a), fp64.

    [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose: the kernel's FP8 output is
    fed straight into the wo_a einsum.]  The pages give no shape; the reading: the heads
    are taken hg = heads_per_group at a time, and group g's hg * 512 dims are contracted
    with its own weight [d_out][hg * 512]:

        y[t, g, o] = sum_k x[t, g, k] * W[g, o, k],   x[t, g, h * 512 + i] = out[t, g * hg + h, i]

    with x and W decoded exactly (``mx_decode``).  The contraction is numpy's einsum.
    """
    s, h, d = x_codes.shape
    hg = int(heads_per_group)
    G = h // hg
    x = mx_decode(x_codes, x_scales).reshape(s, G, hg * d)
    W = mx_decode(w_codes, w_scales)
    return np.einsum("tgk,gok->tgo", x, W)


def select_topk(logits_bits: np.ndarray, k: int) -> np.ndarray:
    """Columns of the k largest logits of one row, ascending.

    The rule the pages give for their top-k kernel [vLLM #64364 "latency_specialized
    decode", Validation: torch.topk's k-th value, the selected columns in ascending order,
    ties toward the lowest column]: order by value (bf16 bits; NaN above every number, as
    torch orders it; -0 equal to +0), break ties by the lower column, keep the first k,
    return them sorted by column.  k larger than the row keeps the whole row.
    """
    bits = np.asarray(logits_bits, dtype=np.uint16)
    n = bits.size
    k = min(int(k), n)
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    v = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(v)
    v = np.where(nan, 0.0, v)
    cols = np.arange(n)
    # np.lexsort sorts by the last key first: NaN first, then larger values, then lower columns
    order = np.lexsort((cols, -v, -nan.astype(np.int64)))
    return np.sort(order[:k])


def build_index(positions: np.ndarray, logits_bits: np.ndarray, n_valid, *, topk: int, window: int,
                self_in_window: bool, n_swa: int, cmp_base: int, k_cmp: int):
    """Index rows of the step, the step before it [vLLM #56344 "Deepseek V41 Attention
    MegaKernel", Purpose: combine_topk_swa_indices builds each token's row of SWA and
    compressed-cache indices and writes its own -1 sentinels].

    Row t: entries 0 .. window-1 are the sliding-window rows of positions
    p - window + s .. p - 1 + s (s = 1 when the token's own row is in its window), each
    ``pos mod n_swa`` or -1 for a negative position; the next k_cmp entries are
    ``cmp_base + c`` for the columns c chosen by ``select_topk`` among the token's first
    ``n_valid[t]`` candidate logits, ascending, then -1 where fewer were chosen; every
    later entry is -1.  ``topk_length[t]`` = window + the number chosen.

    Returns ``(indices i32 [s_q, topk], topk_length i32 [s_q])``.
    """
    positions = np.asarray(positions, dtype=np.int64)
    logits_bits = np.asarray(logits_bits, dtype=np.uint16)
    s_q, n_cand = logits_bits.shape
    nv = np.full(s_q, n_cand, dtype=np.int64) if n_valid is None else np.clip(np.asarray(n_valid, np.int64), 0, n_cand)
    assert window + k_cmp <= topk and window <= n_swa
    idx = np.full((s_q, topk), -1, dtype=np.int32)
    L = np.zeros(s_q, dtype=np.int32)
    s = 1 if self_in_window else 0
    for t in range(s_q):
        p = int(positions[t])
        for j in range(window):
            q = p - window + s + j
            idx[t, j] = q % n_swa if q >= 0 else -1
        sel = select_topk(logits_bits[t, :nv[t]], k_cmp)
        idx[t, window:window + sel.size] = cmp_base + sel
        L[t] = window + sel.size
    return idx, L
