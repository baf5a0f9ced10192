"""MI355X (gfx950) fused sparse-MLA attention step.

The compute runs in ``libsmla.so`` (hand-written HIP kernels behind the C ABI of
``include/smla.h``).  This module only marshals torch tensors (device memory) and the
current HIP stream into that ABI; there is no other implementation to fall back on.

    from prefill_token_amd import sparse_mla_fwd
    sparse_mla_fwd(q, kv_pool, kv_scales, indices, topk_length, positions, norm_w,
                   out_fp8, out_scales, sm_scale=..., rope_dim=64)
"""
from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib
from ._lib import (SMLA_ERR_HIP, SMLA_ERR_NULL, SMLA_ERR_SHAPE, SMLA_ERR_VALUE, SMLA_KV_BF16,
                   SMLA_KV_E4M3_UE8M0, SMLA_OK, LibraryMissing, SmlaDsParams, SmlaIndexParams, SmlaKvInsertParams,
                   SmlaParams, SmlaWoAParams, last_error)

__all__ = [
    "sparse_mla_fwd", "sparse_mla_workspace_size", "sparse_mla_num_splits", "sparse_mla_last_error",
    "sparse_mla_abi_version", "sparse_mla_profile_events", "sparse_mla_fwd_ds_nvfp4", "SmlaDsParams", "sparse_mla_fwd_noalloc", "sparse_mla_noalloc_num_splits", "sparse_mla_kv_insert", "sparse_mla_build_index", "sparse_mla_wo_a", "make_params",
    "make_kv_insert_params", "make_index_params", "SmlaParams", "SmlaKvInsertParams", "SmlaIndexParams", "SmlaError",
    "LibraryMissing",
    "SMLA_OK", "SMLA_ERR_NULL", "SMLA_ERR_SHAPE", "SMLA_ERR_VALUE", "SMLA_ERR_HIP",
    "SMLA_KV_E4M3_UE8M0", "SMLA_KV_BF16",
]


class SmlaError(RuntimeError):
    def __init__(self, code: int, msg: str, fn: str = "sparse_mla_fwd"):
        super().__init__(f"{fn} failed (code {code}): {msg}")
        self.code = code


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


class _Checker:
    """Argument checks of one binding call: dtype, shape, contiguity and device of every
    tensor, before anything reaches the C ABI.  The library itself only sees pointers and
    sizes, so a tensor whose shape disagrees with the others would be read or written out
    of bounds on the device; every such mismatch is a ValueError here instead."""

    def __init__(self, fn: str):
        self.fn = fn
        self.seen = []

    def __call__(self, name, t, dtypes, shape=None, ndim=None, optional=False):
        if t is None:
            if optional:
                return None
            raise ValueError(f"{self.fn}: {name} is required")
        if not hasattr(t, "dtype") or not hasattr(t, "data_ptr"):
            raise ValueError(f"{self.fn}: {name} must be a torch tensor")
        if t.dtype not in dtypes:
            raise ValueError(f"{self.fn}: {name} must have dtype " + " or ".join(str(d) for d in dtypes) +
                             f" (got {t.dtype})")
        if ndim is not None and t.dim() != ndim:
            raise ValueError(f"{self.fn}: {name} must have {ndim} dimensions (got shape {tuple(t.shape)})")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{self.fn}: {name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
        if not t.is_contiguous():
            raise ValueError(f"{self.fn}: {name} must be contiguous")
        self.seen.append((name, t))
        return t

    def done(self):
        """Every tensor checked so far lies on one GPU (checked last, so that the dtype and
        shape rules can be exercised with host tensors)."""
        dev = None
        for name, t in self.seen:
            if t.device.type != "cuda":
                raise ValueError(f"{self.fn}: {name} must be on a GPU (got {t.device})")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{self.fn}: {name} is on {t.device}, other arguments on {dev}")


def _dtypes():
    import torch

    codes = (torch.uint8, torch.float8_e4m3fn)
    return torch, codes


def make_params(*, s_q: int, h_q: int, d: int, rope_dim: int, topk: int, n_rows: int, kv_format: int,
                sm_scale: float, eps: float = 1e-6, theta: float = 1e4, num_splits: int = 0,
                out_f32=None, workspace=None, stream=None) -> SmlaParams:
    p = SmlaParams()
    p.s_q, p.h_q, p.d, p.rope_dim, p.topk, p.kv_format = s_q, h_q, d, rope_dim, topk, kv_format
    p.n_rows = n_rows
    p.sm_scale, p.rms_eps, p.rope_theta = sm_scale, eps, theta
    p.num_splits = num_splits
    p.out_f32 = _ptr(out_f32)
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p.stream = stream
    return p


def sparse_mla_workspace_size(params: SmlaParams) -> int:
    return int(_lib.load().sparse_mla_workspace_size(ctypes.byref(params)))


def sparse_mla_num_splits(params: SmlaParams) -> int:
    return int(_lib.load().sparse_mla_num_splits(ctypes.byref(params)))


def sparse_mla_last_error() -> str:
    return last_error()


def sparse_mla_abi_version() -> int:
    return int(_lib.load().sparse_mla_abi_version())


def sparse_mla_profile_events(before_main=None, after_main=None, after_all=None) -> None:
    """Arm torch.cuda.Event objects (created with enable_timing=True and recorded once, so
    that they exist) to be recorded by this thread's next step call: before its main kernel,
    after it, and after its last kernel."""
    def handle(ev):
        if ev is None:
            return None
        h = int(ev.cuda_event)
        if h == 0:
            raise ValueError("record the event once before arming it (torch creates events lazily)")
        return h
    _lib.load().sparse_mla_profile_events(handle(before_main), handle(after_main), handle(after_all))


def sparse_mla_noalloc_num_splits(params: SmlaParams) -> int:
    return int(_lib.load().sparse_mla_noalloc_num_splits(ctypes.byref(params)))


def _check_fwd(fn, q, kv_pool, kv_scales, indices, topk_length, positions, norm_w, out_fp8, out_scales, out_f32,
               workspace):
    """Checks shared by sparse_mla_fwd and its allocation-free variant; returns
    (s_q, h_q, d, topk, n_rows, kv_format)."""
    torch, codes = _dtypes()
    ck = _Checker(fn)
    ck("q", q, (torch.bfloat16,), ndim=3)
    s_q, h_q, d = q.shape
    ck("kv_pool", kv_pool, (torch.bfloat16,) + codes, ndim=2)
    n_rows = kv_pool.shape[0]
    if kv_pool.shape[1] != d:
        raise ValueError(f"{fn}: kv_pool rows must have d = {d} elements (got {kv_pool.shape[1]})")
    bf16_pool = kv_pool.dtype == torch.bfloat16
    kv_format = SMLA_KV_BF16 if bf16_pool else SMLA_KV_E4M3_UE8M0
    if bf16_pool:
        if kv_scales is not None:
            raise ValueError(f"{fn}: kv_scales must be None for a bf16 pool")
    else:
        if d % 32:
            raise ValueError(f"{fn}: d must be a multiple of 32 (got {d})")
        ck("kv_scales", kv_scales, (torch.uint8,), shape=(n_rows, d // 32))
    ck("indices", indices, (torch.int32,), ndim=2)
    if indices.shape[0] != s_q:
        raise ValueError(f"{fn}: indices must have {s_q} rows (got {indices.shape[0]})")
    topk = indices.shape[1]
    ck("topk_length", topk_length, (torch.int32,), shape=(s_q,))
    ck("positions", positions, (torch.int32,), shape=(s_q,))
    ck("norm_w", norm_w, (torch.float32,), shape=(d,))
    ck("out_fp8", out_fp8, codes, shape=(s_q, h_q, d))
    ck("out_scales", out_scales, (torch.uint8,), shape=(s_q, h_q, d // 32))
    ck("out_f32", out_f32, (torch.float32,), shape=(s_q, h_q, d), optional=True)
    ck("workspace", workspace, (torch.uint8,), ndim=1, optional=True)
    ck.done()
    return s_q, h_q, d, topk, n_rows, kv_format


def sparse_mla_fwd_noalloc(q, kv_pool, kv_scales, indices, topk_length, positions, norm_w, out_fp8, out_scales, *,
                           sm_scale: float, rope_dim: int, eps: float = 1e-6, theta: float = 1e4, out_f32=None,
                           num_splits: int = 0, stream=None) -> None:
    """sparse_mla_fwd without a workspace: the scratch is the library's static device array
    (for callers that cannot allocate, e.g. under graph capture).  Calls that overlap in
    time on one GPU race.  Raises SmlaError on failure."""
    torch, _ = _dtypes()
    s_q, h_q, d, topk, n_rows, kv_format = _check_fwd("sparse_mla_fwd_noalloc", q, kv_pool, kv_scales, indices,
                                                      topk_length, positions, norm_w, out_fp8, out_scales, out_f32,
                                                      None)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    params = make_params(s_q=s_q, h_q=h_q, d=d, rope_dim=rope_dim, topk=topk, n_rows=n_rows,
                         kv_format=kv_format, sm_scale=sm_scale, eps=eps, theta=theta, num_splits=num_splits,
                         out_f32=out_f32, stream=stream)
    rc = _lib.load().sparse_mla_fwd_noalloc(_ptr(q), _ptr(kv_pool), _ptr(kv_scales), _ptr(indices),
                                            _ptr(topk_length), _ptr(positions), _ptr(norm_w), _ptr(out_fp8),
                                            _ptr(out_scales), ctypes.byref(params))
    if rc != SMLA_OK:
        raise SmlaError(rc, last_error(), "sparse_mla_fwd_noalloc")


def sparse_mla_fwd(q, kv_pool, kv_scales, indices, topk_length, positions, norm_w, out_fp8, out_scales, *,
                   sm_scale: float, rope_dim: int, eps: float = 1e-6, theta: float = 1e4, out_f32=None,
                   workspace=None, num_splits: int = 0, stream=None) -> None:
    """Enqueue the fused step on the current (or given) HIP stream.

    q bf16 [s_q, h_q, d]; kv_pool uint8 / float8_e4m3fn [n, d] (E4M3 codes, with
    kv_scales uint8 [n, d/32]) or bf16 [n, d] (kv_scales None); indices / topk_length /
    positions int32; norm_w float32 [d]; out_fp8 uint8 / float8_e4m3fn [s_q, h_q, d];
    out_scales uint8 [s_q, h_q, d/32]; out_f32 optional float32 [s_q, h_q, d].
    ``workspace`` (a uint8 device tensor of at least sparse_mla_workspace_size bytes,
    zero-filled before its first use; each call leaves its scheduler counters zero) is
    allocated here, zero-filled, when none is given.  Calls sharing a workspace must not
    overlap.  Raises SmlaError with the library's message on failure.
    """
    torch, _ = _dtypes()
    s_q, h_q, d, topk, n_rows, kv_format = _check_fwd("sparse_mla_fwd", q, kv_pool, kv_scales, indices, topk_length,
                                                      positions, norm_w, out_fp8, out_scales, out_f32, workspace)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif workspace is None:
        # a workspace allocated here would be zero-filled and freed on torch's current
        # stream, unordered with the kernels enqueued on `stream`
        raise ValueError("sparse_mla_fwd: pass a workspace when enqueuing on an explicit stream")
    params = make_params(s_q=s_q, h_q=h_q, d=d, rope_dim=rope_dim, topk=topk, n_rows=n_rows,
                         kv_format=kv_format, sm_scale=sm_scale, eps=eps, theta=theta, num_splits=num_splits,
                         out_f32=out_f32, workspace=workspace, stream=stream)
    need = sparse_mla_workspace_size(params)
    if need > 0 and workspace is None:
        # its scheduler counters must start at zero (every call leaves them zero); made,
        # used and released on torch's current stream, which the kernels run on
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
        params.workspace = _ptr(workspace)
        params.workspace_bytes = need
    rc = _lib.load().sparse_mla_fwd(_ptr(q), _ptr(kv_pool), _ptr(kv_scales), _ptr(indices), _ptr(topk_length),
                                    _ptr(positions), _ptr(norm_w), _ptr(out_fp8), _ptr(out_scales),
                                    ctypes.byref(params))
    if rc != SMLA_OK:
        raise SmlaError(rc, last_error())


def sparse_mla_fwd_ds_nvfp4(q, swa_pool, swa_scales, cmp_pool, cmp_scales, indices, topk_length, positions, norm_w,
                            out_fp8, out_scales, *, swa_entries: int, sm_scale: float, rope_dim: int,
                            eps: float = 1e-6, theta: float = 1e4, out_f32=None, workspace=None,
                            num_splits: int = 0, stream=None) -> None:
    """Enqueue the step over the two-pool nvfp4_ds_mla cache on the current (or given) stream.

    swa_pool uint8 / float8_e4m3fn [n_swa, 512] + swa_scales uint8 [n_swa, 16] (E4M3 +
    UE8M0); cmp_pool uint8 [n_cmp, 256] (E2M1 pairs, low nibble first) + cmp_scales uint8
    [n_cmp, 32] (E4M3 per 16); index entries j < swa_entries name SWA rows, later entries
    compressed rows.  The rest as sparse_mla_fwd.  Raises SmlaError on failure."""
    torch, _ = _dtypes()
    s_q, h_q, d, topk, n_swa, kv_format = _check_fwd("sparse_mla_fwd_ds_nvfp4", q, swa_pool, swa_scales, indices,
                                                     topk_length, positions, norm_w, out_fp8, out_scales, out_f32,
                                                     workspace)
    if kv_format != SMLA_KV_E4M3_UE8M0:
        raise ValueError("sparse_mla_fwd_ds_nvfp4: the SWA pool must hold E4M3 codes")
    ck = _Checker("sparse_mla_fwd_ds_nvfp4")
    ck("cmp_pool", cmp_pool, (torch.uint8,), ndim=2)
    n_cmp = cmp_pool.shape[0]
    if cmp_pool.shape[1] != d // 2:
        raise ValueError(f"sparse_mla_fwd_ds_nvfp4: cmp_pool rows must have {d // 2} bytes (got {cmp_pool.shape[1]})")
    ck("cmp_scales", cmp_scales, (torch.uint8,), shape=(n_cmp, d // 16))
    ck("q", q, (torch.bfloat16,), ndim=3)
    ck.done()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif workspace is None:
        raise ValueError("sparse_mla_fwd_ds_nvfp4: pass a workspace when enqueuing on an explicit stream")
    dp = SmlaDsParams()
    dp.base = make_params(s_q=s_q, h_q=h_q, d=d, rope_dim=rope_dim, topk=topk, n_rows=n_swa, kv_format=kv_format,
                          sm_scale=sm_scale, eps=eps, theta=theta, num_splits=num_splits, out_f32=out_f32,
                          workspace=workspace, stream=stream)
    dp.n_cmp_rows, dp.swa_entries, dp.reserved = n_cmp, swa_entries, 0
    need = sparse_mla_workspace_size(dp.base)
    if need > 0 and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
        dp.base.workspace = _ptr(workspace)
        dp.base.workspace_bytes = need
    rc = _lib.load().sparse_mla_fwd_ds_nvfp4(_ptr(q), _ptr(swa_pool), _ptr(swa_scales), _ptr(cmp_pool),
                                             _ptr(cmp_scales), _ptr(indices), _ptr(topk_length), _ptr(positions),
                                             _ptr(norm_w), _ptr(out_fp8), _ptr(out_scales), ctypes.byref(dp))
    if rc != SMLA_OK:
        raise SmlaError(rc, last_error(), "sparse_mla_fwd_ds_nvfp4")


def make_kv_insert_params(*, n: int, rope_dim: int, n_swa: int, n_rows: int, d: int = 512, eps: float = 1e-6,
                          theta: float = 1e4, stream=None) -> SmlaKvInsertParams:
    p = SmlaKvInsertParams()
    p.n, p.d, p.rope_dim, p.n_swa, p.n_rows = n, d, rope_dim, n_swa, n_rows
    p.rms_eps, p.rope_theta = eps, theta
    p.stream = stream
    return p


def sparse_mla_kv_insert(kv, positions, norm_w, kv_pool, kv_scales, *, rope_dim: int, n_swa: int,
                         eps: float = 1e-6, theta: float = 1e4, stream=None) -> None:
    """Enqueue the KV insert on the current (or given) HIP stream.

    kv bf16 [n, 512]; positions int32 [n] (negative = skip); norm_w float32 [512];
    kv_pool uint8 / float8_e4m3fn [n_rows, 512] and kv_scales uint8 [n_rows, 16], whose
    rows ``positions mod n_swa`` are overwritten.  Raises SmlaError on failure.
    """
    torch, codes = _dtypes()
    ck = _Checker("sparse_mla_kv_insert")
    ck("kv", kv, (torch.bfloat16,), ndim=2)
    n, d = kv.shape
    ck("positions", positions, (torch.int32,), shape=(n,))
    ck("norm_w", norm_w, (torch.float32,), shape=(d,))
    ck("kv_pool", kv_pool, codes, ndim=2)
    if kv_pool.shape[1] != d:
        raise ValueError(f"sparse_mla_kv_insert: kv_pool rows must have {d} elements (got {kv_pool.shape[1]})")
    ck("kv_scales", kv_scales, (torch.uint8,), shape=(kv_pool.shape[0], d // 32))
    ck.done()
    if stream is None:
        stream = torch.cuda.current_stream(kv.device).cuda_stream
    params = make_kv_insert_params(n=n, d=d, rope_dim=rope_dim, n_swa=n_swa, n_rows=kv_pool.shape[0], eps=eps,
                                   theta=theta, stream=stream)
    rc = _lib.load().sparse_mla_kv_insert(_ptr(kv), _ptr(positions), _ptr(norm_w), _ptr(kv_pool), _ptr(kv_scales),
                                          ctypes.byref(params))
    if rc != SMLA_OK:
        raise SmlaError(rc, last_error(), "sparse_mla_kv_insert")


def make_index_params(*, s_q: int, n_cand: int, topk: int, window: int, self_in_window: bool, n_swa: int,
                      cmp_base: int, k_cmp: int, stream=None) -> SmlaIndexParams:
    p = SmlaIndexParams()
    p.s_q, p.n_cand, p.topk, p.window = s_q, n_cand, topk, window
    p.self_in_window, p.n_swa, p.cmp_base, p.k_cmp = int(bool(self_in_window)), n_swa, cmp_base, k_cmp
    p.stream = stream
    return p


def sparse_mla_build_index(positions, logits, n_valid, indices, topk_length, *, window: int, self_in_window: bool,
                           n_swa: int, cmp_base: int, k_cmp: int, stream=None) -> None:
    """Enqueue the index-row builder on the current (or given) HIP stream.

    positions int32 [s_q]; logits bf16 [s_q, n_cand]; n_valid int32 [s_q] or None;
    indices int32 [s_q, topk] and topk_length int32 [s_q] are written.  Raises SmlaError.
    """
    torch, _ = _dtypes()
    ck = _Checker("sparse_mla_build_index")
    ck("logits", logits, (torch.bfloat16,), ndim=2)
    s_q, n_cand = logits.shape
    ck("positions", positions, (torch.int32,), shape=(s_q,))
    ck("n_valid", n_valid, (torch.int32,), shape=(s_q,), optional=True)
    ck("indices", indices, (torch.int32,), ndim=2)
    if indices.shape[0] != s_q:
        raise ValueError(f"sparse_mla_build_index: indices must have {s_q} rows (got {indices.shape[0]})")
    ck("topk_length", topk_length, (torch.int32,), shape=(s_q,))
    ck.done()
    if stream is None:
        stream = torch.cuda.current_stream(logits.device).cuda_stream
    params = make_index_params(s_q=s_q, n_cand=n_cand, topk=indices.shape[1], window=window,
                               self_in_window=self_in_window, n_swa=n_swa, cmp_base=cmp_base, k_cmp=k_cmp,
                               stream=stream)
    rc = _lib.load().sparse_mla_build_index(_ptr(positions), _ptr(logits), _ptr(n_valid), _ptr(indices),
                                            _ptr(topk_length), ctypes.byref(params))
    if rc != SMLA_OK:
        raise SmlaError(rc, last_error(), "sparse_mla_build_index")


def sparse_mla_wo_a(x_fp8, x_scales, w_fp8, w_scales, y, *, heads_per_group: int = 1, stream=None) -> None:
    """Enqueue the FP8 output consumer (wo_a) on the current (or given) HIP stream.

    x_fp8 uint8 [s_q, h_q, 512] and x_scales uint8 [s_q, h_q, 16] (sparse_mla_fwd's
    outputs); w_fp8 uint8 [h_q / hg, d_out, hg * 512], w_scales uint8 [h_q / hg, d_out,
    hg * 16]; y bfloat16 [s_q, h_q / hg, d_out] is written.  Raises SmlaError.
    """
    torch, codes = _dtypes()
    ck = _Checker("sparse_mla_wo_a")
    ck("x_fp8", x_fp8, codes, ndim=3)
    s_q, h_q, d = x_fp8.shape
    hg = int(heads_per_group)
    if hg < 1 or h_q % hg:
        raise ValueError(f"sparse_mla_wo_a: heads_per_group must divide h_q = {h_q} (got {hg})")
    G = h_q // hg
    ck("x_scales", x_scales, (torch.uint8,), shape=(s_q, h_q, d // 32))
    ck("w_fp8", w_fp8, codes, ndim=3)
    d_out = w_fp8.shape[1]
    if tuple(w_fp8.shape) != (G, d_out, hg * d):
        raise ValueError(f"sparse_mla_wo_a: w_fp8 must have shape {(G, d_out, hg * d)} (got {tuple(w_fp8.shape)})")
    ck("w_scales", w_scales, (torch.uint8,), shape=(G, d_out, hg * d // 32))
    ck("y", y, (torch.bfloat16,), shape=(s_q, G, d_out))
    ck.done()
    if stream is None:
        stream = torch.cuda.current_stream(x_fp8.device).cuda_stream
    p = SmlaWoAParams()
    p.s_q, p.h_q, p.d, p.heads_per_group, p.d_out = s_q, h_q, d, hg, d_out
    p.stream = stream
    rc = _lib.load().sparse_mla_wo_a(_ptr(x_fp8), _ptr(x_scales), _ptr(w_fp8), _ptr(w_scales), _ptr(y),
                                     ctypes.byref(p))
    if rc != SMLA_OK:
        raise SmlaError(rc, last_error(), "sparse_mla_wo_a")
