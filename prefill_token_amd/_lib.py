"""ctypes view of the C ABI declared in include/smla.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsmla.so")
DEBUG_LIB_PATH = os.path.join(HERE, "libsmla_debug.so")

SMLA_ABI_VERSION = 5  # the layout of the structures below and the exported functions
SMLA_NOALLOC_SCRATCH_BYTES = 34 << 20
SMLA_DEBUG_WORD_OFFSET = 8
SMLA_DEBUG_BAD_INDEX = 1
SMLA_DEBUG_BAD_SCALE = 2

SMLA_OK = 0
SMLA_ERR_NULL = 1
SMLA_ERR_SHAPE = 2
SMLA_ERR_VALUE = 3
SMLA_ERR_HIP = 4

SMLA_KV_E4M3_UE8M0 = 0
SMLA_KV_BF16 = 1


class SmlaParams(ctypes.Structure):
    """Mirror of ``smla_params`` (same field order and C layout)."""

    _fields_ = [
        ("s_q", ctypes.c_int32),
        ("h_q", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
        ("n_rows", ctypes.c_int64),
        ("sm_scale", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
        ("rope_theta", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("out_f32", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
    ]


class SmlaDsParams(ctypes.Structure):
    """Mirror of ``smla_ds_params`` (the two-pool nvfp4_ds_mla step)."""

    _fields_ = [
        ("base", SmlaParams),
        ("n_cmp_rows", ctypes.c_int64),
        ("swa_entries", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class SmlaKvInsertParams(ctypes.Structure):
    """Mirror of ``smla_kv_insert_params``."""

    _fields_ = [
        ("n", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("n_swa", ctypes.c_int32),
        ("n_rows", ctypes.c_int64),
        ("rms_eps", ctypes.c_float),
        ("rope_theta", ctypes.c_float),
        ("stream", ctypes.c_void_p),
    ]


class SmlaIndexParams(ctypes.Structure):
    """Mirror of ``smla_index_params``."""

    _fields_ = [
        ("s_q", ctypes.c_int32),
        ("n_cand", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("self_in_window", ctypes.c_int32),
        ("n_swa", ctypes.c_int32),
        ("cmp_base", ctypes.c_int32),
        ("k_cmp", ctypes.c_int32),
        ("stream", ctypes.c_void_p),
    ]


class SmlaWoAParams(ctypes.Structure):
    """Mirror of ``smla_wo_a_params``."""

    _fields_ = [
        ("s_q", ctypes.c_int32),
        ("h_q", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("heads_per_group", ctypes.c_int32),
        ("d_out", ctypes.c_int32),
        ("stream", ctypes.c_void_p),
    ]


_lib = None


class LibraryMissing(RuntimeError):
    pass


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise LibraryMissing(
            f"{path} is missing: build it with `python -m prefill_token_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.sparse_mla_fwd.restype = ctypes.c_int
    lib.sparse_mla_fwd.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.POINTER(SmlaParams)]
    lib.sparse_mla_workspace_size.restype = ctypes.c_size_t
    lib.sparse_mla_workspace_size.argtypes = [ctypes.POINTER(SmlaParams)]
    lib.sparse_mla_num_splits.restype = ctypes.c_int
    lib.sparse_mla_num_splits.argtypes = [ctypes.POINTER(SmlaParams)]
    lib.sparse_mla_last_error.restype = ctypes.c_char_p
    lib.sparse_mla_last_error.argtypes = []
    lib.sparse_mla_kv_insert.restype = ctypes.c_int
    lib.sparse_mla_kv_insert.argtypes = [P, P, P, P, P, ctypes.POINTER(SmlaKvInsertParams)]
    lib.sparse_mla_build_index.restype = ctypes.c_int
    lib.sparse_mla_build_index.argtypes = [P, P, P, P, P, ctypes.POINTER(SmlaIndexParams)]
    lib.sparse_mla_wo_a.restype = ctypes.c_int
    lib.sparse_mla_wo_a.argtypes = [P, P, P, P, P, ctypes.POINTER(SmlaWoAParams)]
    lib.sparse_mla_abi_version.restype = ctypes.c_int
    lib.sparse_mla_abi_version.argtypes = []
    lib.sparse_mla_debug_checks.restype = ctypes.c_int
    lib.sparse_mla_debug_checks.argtypes = []
    lib.sparse_mla_fwd_noalloc.restype = ctypes.c_int
    lib.sparse_mla_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.POINTER(SmlaParams)]
    lib.sparse_mla_fwd_ds_nvfp4.restype = ctypes.c_int
    lib.sparse_mla_fwd_ds_nvfp4.argtypes = [P, P, P, P, P, P, P, P, P, P, P, ctypes.POINTER(SmlaDsParams)]
    lib.sparse_mla_noalloc_num_splits.restype = ctypes.c_int
    lib.sparse_mla_noalloc_num_splits.argtypes = [ctypes.POINTER(SmlaParams)]
    lib.sparse_mla_profile_events.restype = ctypes.c_int
    lib.sparse_mla_profile_events.argtypes = [P, P, P]
    got = lib.sparse_mla_abi_version()
    if got != SMLA_ABI_VERSION:
        raise LibraryMissing(f"{path} has ABI version {got}, this binding needs {SMLA_ABI_VERSION}: rebuild it with "
                             "`python -m prefill_token_amd.build`")
    return lib


def load() -> ctypes.CDLL:
    """Load the in-tree libsmla.so; raises LibraryMissing if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


_debug_lib = None


def load_debug() -> ctypes.CDLL:
    """Load the in-tree debug build libsmla_debug.so (same entry points, with the device-side
    precondition checks); raises LibraryMissing if it has not been built."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _open(DEBUG_LIB_PATH)
    return _debug_lib


def last_error() -> str:
    return load().sparse_mla_last_error().decode()
