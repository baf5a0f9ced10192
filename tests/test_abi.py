"""The C ABI on the host (no GPU needed): the library loads, exports every function
include/smla.h declares, and rejects bad arguments with the documented codes before
any HIP call.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import prefill_token_amd as smla
from prefill_token_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from prefill_token_amd import build

        build.build()
    return _lib.load()


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(sparse_mla_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "sparse_mla_fwd" in names and len(names) >= 5
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    # 2: sparse_mla_wo_a, the item order in the workspace; 3: the debug build's error word;
    # 5: sparse_mla_profile_events
    assert smla.sparse_mla_abi_version() == 5 == smla._lib.SMLA_ABI_VERSION


def test_profile_events_arm_and_disarm_without_a_gpu(lib):
    # arming takes plain handles; a step call that fails its checks consumes them without
    # touching them (fake handles are never dereferenced)
    assert lib.sparse_mla_profile_events(None, None, None) == smla.SMLA_OK
    assert lib.sparse_mla_profile_events(FAKE, FAKE, FAKE) == smla.SMLA_OK
    p = good(h_q=65)
    assert lib.sparse_mla_fwd(*([FAKE] * 9), ctypes.byref(p)) == smla.SMLA_ERR_SHAPE
    assert lib.sparse_mla_profile_events(None, None, None) == smla.SMLA_OK


def test_debug_build_exports_the_same_symbols_and_says_so(lib):
    dbg = _lib.load_debug()
    for n in declared_functions():
        assert hasattr(dbg, n), n
    assert lib.sparse_mla_debug_checks() == 0 and dbg.sparse_mla_debug_checks() == 1
    assert dbg.sparse_mla_abi_version() == lib.sparse_mla_abi_version()
    # the debug build rejects bad arguments exactly as the production build does
    p = good(h_q=65)
    assert dbg.sparse_mla_fwd(*([FAKE] * 9), ctypes.byref(p)) == smla.SMLA_ERR_SHAPE


def test_debug_word_constants_match_header():
    text = open(os.path.join(ROOT, "include", "smla.h")).read()
    for name, val in (("SMLA_DEBUG_WORD_OFFSET", _lib.SMLA_DEBUG_WORD_OFFSET),
                      ("SMLA_DEBUG_BAD_INDEX", _lib.SMLA_DEBUG_BAD_INDEX),
                      ("SMLA_DEBUG_BAD_SCALE", _lib.SMLA_DEBUG_BAD_SCALE)):
        m = re.search(r"#define " + name + r" (\d+)u?", text)
        assert m and int(m.group(1)) == val, name


def test_struct_layout_matches_header():
    # int32 x6, int64, float x3, int32, pointers: offsets fixed by the C layout
    P = smla.SmlaParams
    assert P.n_rows.offset == 24 and P.sm_scale.offset == 32 and P.num_splits.offset == 44
    assert P.out_f32.offset == 48 and P.stream.offset == 72 and ctypes.sizeof(P) == 80


def good(**kw):
    base = dict(s_q=4, h_q=64, d=512, rope_dim=64, topk=640, n_rows=10240, kv_format=0, sm_scale=0.0442)
    base.update(kw)
    return smla.make_params(**base)


FAKE = 0x1000  # a non-null pointer the host never dereferences


def call(lib, p, *, null=None, kv_scales=True):
    ptrs = [FAKE] * 9
    if not kv_scales:
        ptrs[2] = None
    if null is not None:
        ptrs[null] = None
    return lib.sparse_mla_fwd(*ptrs, ctypes.byref(p) if p is not None else None)


def test_null_params(lib):
    assert lib.sparse_mla_fwd(*([FAKE] * 9), None) == smla.SMLA_ERR_NULL
    assert "params" in smla.sparse_mla_last_error()


@pytest.mark.parametrize("which", [0, 1, 3, 4, 5, 6, 7, 8])
def test_null_arrays(lib, which):
    p = good(num_splits=1)
    assert call(lib, p, null=which) == smla.SMLA_ERR_NULL


def test_null_scales_for_fp8_pool(lib):
    assert call(lib, good(num_splits=1), kv_scales=False) == smla.SMLA_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(d=256), smla.SMLA_ERR_SHAPE),
    (dict(d=512, kv_format=1), smla.SMLA_ERR_SHAPE),
    (dict(h_q=0), smla.SMLA_ERR_SHAPE),
    (dict(h_q=65), smla.SMLA_ERR_SHAPE),
    (dict(rope_dim=24), smla.SMLA_ERR_SHAPE),
    (dict(rope_dim=528), smla.SMLA_ERR_SHAPE),
    (dict(rope_dim=-16), smla.SMLA_ERR_SHAPE),
    (dict(topk=-1), smla.SMLA_ERR_SHAPE),
    (dict(topk=70000), smla.SMLA_ERR_SHAPE),
    (dict(n_rows=(1 << 32) // 512), smla.SMLA_ERR_SHAPE),  # a 4 GiB pool
    (dict(s_q=-1), smla.SMLA_ERR_VALUE),
    (dict(n_rows=0), smla.SMLA_ERR_VALUE),
    (dict(kv_format=7), smla.SMLA_ERR_VALUE),
    (dict(sm_scale=0.0), smla.SMLA_ERR_VALUE),
    (dict(sm_scale=float("nan")), smla.SMLA_ERR_VALUE),
    (dict(sm_scale=float("inf")), smla.SMLA_ERR_VALUE),
    (dict(eps=0.0), smla.SMLA_ERR_VALUE),
    (dict(eps=-1e-6), smla.SMLA_ERR_VALUE),
    (dict(theta=float("nan")), smla.SMLA_ERR_VALUE),
    (dict(num_splits=-1), smla.SMLA_ERR_VALUE),
    (dict(num_splits=65), smla.SMLA_ERR_VALUE),
])
def test_rejected_parameters(lib, kw, code):
    p = good(**kw)
    assert call(lib, p) == code
    assert smla.sparse_mla_last_error() != ""
    assert smla.sparse_mla_workspace_size(p) == 0 and smla.sparse_mla_num_splits(p) == 0


@pytest.mark.parametrize("which,off", [(0, 8), (1, 4), (2, 2), (6, 4), (7, 1)])
def test_misaligned_pointers(lib, which, off):
    p = good(num_splits=1)
    ptrs = [FAKE] * 9
    ptrs[which] = FAKE + off
    assert lib.sparse_mla_fwd(*ptrs, ctypes.byref(p)) == smla.SMLA_ERR_VALUE
    assert "aligned" in smla.sparse_mla_last_error()


def test_misaligned_out_f32(lib):
    p = good(num_splits=1)
    p.out_f32 = FAKE + 4
    assert call(lib, p) == smla.SMLA_ERR_VALUE


def test_workspace_required_when_split(lib):
    p = good(s_q=4)  # few tokens: automatic splitting needs a workspace
    ns = smla.sparse_mla_num_splits(p)
    assert ns > 1
    need = smla.sparse_mla_workspace_size(p)
    assert need == 256 + 4 * ns * 64 * (512 + 2) * 4  # scheduler counters, then partials
    assert call(lib, p) == smla.SMLA_ERR_VALUE  # no workspace given
    assert "workspace" in smla.sparse_mla_last_error()
    p.workspace, p.workspace_bytes = FAKE, need - 1
    assert call(lib, p) == smla.SMLA_ERR_VALUE


def test_split_choice():
    assert smla.sparse_mla_num_splits(good(s_q=1)) == 10   # one split per 64-entry tile
    # (these assume 256 compute units: the count without a GPU, and MI355X's)
    assert smla.sparse_mla_num_splits(good(s_q=4)) == 10
    assert smla.sparse_mla_num_splits(good(s_q=32)) == 5   # two tiles per split past 64 tiles of work
    assert smla.sparse_mla_num_splits(good(s_q=64)) == 4   # three tiles: 256 items
    assert smla.sparse_mla_num_splits(good(s_q=96)) == 2
    assert smla.sparse_mla_num_splits(good(s_q=129)) == 1  # no split count keeps one round
    assert smla.sparse_mla_num_splits(good(s_q=2123)) == 1
    assert smla.sparse_mla_num_splits(good(s_q=1, num_splits=3)) == 3
    assert smla.sparse_mla_num_splits(good(s_q=1, num_splits=64)) == 10  # capped at the tile count
    # the scheduler counters, then the unsplit call's item order (s_q int32, 256-byte units)
    assert smla.sparse_mla_workspace_size(good(s_q=2123)) == 256 + 8704


def test_zero_tokens_is_a_noop(lib):
    p = good(s_q=0)
    assert lib.sparse_mla_fwd(*([None] * 9), ctypes.byref(p)) == smla.SMLA_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(_lib.LibraryMissing):
        _lib.load()


# ---------------------------------------------------------------- KV insert


def good_insert(**kw):
    base = dict(n=4, rope_dim=64, n_swa=8192, n_rows=10240)
    base.update(kw)
    return smla.make_kv_insert_params(**base)


def call_insert(lib, p, null=None, off=None):
    ptrs = [FAKE] * 5
    if null is not None:
        ptrs[null] = None
    if off is not None:
        ptrs[off[0]] = FAKE + off[1]
    return lib.sparse_mla_kv_insert(*ptrs, ctypes.byref(p) if p is not None else None)


def test_insert_struct_layout():
    P = smla.SmlaKvInsertParams
    assert P.n_rows.offset == 16 and P.rms_eps.offset == 24 and P.stream.offset == 32 and ctypes.sizeof(P) == 40


@pytest.mark.parametrize("kw,code", [
    (dict(d=128), smla.SMLA_ERR_SHAPE),
    (dict(rope_dim=24), smla.SMLA_ERR_SHAPE),
    (dict(rope_dim=528), smla.SMLA_ERR_SHAPE),
    (dict(n_rows=0), smla.SMLA_ERR_SHAPE),
    (dict(n_rows=(1 << 32) // 512), smla.SMLA_ERR_SHAPE),
    (dict(n=-1), smla.SMLA_ERR_VALUE),
    (dict(n_swa=0), smla.SMLA_ERR_VALUE),
    (dict(n_swa=10241), smla.SMLA_ERR_VALUE),
    (dict(eps=0.0), smla.SMLA_ERR_VALUE),
    (dict(theta=float("inf")), smla.SMLA_ERR_VALUE),
])
def test_insert_rejected_parameters(lib, kw, code):
    assert call_insert(lib, good_insert(**kw)) == code
    assert smla.sparse_mla_last_error() != ""


@pytest.mark.parametrize("which", range(5))
def test_insert_null_arrays(lib, which):
    assert call_insert(lib, good_insert(), null=which) == smla.SMLA_ERR_NULL


@pytest.mark.parametrize("which,off", [(0, 8), (2, 4), (3, 8), (4, 2)])
def test_insert_misaligned(lib, which, off):
    assert call_insert(lib, good_insert(), off=(which, off)) == smla.SMLA_ERR_VALUE
    assert "aligned" in smla.sparse_mla_last_error()


def test_insert_null_params_and_empty(lib):
    assert lib.sparse_mla_kv_insert(*([FAKE] * 5), None) == smla.SMLA_ERR_NULL
    assert lib.sparse_mla_kv_insert(*([None] * 5), ctypes.byref(good_insert(n=0))) == smla.SMLA_OK


# ---------------------------------------------------------------- index-row builder


def good_index(**kw):
    base = dict(s_q=4, n_cand=2048, topk=640, window=128, self_in_window=False, n_swa=8192, cmp_base=8192, k_cmp=512)
    base.update(kw)
    return smla.make_index_params(**base)


def test_index_struct_layout():
    P = smla.SmlaIndexParams
    assert P.k_cmp.offset == 28 and P.stream.offset == 32 and ctypes.sizeof(P) == 40


@pytest.mark.parametrize("kw,code", [
    (dict(s_q=-1), smla.SMLA_ERR_VALUE),
    (dict(n_cand=65537), smla.SMLA_ERR_SHAPE),
    (dict(n_swa=0), smla.SMLA_ERR_VALUE),
    (dict(window=8193), smla.SMLA_ERR_SHAPE),
    (dict(k_cmp=-1), smla.SMLA_ERR_SHAPE),
    (dict(topk=639), smla.SMLA_ERR_SHAPE),
    (dict(topk=70000, k_cmp=60000), smla.SMLA_ERR_SHAPE),
    (dict(cmp_base=-1), smla.SMLA_ERR_VALUE),
    (dict(cmp_base=0x7FFFFFFF - 100), smla.SMLA_ERR_VALUE),
])
def test_index_rejected_parameters(lib, kw, code):
    p = good_index(**kw)
    assert lib.sparse_mla_build_index(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(p)) == code
    assert smla.sparse_mla_last_error() != ""


def test_index_self_in_window_flag(lib):
    p = good_index()
    p.self_in_window = 2
    assert lib.sparse_mla_build_index(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(p)) == smla.SMLA_ERR_VALUE


@pytest.mark.parametrize("which", [0, 1, 3, 4])
def test_index_null_arrays(lib, which):
    ptrs = [FAKE] * 5
    ptrs[which] = None
    assert lib.sparse_mla_build_index(*ptrs, ctypes.byref(good_index())) == smla.SMLA_ERR_NULL


def test_index_misaligned_logits_and_empty(lib):
    assert lib.sparse_mla_build_index(FAKE, FAKE + 1, FAKE, FAKE, FAKE, ctypes.byref(good_index())) == smla.SMLA_ERR_VALUE
    assert lib.sparse_mla_build_index(*([None] * 5), ctypes.byref(good_index(s_q=0))) == smla.SMLA_OK


def good_wo_a(**kw):
    p = smla.SmlaWoAParams()
    base = dict(s_q=4, h_q=64, d=512, heads_per_group=1, d_out=128)
    base.update(kw)
    for k, v in base.items():
        setattr(p, k, v)
    return p


def test_wo_a_struct_layout():
    P = smla.SmlaWoAParams
    assert P.d_out.offset == 16 and P.stream.offset == 24 and ctypes.sizeof(P) == 32


@pytest.mark.parametrize("kw,code", [
    (dict(s_q=-1), smla.SMLA_ERR_VALUE),
    (dict(d=256), smla.SMLA_ERR_SHAPE),
    (dict(h_q=0), smla.SMLA_ERR_SHAPE),
    (dict(h_q=129), smla.SMLA_ERR_SHAPE),
    (dict(heads_per_group=3), smla.SMLA_ERR_SHAPE),
    (dict(heads_per_group=0), smla.SMLA_ERR_SHAPE),
    (dict(heads_per_group=128), smla.SMLA_ERR_SHAPE),
    (dict(d_out=64), smla.SMLA_ERR_SHAPE),
    (dict(d_out=200), smla.SMLA_ERR_SHAPE),
    (dict(d_out=4224), smla.SMLA_ERR_SHAPE),
    (dict(s_q=140000, h_q=64), smla.SMLA_ERR_SHAPE),
])
def test_wo_a_rejected_parameters(lib, kw, code):
    p = good_wo_a(**kw)
    assert lib.sparse_mla_wo_a(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(p)) == code
    assert smla.sparse_mla_last_error() != ""


@pytest.mark.parametrize("which", [0, 1, 2, 3, 4])
def test_wo_a_null_and_misaligned(lib, which):
    ptrs = [FAKE] * 5
    ptrs[which] = None
    assert lib.sparse_mla_wo_a(*ptrs, ctypes.byref(good_wo_a())) == smla.SMLA_ERR_NULL
    ptrs[which] = FAKE + 4
    assert lib.sparse_mla_wo_a(*ptrs, ctypes.byref(good_wo_a())) == smla.SMLA_ERR_VALUE


def test_wo_a_null_params_and_empty(lib):
    assert lib.sparse_mla_wo_a(*([FAKE] * 5), None) == smla.SMLA_ERR_NULL
    assert lib.sparse_mla_wo_a(*([None] * 5), ctypes.byref(good_wo_a(s_q=0))) == smla.SMLA_OK


# ---------------------------------------------------------------- allocation-free variant


def test_noalloc_split_choice_and_limits(lib):
    scratch = _lib.SMLA_NOALLOC_SCRATCH_BYTES
    for s_q in (1, 4, 16, 32, 64, 96, 129, 2123):
        p = good(s_q=s_q)
        ns = smla.sparse_mla_num_splits(p)
        # the same count as sparse_mla_fwd whenever that call's scratch fits the static array
        assert smla.sparse_mla_workspace_size(p) <= scratch
        assert lib.sparse_mla_noalloc_num_splits(ctypes.byref(p)) == ns
    # an explicit split count whose partials cannot fit is rejected before any HIP call
    p = good(s_q=300, num_splits=4)
    assert smla.sparse_mla_workspace_size(p) > scratch
    assert lib.sparse_mla_noalloc_num_splits(ctypes.byref(p)) == 0
    assert lib.sparse_mla_fwd_noalloc(*([FAKE] * 9), ctypes.byref(p)) == smla.SMLA_ERR_VALUE
    assert "static scratch" in smla.sparse_mla_last_error()
    # the same argument checks as sparse_mla_fwd
    assert lib.sparse_mla_fwd_noalloc(*([FAKE] * 9), ctypes.byref(good(h_q=65))) == smla.SMLA_ERR_SHAPE
    ptrs = [FAKE] * 9
    ptrs[0] = None
    assert lib.sparse_mla_fwd_noalloc(*ptrs, ctypes.byref(good())) == smla.SMLA_ERR_NULL
    ptrs[0] = FAKE + 8
    assert lib.sparse_mla_fwd_noalloc(*ptrs, ctypes.byref(good())) == smla.SMLA_ERR_VALUE
    assert lib.sparse_mla_fwd_noalloc(*([None] * 9), ctypes.byref(good(s_q=0))) == smla.SMLA_OK


def test_noalloc_scratch_constant_matches_header():
    text = open(os.path.join(ROOT, "include", "smla.h")).read()
    m = re.search(r"#define SMLA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.SMLA_NOALLOC_SCRATCH_BYTES


# ---------------------------------------------------------------- two-pool (nvfp4_ds_mla) step


def good_ds(**kw):
    n_cmp = kw.pop("n_cmp_rows", 2048)
    swa_entries = kw.pop("swa_entries", 128)
    reserved = kw.pop("reserved", 0)
    dp = smla.SmlaDsParams()
    dp.base = good(**kw)
    dp.n_cmp_rows, dp.swa_entries, dp.reserved = n_cmp, swa_entries, reserved
    return dp


def call_ds(lib, dp, null=None, off=None):
    ptrs = [FAKE] * 11
    if null is not None:
        ptrs[null] = None
    if off is not None:
        ptrs[off[0]] = FAKE + off[1]
    return lib.sparse_mla_fwd_ds_nvfp4(*ptrs, ctypes.byref(dp) if dp is not None else None)


def test_ds_struct_layout():
    P = smla.SmlaDsParams
    assert P.n_cmp_rows.offset == 80 and P.swa_entries.offset == 88 and ctypes.sizeof(P) == 96


@pytest.mark.parametrize("kw,code", [
    (dict(d=128), smla.SMLA_ERR_SHAPE),
    (dict(d=128, kv_format=1), smla.SMLA_ERR_SHAPE),
    (dict(rope_dim=128), smla.SMLA_ERR_SHAPE),
    (dict(n_cmp_rows=0), smla.SMLA_ERR_SHAPE),
    (dict(n_cmp_rows=(1 << 32) // 256), smla.SMLA_ERR_SHAPE),
    (dict(swa_entries=100), smla.SMLA_ERR_SHAPE),
    (dict(swa_entries=-64), smla.SMLA_ERR_SHAPE),
    (dict(reserved=1), smla.SMLA_ERR_VALUE),
    (dict(h_q=65), smla.SMLA_ERR_SHAPE),
    (dict(sm_scale=0.0), smla.SMLA_ERR_VALUE),
])
def test_ds_rejected_parameters(lib, kw, code):
    assert call_ds(lib, good_ds(num_splits=1, **kw)) == code
    assert smla.sparse_mla_last_error() != ""


@pytest.mark.parametrize("which", [0, 1, 2, 3, 4, 6, 7, 8, 9, 10])
def test_ds_null_arrays(lib, which):
    assert call_ds(lib, good_ds(num_splits=1), null=which) == smla.SMLA_ERR_NULL


@pytest.mark.parametrize("which,off", [(0, 8), (1, 4), (3, 8), (4, 2), (9, 1)])
def test_ds_misaligned(lib, which, off):
    assert call_ds(lib, good_ds(num_splits=1), off=(which, off)) == smla.SMLA_ERR_VALUE
    assert "aligned" in smla.sparse_mla_last_error()


def test_ds_null_params_workspace_and_empty(lib):
    assert lib.sparse_mla_fwd_ds_nvfp4(*([FAKE] * 11), None) == smla.SMLA_ERR_NULL
    assert call_ds(lib, good_ds(s_q=4)) == smla.SMLA_ERR_VALUE  # a split call without a workspace
    assert "workspace" in smla.sparse_mla_last_error()
    assert lib.sparse_mla_fwd_ds_nvfp4(*([None] * 11), ctypes.byref(good_ds(s_q=0))) == smla.SMLA_OK
