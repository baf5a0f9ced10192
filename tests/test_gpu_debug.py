"""GPU: the debug build's error word and calls on a side stream.

libsmla_debug.so (the same kernels compiled with SMLA_DEBUG_CHECKS) reports an index
entry read (j < topk_length) outside [-1, n_rows) and a read row whose UE8M0 scales lie
outside [10, 246] in the u32 at byte 8 of the workspace, and still completes the call
normally: a bad id reads as an empty slot.  Checked on the production path (d = 512,
E4M3 pool) split and unsplit, and on the generic path (d = 128 E4M3 pool); entries past
topk_length and unreferenced rows never flag; the production library never writes the
word.  The side-stream test runs the step on a non-default stream with its own
workspace and compares with the default stream bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

from prefill_token_amd import _lib, inputs, make_params, sparse_mla_workspace_size

from parity import compare, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


def call(lib, inp, num_splits=0):
    """One sparse_mla_fwd call through the given library's C ABI; returns (codes, scales,
    f32, error word)."""
    t = to_device(inp)
    s_q, h, d = inp["q"].shape
    out_fp8 = torch.zeros((s_q, h, d), dtype=torch.uint8, device="cuda")
    out_sc = torch.zeros((s_q, h, d // 32), dtype=torch.uint8, device="cuda")
    out_f32 = torch.zeros((s_q, h, d), dtype=torch.float32, device="cuda")
    p = make_params(s_q=s_q, h_q=h, d=d, rope_dim=inp["rope_dim"], topk=inp["topk"], n_rows=inp["n_rows"],
                    kv_format=inp["kv_format"], sm_scale=inp["sm_scale"], eps=inp["eps"], theta=inp["theta"],
                    num_splits=num_splits, out_f32=out_f32)
    ws = torch.zeros(max(sparse_mla_workspace_size(p), 256), dtype=torch.uint8, device="cuda")
    p.workspace, p.workspace_bytes = ws.data_ptr(), ws.numel()
    p.stream = torch.cuda.current_stream().cuda_stream
    ptr = lambda x: None if x is None else x.data_ptr()  # noqa: E731
    rc = lib.sparse_mla_fwd(ptr(t["q"]), ptr(t["kv_pool"]), ptr(t["kv_scales"]), ptr(t["indices"]),
                            ptr(t["topk_length"]), ptr(t["positions"]), ptr(t["norm_w"]), ptr(out_fp8), ptr(out_sc),
                            ctypes.byref(p))
    assert rc == 0, lib.sparse_mla_last_error()
    torch.cuda.synchronize()
    word = int(ws[_lib.SMLA_DEBUG_WORD_OFFSET:_lib.SMLA_DEBUG_WORD_OFFSET + 4].cpu().numpy().view(np.uint32)[0])
    return dict(codes=out_fp8.cpu().numpy(), scales=out_sc.cpu().numpy(), f32=out_f32.cpu().numpy()), word


def sanitized(inp):
    """The same inputs with every id outside [-1, n_rows) replaced by -1 (what the kernels read)."""
    out = dict(inp)
    idx = inp["indices"].copy()
    idx[(idx < -1) | (idx >= inp["n_rows"])] = -1
    out["indices"] = idx
    return out


@pytest.mark.parametrize("ns", [0, 1, 3])
def test_bad_ids_set_the_word_and_read_as_empty(ns):
    inp = inputs.make("decode_sq64", seed=71, s_q=5)
    inp["indices"][0, 10] = inp["n_rows"] + 5
    inp["indices"][2, 300] = -7
    inp["indices"][4, 639] = 2 ** 30
    g, word = call(_lib.load_debug(), inp, ns)
    print("debug word", word, flush=True)
    assert word == _lib.SMLA_DEBUG_BAD_INDEX
    compare(g, run_oracle(sanitized(inp)))
    g2, word2 = call(_lib.load(), inp, ns)  # the production build: same output, word untouched
    assert word2 == 0
    for k in ("codes", "scales", "f32"):
        assert np.array_equal(g[k], g2[k]), k


def test_bad_ids_past_the_length_do_not_flag():
    inp = inputs.make("decode_sq64", seed=72, s_q=3)
    inp["topk_length"][:] = [100, 0, 640]
    inp["indices"][0, 100:] = inp["n_rows"] + 1
    inp["indices"][1, :] = -5
    g, word = call(_lib.load_debug(), inp)
    assert word == 0
    compare(g, run_oracle(inp))


def test_bad_scales_of_read_rows_set_the_word():
    inp = inputs.make("decode_sq64", seed=73, s_q=3)
    used = np.unique(inp["indices"][inp["indices"] >= 0])
    unused = np.setdiff1d(np.arange(inp["n_rows"]), used)
    inp["kv_scales"][unused[:50]] = 3  # never read: no flag
    _, word = call(_lib.load_debug(), inp)
    assert word == 0
    inp["kv_scales"][used[7], 4] = 250
    _, word = call(_lib.load_debug(), inp)
    assert word == _lib.SMLA_DEBUG_BAD_SCALE


def test_generic_path_d128():
    rng = np.random.default_rng(74)
    inp = inputs.make("tiny")
    pool, sc = inputs.mx_pool(rng.standard_normal((256, 128)).astype(np.float32))
    inp.update(kv_pool=pool, kv_scales=sc, kv_format=inputs.KV_E4M3_UE8M0)
    g, word = call(_lib.load_debug(), inp)
    assert word == 0
    compare(g, run_oracle(inp))
    inp["indices"][1, 3] = 4096
    sc = sc.copy()
    row2 = inp["indices"][2]
    sc[row2[row2 >= 0][0]] = 1  # a read row's scales below the range
    inp["kv_scales"] = sc
    g, word = call(_lib.load_debug(), inp)
    assert word == _lib.SMLA_DEBUG_BAD_INDEX | _lib.SMLA_DEBUG_BAD_SCALE


def test_side_stream_with_its_own_workspace():
    from prefill_token_amd import SmlaError, sparse_mla_fwd

    inp = inputs.make("decode_sq64", seed=75, s_q=16)
    ref = run_gpu(inp)
    t = to_device(inp)
    s_q, h, d = inp["q"].shape
    side = torch.cuda.Stream()
    p = make_params(s_q=s_q, h_q=h, d=d, rope_dim=inp["rope_dim"], topk=inp["topk"], n_rows=inp["n_rows"],
                    kv_format=inp["kv_format"], sm_scale=inp["sm_scale"])
    ws = torch.zeros(sparse_mla_workspace_size(p), dtype=torch.uint8, device="cuda")
    out_fp8 = torch.empty((s_q, h, d), dtype=torch.uint8, device="cuda")
    out_sc = torch.empty((s_q, h, d // 32), dtype=torch.uint8, device="cuda")
    out_f32 = torch.empty((s_q, h, d), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    args = (t["q"], t["kv_pool"], t["kv_scales"], t["indices"], t["topk_length"], t["positions"], t["norm_w"],
            out_fp8, out_sc)
    kw = dict(sm_scale=inp["sm_scale"], rope_dim=inp["rope_dim"], eps=inp["eps"], theta=inp["theta"],
              out_f32=out_f32)
    with pytest.raises(ValueError, match="workspace"):
        sparse_mla_fwd(*args, stream=side.cuda_stream, **kw)
    for _ in range(3):
        sparse_mla_fwd(*args, stream=side.cuda_stream, workspace=ws, **kw)
    side.synchronize()
    assert np.array_equal(out_fp8.cpu().numpy(), ref["codes"]) and np.array_equal(out_sc.cpu().numpy(), ref["scales"])
    assert np.array_equal(out_f32.cpu().numpy(), ref["f32"])
    assert int(ws[:256].count_nonzero()) == 0
    assert SmlaError is not None
