"""GPU: the allocation-free entry point (sparse_mla_fwd_noalloc) through the C ABI.

Its scratch is the library's static device array instead of a caller's workspace.  Calls
in a row of decreasing size -- an unsplit call with more tokens than compute units (the
item order in the scratch), a split call (partials in the scratch), a smaller split call --
must each reproduce sparse_mla_fwd (same split count, own zero-filled workspace) bit for
bit, and the oracle by the parity rules; the array keeps the previous call's contents, so
a stale counter, order entry or partial would show.  Then the call captured in a HIP graph
is replayed several times, with eager work between the replays, against the eager result.
"""
import ctypes

import numpy as np
import pytest
import torch

from prefill_token_amd import _lib, inputs, make_params, sparse_mla_workspace_size

from parity import compare, run_oracle, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


def _outputs(inp):
    s_q, h, d = inp["q"].shape
    # start from values the step never writes, so that a skipped token cannot pass
    return (torch.full((s_q, h, d), 0xFF, dtype=torch.uint8, device="cuda"),
            torch.full((s_q, h, d // 32), 0xFF, dtype=torch.uint8, device="cuda"),
            torch.full((s_q, h, d), float("nan"), dtype=torch.float32, device="cuda"))


def _call(fn, t, inp, outs, num_splits=0, workspace=None):
    s_q, h, d = inp["q"].shape
    out_fp8, out_sc, out_f32 = outs
    p = make_params(s_q=s_q, h_q=h, d=d, rope_dim=inp["rope_dim"], topk=inp["topk"], n_rows=inp["n_rows"],
                    kv_format=inp["kv_format"], sm_scale=inp["sm_scale"], eps=inp["eps"], theta=inp["theta"],
                    num_splits=num_splits, out_f32=out_f32, workspace=workspace)
    p.stream = torch.cuda.current_stream().cuda_stream
    ptr = lambda x: None if x is None else x.data_ptr()  # noqa: E731
    rc = fn(ptr(t["q"]), ptr(t["kv_pool"]), ptr(t["kv_scales"]), ptr(t["indices"]), ptr(t["topk_length"]),
            ptr(t["positions"]), ptr(t["norm_w"]), ptr(out_fp8), ptr(out_sc), ctypes.byref(p))
    assert rc == 0, _lib.load().sparse_mla_last_error()
    return p


def _host(outs):
    torch.cuda.synchronize()
    return dict(codes=outs[0].cpu().numpy(), scales=outs[1].cpu().numpy(), f32=outs[2].cpu().numpy())


def test_noalloc_matches_the_workspace_entry_point():
    lib = _lib.load()
    cases = [inputs.make("decode_sq1024", seed=91, s_q=300),  # unsplit, item order
             inputs.make("decode_sq64", seed=92, s_q=64),     # 4 splits
             inputs.make("decode_sq64", seed=93, s_q=3)]      # 10 splits, a smaller call last
    for inp in cases:
        t = to_device(inp)
        outs_n = _outputs(inp)
        p = _call(lib.sparse_mla_fwd_noalloc, t, inp, outs_n)
        ns = lib.sparse_mla_noalloc_num_splits(ctypes.byref(p))
        got = _host(outs_n)
        outs_w = _outputs(inp)
        need = sparse_mla_workspace_size(make_params(
            s_q=inp["s_q"], h_q=inp["h"], d=inp["d"], rope_dim=inp["rope_dim"], topk=inp["topk"],
            n_rows=inp["n_rows"], kv_format=inp["kv_format"], sm_scale=inp["sm_scale"], num_splits=ns))
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        _call(lib.sparse_mla_fwd, t, inp, outs_w, num_splits=ns, workspace=ws)
        ref = _host(outs_w)
        for k in ("codes", "scales", "f32"):
            assert got[k].tobytes() == ref[k].tobytes(), (inp["s_q"], ns, k)
        st = compare(got, run_oracle(inp))
        print("noalloc", inp["s_q"], "tokens", ns, "splits", st, flush=True)


def test_noalloc_graph_replays():
    lib = _lib.load()
    inp = inputs.make("decode_sq64", seed=94, s_q=16)
    t = to_device(inp)
    outs = _outputs(inp)
    _call(lib.sparse_mla_fwd_noalloc, t, inp, outs)
    eager = _host(outs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(lib.sparse_mla_fwd_noalloc, t, inp, outs)
    for r in range(3):
        for o in outs:
            o.fill_(0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = _host(outs)
        for k in ("codes", "scales", "f32"):
            assert got[k].tobytes() == eager[k].tobytes(), (r, k)
    compare(eager, run_oracle(inp))
