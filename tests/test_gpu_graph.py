"""GPU: sparse_mla_fwd captured in a HIP graph (through torch.cuda.CUDAGraph).

The call enqueues only kernels (no memset, no allocation) and leaves its workspace
counters zero, so a captured call can be replayed any number of times.  Each case
replays the graph several times with eager work and synchronizations in between and
checks every replay against the eager result bit for bit; then new inputs are copied
into the captured buffers and the replay is checked against the oracle.  Cases: the
split path (4 splits + combine), the path with more tokens than compute units (item
order kernel + persistent kernel), and the split path with more than 8 splits.
"""
import numpy as np
import pytest
import torch

from prefill_token_amd import inputs, sparse_mla_fwd, sparse_mla_workspace_size, make_params

from parity import compare, run_oracle, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


def _case(name, seed, s_q):
    return inputs.make(name, seed=seed, s_q=s_q)


@pytest.mark.parametrize("name,s_q,ns", [("decode_sq64", 64, 4), ("decode_sq1024", 300, 0), ("decode_sq1", 1, 10)])
def test_graph_replays(name, s_q, ns):
    inp = _case(name, 61, s_q)
    t = to_device(inp)
    s, h, d = inp["q"].shape
    p = make_params(s_q=s, h_q=h, d=d, rope_dim=inp["rope_dim"], topk=inp["topk"], n_rows=inp["n_rows"],
                    kv_format=inp["kv_format"], sm_scale=inp["sm_scale"], num_splits=ns)
    ws = torch.zeros(max(sparse_mla_workspace_size(p), 1), dtype=torch.uint8, device="cuda")
    out_fp8 = torch.empty((s, h, d), dtype=torch.uint8, device="cuda")
    out_sc = torch.empty((s, h, d // 32), dtype=torch.uint8, device="cuda")
    out_f32 = torch.empty((s, h, d), dtype=torch.float32, device="cuda")

    def call():
        sparse_mla_fwd(t["q"], t["kv_pool"], t["kv_scales"], t["indices"], t["topk_length"], t["positions"],
                       t["norm_w"], out_fp8, out_sc, sm_scale=inp["sm_scale"], rope_dim=inp["rope_dim"],
                       eps=inp["eps"], theta=inp["theta"], out_f32=out_f32, num_splits=ns, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = (out_fp8.clone(), out_sc.clone(), out_f32.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    scratch = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for rep in range(4):
        out_fp8.fill_(0xFF)
        out_sc.fill_(0xFF)
        out_f32.fill_(float("nan"))
        scratch.normal_()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_fp8, eager[0]) and torch.equal(out_sc, eager[1]), ("replay differs", rep)
        assert torch.equal(out_f32.view(torch.int32), eager[2].view(torch.int32)), ("replay f32 differs", rep)
        assert int(ws[:256].count_nonzero()) == 0, ("counters not reset", rep)
    # new inputs in the captured buffers: the replay computes them
    inp2 = _case(name, 62, s_q)
    t2 = to_device(inp2)
    for k in ("q", "kv_pool", "kv_scales", "indices", "topk_length", "positions", "norm_w"):
        t[k].copy_(t2[k])
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    got = dict(codes=out_fp8.cpu().numpy(), scales=out_sc.cpu().numpy(), f32=out_f32.cpu().numpy())
    st = compare(got, run_oracle(inp2))
    print(name, s_q, ns, "graph replay on new inputs", st, flush=True)
