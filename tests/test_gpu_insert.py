"""GPU parity of the KV insert (the pool-row producer) against the fp64 oracle.

The kernel decides every code and exponent from fp64 values, so the whole pool and its
scales are compared bit for bit: the rows the call writes and every row it must leave
alone.  Cases: the three insert workloads at full size (1 and 64 decode tokens, the
2123-token prefill chunk, whose positions wrap around the 8192-row window), rope_dim
0 / 16 / 512, negative positions (skipped), an empty call, extreme norm weights (block
exponents far from 127), all-zero and negative-zero rows, and an end-to-end check: rows
written by the insert are gathered by sparse_mla_fwd.
"""
import numpy as np
import pytest
import torch

import oracle
from prefill_token_amd import inputs

from parity import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

# the library takes rms_eps and rope_theta as float32: the oracle gets the same values
F32 = lambda v: float(np.float32(v))  # noqa: E731


def run_insert_gpu(c, rope_dim=None):
    from prefill_token_amd import sparse_mla_kv_insert

    dev = "cuda"
    kv = torch.from_numpy(c["kv"].view(np.int16)).to(dev).view(torch.bfloat16)
    pos = torch.from_numpy(c["positions"]).to(dev)
    w = torch.from_numpy(c["norm_w"]).to(dev)
    pool = torch.from_numpy(c["kv_pool"]).to(dev)
    sc = torch.from_numpy(c["kv_scales"]).to(dev)
    sparse_mla_kv_insert(kv, pos, w, pool, sc, rope_dim=c["rope_dim"] if rope_dim is None else rope_dim,
                         n_swa=c["n_swa"], eps=c["eps"], theta=c["theta"])
    torch.cuda.synchronize()
    return pool.cpu().numpy(), sc.cpu().numpy()


def run_insert_oracle(c, rope_dim=None):
    return oracle.kv_insert(c["kv"], c["positions"], c["norm_w"], c["kv_pool"], c["kv_scales"], n_swa=c["n_swa"],
                            eps=F32(c["eps"]), theta=F32(c["theta"]),
                            rope_dim=c["rope_dim"] if rope_dim is None else rope_dim)


def check(c, rope_dim=None):
    gp, gs = run_insert_gpu(c, rope_dim)
    rp, rs = run_insert_oracle(c, rope_dim)
    bad_rows = np.nonzero((gp != rp).any(axis=1) | (gs != rs).any(axis=1))[0]
    print(c["name"], "n", c["n"], "rope_dim", c["rope_dim"] if rope_dim is None else rope_dim,
          "mismatched rows", bad_rows[:8].tolist(), flush=True)
    assert bad_rows.size == 0
    return gp, gs


@pytest.mark.parametrize("name", list(inputs.INSERT_WORKLOADS))
def test_insert_workloads(name):
    c = inputs.make_insert(name)
    gp, _ = check(c)
    rows = c["positions"] % c["n_swa"]
    assert not np.array_equal(gp[rows], c["kv_pool"][rows])  # the rows were written


@pytest.mark.parametrize("r", [0, 16, 512])
def test_insert_rope_dims(r):
    check(inputs.make_insert("insert_decode_sq64", seed=51, n=40), rope_dim=r)


def test_insert_negative_positions_and_empty():
    c = inputs.make_insert("insert_decode_sq64", seed=52, n=20)
    c["positions"][[0, 7, 19]] = [-1, -5, -2147483648]
    check(c)
    c0 = inputs.make_insert("insert_decode_sq64", seed=53, n=0)
    gp, gs = run_insert_gpu(c0)
    assert np.array_equal(gp, c0["kv_pool"]) and np.array_equal(gs, c0["kv_scales"])


@pytest.mark.parametrize("w_scale", [1e-37, 1e-30, 3e-12, 7e20, 1e30])
def test_insert_extreme_weights(w_scale):
    c = inputs.make_insert("insert_decode_sq64", seed=54, n=16)
    c["norm_w"] = (c["norm_w"] * np.float32(w_scale)).astype(np.float32)
    _, gs = check(c)
    rows = c["positions"] % c["n_swa"]
    print("exponents", int(gs[rows].min()), int(gs[rows].max()), flush=True)


def test_insert_zero_rows():
    c = inputs.make_insert("insert_decode_sq64", seed=55, n=4)
    c["kv"][0] = 0
    c["kv"][1] = 0x8000  # -0.0
    c["kv"][2, :256] = 0
    c["norm_w"][::3] *= -1
    check(c)


def test_inserted_rows_feed_the_step():
    # Insert 64 decode tokens into the decode pool, then attend over index rows that
    # point at the new rows (and others): the attention reads exactly what was written.
    att = inputs.make("decode_sq64", seed=56, s_q=8)
    c = inputs.make_insert("insert_decode_sq64", seed=57)
    c["kv_pool"], c["kv_scales"] = att["kv_pool"], att["kv_scales"]
    gp, gs = check(c)
    rows = (c["positions"] % c["n_swa"]).astype(np.int32)
    att["kv_pool"], att["kv_scales"] = gp, gs
    att["indices"][:, :64] = rows[None, :]
    st = compare(run_gpu(att), run_oracle(att))
    print("end-to-end", st, flush=True)


@pytest.mark.parametrize("tiny", [1e-36, 1e-30])
def test_tiny_norm_rows_feed_the_step(tiny):
    # Rows whose first blocks are tiny (norm weight ~1e-36 on dims 0..95): the insert codes
    # them at its exponent floor (10), the smallest scale the step decodes exactly; the
    # step then attends over index rows made of nothing but these rows, so its output is
    # a mix of them, and must match the oracle on the same pool bytes.
    att = inputs.make("decode_sq64", seed=58, s_q=6)
    c = inputs.make_insert("insert_decode_sq64", seed=59)
    c["norm_w"][:96] = (c["norm_w"][:96] * np.float32(tiny)).astype(np.float32)
    c["kv_pool"], c["kv_scales"] = att["kv_pool"], att["kv_scales"]
    gp, gs = check(c)
    rows = (c["positions"] % c["n_swa"]).astype(np.int32)
    assert int(gs[rows, :3].min()) >= 10
    if tiny < 1e-35:
        assert (gs[rows, :3] == 10).any()
    att["kv_pool"], att["kv_scales"] = gp, gs
    att["indices"][:, :] = -1
    att["indices"][:, :64] = rows[None, :]
    att["indices"][:, 200:264] = rows[None, ::-1]
    st = compare(run_gpu(att), run_oracle(att))
    print("tiny-norm rows end to end", tiny, st, flush=True)
