"""GPU parity of the index-row builder against the oracle: rows and lengths bit for bit.

Cases: the four builder workloads at full size (1 and 64 decode tokens over 2048
candidates, 1024 ragged decode tokens and the 2123-token prefill chunk over 16384), ties
everywhere (few distinct logits), NaN / -0 / +-inf logits, all-equal rows, no valid
candidates, fewer candidates than k, no candidate row at all (n_valid NULL), an empty
window, k = 0, positions before the window fills, candidate counts around 8192 and
16384 (a thread's share doubles; the last count whose keys stay in registers), 65536
candidates (the largest LDS case), a wide -1 tail, and an end-to-end check: rows built on the GPU drive
sparse_mla_fwd against the oracle.
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


def run_gpu_index(c, use_nv=True):
    from prefill_token_amd import sparse_mla_build_index

    dev = "cuda"
    pos = torch.from_numpy(c["positions"]).to(dev)
    lg = torch.from_numpy(c["logits"].view(np.int16)).to(dev).view(torch.bfloat16)
    nv = torch.from_numpy(c["n_valid"]).to(dev) if use_nv else None
    idx = torch.full((c["n"], c["topk"]), 12345, dtype=torch.int32, device=dev)  # stale contents
    L = torch.full((c["n"],), 777, dtype=torch.int32, device=dev)
    sparse_mla_build_index(pos, lg, nv, idx, L, window=c["window"], self_in_window=c["self_in_window"],
                           n_swa=c["n_swa"], cmp_base=c["cmp_base"], k_cmp=c["k_cmp"])
    torch.cuda.synchronize()
    return idx.cpu().numpy(), L.cpu().numpy()


def check(c, use_nv=True):
    gi, gl = run_gpu_index(c, use_nv)
    ri, rl = oracle.build_index(c["positions"], c["logits"], c["n_valid"] if use_nv else None, topk=c["topk"],
                                window=c["window"], self_in_window=c["self_in_window"], n_swa=c["n_swa"],
                                cmp_base=c["cmp_base"], k_cmp=c["k_cmp"])
    bad = np.nonzero((gi != ri).any(axis=1) | (gl != rl))[0]
    print(c["name"], "n", c["n"], "n_cand", c["n_cand"], "k", c["k_cmp"], "mismatched rows", bad[:8].tolist(),
          flush=True)
    assert bad.size == 0
    return gi, gl


@pytest.mark.parametrize("name", list(inputs.INDEX_WORKLOADS))
def test_index_workloads(name):
    check(inputs.make_index(name))


def test_index_special_values():
    c = inputs.make_index("index_decode_sq64", seed=61, n=12)
    lg = c["logits"]
    rng = np.random.default_rng(61)
    for t in range(12):
        cols = rng.choice(c["n_cand"], size=40, replace=False)
        lg[t, cols[:10]] = 0x7FC0  # NaN
        lg[t, cols[10:20]] = 0x8000  # -0
        lg[t, cols[20:25]] = 0x7F80  # +inf
        lg[t, cols[25:30]] = 0xFF80  # -inf
        lg[t, cols[30:40]] = 0xFFC1  # negative-signed NaN
    lg[5, :] = lg[5, 0]  # one row all equal
    check(c)


@pytest.mark.parametrize("nv_case", ["zero", "few", "exact", "none"])
def test_index_valid_counts(nv_case):
    c = inputs.make_index("index_decode_sq64", seed=62, n=8)
    if nv_case == "zero":
        c["n_valid"][:] = 0
    elif nv_case == "few":
        c["n_valid"][:] = [1, 5, 100, 511, 512, 513, -3, 99999]
    elif nv_case == "exact":
        c["n_valid"][:] = c["k_cmp"]
    check(c, use_nv=nv_case != "none")


def test_index_shapes():
    c = inputs.make_index("index_decode_sq64", seed=63, n=6)
    c["positions"][:] = [0, 1, 50, 127, 128, 129]
    for window, self_in, k, topk in [(0, False, 512, 512), (128, True, 0, 640), (128, False, 64, 1000), (8, True, 700, 708)]:
        c.update(window=window, self_in_window=self_in, k_cmp=k, topk=topk)
        check(c)


def test_index_candidate_count_not_a_multiple_of_8():
    # rows of 2052 candidates: even rows start 16-byte aligned and end in a partial group
    # of 8 columns, odd rows are not aligned
    rng = np.random.default_rng(97)
    n_cand = 2052
    c = dict(name="index_2052", n=4, n_cand=n_cand, positions=np.array([9, 300, 40000, 2], dtype=np.int32),
             logits=inputs.bf16_bits((np.round(rng.standard_normal((4, n_cand)) * 8) / 8).astype(np.float32)),
             n_valid=np.array([n_cand, 2050, 2049, 300], dtype=np.int32), topk=640, window=128,
             self_in_window=False, n_swa=8192, cmp_base=8192, k_cmp=512)
    # the largest logits in the last columns, so that they must be found
    c["logits"][:, -4:] = inputs.bf16_bits(np.full((4, 4), 9.0, dtype=np.float32))
    check(c)


@pytest.mark.parametrize("n_cand", [4095, 4096, 8191, 8192, 8193, 16383, 16384, 16385])
def test_index_candidate_count_boundaries(n_cand):
    # around the valid counts where a thread's share of the row grows from 8 to 16 columns
    # (8192) and where the builder moves from keys in registers (up to 16384 candidates) to
    # keys in LDS; counts that are not a multiple of 8 read the row column by column
    rng = np.random.default_rng(n_cand)
    n = 5
    c = dict(name=f"index_{n_cand}", n=n, n_cand=n_cand, positions=rng.integers(0, 40000, size=n).astype(np.int32),
             logits=inputs.bf16_bits((np.round(rng.standard_normal((n, n_cand)) * 8) / 8).astype(np.float32)),
             n_valid=np.array([n_cand, n_cand - 1, n_cand // 2 + 3, 513, 64], dtype=np.int32), topk=640,
             window=128, self_in_window=False, n_swa=8192, cmp_base=8192, k_cmp=512)
    c["logits"][0, -3:] = inputs.bf16_bits(np.full(3, 9.0, dtype=np.float32))  # the largest in the last columns
    check(c)


def test_index_largest_candidate_row():
    rng = np.random.default_rng(64)
    n_cand = 65536
    c = dict(name="index_65536", n=3, n_cand=n_cand, positions=np.array([5, 40000, 9], dtype=np.int32),
             logits=inputs.bf16_bits((np.round(rng.standard_normal((3, n_cand)) * 4) / 4).astype(np.float32)),
             n_valid=np.array([n_cand, 70000, 1000], dtype=np.int32), topk=2176, window=128, self_in_window=False,
             n_swa=8192, cmp_base=8192, k_cmp=2048)
    check(c)


def test_built_rows_feed_the_step():
    att = inputs.make("decode_sq64", seed=65, s_q=8)
    c = inputs.make_index("index_decode_sq64", seed=66, n=8)
    c["positions"] = att["positions"].copy()
    gi, gl = check(c)
    att["indices"], att["topk_length"] = gi, gl
    st = compare(run_gpu(att), run_oracle(att))
    print("end-to-end", st, flush=True)
