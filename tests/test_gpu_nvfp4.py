"""GPU parity of the step over the two-pool nvfp4_ds_mla cache (sparse_mla_fwd_ds_nvfp4)
against the fp64 oracle's two-pool step, by the rules of tests/parity.py.

Workloads in the two-pool form (E4M3 + UE8M0 SWA rows, NVFP4 compressed rows, entries
0 .. 127 SWA, 128 .. 639 compressed): decode s_q = 1 and 64 (split calls, the combine),
the 1024-token ragged decode and the 2123-token prefill with every token checked; forced
split counts; all entries in one segment (swa_entries 0 and 640); empty, all-sentinel and
short rows; stale ids past the length pointing outside either pool; fewer heads; no
rotary dims; split calls at rotary widths 0, 32 and 96 (both combine formats); 17 and 32
splits of 2000-entry rows (the combine's chunks of 16); tiny and huge compressed-row
scales."""
import numpy as np
import pytest
import torch

import oracle
from prefill_token_amd import inputs

from parity import compare, run_gpu_ds, run_oracle_ds

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


def check(inp, **kw):
    g = run_gpu_ds(inp, **kw)
    st = compare(g, run_oracle_ds(inp))
    print(inp["name"], kw, st, flush=True)
    return g, st


@pytest.mark.parametrize("name", ["decode_sq1", "decode_sq64"])
def test_decode(name):
    check(inputs.make_ds_nvfp4(name))


@pytest.mark.parametrize("name", ["decode_sq1024", "prefill_sq2123"])
def test_full_size_every_token(name):
    inp = inputs.make_ds_nvfp4(name)
    full = run_gpu_ds(inp)
    bench = run_gpu_ds(inp, with_f32=False)
    assert np.array_equal(full["codes"], bench["codes"]) and np.array_equal(full["scales"], bench["scales"])
    assert int((full["scales"] == 0xFF).sum()) == 0, "tokens left unwritten"
    st = compare(full, run_oracle_ds(inp))
    print(name, "nvfp4 all tokens", st, flush=True)


@pytest.mark.parametrize("ns", [1, 3, 10])
def test_forced_splits(ns):
    check(inputs.make_ds_nvfp4("decode_sq64", seed=201, s_q=6), num_splits=ns)


@pytest.mark.parametrize("swa_entries", [0, 640])
def test_one_segment(swa_entries):
    inp = inputs.make_ds_nvfp4("decode_sq64", seed=202, s_q=5)
    idx = inp["indices"]
    rng = np.random.default_rng(swa_entries)
    if swa_entries == 0:
        idx[:, :] = rng.integers(0, inp["cmp_codes"].shape[0], idx.shape)
    else:
        idx[:, :] = rng.integers(0, inp["swa_codes"].shape[0], idx.shape)
    idx[rng.random(idx.shape) < 0.1] = -1
    inp["swa_entries"] = swa_entries
    check(inp)
    check(inp, num_splits=1)


def test_edges():
    inp = inputs.make_ds_nvfp4("decode_sq64", seed=203, s_q=7)
    idx = inp["indices"]
    inp["topk_length"] = np.array([0, 1, 64, 129, 640, 200, 640], dtype=np.int32)
    idx[1, 0] = 3                          # a single SWA entry
    idx[3, :] = -1
    idx[3, 128] = 5                        # a single compressed entry
    idx[5, 200:] = 10 ** 6                 # stale ids past the length, outside either pool
    idx[6, :] = -1                         # all sentinels
    for ns in (0, 1):
        g, _ = check(inp, num_splits=ns)
        assert (g["f32"][0] == 0).all() and (g["f32"][6] == 0).all()


def test_fewer_heads_and_no_rope():
    inp = inputs.make_ds_nvfp4("decode_sq64", seed=204, s_q=3)
    inp["q"] = np.ascontiguousarray(inp["q"][:, :8])
    check(inp)
    inp["rope_dim"] = 0
    check(inp, num_splits=1)


@pytest.mark.parametrize("rope", [0, 32, 96])
@pytest.mark.parametrize("ns", [3, 10])
def test_split_combines_by_rotary_width(rope, ns):
    # rotary widths 0 and 64 send the split partials to the register-order combines (3
    # splits: four per thread, 10: one per thread), other widths to the generic combine
    inp = inputs.make_ds_nvfp4("decode_sq64", seed=206 + rope, s_q=3)
    inp["rope_dim"] = rope
    check(inp, num_splits=ns)


@pytest.mark.parametrize("ns", [17, 32])
def test_many_splits(ns):
    # more than 16 splits per token: the two-pool kernel's register-order partials merged
    # by the combine in chunks of 16.  Rows of 2000 entries: 128 SWA, then 1872 compressed
    inp = inputs.make_ds_nvfp4("decode_sq64", seed=230 + ns, s_q=3)
    rng = np.random.default_rng(ns)
    topk = 2000
    idx = np.empty((3, topk), dtype=np.int32)
    idx[:, :128] = rng.integers(0, inp["swa_codes"].shape[0], (3, 128))
    idx[:, 128:] = rng.integers(0, inp["cmp_codes"].shape[0], (3, topk - 128))
    idx[rng.random(idx.shape) < 0.1] = -1
    inp["indices"], inp["topk"] = idx, topk
    inp["topk_length"] = np.array([topk, 1500, 1100], dtype=np.int32)
    check(inp, num_splits=ns)


@pytest.mark.parametrize("lo,hi", [(0x10, 0x20), (0x60, 0x70)])
def test_compressed_scale_range(lo, hi):
    # compressed rows far from unit scale (E4M3 scales from 2^-5 to 2^7 or so); the softmax
    # scale is divided by the largest so that the scores stay O(1)
    inp = inputs.make_ds_nvfp4("decode_sq64", seed=205, s_q=4)
    rng = np.random.default_rng(lo)
    inp["cmp_scales"] = rng.integers(lo, hi, inp["cmp_scales"].shape).astype(np.uint8)
    big = float(oracle.e4m3_decode(np.array([hi - 1], np.uint8))[0])
    inp["sm_scale"] = inp["sm_scale"] / max(big / 0.3, 1.0)
    check(inp)
