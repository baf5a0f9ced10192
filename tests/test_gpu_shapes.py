"""GPU parity of the step on shapes the decode and prefill workloads do not reach: head
counts that leave part of a 32-head MFMA block empty, token counts around the multiples
the split choice and the persistent grid work in, rotary widths other than 64 (the
general kernel, its rotary staging above the raw tiles or at offset 0), index rows whose
width is not a multiple of the 64-entry tile, no entries at all, and rows whose scores
rise tile after tile (the running reference raised mid-row, past its lazy-rescale
margin), and more than 16 splits per token (the combine's chunks of 16)."""
import math

import numpy as np
import pytest
import torch

from prefill_token_amd import inputs

from parity import compare, run_gpu, run_oracle, tie_aware_tolerance

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


def check(inp, extra=None, **kw):
    g = run_gpu(inp, **kw)
    st = compare(g, run_oracle(inp), extra=extra)
    print(inp["name"], inp["q"].shape, "rope", inp["rope_dim"], "topk", inp["indices"].shape[1], kw, st, flush=True)
    return g, st


@pytest.mark.parametrize("h", [1, 8, 20, 33, 64])
def test_head_counts(h):
    inp = inputs.make("decode_sq64", seed=300 + h, s_q=5)
    inp["q"] = np.ascontiguousarray(inp["q"][:, :h])
    inp["h"] = h
    check(inp)


@pytest.mark.parametrize("r", [0, 16, 128, 512])
def test_rotary_widths(r):
    inp = inputs.make("decode_sq64", seed=310 + r, s_q=3)
    inp["rope_dim"] = r
    check(inp)


@pytest.mark.parametrize("s_q", [7, 9, 63, 65, 257])
def test_token_counts(s_q):
    check(inputs.make("decode_sq64", seed=320 + s_q, s_q=s_q))


@pytest.mark.parametrize("topk", [1, 31, 33, 100, 2000])
def test_row_widths(topk):
    inp = inputs.make("decode_sq64", seed=330 + topk, s_q=6)
    rng = np.random.default_rng(topk)
    n_rows = inp["kv_pool"].shape[0]
    idx = rng.integers(0, n_rows, (6, topk)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.1] = -1
    inp["indices"] = idx
    inp["topk"] = topk
    inp["topk_length"] = np.array([topk, topk - 1, 0, max(topk // 2, 1), topk + 7, -3], dtype=np.int32)
    g, _ = check(inp)
    assert (g["f32"][2] == 0).all() and (g["f32"][5] == 0).all()


def test_no_entries():
    inp = inputs.make("decode_sq64", seed=340, s_q=4)
    inp["indices"] = np.zeros((4, 0), dtype=np.int32)
    inp["topk"] = 0
    inp["topk_length"] = np.array([0, 5, 0, 1], dtype=np.int32)
    g, _ = check(inp)
    assert (g["f32"] == 0).all()


@pytest.mark.parametrize("seed", [350, 351])
def test_scores_rising_slab_after_slab(seed):
    # entry j of a row reads pool row j, whose latent is scaled by 1 + 0.25 (j // 32): the
    # scores of entries 32 s .. 32 s + 31 are 1 + s/4 times those of the first 32, so the
    # tile maxima climb by more than the lazy-rescale margin several times along the row;
    # the softmax is then sharp, hence the tie-aware tolerance
    inp = inputs.make("decode_sq64", seed=seed, s_q=4)
    rng = np.random.default_rng(seed)
    topk = 640
    lat = rng.standard_normal((topk, 512)).astype(np.float32)
    lat *= (1.0 + 0.25 * (np.arange(topk) // 32))[:, None].astype(np.float32)
    inp["kv_pool"], inp["kv_scales"] = inputs.mx_pool(lat)
    inp["n_rows"] = topk
    inp["indices"] = np.tile(np.arange(topk, dtype=np.int32), (4, 1))
    inp["topk_length"] = np.array([topk, topk, 500, 321], dtype=np.int32)
    inp["sm_scale"] = 4.0 / math.sqrt(512)
    check(inp, extra=tie_aware_tolerance(inp))


@pytest.mark.parametrize("ns", [17, 20, 32])
def test_many_splits(ns):
    # more than 16 splits per token: the combine merges them in chunks of 16, raising its
    # running maximum (and rescaling the sums so far) between chunks.  Rows of 2000 random
    # entries, and rows whose scores rise along the row (entry j reads pool row j, scaled
    # by 1 + j / 400), so that a later chunk holds the largest m
    inp = inputs.make("decode_sq64", seed=360 + ns, s_q=3)
    rng = np.random.default_rng(ns)
    topk = 2000
    n_rows = inp["kv_pool"].shape[0]
    idx = rng.integers(0, n_rows, (3, topk)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.1] = -1
    inp["indices"], inp["topk"] = idx, topk
    inp["topk_length"] = np.array([topk, 1500, 1100], dtype=np.int32)
    check(inp, num_splits=ns)
    rising = inputs.make("decode_sq64", seed=370 + ns, s_q=2)
    lat = rng.standard_normal((topk, 512)).astype(np.float32)
    lat *= (1.0 + np.arange(topk) / 400.0)[:, None].astype(np.float32)
    rising["kv_pool"], rising["kv_scales"] = inputs.mx_pool(lat)
    rising["n_rows"] = topk
    rising["indices"] = np.tile(np.arange(topk, dtype=np.int32), (2, 1))
    rising["topk"] = topk
    rising["topk_length"] = np.array([topk, 1300], dtype=np.int32)
    check(rising, extra=tie_aware_tolerance(rising), num_splits=ns)
