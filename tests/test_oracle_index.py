"""Pins for the oracle's index-row builder and its top-k selection rule.

Independent references: torch.topk (library routine) for the multiset of selected
values, including NaN, which torch ranks above every number; a brute force over all
k-subsets of tiny rows for the tie rule (of the subsets holding the k largest values, the
kept one is the one with the smallest column sum, i.e. the lowest tied columns); closed
forms for the sliding-window part; and the workload generator's own window rows.
"""
import itertools

import numpy as np
import pytest
import torch

from prefill_token_amd import inputs


def _bits(vals):
    return inputs.bf16_bits(np.asarray(vals, dtype=np.float32))


def _vals(bits):
    return inputs.bf16_values(bits).astype(np.float64)


@pytest.mark.parametrize("n,k,levels", [(2048, 512, 8), (16384, 512, 64), (300, 512, 4), (1000, 1, 3), (64, 64, 2)])
def test_selected_values_match_torch_topk(oracle_mod, n, k, levels):
    rng = np.random.default_rng(n + k)
    # few distinct values, as real indexer logits have: many ties at the k-th value
    x = np.round(rng.standard_normal(n) * levels) / levels
    x[rng.choice(n, size=max(1, n // 100), replace=False)] = np.nan
    x[rng.choice(n, size=max(1, n // 200), replace=False)] = -0.0
    b = _bits(x)
    sel = oracle_mod.select_topk(b, k)
    assert sel.size == min(k, n) and (np.diff(sel) > 0).all()
    t = torch.from_numpy(_vals(b))
    ref = torch.topk(t, min(k, n)).values.numpy()
    got = _vals(b)[sel]
    assert np.isnan(got).sum() == np.isnan(ref).sum()
    assert np.array_equal(np.sort(got[~np.isnan(got)]), np.sort(ref[~np.isnan(ref)]))


def test_tie_rule_brute_force(oracle_mod):
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, n + 1))
        x = rng.integers(-2, 3, size=n).astype(np.float64)
        if rng.random() < 0.3:
            x[rng.integers(0, n)] = np.nan
        b = _bits(x)
        v = _vals(b)
        key = np.where(np.isnan(v), np.inf, v)  # NaN ranks above every number here
        key = np.where(np.isnan(v), 1e300, key)
        best = None
        target = np.sort(key)[::-1][:k]
        for S in itertools.combinations(range(n), k):
            if np.array_equal(np.sort(key[list(S)])[::-1], target):
                if best is None or sum(S) < sum(best):
                    best = S
        assert list(oracle_mod.select_topk(b, k)) == list(best), (x, k)


def test_window_closed_forms(oracle_mod):
    n_swa, W = 8192, 128
    pos = np.array([0, 5, 127, 128, 8191, 8200, 30000], dtype=np.int32)
    logits = np.zeros((pos.size, 16), dtype=np.uint16)
    for s in (0, 1):
        idx, L = oracle_mod.build_index(pos, logits, None, topk=160, window=W, self_in_window=bool(s), n_swa=n_swa,
                                        cmp_base=n_swa, k_cmp=16)
        for t, p in enumerate(pos):
            q = p - W + s + np.arange(W)
            exp = np.where(q >= 0, q % n_swa, -1)
            assert np.array_equal(idx[t, :W], exp)
            assert np.array_equal(idx[t, W:W + 16], n_swa + np.arange(16))  # all-equal logits: lowest columns
            assert (idx[t, W + 16:] == -1).all() and L[t] == W + 16


def test_fewer_candidates_than_k(oracle_mod):
    rng = np.random.default_rng(6)
    logits = _bits(rng.standard_normal((3, 600)))
    nv = np.array([0, 100, 5000])
    idx, L = oracle_mod.build_index(np.array([10, 20, 30]), logits, nv, topk=700, window=128, self_in_window=False,
                                    n_swa=8192, cmp_base=8192, k_cmp=512)
    assert L.tolist() == [128, 228, 640]
    assert (idx[0, 128:] == -1).all()
    assert np.array_equal(idx[1, 128:228], 8192 + np.arange(100)) and (idx[1, 228:] == -1).all()
    assert (idx[2, 128:640] >= 8192).all() and (idx[2, 640:] == -1).all()


@pytest.mark.parametrize("name,s", [("decode_sq64", 0), ("prefill_sq184", 1)])
def test_window_matches_workload_recipe(oracle_mod, name, s):
    inp = inputs.make(name, s_q=16)
    logits = np.zeros((16, 8), dtype=np.uint16)
    idx, _ = oracle_mod.build_index(inp["positions"], logits, None, topk=640, window=128, self_in_window=bool(s),
                                    n_swa=inp["n_swa"], cmp_base=inp["n_swa"], k_cmp=8)
    gen = inp["indices"][:, :128]
    keep = gen >= 0  # the generator masks ~10 % of decode entries with -1
    assert np.array_equal(idx[:, :128][keep], gen[keep])
