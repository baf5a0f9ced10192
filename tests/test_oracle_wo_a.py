"""Pins of the oracle's output projection (wo_a), the consumer of the step's FP8 output.

The pages print no values for it; the oracle is pinned by a library route (torch's CPU
float8_e4m3fn cast for the decode and torch.matmul per group in fp64), closed forms (a
one-hot weight selects one input element; a weight scale one higher doubles the output
exactly), the group structure (two heads per group equal the sum of two one-head
projections with the weight's halves) and brute force on a tiny case.
"""
import numpy as np
import pytest
import torch

import oracle
from prefill_token_amd import inputs


def _case(seed=5, n=5, hg=1, d_out=128, h=8):
    rng = np.random.default_rng(seed)
    d = 512
    G = h // hg
    x, xs = inputs.mx_pool(rng.standard_normal((n * h, d)).astype(np.float32) * np.float32(0.05))
    w, ws = inputs.mx_pool(rng.standard_normal((G * d_out, hg * d)).astype(np.float32) / np.float32(23.0))
    return (x.reshape(n, h, d), xs.reshape(n, h, d // 32), w.reshape(G, d_out, hg * d),
            ws.reshape(G, d_out, hg * d // 32))


def _torch_route(x, xs, w, ws, hg):
    def deq(c, s):
        v = torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).to(torch.float64)
        sc = torch.from_numpy(np.ascontiguousarray(s)).to(torch.float64)
        return v * torch.pow(2.0, sc - 127.0).repeat_interleave(32, dim=-1)

    X, W = deq(x, xs), deq(w, ws)
    n, h, d = X.shape
    G = h // hg
    Xg = X.reshape(n, G, hg * d)
    return torch.stack([torch.matmul(Xg[:, g, :], W[g].T) for g in range(G)], dim=1).numpy()


def test_mx_decode_against_torch_cast():
    x, xs, _, _ = _case()
    ref = torch.from_numpy(x).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = ref * np.repeat(np.exp2(xs.astype(np.float64) - 127), 32, axis=-1)
    assert np.array_equal(oracle.mx_decode(x, xs), ref)


@pytest.mark.parametrize("hg", [1, 2, 8])
def test_against_library_route(hg):
    x, xs, w, ws = _case(hg=hg)
    y = oracle.wo_a(x, xs, w, ws, hg)
    ref = _torch_route(x, xs, w, ws, hg)
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15)


def test_one_hot_weight_selects_an_input():
    x, xs, w, ws = _case(hg=2, h=4)
    w = np.zeros_like(w)
    ws = np.full_like(ws, 127)
    G, d_out, K = w.shape
    picks = [(0, 3, 7), (1, 0, 512 + 31), (1, 127, 1023)]
    for g, o, k in picks:
        w[g, o, k] = 0x38  # E4M3 1.0
    y = oracle.wo_a(x, xs, w, ws, 2)
    X = oracle.mx_decode(x, xs)
    expect = np.zeros_like(y)
    for g, o, k in picks:
        expect[:, g, o] = X[:, 2 * g + k // 512, k % 512]
    assert np.array_equal(y, expect)


def test_weight_scale_doubles_output_exactly():
    x, xs, w, ws = _case()
    y = oracle.wo_a(x, xs, w, ws)
    assert np.array_equal(oracle.wo_a(x, xs, w, ws + 1), 2 * y)
    assert np.array_equal(oracle.wo_a(x, xs - 1, w, ws), y / 2)


def test_two_heads_per_group_is_the_sum_of_halves():
    x, xs, w, ws = _case(hg=2, h=4)
    y2 = oracle.wo_a(x, xs, w, ws, 2)
    for g in range(2):
        xa, xsa = x[:, 2 * g:2 * g + 1], xs[:, 2 * g:2 * g + 1]
        xb, xsb = x[:, 2 * g + 1:2 * g + 2], xs[:, 2 * g + 1:2 * g + 2]
        ya = oracle.wo_a(xa, xsa, w[g:g + 1, :, :512], ws[g:g + 1, :, :16], 1)
        yb = oracle.wo_a(xb, xsb, w[g:g + 1, :, 512:], ws[g:g + 1, :, 16:], 1)
        np.testing.assert_allclose(y2[:, g], (ya + yb)[:, 0], rtol=1e-12, atol=1e-15)


def test_brute_force_tiny():
    x, xs, w, ws = _case(n=2, h=2, hg=2, d_out=128)
    y = oracle.wo_a(x, xs, w, ws, 2)
    X = oracle.mx_decode(x, xs).reshape(2, 1, 1024)
    W = oracle.mx_decode(w, ws)
    for t in range(2):
        for o in (0, 1, 64, 127):
            acc = 0.0
            for k in range(1024):
                acc += X[t, 0, k] * W[0, o, k]
            assert abs(y[t, 0, o] - acc) <= 1e-12 * max(1.0, abs(acc))
