"""GPU parity of the output projection (wo_a): the HIP kernel through the C ABI against the
fp64 oracle on the same seeded inputs.

Tolerance, from the arithmetic: each product of two E4M3 values with power-of-two scales is
exact in f32 and the K = 512 * hg products are summed in f32 (error at most
K * 2^-24 * sum |x_k w_k|), then rounded once to bf16 (8 significant bits: at most 2^-8
of the value).  The test allows 2^-8 |y| + 2 K 2^-24 sum |x_k w_k|; a wrong scale,
element or operand order is off by far more.  Also counted: outputs equal to the oracle rounded to bf16.
Cases: the three workloads, 2 / 4 / 64 heads per group, 1 / 16 / 128 heads, 256 outputs,
token counts that leave ragged token tiles, all-zero input, and the step's own output
fed in.
"""
import numpy as np
import pytest
import torch

import oracle
from prefill_token_amd import inputs, sparse_mla_wo_a

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


def run_gpu(c):
    dev = "cuda"
    x = torch.from_numpy(c["x"]).to(dev)
    xs = torch.from_numpy(c["x_scales"]).to(dev)
    w = torch.from_numpy(c["w"]).to(dev)
    ws = torch.from_numpy(c["w_scales"]).to(dev)
    G = c["h"] // c["heads_per_group"]
    y = torch.full((c["n"], G, c["d_out"]), float("nan"), dtype=torch.bfloat16, device=dev)
    sparse_mla_wo_a(x, xs, w, ws, y, heads_per_group=c["heads_per_group"])
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def bf16_round(a):
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def check(c, label="", n_sample=None):
    g = run_gpu(c)
    assert np.isfinite(g).all(), "outputs left unwritten"
    hg = c["heads_per_group"]
    x, xs = c["x"], c["x_scales"]
    if n_sample is not None and c["n"] > n_sample:
        # full-size call; the oracle on sampled tokens (first and last of the ragged tiles too)
        rng = np.random.default_rng(0)
        tok = set(rng.choice(c["n"], size=n_sample, replace=False).tolist()) | {0, 31, 32, c["n"] - 1}
        tok = np.array(sorted(tok))
        g, x, xs = g[tok], x[tok], xs[tok]
    ref = oracle.wo_a(x, xs, c["w"], c["w_scales"], hg)
    # sum |x_k w_k|: the same projection of the magnitudes (sign bits cleared)
    mag = oracle.wo_a((x & 0x7F).astype(np.uint8), xs, (c["w"] & 0x7F).astype(np.uint8), c["w_scales"], hg)
    K = 512 * hg
    tol = 2.0 ** -8 * np.abs(ref) + 2 * K * 2.0 ** -24 * mag
    err = np.abs(g - ref)
    assert (err <= tol).all(), f"{int((err > tol).sum())} outputs beyond tolerance, worst {(err / np.maximum(tol, 1e-300)).max():.3g}x"
    same = float((g == bf16_round(ref)).mean())
    print(c["name"], label, "max err / tol", float((err / np.maximum(tol, 1e-300)).max()), "equal to rounded oracle", same,
          flush=True)
    return g, ref


@pytest.mark.parametrize("name", list(inputs.WO_A_WORKLOADS))
def test_wo_a_workloads(name):
    check(inputs.make_wo_a(name), n_sample=96)


@pytest.mark.parametrize("hg", [2, 4, 64])
def test_wo_a_heads_per_group(hg):
    check(inputs.make_wo_a("wo_a_decode_sq64", seed=71, n=40, heads_per_group=hg), f"hg={hg}")


@pytest.mark.parametrize("n", [1, 31, 32, 33, 100])
def test_wo_a_ragged_tokens_and_wider_output(n):
    check(inputs.make_wo_a("wo_a_decode_sq64", seed=72, n=n, d_out=256), f"n={n}")


@pytest.mark.parametrize("h,hg", [(1, 1), (16, 2), (128, 8)])
def test_wo_a_head_counts(h, hg):
    rng = np.random.default_rng(76 + h)
    n, d_out = 37, 128
    G = h // hg
    x, xs = inputs.mx_pool(rng.standard_normal((n * h, 512)).astype(np.float32) * np.float32(0.05))
    w, ws = inputs.mx_pool(rng.standard_normal((G * d_out, hg * 512)).astype(np.float32) / np.float32(40.0))
    c = dict(name=f"wo_a_h{h}", n=n, h=h, d=512, heads_per_group=hg, d_out=d_out, x=x.reshape(n, h, 512),
             x_scales=xs.reshape(n, h, 16), w=w.reshape(G, d_out, hg * 512), w_scales=ws.reshape(G, d_out, hg * 16))
    check(c, f"h={h} hg={hg}")


def test_wo_a_zero_input_gives_zero():
    c = inputs.make_wo_a("wo_a_decode_sq64", seed=73, n=9)
    c["x"] = np.zeros_like(c["x"])
    g = run_gpu(c)
    assert np.array_equal(g, np.zeros_like(g))


def test_step_output_feeds_wo_a():
    # sparse_mla_fwd's out_fp8 / out_scales, as they are, are wo_a's input
    from parity import run_gpu as run_step

    inp = inputs.make("decode_sq64", seed=74, s_q=12)
    out = run_step(inp, with_f32=False)
    c = inputs.make_wo_a("wo_a_decode_sq64", seed=75, n=12)
    c["x"], c["x_scales"] = out["codes"], out["scales"]
    check(c, "step output")
