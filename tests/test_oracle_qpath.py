"""Pins for the oracle's query path: per-head RMSNorm and rotate-half RoPE / inverse RoPE.

Independent references: torch.nn.functional.rms_norm in fp64 (library routine), the
rotate-half routine and default frequency table of ``transformers``' Llama rotary
embedding (library routine), a complex-number formulation of the same rotation, and
closed forms / invariants (p = 0 is the identity, inverse after forward is the
identity, rotations keep the norm, scores depend only on the position difference).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F


def test_rmsnorm_constant_vector_closed_form(oracle_mod):
    d, eps = 128, 1e-6
    rng = np.random.default_rng(1)
    w = rng.normal(1.0, 0.1, size=d)
    for c in [-3.0, 1e-4, 0.5, 7.25]:
        y = oracle_mod.rmsnorm(np.full(d, c), w, eps)
        ref = np.sign(c) * w * abs(c) / np.sqrt(c * c + eps)
        np.testing.assert_allclose(y, ref, rtol=1e-14, atol=0)


def test_rmsnorm_matches_library_fp64(oracle_mod):
    rng = np.random.default_rng(2)
    for d in [128, 512]:
        x = rng.standard_normal(d) * 3.0
        w = rng.normal(1.0, 0.1, size=d)
        y = oracle_mod.rmsnorm(x, w, 1e-6)
        ref = F.rms_norm(torch.from_numpy(x)[None], (d,), weight=torch.from_numpy(w), eps=1e-6)[0].numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)


def test_rmsnorm_scale_invariance(oracle_mod):
    rng = np.random.default_rng(3)
    x = rng.standard_normal(512)
    w = np.ones(512)
    np.testing.assert_allclose(oracle_mod.rmsnorm(17.0 * x, w, 1e-12), oracle_mod.rmsnorm(x, w, 1e-12), rtol=1e-10)


def _rot_complex(y, r, pos, theta, direction):
    """Same rotation written as complex multiplication: (a + ib) * exp(i*angle)."""
    d = y.shape[-1]
    o0, half = d - r, r // 2
    i = np.arange(half)
    ang = direction * pos * theta ** (-(2.0 * i) / r)
    z = (y[o0:o0 + half] + 1j * y[o0 + half:]) * np.exp(1j * ang)
    out = y.copy()
    out[o0:o0 + half] = z.real
    out[o0 + half:] = z.imag
    return out


@pytest.mark.parametrize("d,r", [(128, 32), (512, 64), (64, 64), (512, 2)])
def test_rope_complex_formulation(oracle_mod, d, r):
    rng = np.random.default_rng(4)
    for pos in [0, 1, 77, 4095, 32767]:
        y = rng.standard_normal(d)
        for direction in (1, -1):
            got = oracle_mod.rope(y, r, pos, 10000.0, direction)
            ref = _rot_complex(y, r, pos, 10000.0, direction)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)
            # the non-rotary dims are untouched
            assert np.array_equal(got[: d - r], y[: d - r])


def test_rope_matches_transformers_rotate_half(oracle_mod):
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    r = 64
    cfg = LlamaConfig(hidden_size=r, num_attention_heads=1, head_dim=r, rope_theta=10000.0,
                      max_position_embeddings=4096)
    emb = LlamaRotaryEmbedding(config=cfg)
    # the frequency table: inv_freq_i = base^(-2i/r)
    i = np.arange(r // 2)
    np.testing.assert_allclose(emb.inv_freq.double().numpy(), 10000.0 ** (-(2.0 * i) / r), rtol=1e-6)
    rng = np.random.default_rng(5)
    positions = np.array([0, 1, 5, 33, 63])
    x = rng.standard_normal((len(positions), r))
    cos, sin = emb(torch.zeros(1, 1, len(positions), r), torch.from_numpy(positions)[None])
    qt = torch.from_numpy(x)[None, None].float()  # [1, 1, S, r]
    ref, _ = apply_rotary_pos_emb(qt, qt, cos, sin)
    ref = ref[0, 0].double().numpy()
    for k, p in enumerate(positions):
        got = oracle_mod.rope(x[k], r, float(p), 10000.0, 1)
        np.testing.assert_allclose(got, ref[k], rtol=0, atol=2e-5)


def test_rope_identity_and_inverse(oracle_mod):
    rng = np.random.default_rng(6)
    for d, r in [(128, 32), (512, 64)]:
        y = rng.standard_normal(d)
        assert np.array_equal(oracle_mod.rope(y, r, 0.0, 10000.0, 1), y)
        for pos in [3, 1000, 32767]:
            fwd = oracle_mod.rope(y, r, pos, 10000.0, 1)
            back = oracle_mod.rope(fwd, r, pos, 10000.0, -1)
            np.testing.assert_allclose(back, y, rtol=0, atol=1e-12)
            np.testing.assert_allclose(np.linalg.norm(fwd), np.linalg.norm(y), rtol=1e-14)


def test_rope_relative_position(oracle_mod):
    rng = np.random.default_rng(7)
    d, r = 512, 64
    a, b = rng.standard_normal(d), rng.standard_normal(d)
    for p, q in [(10, 3), (30000, 29872), (128, 0), (5, 5)]:
        lhs = oracle_mod.rope(a, r, p, 1e4, 1) @ oracle_mod.rope(b, r, q, 1e4, 1)
        rhs = oracle_mod.rope(a, r, p - q, 1e4, 1) @ b
        np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-9)
