"""Pins for the oracle's KV insert (the producer of the pool rows the step gathers).

Independent references: torch.nn.functional.rms_norm in fp64 (library routine), the
rotation written as complex multiplication, torch's CPU float8_e4m3fn cast (library
routine), and the definition of the minimal power-of-two block scale, floored at 2^(10-127)
(the smallest exponent the step decodes exactly).  A plausible
mistake anywhere -- RoPE before the norm, a flipped rotation, a dropped weight, the
wrong row, a wrong exponent -- moves a dequantized value by far more than half an E4M3
step, or a code away from the library's cast, and fails here.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from prefill_token_amd import inputs


def _ref_rows(kv_bits, positions, w, eps, theta, r):
    """RoPE(RMSNorm(kv)) in fp64 from library routines and the complex form of the rotation."""
    x = inputs.bf16_values(kv_bits).astype(np.float64)
    y = F.rms_norm(torch.from_numpy(x), (x.shape[1],), weight=torch.from_numpy(np.asarray(w, np.float64)),
                   eps=eps).numpy()
    if r:
        d = x.shape[1]
        o0, half = d - r, r // 2
        ang = positions[:, None].astype(np.float64) * theta ** (-(2.0 * np.arange(half)) / r)[None, :]
        z = (y[:, o0:o0 + half] + 1j * y[:, o0 + half:]) * np.exp(1j * ang)
        y = y.copy()
        y[:, o0:o0 + half] = z.real
        y[:, o0 + half:] = z.imag
    return y


def _case(seed, n, n_rows=4096, n_swa=1024, r=64, w_scale=1.0):
    rng = np.random.default_rng(seed)
    kv = inputs.bf16_bits(rng.standard_normal((n, 512), dtype=np.float32) * 3.0)
    w = inputs.bf16_values(inputs.bf16_bits(rng.normal(1.0, 0.1, 512).astype(np.float32))) * w_scale
    positions = rng.choice(np.arange(32768), size=n, replace=False).astype(np.int32)
    # distinct rows: drop repeats modulo n_swa
    _, keep = np.unique(positions % n_swa, return_index=True)
    positions = positions[np.sort(keep)]
    kv = kv[np.sort(keep)]
    pool = rng.integers(0, 256, size=(n_rows, 512), dtype=np.uint8)
    sc = rng.integers(100, 140, size=(n_rows, 16), dtype=np.uint8)
    return kv, positions, w.astype(np.float32), pool, sc, n_swa, r


@pytest.mark.parametrize("r,w_scale", [(64, 1.0), (0, 1.0), (512, 1.0), (16, 3e-20), (64, 5e25), (64, 1e-36)])
def test_insert_against_library_pipeline(oracle_mod, r, w_scale):
    kv, pos, w, pool, sc, n_swa, r = _case(30 + r, 40, r=r, w_scale=w_scale)
    eps, theta = 1e-6, 1e4
    got_pool, got_sc = oracle_mod.kv_insert(kv, pos, w, pool, sc, n_swa=n_swa, eps=eps, theta=theta, rope_dim=r)
    rows = pos % n_swa
    # untouched rows keep their bytes
    other = np.setdiff1d(np.arange(pool.shape[0]), rows)
    assert np.array_equal(got_pool[other], pool[other]) and np.array_equal(got_sc[other], sc[other])
    y = _ref_rows(kv, pos, w, eps, theta, r)
    blocks = np.abs(y).reshape(len(pos), 16, 32).max(axis=2)
    # exponent: the smallest e >= 10 with 448 * 2^(e-127) >= amax (decided by the definition)
    e = np.ceil(np.log2(blocks / 448.0)).astype(np.int64) + 127
    e = np.clip(e, 10, 254)
    assert (448.0 * np.exp2(e - 127.0) >= blocks).all()
    assert ((448.0 * np.exp2(e - 128.0) < blocks) | (e == 10)).all()
    assert np.array_equal(got_sc[rows].astype(np.int64), e)
    if w_scale < 1e-30:
        assert (e == 10).any()  # the floor is exercised
    # codes: within half an E4M3 step of the exact scaled value ...
    scaled = y * np.exp2(127.0 - np.repeat(e, 32, axis=1))
    deq = torch.from_numpy(got_pool[rows].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    k = np.floor(np.log2(np.maximum(np.abs(scaled), 2.0 ** -6)))
    half_step = np.exp2(k - 4)
    assert (np.abs(deq - scaled) <= half_step * (1 + 1e-9)).all()
    # ... and equal to the library's RNE cast away from rounding midpoints
    lib = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    frac = np.abs(scaled) / (2 * half_step)
    near_mid = np.abs(frac - np.floor(frac) - 0.5) < 1e-6
    assert np.array_equal(got_pool[rows][~near_mid], lib[~near_mid])


def test_insert_skips_negative_positions_and_later_token_wins(oracle_mod):
    kv, pos, w, pool, sc, n_swa, r = _case(41, 6)
    pos = pos.copy()
    pos[2] = -1
    pos[4] = pos[1] + n_swa  # lands on token 1's row, after it
    got_pool, got_sc = oracle_mod.kv_insert(kv, pos, w, pool, sc, n_swa=n_swa, eps=1e-6, theta=1e4, rope_dim=r)
    alone, alone_sc = oracle_mod.kv_insert(kv[4:5], pos[4:5], w, pool, sc, n_swa=n_swa, eps=1e-6, theta=1e4,
                                           rope_dim=r)
    row = pos[4] % n_swa
    assert np.array_equal(got_pool[row], alone[row]) and np.array_equal(got_sc[row], alone_sc[row])
    # a skipped token writes nothing: the result equals the call without it
    keep = np.array([0, 1, 3, 4, 5])
    ref_pool, ref_sc = oracle_mod.kv_insert(kv[keep], pos[keep], w, pool, sc, n_swa=n_swa, eps=1e-6, theta=1e4,
                                            rope_dim=r)
    assert np.array_equal(got_pool, ref_pool) and np.array_equal(got_sc, ref_sc)


def test_insert_zero_row(oracle_mod):
    kv, pos, w, pool, sc, n_swa, r = _case(42, 2)
    kv = np.zeros_like(kv)
    kv[1] = 0x8000  # -0.0 in bf16
    got_pool, got_sc = oracle_mod.kv_insert(kv, pos, w, pool, sc, n_swa=n_swa, eps=1e-6, theta=1e4, rope_dim=0)
    rows = pos % n_swa
    assert (got_sc[rows] == 10).all()  # the exponent floor
    # y = x * inv * w: the sign of zero follows x and w (w > 0 here)
    assert (got_pool[rows[0]] == 0x00).all() and (got_pool[rows[1]] == 0x80).all()
