"""Pins for the oracle's number formats: E4M3FN decode/encode and the UE8M0 block rule.

Independent references: torch's CPU float8_e4m3fn cast (a library routine), the OCP
8-bit floating point specification's table of special values (closed forms), and the
mathematical definition of the minimal power-of-two block scale.  The encode sweep
spans five magnitude decades plus every midpoint between adjacent codes, the method
the pages use for their bitwise quantizer test
[SGLang #39370 "[DSV4.1] Combine DSpark decode and prefill kernel optimizations",
commit note on the MXFP8 epilogue].
"""
import math

import numpy as np
import pytest
import torch


def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode_f32(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x, dtype=np.float32).copy()).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_decode_exhaustive(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle_mod.e4m3_decode(codes)
    ref = torch_decode(codes)
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert (nan_g == nan_r).all()
    assert set(np.nonzero(nan_g)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan_g], ref[~nan_r])


def test_e4m3_special_values_from_spec(oracle_mod):
    # OCP OFP8 spec, E4M3: max normal S.1111.110 = 448, min normal S.0001.000 = 2^-6,
    # max subnormal S.0000.111 = 7 * 2^-9, min subnormal S.0000.001 = 2^-9, bias 7.
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0, 0x3C: 1.5}
    for c, v in cases.items():
        assert oracle_mod.e4m3_decode([c])[0] == v, hex(c)
        assert oracle_mod.e4m3_encode([v])[0] == c, hex(c)
    assert oracle_mod.e4m3_encode([-0.0])[0] == 0x80


def _sweep_values():
    vals = []
    # five magnitude decades, dense log grid, both signs
    for dec in range(-3, 2):
        g = np.geomspace(10.0 ** dec, 10.0 ** (dec + 1), 4001, dtype=np.float64)
        vals.append(g.astype(np.float32))
    # every midpoint between adjacent finite positive codes, and one float32 ulp either side
    pos = torch_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
             pos.astype(np.float32)]
    # the subnormal range and below
    vals.append(np.linspace(0, 2.0 ** -6, 2049, dtype=np.float32))
    v = np.concatenate(vals)
    v = v[np.abs(v) <= 448.0]
    return np.concatenate([v, -v])


def test_e4m3_encode_rne_sweep(oracle_mod):
    x = _sweep_values()
    got = oracle_mod.e4m3_encode(x.astype(np.float64))
    ref = torch_encode_f32(x)
    # +0 and -0 are the same value; torch keeps the sign like the oracle does
    same = (got == ref) | (((got & 0x7F) == 0) & ((ref & 0x7F) == 0))
    bad = np.nonzero(~same)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_encode_ties_to_even(oracle_mod):
    # 1.0625 lies halfway between 1.0 (0x38, even) and 1.125 (0x39): even wins.
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even).
    assert oracle_mod.e4m3_encode([1.0625, 1.1875])[0] == 0x38
    assert oracle_mod.e4m3_encode([1.1875])[0] == 0x3A
    # halfway between 0 and the smallest subnormal rounds to 0; just above rounds up
    assert oracle_mod.e4m3_encode([2.0 ** -10])[0] == 0x00
    assert oracle_mod.e4m3_encode([2.0 ** -10 * (1 + 2 ** -30)])[0] == 0x01


def test_ue8m0_closed_forms(oracle_mod):
    # 448 * 2^k is exactly representable: the smallest scale that covers it is 2^k.
    ks = np.arange(-127, 128)
    amax = np.ldexp(448.0, ks)
    assert np.array_equal(oracle_mod.ue8m0_exponent(amax), ks + 127)
    # just above 448 * 2^k needs the next power of two
    ks2 = np.arange(-127, 127)
    amax2 = np.ldexp(448.0 * (1 + 2.0 ** -40), ks2)
    assert np.array_equal(oracle_mod.ue8m0_exponent(amax2), ks2 + 128)
    # zero -> e = 0 (through the clamp); huge -> clamp at 254; tiny -> 0
    assert oracle_mod.ue8m0_exponent([0.0, 1e-300, 1e300]).tolist() == [0, 0, 254]
    # hand-worked: 448*2^-8 = 1.75 >= 1 > 0.875, 448*2^-7 = 3.5 >= 3.5 > 1.75
    assert oracle_mod.ue8m0_exponent([1.0, 3.0, 3.5, 3.5000001]).tolist() == [119, 120, 120, 121]


def test_ue8m0_is_ceil_not_nearest(oracle_mod):
    # torch's e8m0 cast rounds to nearest; the block rule must round the scale UP so
    # that amax / S never exceeds 448.  amax = 448 * 2.5 needs S = 4 (e = 129).
    assert oracle_mod.ue8m0_exponent([448.0 * 2.5])[0] == 129
    near = torch.tensor([2.5], dtype=torch.float32).to(torch.float8_e8m0fnu).to(torch.float32).item()
    assert near == 2.0  # the library cast would under-scale this block


def test_ue8m0_minimality_random(oracle_mod):
    rng = np.random.default_rng(7)
    amax = np.exp(rng.uniform(-80, 80, size=20000))
    e = oracle_mod.ue8m0_exponent(amax).astype(np.int64)
    S = np.ldexp(1.0, e - 127)
    assert (448.0 * S >= amax).all()
    assert (448.0 * S / 2 < amax).all()


def test_quantize_blocks_against_library_cast(oracle_mod):
    rng = np.random.default_rng(11)
    rows = []
    for mag in [1e-30, 1e-3, 1.0, 37.0, 1e6]:
        rows.append((rng.standard_normal((64, 128)) * mag).astype(np.float32))
    o = np.concatenate(rows).astype(np.float64)
    o[3, 32:64] = 0.0  # an all-zero block
    codes, scales = oracle_mod.quantize_blocks(o)
    blocks = o.reshape(o.shape[0], -1, 32)
    amax = np.abs(blocks).max(axis=2)
    S = np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert (448.0 * S >= amax).all()
    nz = amax > 0
    assert (448.0 * S[nz] / 2 < amax[nz]).all()
    assert (scales[3, 1] == 0) and (codes[3, 32:64] == 0).all()
    # o / S is exact in float32 (power-of-two scaling of float32 values), so torch's
    # cast of it is the reference rounding
    scaled = (blocks / S[..., None]).reshape(o.shape).astype(np.float32)
    ref = torch_encode_f32(scaled)
    same = (codes == ref) | (((codes & 0x7F) == 0) & ((ref & 0x7F) == 0))
    assert same.all()
    # round-to-nearest: the decoded code is within half of the local E4M3 step of o / S
    x = blocks / S[..., None]
    deq = torch_decode(codes).reshape(blocks.shape)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.abs(x)))
    step = np.ldexp(1.0, (np.maximum(np.where(np.isfinite(ex), ex, -6), -6) - 3).astype(np.int64))
    assert (np.abs(deq - x) <= step / 2).all()
