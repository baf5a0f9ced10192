"""GPU parity: the HIP library through its C ABI against the fp64 oracle on the same
seeded inputs (rules in tests/parity.py).

Workloads: the tiny case and both small decode cases in full; the s_q = 1024 decode and
the 2123-token prefill at full size in the benchmark's launch configuration, every token
checked; ten seeds each of the 64-token decode and the 400-token ragged decode.  The
sharp-softmax regime (scores 16x their natural size, and pools far from unit scale) is
checked with a tolerance derived from the softmax's sensitivity to the kernel's score
error (tie-aware: near-tied top rows may mix either way).  Edge cases: every tile boundary of
topk_length, empty and all-sentinel rows, stale ids beyond topk_length pointing at rows
that decode to NaN, duplicates, position 0, fewer heads, no rotary dims, the E4M3 pool at
d = 128, the ends of the exact scale range, forced split counts, bit-reproducibility, and
one workspace shared by successive calls of different shapes (its scheduler counters are
left zero by every call), and the per-kernel profiling events (no effect on the outputs).
"""
import ctypes

import numpy as np
import pytest
import torch

from prefill_token_amd import inputs

from parity import compare, run_gpu, run_oracle, tie_aware_tolerance, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


def check(inp, **kw):
    gpu = run_gpu(inp, **kw)
    ref = run_oracle(inp)
    st = compare(gpu, ref)
    print(inp["name"], kw, st, flush=True)
    return gpu, ref, st


def test_tiny():
    check(inputs.make("tiny"))


@pytest.mark.parametrize("seed", [None, 7])
def test_decode_sq1(seed):
    check(inputs.make("decode_sq1", seed=seed))


def test_decode_sq64():
    check(inputs.make("decode_sq64"))


@pytest.mark.parametrize("ns", [1, 2, 3, 5, 7, 10])
def test_decode_forced_splits(ns):
    check(inputs.make("decode_sq64", seed=101, s_q=8), num_splits=ns)


@pytest.mark.parametrize("s_q,ns", [(40, 8), (30, 10)])
def test_split_combine_kernels(s_q, ns):
    # more (token, split) items than compute units, so the persistent kernel takes split
    # items from its queue; then the combine for ns <= 8 and the one for ns > 8
    check(inputs.make("decode_sq64", seed=102, s_q=s_q), num_splits=ns)


def _full(name, **make_kw):
    """Every token of a full-size workload against the oracle, in the benchmark's launch
    configuration (no f32 output) and with the f32 output (whose codes must agree)."""
    inp = inputs.make(name, **make_kw)
    dev = to_device(inp)
    full = run_gpu(inp, dev_inputs=dev)                  # with out_f32
    bench = run_gpu(inp, dev_inputs=dev, with_f32=False)  # the benchmark's launch configuration
    assert np.array_equal(full["codes"], bench["codes"]) and np.array_equal(full["scales"], bench["scales"])
    assert int((full["scales"] == 0xFF).sum()) == 0, "tokens left unwritten"
    st = compare(full, run_oracle(inp))
    print(name, make_kw, "all", inp["s_q"], "tokens", st, flush=True)
    return st


def test_decode_sq1024_every_token():
    _full("decode_sq1024")


def test_prefill_sq2123_every_token():
    _full("prefill_sq2123")


def test_ragged_more_than_4096_tokens():
    # the item order is built in passes of 4096 tokens above that count
    _full("decode_sq1024", seed=5, s_q=4500)


@pytest.mark.parametrize("seed", range(1001, 1011))
def test_decode_sq64_seeds(seed):
    check(inputs.make("decode_sq64", seed=seed))


@pytest.mark.parametrize("seed", range(2001, 2011))
def test_ragged_400_seeds(seed):
    # the 400-token ragged decode (lengths 0 .. 640, one split per token): the case with
    # the largest measured error (rows with one or two valid entries)
    inp = inputs.make("decode_sq1024", seed=seed, s_q=400)
    L = inp["topk_length"].copy()
    L[:8] = [0, 1, 2, 3, 64, 65, 639, 640]
    inp["topk_length"] = L
    check(inp)


def _decode_case(seed, s_q=8):
    return inputs.make("decode_sq64", seed=seed, s_q=s_q)


def test_topk_length_edges():
    inp = _decode_case(11, s_q=10)
    inp["topk_length"] = np.array([0, 1, 63, 64, 65, 127, 128, 639, 640, 5000], dtype=np.int32)
    inp["indices"][inp["indices"] < 0] = 17  # no sentinels: the length alone decides
    for ns in (0, 1, 4):
        check(inp, num_splits=ns)


def test_ragged_lengths_longest_first():
    # More tokens than compute units, one split each: the tokens are taken in order of
    # descending tile count.  Lengths span empty rows, every tile count and values past
    # topk; every token is checked.
    inp = inputs.make("decode_sq1024", seed=31, s_q=400)
    L = inp["topk_length"].copy()
    L[:16] = [0, -3, 1, 64, 65, 640, 700, 5000, 128, 0, 639, 2, 200, 384, 512, 576]
    inp["topk_length"] = L
    check(inp)
    check(inp, num_splits=1)


def test_equal_rows_with_huge_scores():
    # Every pool row is one row with block scale 200: a head's scores are all equal and of
    # size ~1e26, positive for some heads (the running max is raised) and negative for
    # others (the initial reference is lowered to them); every output is that row after
    # inverse RoPE.
    inp = inputs.make("decode_sq64", seed=81, s_q=6)
    inp["kv_pool"][:] = inp["kv_pool"][5].copy()
    inp["kv_scales"][:] = 200
    for ns in (0, 1, 3):
        check(inp, num_splits=ns)


def test_empty_and_sentinel_rows():
    inp = _decode_case(12, s_q=4)
    inp["indices"][0, :] = -1
    inp["topk_length"][1] = 0
    inp["indices"][2, :] = -1
    inp["indices"][2, 300] = 5  # a single valid entry in the middle of the row
    for ns in (0, 1):
        gpu, ref, _ = check(inp, num_splits=ns)
        assert (gpu["f32"][0] == 0).all() and (gpu["f32"][1] == 0).all()
        assert (gpu["scales"][0] == 0).all() and ((gpu["codes"][0] & 0x7F) == 0).all()


def test_stale_indices_point_at_nan_rows():
    inp = _decode_case(13, s_q=4)
    pool = inp["kv_pool"].copy()
    pool[:16, :] = 0x7F  # rows 0..15 decode to NaN
    inp["kv_pool"] = pool
    idx = inp["indices"]
    idx[(idx >= 0) & (idx < 16)] += 16
    inp["topk_length"] = np.array([100, 37, 640, 0], dtype=np.int32)
    for t, L in enumerate(inp["topk_length"]):
        idx[t, L:] = np.arange(640 - L) % 16  # every entry past the length points at a NaN row
    gpu, _, _ = check(inp)
    assert np.isfinite(gpu["f32"]).all()


def test_duplicates():
    inp = _decode_case(14, s_q=3)
    inp["indices"][:, 320:] = inp["indices"][:, 128:448]
    check(inp)


def test_position_zero_and_small():
    inp = _decode_case(15, s_q=4)
    inp["positions"] = np.array([0, 1, 2, 127], dtype=np.int32)
    check(inp)


@pytest.mark.parametrize("h", [1, 8, 16, 33, 48])
def test_fewer_heads(h):
    inp = _decode_case(16, s_q=3)
    inp["q"] = np.ascontiguousarray(inp["q"][:, :h])
    check(inp)


def test_rope_dim_zero_and_full():
    inp = _decode_case(17, s_q=3)
    for r in (0, 512):
        inp["rope_dim"] = r
        check(inp)


def test_fp8_pool_d128():
    rng = np.random.default_rng(18)
    inp = inputs.make("tiny")
    pool, sc = inputs.mx_pool(rng.standard_normal((256, 128)).astype(np.float32))
    inp.update(kv_pool=pool, kv_scales=sc, kv_format=inputs.KV_E4M3_UE8M0, name="tiny_fp8")
    check(inp)


@pytest.mark.parametrize("lo,hi", [(20, 20), (200, 200), (100, 140)])
def test_scale_range_ends(lo, hi):
    # Pools far from unit scale (tiny and huge latents, and rows whose 32-element blocks
    # span 2^40), first with the softmax scale divided by the largest block scale
    # (relative to the generator's natural scale) so that the scores stay O(1) and the
    # plain 1e-2 rule applies; then at the unscaled softmax scale, where the scores are
    # astronomically large and the softmax one-hot, under the tie-aware tolerance.
    inp = _decode_case(19, s_q=4)
    natural = float(np.mean(inp["kv_scales"]))  # the generator's scale for N(0, 1) latents
    rng = np.random.default_rng(lo + hi)
    inp["kv_scales"] = rng.integers(lo, hi + 1, size=inp["kv_scales"].shape).astype(np.uint8)
    sharp = dict(inp)
    inp["sm_scale"] = inp["sm_scale"] / 2.0 ** (hi - natural)
    check(inp)
    if hi - natural < 100:  # scores stay inside the f32 range
        extra = tie_aware_tolerance(sharp)
        for ns in (0, 1):
            st = compare(run_gpu(sharp, num_splits=ns), run_oracle(sharp), extra=extra)
            print("scale range, unscaled softmax", lo, hi, ns, st, flush=True)


@pytest.mark.parametrize("seed", [501, 502, 503])
def test_sharp_softmax_tie_aware(seed):
    # scores 16x their natural size: most heads near one-hot, some with near-tied top rows
    inp = _decode_case(seed, s_q=8)
    inp["sm_scale"] *= 16.0
    extra = tie_aware_tolerance(inp)
    ref = run_oracle(inp)
    for ns in (0, 1):
        st = compare(run_gpu(inp, num_splits=ns), ref, extra=extra)
        print("sharp softmax", seed, ns, "heads with extra tolerance > 1e-3:", int((extra > 1e-3).sum()), st,
              flush=True)


def test_bit_reproducible():
    inp = _decode_case(20, s_q=16)
    dev = to_device(inp)
    for ns in (0, 1, 5):
        a = run_gpu(inp, dev_inputs=dev, num_splits=ns)
        b = run_gpu(inp, dev_inputs=dev, num_splits=ns)
        for k in ("codes", "scales", "f32"):
            assert a[k].tobytes() == b[k].tobytes(), (ns, k)


def test_workspace_reused_across_calls():
    # The first 256 bytes of the workspace are the work-item counters: every call must
    # leave them zero, so one zero-filled workspace serves successive calls of any shape.
    from prefill_token_amd import make_params, sparse_mla_workspace_size

    cases = [_decode_case(21, s_q=300), _decode_case(22, s_q=3), _decode_case(23, s_q=300)]
    need = 0
    for inp in cases:
        s_q, h, d = inp["q"].shape
        for ns in (0, 1, 4):
            p = make_params(s_q=s_q, h_q=h, d=d, rope_dim=inp["rope_dim"], topk=inp["topk"], n_rows=inp["n_rows"],
                            kv_format=inp["kv_format"], sm_scale=inp["sm_scale"], num_splits=ns)
            need = max(need, sparse_mla_workspace_size(p))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for inp in cases:
        dev = to_device(inp)
        for ns in (0, 1, 4):
            a = run_gpu(inp, dev_inputs=dev, num_splits=ns, workspace=ws)
            assert int(ws[:256].count_nonzero()) == 0, ("counters not reset", ns)
            b = run_gpu(inp, dev_inputs=dev, num_splits=ns)  # a fresh workspace
            for k in ("codes", "scales", "f32"):
                assert a[k].tobytes() == b[k].tobytes(), (ns, k)
    compare(run_gpu(cases[0], workspace=ws), run_oracle(cases[0]))


def test_profile_events_time_each_kernel():
    # sparse_mla_profile_events arms three events for this thread's next step call: before
    # its main kernel, after it, after its last kernel.  Arming changes no output, and every
    # step call consumes the armed events, also one that fails its checks.
    from prefill_token_amd import _lib, make_params, sparse_mla_profile_events

    inp = _decode_case(24, s_q=16)
    dev = to_device(inp)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()  # torch creates its events on first record
    torch.cuda.synchronize()
    whole = {}
    for ns in (1, 4):
        ref = run_gpu(inp, dev_inputs=dev, num_splits=ns)
        evs[3].record()
        sparse_mla_profile_events(evs[0], evs[1], evs[2])
        got = run_gpu(inp, dev_inputs=dev, num_splits=ns)
        main, tail, whole[ns] = evs[0].elapsed_time(evs[1]), evs[1].elapsed_time(evs[2]), evs[3].elapsed_time(evs[2])
        assert main > 0 and tail >= 0 and main + tail <= whole[ns] + 1e-3, (ns, main, tail, whole[ns])
        if ns == 4:
            assert tail > 0  # the split combine runs between the second and the third event
        for k in ("codes", "scales", "f32"):
            assert got[k].tobytes() == ref[k].tobytes(), (ns, k)
    # a call that fails its checks consumes the armed events: the next call records none
    for e in evs[:3]:
        e.record()
    torch.cuda.synchronize()
    sparse_mla_profile_events(evs[0], evs[1], evs[2])
    bad = make_params(s_q=1, h_q=65, d=512, rope_dim=64, topk=640, n_rows=10, kv_format=0, sm_scale=0.1)
    assert _lib.load().sparse_mla_fwd(*([None] * 9), ctypes.byref(bad)) != 0
    run_gpu(inp, dev_inputs=dev, num_splits=4)
    assert evs[0].elapsed_time(evs[2]) < 0.5 * whole[4]
