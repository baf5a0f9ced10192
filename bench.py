#!/usr/bin/env python3
"""Benchmark of the fused sparse-MLA step (sparse_mla_fwd) on one MI355X.

A step is one sparse_mla_fwd call over one batch of seeded synthetic inputs (inputs
resident in HBM).  Timing follows the pages' kernel benchmark [vLLM #58872, Test Plan:
one captured graph per case, the L2 flushed before every replay outside the timed
interval, the median of many replays]: each timed step flushes the caches (a 1 GiB
fill), synchronizes, then launches ONE call between two HIP events on the launch stream;
a GPU spin queued before the first event keeps the host's launch latency out of the span.
On ROCm a one-call graph replay adds about 9 us of graph-launch work inside such a span
(a one-kernel graph of a trivial add reads about 13 us against 6 us launched directly),
so the calls are launched directly; the graph replays are checked for identical output
and their cold figures reported beside the direct ones, with the protocol's own
overheads measured in the same run.  The headline workload is the s_q = 1 decode (h_q = 64,
d = 512 with 64 rotary dims, topk 128 SWA + 512 compressed, E4M3 + UE8M0 pools); the
s_q = 64 / 1024 decodes and the 2123-token prefill (and the pages' s_q = 256 and
184-token rows) are measured after the timed region and reported under "configs", each
with at least 50 cold samples.  Warm figures (graphs of 10 back-to-back calls, caches
hot) are kept beside them, labelled warm.

Prints one JSON line:
  value        tokens/s of the headline workload: s_q / the mean cold span of the K timed
               steps
  roofline     the dominant kernel (smla_ws) of the headline call: its algorithmic HBM
               bytes / its mean cold span between the library's profiling events
               (sparse_mla_profile_events), against 8 TB/s (and against the copy bandwidth
               measured in the same run); the whole call's figure beside it
  cpu_baseline the fp64 oracle on the headline workload's own arrays (median of 3 runs),
               on the host cores; per-config oracle medians under "cpu_oracle_configs"
  measured_peaks  device-copy bandwidth and pure MFMA-loop rates (bf16, E4M3) measured
               in the same run, beside the published peaks
  configs      per workload: cold median / p10 / p90 / mean us per call, warm us per call,
               tokens/s, HBM and MFMA fractions (cold, and warm labelled as such)
  kv_insert    the KV-insert entry point (the pool-row producer) on its three workloads:
               us/call, tokens/s, algorithmic HBM bytes / mean duration against 8 TB/s
  build_index  the index-row builder on its four workloads, the same figures
  two_pool_nvfp4  the step over the two-pool nvfp4_ds_mla cache (sparse_mla_fwd_ds_nvfp4) on
               the decode s_q = 1 / 64 / 1024 and 2123-token prefill workloads, the same figures
  wo_a         the output projection (the step's FP8 output consumer) on its three
               workloads: us/call, tokens/s, HBM and fp8 MFMA fractions

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Counter helpers (for the HBM traffic figure, see profiles/):
  python bench.py --copy-probe MIB    plain device-to-device copies of MIB MiB (the
                                      reference kernel for FETCH_SIZE / WRITE_SIZE)
  python bench.py --traffic-from DIR --workload W
                                      turn the four rocprofv3 --pmc CSVs under DIR
                                      (fetch/, write/, copy_fetch/, copy_write/) into
                                      profiles/traffic_<W>.json
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse_mla_fwd µs/call + tokens/s and % HBM/MFMA roofline at s_q=1/64/1024"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA (the output projection's arithmetic)
PAGES_US_SQ1 = 22.7            # pages' fused kernel at s_q = 1 (GB200, TP4, CUDA graph): context only
EXTRA = ["decode_sq64", "decode_sq1024", "prefill_sq2123", "decode_sq256", "prefill_sq184"]
TWO_POOL = ["decode_sq1", "decode_sq64", "decode_sq1024", "prefill_sq2123"]
FLUSH_BYTES = 1 << 30          # larger than the 256 MB MALL + 8 x 4 MB L2
CALLS_PER_GRAPH = 10           # warm replays hold this many back-to-back calls
MIN_COLD_SAMPLES = 50          # cold single-call replays per workload, whatever --steps is
SPIN_CYCLES = 500000           # GPU spin before each timed call: covers the host-side launch


def upload(inp, torch, device):
    t = {"q": torch.from_numpy(inp["q"].view(np.int16)).to(device).view(torch.bfloat16)}
    t["kv_pool"] = torch.from_numpy(inp["kv_pool"]).to(device)
    t["kv_scales"] = torch.from_numpy(inp["kv_scales"]).to(device)
    for k in ("indices", "topk_length", "positions"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.int32)).to(device)
    t["norm_w"] = torch.from_numpy(np.ascontiguousarray(inp["norm_w"], dtype=np.float32)).to(device)
    return t


def work_model(inp):
    """Algorithmic flops and bytes of one call (valid entries only)."""
    from prefill_token_amd import inputs

    s_q, h, d = inp["q"].shape
    nv = inputs.valid_rows(inp).astype(np.int64)
    row_bytes = d + d // 32
    flops = 4.0 * h * d * float(nv.sum())
    L = np.minimum(inp["topk_length"], inp["topk"])
    cols = np.arange(inp["topk"])[None, :]
    valid = (cols < L[:, None]) & (inp["indices"] >= 0)
    distinct = np.unique(inp["indices"][valid]).size
    per_tok_fixed = 2 * h * d + 4 * inp["topk"] + 8 + h * d + h * d // 32
    gathered = float(s_q * per_tok_fixed + row_bytes * nv.sum())
    compulsory = float(s_q * per_tok_fixed + row_bytes * distinct)
    return dict(flops=flops, gathered_bytes=gathered, compulsory_bytes=compulsory, valid_rows=int(nv.sum()),
                distinct_rows=int(distinct))


def upload_ds(inp, torch, device):
    t = {"q": torch.from_numpy(inp["q"].view(np.int16)).to(device).view(torch.bfloat16)}
    for k in ("swa_codes", "swa_scales", "cmp_codes", "cmp_scales"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(device)
    for k in ("indices", "topk_length", "positions"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.int32)).to(device)
    t["norm_w"] = torch.from_numpy(np.ascontiguousarray(inp["norm_w"], dtype=np.float32)).to(device)
    return t


def work_model_ds(inp):
    """Algorithmic flops and bytes of one two-pool call: SWA rows 512 + 16 bytes, compressed
    rows 256 + 32 bytes, distinct rows counted per pool."""
    s_q, h, d = inp["q"].shape
    L = np.minimum(inp["topk_length"], inp["topk"])
    cols = np.arange(inp["topk"])[None, :]
    valid = (cols < L[:, None]) & (inp["indices"] >= 0)
    swa = valid & (cols < inp["swa_entries"])
    cmp_ = valid & (cols >= inp["swa_entries"])
    swa_b, cmp_b = d + d // 32, d // 2 + d // 16
    nv = int(valid.sum())
    per_tok_fixed = 2 * h * d + 4 * inp["topk"] + 8 + h * d + h * d // 32
    gathered = float(s_q * per_tok_fixed + swa_b * swa.sum() + cmp_b * cmp_.sum())
    distinct_swa = np.unique(inp["indices"][swa]).size
    distinct_cmp = np.unique(inp["indices"][cmp_]).size
    compulsory = float(s_q * per_tok_fixed + swa_b * distinct_swa + cmp_b * distinct_cmp)
    return dict(flops=4.0 * h * d * nv, gathered_bytes=gathered, compulsory_bytes=compulsory, valid_rows=nv,
                distinct_rows=int(distinct_swa + distinct_cmp), swa_row_bytes=swa_b, cmp_row_bytes=cmp_b)


def kernel_names(s_q, ns, torch, device):
    """The kernels one call launches (d = 512 E4M3 pool, the persistent kernel's path)."""
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    if ns > 1:
        return "smla_ws + " + ("smla_combine_lm4" if ns <= 8 else "smla_combine_lm1")
    return "smla_order + smla_ws" if s_q > cus else "smla_ws"


class ColdTimer:
    """Cold single-call timing: flush the caches (1 GiB fill), synchronize, queue a short
    GPU spin, then an event, the replay, an event.  The spin keeps the GPU busy while the
    host submits the event and the replay, so the span holds the call and not the launch
    latency; the flush and the synchronization lie outside the span."""

    def __init__(self, torch, device):
        self.torch = torch
        self.flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=device)
        self.stream = torch.cuda.current_stream()
        try:
            torch.cuda._sleep(10)
            self.spin = True
        except Exception:  # pragma: no cover - torch builds without the spin kernel
            self.spin = False

    def run(self, replay, n):
        torch = self.torch
        out = []
        for _ in range(n):
            self.flush.zero_()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if self.spin:
                torch.cuda._sleep(SPIN_CYCLES)
            a.record(self.stream)
            replay()
            b.record(self.stream)
            b.synchronize()
            out.append(a.elapsed_time(b) * 1e3)
        return np.array(out)


def measure(name, steps, warmup, torch, device, cold_timer, timed_steps=None, two_pool=False):
    """Time one workload.  Returns (result dict, wall seconds of the timed steps, number of
    timed steps): the timed steps are cold single-call replays (timed_steps of them for the
    headline; at least MIN_COLD_SAMPLES for every workload), then warm graphs of 10 calls.
    two_pool: the same workload over the two-pool nvfp4_ds_mla cache (sparse_mla_fwd_ds_nvfp4)."""
    from prefill_token_amd import (inputs, make_params, sparse_mla_fwd, sparse_mla_fwd_ds_nvfp4,
                                   sparse_mla_num_splits, sparse_mla_profile_events, sparse_mla_workspace_size)

    inp = inputs.make_ds_nvfp4(name) if two_pool else inputs.make(name)
    t = upload_ds(inp, torch, device) if two_pool else upload(inp, torch, device)
    s_q, h, d = inp["q"].shape
    out_fp8 = torch.empty((s_q, h, d), dtype=torch.uint8, device=device)
    out_sc = torch.empty((s_q, h, d // 32), dtype=torch.uint8, device=device)
    p = make_params(s_q=s_q, h_q=h, d=d, rope_dim=inp["rope_dim"], topk=inp["topk"],
                    n_rows=inp["n_swa_rows"] if two_pool else inp["n_rows"],
                    kv_format=inputs.KV_E4M3_UE8M0 if two_pool else inp["kv_format"], sm_scale=inp["sm_scale"])
    ns, need = sparse_mla_num_splits(p), sparse_mla_workspace_size(p)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=device)  # counters start at zero

    def call():
        if two_pool:
            sparse_mla_fwd_ds_nvfp4(t["q"], t["swa_codes"], t["swa_scales"], t["cmp_codes"], t["cmp_scales"],
                                    t["indices"], t["topk_length"], t["positions"], t["norm_w"], out_fp8, out_sc,
                                    swa_entries=inp["swa_entries"], sm_scale=inp["sm_scale"],
                                    rope_dim=inp["rope_dim"], eps=inp["eps"], theta=inp["theta"],
                                    workspace=ws if need else None)
        else:
            sparse_mla_fwd(t["q"], t["kv_pool"], t["kv_scales"], t["indices"], t["topk_length"], t["positions"],
                           t["norm_w"], out_fp8, out_sc, sm_scale=inp["sm_scale"], rope_dim=inp["rope_dim"],
                           eps=inp["eps"], theta=inp["theta"], workspace=ws if need else None)

    for _ in range(max(warmup, 1)):
        call()
    torch.cuda.synchronize()
    eager_ref = (out_fp8.clone(), out_sc.clone())
    graph1 = torch.cuda.CUDAGraph()  # one call: the cold timed steps
    with torch.cuda.graph(graph1):
        call()
    graphg = torch.cuda.CUDAGraph()  # CALLS_PER_GRAPH back-to-back calls: warm figures
    with torch.cuda.graph(graphg):
        for _ in range(CALLS_PER_GRAPH):
            call()
    for g in (graph1, graphg):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_fp8, eager_ref[0]) and torch.equal(out_sc, eager_ref[1]), "graph replay differs"

    # cold: the timed steps, each one call launched directly on the stream (the GPU spin
    # queued before the first event hides the host's launch); the single-call graph
    # replays are measured the same way and reported beside them
    n = max(1, timed_steps if timed_steps is not None else MIN_COLD_SAMPLES)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cold = cold_timer.run(call, n)
    wall = time.perf_counter() - t0
    if n < MIN_COLD_SAMPLES:  # more samples for the reported distribution
        cold_all = np.concatenate([cold, cold_timer.run(call, MIN_COLD_SAMPLES - n)])
    else:
        cold_all = cold
    assert torch.equal(out_fp8, eager_ref[0]), "call after flush differs"
    cold_graph = cold_timer.run(graph1.replay, MIN_COLD_SAMPLES)
    assert torch.equal(out_fp8, eager_ref[0]), "replay after flush differs"

    # the main kernel on its own: the same cold protocol with the library's profiling
    # events armed (recorded on the launch stream just before the main kernel, between it
    # and the split combine, and after the call), in a pass of its own so that the timed
    # steps above carry no extra event records
    prof = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(MIN_COLD_SAMPLES)]
    for trio in prof:
        for e in trio:
            e.record()  # torch creates its events on first record
    torch.cuda.synchronize()
    used = [0]

    def armed_call():
        sparse_mla_profile_events(*prof[used[0]])
        used[0] += 1
        call()

    cold_timer.run(armed_call, MIN_COLD_SAMPLES)
    assert torch.equal(out_fp8, eager_ref[0]), "armed call differs"
    main_us = np.array([a.elapsed_time(b) * 1e3 for a, b, _ in prof])
    after_us = np.array([b.elapsed_time(c) * 1e3 for _, b, c in prof])

    # warm: graphs of CALLS_PER_GRAPH back-to-back calls, caches hot
    stream = torch.cuda.current_stream()
    reps = max(2, MIN_COLD_SAMPLES // CALLS_PER_GRAPH)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        graphg.replay()
        b.record(stream)
    torch.cuda.synchronize()
    warm = np.array([a.elapsed_time(b) * 1e3 / CALLS_PER_GRAPH for a, b in ev])

    wm = work_model_ds(inp) if two_pool else work_model(inp)
    cold_mean = float(cold.mean())
    cold_med = float(np.median(cold_all))
    warm_mean = float(warm.mean())
    res = dict(
        workload=name, description=inp["description"], s_q=s_q, num_splits=ns,
        kernels=("smla_nv" + (" + smla_combine<512>" if ns > 1 else "")) if two_pool
        else kernel_names(s_q, ns, torch, device),
        timing="cold: caches flushed before each call (one direct launch, a GPU spin queued before the first "
               "event), HIP events on the launch stream; graph_cold: the same with a one-call graph replay",
        cold_samples=int(cold_all.size),
        us_per_call_median=cold_med, us_per_call_p10=float(np.percentile(cold_all, 10)),
        us_per_call_p90=float(np.percentile(cold_all, 90)), us_per_call_mean=float(cold_all.mean()),
        us_per_call_timed_mean=cold_mean,
        us_per_call_graph_cold_median=float(np.median(cold_graph)),
        main_kernel="smla_nv" if two_pool else "smla_ws",
        main_kernel_cold_us_mean=float(main_us.mean()), main_kernel_cold_us_median=float(np.median(main_us)),
        after_main_cold_us_mean=float(after_us.mean()),
        main_kernel_bytes=wm["compulsory_bytes"] - (s_q * (h * d + h * d // 32) if ns > 1 else 0),
        us_per_call_warm_mean=warm_mean, us_per_call_warm_median=float(np.median(warm)),
        calls_per_warm_graph=CALLS_PER_GRAPH,
        tokens_per_s=s_q / (cold_med * 1e-6), tokens_per_s_warm=s_q / (warm_mean * 1e-6),
        hbm_compulsory_GBs=wm["compulsory_bytes"] / (cold_med * 1e-6) / 1e9,
        hbm_compulsory_frac=wm["compulsory_bytes"] / (cold_med * 1e-6) / 1e9 / HBM_PEAK_GBS,
        gather_effective_GBs=wm["gathered_bytes"] / (cold_med * 1e-6) / 1e9,
        mfma_TFLOPs=wm["flops"] / (cold_med * 1e-6) / 1e12,
        mfma_frac=wm["flops"] / (cold_med * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS,
        hbm_compulsory_frac_warm=wm["compulsory_bytes"] / (warm_mean * 1e-6) / 1e9 / HBM_PEAK_GBS,
        mfma_frac_warm=wm["flops"] / (warm_mean * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS,
        **wm,
    )
    return res, wall, n


def timing_overheads(torch, device, cold_timer):
    """What the cold protocol reads for no work: an empty event pair, and one tiny kernel
    (a 1024-element add) launched directly and as a one-kernel graph replay."""
    x = torch.zeros(1024, device=device)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        x.add_(1.0)
    torch.cuda.synchronize()
    return {"event_pair_us": float(np.median(cold_timer.run(lambda: None, MIN_COLD_SAMPLES))),
            "tiny_kernel_direct_us": float(np.median(cold_timer.run(lambda: x.add_(1.0), MIN_COLD_SAMPLES))),
            "tiny_kernel_graph_replay_us": float(np.median(cold_timer.run(g.replay, MIN_COLD_SAMPLES)))}


def measured_peaks(torch, device):
    """Device-copy bandwidth (bytes read + written per second, a 1 GiB torch copy) and the
    MFMA-loop rates of libsmla_probe.so (bf16 and E4M3), median of 5 launches each."""
    import ctypes

    out = {}
    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    out["copy_GBs"] = 2.0 * nbytes / float(np.median(ts)) / 1e9
    del src, dst
    try:
        from prefill_token_amd.build import PROBE_LIB_PATH

        lib = ctypes.CDLL(PROBE_LIB_PATH)
        lib.smla_probe_mfma.restype = ctypes.c_double
        lib.smla_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        cus = torch.cuda.get_device_properties(device).multi_processor_count
        blocks = 2 * cus  # two 4-wave workgroups per CU: two waves per SIMD
        buf = torch.empty(blocks, dtype=torch.float32, device=device)
        stream = torch.cuda.current_stream().cuda_stream
        for kind, key, iters in ((0, "mfma_bf16_TFLOPs", 4000), (1, "mfma_fp8_TFLOPs", 2000)):
            flops = lib.smla_probe_mfma(kind, iters, blocks, stream, buf.data_ptr())
            torch.cuda.synchronize()
            ts = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                flops = lib.smla_probe_mfma(kind, iters, blocks, stream, buf.data_ptr())
                b.record()
                b.synchronize()
                ts.append(a.elapsed_time(b) * 1e-3)
            if flops > 0:
                out[key] = flops / float(np.median(ts)) / 1e12
    except OSError:
        pass
    out["note"] = ("copy: 1 GiB device copy, read + write bytes / time; MFMA: 8 independent accumulator chains per "
                   "wave, two waves per SIMD, v_mfma_f32_32x32x16_bf16 / v_mfma_scale_f32_32x32x64_f8f6f4")
    return out


def measure_insert(name, steps, torch, device):
    """Time the KV insert (the pool-row producer) on one insert workload.

    Algorithmic bytes per token: the bf16 latent read (2 d), its position (4), the E4M3
    row and its UE8M0 scales written (d + d/32); plus norm_w (4 d) once per call."""
    from prefill_token_amd import inputs, sparse_mla_kv_insert

    c = inputs.make_insert(name)
    kv = torch.from_numpy(c["kv"].view(np.int16)).to(device).view(torch.bfloat16)
    pos = torch.from_numpy(c["positions"]).to(device)
    w = torch.from_numpy(c["norm_w"]).to(device)
    pool = torch.from_numpy(c["kv_pool"]).to(device)
    sc = torch.from_numpy(c["kv_scales"]).to(device)

    def call():
        sparse_mla_kv_insert(kv, pos, w, pool, sc, rope_dim=c["rope_dim"], n_swa=c["n_swa"], eps=c["eps"],
                             theta=c["theta"])

    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(CALLS_PER_GRAPH):
            call()
    stream = torch.cuda.current_stream()
    reps = max(1, steps // CALLS_PER_GRAPH)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    g.replay()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 / CALLS_PER_GRAPH for a, b in ev])
    n, d = c["n"], c["d"]
    nbytes = float(n * (2 * d + 4 + d + d // 32) + 4 * d)
    mean_us = float(us.mean())
    return dict(workload=name, kernel="kv_insert_kernel", tokens=n, us_per_call_mean=mean_us,
                us_per_call_median=float(np.median(us)), tokens_per_s=n / (mean_us * 1e-6),
                bytes_per_call=nbytes, hbm_GBs=nbytes / (mean_us * 1e-6) / 1e9,
                hbm_frac=nbytes / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS)


def measure_index(name, steps, torch, device):
    """Time the index-row builder on one workload.  Algorithmic bytes per token: the
    valid candidate logits read (2 n_valid), the position and n_valid (8), the index row
    and its length written (4 topk + 4)."""
    from prefill_token_amd import inputs, sparse_mla_build_index

    c = inputs.make_index(name)
    pos = torch.from_numpy(c["positions"]).to(device)
    lg = torch.from_numpy(c["logits"].view(np.int16)).to(device).view(torch.bfloat16)
    nv = torch.from_numpy(c["n_valid"]).to(device)
    idx = torch.empty((c["n"], c["topk"]), dtype=torch.int32, device=device)
    L = torch.empty((c["n"],), dtype=torch.int32, device=device)

    def call():
        sparse_mla_build_index(pos, lg, nv, idx, L, window=c["window"], self_in_window=c["self_in_window"],
                               n_swa=c["n_swa"], cmp_base=c["cmp_base"], k_cmp=c["k_cmp"])

    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(CALLS_PER_GRAPH):
            call()
    stream = torch.cuda.current_stream()
    reps = max(1, steps // CALLS_PER_GRAPH)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    g.replay()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 / CALLS_PER_GRAPH for a, b in ev])
    n = c["n"]
    nbytes = float(2 * np.minimum(c["n_valid"], c["n_cand"]).sum() + n * (8 + 4 * c["topk"] + 4))
    mean_us = float(us.mean())
    kernel = ("build_index_reg<16, 256>" if c["n_cand"] <= 4096 else
              "build_index_reg<64, 256>" if c["n_cand"] <= 16384 else "build_index_kernel")
    return dict(workload=name, kernel=kernel, tokens=n, n_cand=c["n_cand"], us_per_call_mean=mean_us,
                us_per_call_median=float(np.median(us)), tokens_per_s=n / (mean_us * 1e-6), bytes_per_call=nbytes,
                hbm_GBs=nbytes / (mean_us * 1e-6) / 1e9, hbm_frac=nbytes / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS)


def measure_wo_a(name, steps, torch, device):
    """Time the output projection (wo_a) on one workload.  Algorithmic bytes: the E4M3
    input and its scales (528 per token and head), the weight and its scales (read once),
    the bf16 output; flops 2 * tokens * heads * 512 * d_out."""
    from prefill_token_amd import inputs, sparse_mla_wo_a

    c = inputs.make_wo_a(name)
    x = torch.from_numpy(c["x"]).to(device)
    xs = torch.from_numpy(c["x_scales"]).to(device)
    w = torch.from_numpy(c["w"]).to(device)
    ws = torch.from_numpy(c["w_scales"]).to(device)
    G = c["h"] // c["heads_per_group"]
    y = torch.empty((c["n"], G, c["d_out"]), dtype=torch.bfloat16, device=device)

    def call():
        sparse_mla_wo_a(x, xs, w, ws, y, heads_per_group=c["heads_per_group"])

    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(CALLS_PER_GRAPH):
            call()
    stream = torch.cuda.current_stream()
    reps = max(1, steps // CALLS_PER_GRAPH)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    g.replay()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 / CALLS_PER_GRAPH for a, b in ev])
    n, h, dout = c["n"], c["h"], c["d_out"]
    nbytes = float(n * h * 528 + G * dout * c["heads_per_group"] * 528 + n * G * dout * 2)
    flops = 2.0 * n * h * 512 * dout
    mean_us = float(us.mean())
    return dict(workload=name, kernel="wo_a_kernel", tokens=n, heads=h, heads_per_group=c["heads_per_group"],
                d_out=dout, us_per_call_mean=mean_us, us_per_call_median=float(np.median(us)),
                tokens_per_s=n / (mean_us * 1e-6), bytes_per_call=nbytes, flops_per_call=flops,
                hbm_GBs=nbytes / (mean_us * 1e-6) / 1e9, hbm_frac=nbytes / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                mfma_TFLOPs=flops / (mean_us * 1e-6) / 1e12,
                mfma_frac_fp8=flops / (mean_us * 1e-6) / 1e12 / MFMA_FP8_PEAK_TFLOPS)


def _oracle_run(inp):
    import oracle

    args = (inp["q"], inp["kv_pool"], inp["kv_scales"], inp["indices"], inp["topk_length"], inp["positions"],
            inp["norm_w"])
    kw = dict(sm_scale=inp["sm_scale"], eps=inp["eps"], theta=inp["theta"], rope_dim=inp["rope_dim"])
    return oracle.sparse_mla(*args, **kw)


def oracle_median(inp, min_seconds=0.0):
    """Median wall time of 3 oracle runs over a workload's own arrays; a run repeats the
    whole workload until it lasts min_seconds (so that one-token workloads are timed over
    many repetitions).  Returns (seconds per workload, repetitions per run, runs)."""
    runs, reps = [], 1
    t0 = time.perf_counter()
    _oracle_run(inp)
    one = time.perf_counter() - t0
    if min_seconds > 0 and one < min_seconds:
        reps = int(math.ceil(min_seconds / max(one, 1e-6)))
    for _ in range(3):
        t0 = time.perf_counter()
        for _ in range(reps):
            _oracle_run(inp)
        runs.append((time.perf_counter() - t0) / reps)
    return float(np.median(runs)), reps, runs


def cpu_baseline(head_name, configs, torch, device, seconds):
    """The oracle (as it stands) on the host cores: the headline workload's own arrays
    (median of 3 runs, each repeating the workload for about seconds / 3), and every config
    workload's own arrays (median of 3 runs).  Also the headline's GPU-vs-oracle pre-quant
    error on those arrays."""
    import oracle
    from prefill_token_amd import inputs, sparse_mla_fwd

    inp = inputs.make(head_name)
    per, reps, runs = oracle_median(inp, min_seconds=seconds / 3.0)
    o, _, _ = _oracle_run(inp)
    t = upload(inp, torch, device)
    out_fp8 = torch.empty(inp["q"].shape, dtype=torch.uint8, device=device)
    out_sc = torch.empty(inp["q"].shape[:2] + (inp["d"] // 32,), dtype=torch.uint8, device=device)
    out_f32 = torch.empty(inp["q"].shape, dtype=torch.float32, device=device)
    sparse_mla_fwd(t["q"], t["kv_pool"], t["kv_scales"], t["indices"], t["topk_length"], t["positions"],
                   t["norm_w"], out_fp8, out_sc, out_f32=out_f32, sm_scale=inp["sm_scale"], eps=inp["eps"],
                   theta=inp["theta"], rope_dim=inp["rope_dim"])
    torch.cuda.synchronize()
    g = out_f32.cpu().numpy().astype(np.float64)
    blk = o.reshape(*o.shape[:-1], -1, 32)
    amax = np.abs(blk).max(-1)
    err = np.abs(g.reshape(blk.shape) - blk).max(-1) / np.maximum(amax, 1e-300)
    cores = oracle.num_threads()
    head = {
        "value": inp["s_q"] / per, "unit": "tokens/s", "cores": min(cores, max(inp["s_q"], 1)), "kind": "oracle",
        "sample": f"the {head_name} workload's own arrays ({inp['s_q']} token(s)); median of 3 runs of {reps} "
                  f"repetition(s) each ({sum(runs) * reps:.1f} s in all); OpenMP over tokens",
        "seconds_per_call": per, "gpu_vs_oracle_max_rel_block_err": float(err.max()),
    }
    per_cfg = []
    for name in configs:
        c = inputs.make(name)
        sec, _, runs = oracle_median(c)
        per_cfg.append({"workload": name, "s_q": c["s_q"], "seconds_median_of_3": sec,
                        "runs_s": runs, "tokens_per_s": c["s_q"] / sec,
                        "cores": min(cores, c["s_q"])})
    return head, per_cfg


def host_info():
    info = {"nproc": os.cpu_count(), "machine": platform.machine()}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
    except Exception:
        pass
    return info


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "prefill_token_amd", "csrc")
    for fn in sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".cpp", ".h"))):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(digest, workload, kernel=None):
    """HBM bytes per launch of one kernel (or per call, all kernels) from the committed
    rocprofv3 counter summary of this workload, if it was taken on the current kernel
    sources: scaled FETCH_SIZE + WRITE_SIZE medians."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_digest") != digest:
            return None
        if kernel is None:
            return float(rec["hbm_bytes_per_call"])
        k = rec["kernels"][kernel]
        return 1024.0 * (k["FETCH_SIZE_KiB_median"] * rec["FETCH_SIZE_copy_factor"] +
                         k["WRITE_SIZE_KiB_median"] * rec["WRITE_SIZE_copy_factor"])
    except Exception:
        return None


COPY_PROBE_REPS = 8


def copy_probe(mib):
    """A plain device copy of known size, for scaling the memory counters."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(COPY_PROBE_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "reps": COPY_PROBE_REPS}), flush=True)


def _counter_rows(folder, counter):
    import csv
    import glob

    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    rows = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def traffic_from(folder, copy_mib, workload):
    """HBM bytes per sparse_mla_fwd call of one workload from rocprofv3 --pmc runs:
    the median FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each of its kernels, each
    scaled by (known bytes / counter reading) of a plain copy of copy_mib MiB."""
    out = {"source_digest": source_digest(), "workload": workload, "copy_probe_mib": copy_mib, "kernels": {}}
    total = 0.0
    for counter, sub, csub in (("FETCH_SIZE", "fetch", "copy_fetch"), ("WRITE_SIZE", "write", "copy_write")):
        crow = [v for k, v in _counter_rows(os.path.join(folder, csub), counter) if "copy" in k.lower()]
        if not crow:
            raise SystemExit(f"no copy kernel rows for {counter}")
        factor = (copy_mib * 1024.0) / float(np.median(crow))
        out[f"{counter}_copy_factor"] = factor
        rows = _counter_rows(os.path.join(folder, sub), counter)
        for kname in ("smla_order", "smla_ws", "smla_combine"):
            vals = [v for k, v in rows if kname in k]
            if not vals:
                continue
            kib = float(np.median(vals))
            out["kernels"].setdefault(kname, {})[counter + "_KiB_median"] = kib
            out["kernels"][kname]["dispatches"] = len(vals)
            total += kib * factor * 1024.0
    out["hbm_bytes_per_call"] = total
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_sq1")
    ap.add_argument("--extra", default=",".join(EXTRA), help="comma-separated workloads after the timed region")
    ap.add_argument("--two-pool", default=",".join(TWO_POOL),
                    help="comma-separated workloads measured over the two-pool nvfp4_ds_mla cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-insert", action="store_true",
                    help="skip the KV-insert and index-row-builder measurements")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB")
    ap.add_argument("--traffic-from", default="", metavar="DIR")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.traffic_from:
        traffic_from(args.traffic_from, 256, args.workload)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only: the step runs on a single MI355X and "
                                   "has no multi-GPU path; run with --gpus 1"}), flush=True)
        sys.exit(2)

    import torch

    from prefill_token_amd import _lib

    _lib.load()  # fails loudly when the HIP library has not been built
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    cold_timer = ColdTimer(torch, device)

    head, wall, n = measure(args.workload, args.steps, args.warmup, torch, device, cold_timer,
                            timed_steps=args.steps)
    configs = [head]
    for name in [x for x in args.extra.split(",") if x and x != args.workload]:
        r, _, _ = measure(name, args.steps, args.warmup, torch, device, cold_timer)
        configs.append(r)
    for r in configs:
        print(f"# {r['workload']}: cold {r['us_per_call_median']:.2f} us/call (p10 {r['us_per_call_p10']:.2f}, "
              f"p90 {r['us_per_call_p90']:.2f}), warm {r['us_per_call_warm_mean']:.2f} us, "
              f"{r['tokens_per_s']:.4g} tok/s, HBM {100 * r['hbm_compulsory_frac']:.1f}%, "
              f"MFMA {100 * r['mfma_frac']:.1f}%", file=sys.stderr, flush=True)
    two_pool = []
    for name in [x for x in args.two_pool.split(",") if x]:
        r, _, _ = measure(name, args.steps, args.warmup, torch, device, cold_timer, two_pool=True)
        two_pool.append(r)
        print(f"# {name} two-pool nvfp4: cold {r['us_per_call_median']:.2f} us/call, warm "
              f"{r['us_per_call_warm_mean']:.2f} us, {r['tokens_per_s']:.4g} tok/s, "
              f"HBM {100 * r['hbm_compulsory_frac']:.1f}%, MFMA {100 * r['mfma_frac']:.1f}%", file=sys.stderr,
              flush=True)
    overheads = timing_overheads(torch, device, cold_timer)
    print(f"# cold-protocol overheads: {json.dumps(overheads)}", file=sys.stderr, flush=True)
    del cold_timer

    inserts = []
    if not args.no_insert:
        from prefill_token_amd import inputs

        for name in inputs.INSERT_WORKLOADS:
            r = measure_insert(name, args.steps, torch, device)
            inserts.append(r)
            print(f"# {name}: {r['us_per_call_mean']:.2f} us/call, {r['tokens_per_s']:.4g} tok/s, "
                  f"HBM {100 * r['hbm_frac']:.1f}%", file=sys.stderr, flush=True)

    builds = []
    if not args.no_insert:
        from prefill_token_amd import inputs

        for name in inputs.INDEX_WORKLOADS:
            r = measure_index(name, args.steps, torch, device)
            builds.append(r)
            print(f"# {name}: {r['us_per_call_mean']:.2f} us/call, {r['tokens_per_s']:.4g} tok/s, "
                  f"HBM {100 * r['hbm_frac']:.1f}%", file=sys.stderr, flush=True)

    projs = []
    if not args.no_insert:
        from prefill_token_amd import inputs

        for name in inputs.WO_A_WORKLOADS:
            r = measure_wo_a(name, args.steps, torch, device)
            projs.append(r)
            print(f"# {name}: {r['us_per_call_mean']:.2f} us/call, {r['tokens_per_s']:.4g} tok/s, "
                  f"HBM {100 * r['hbm_frac']:.1f}%, MFMA(fp8) {100 * r['mfma_frac_fp8']:.1f}%", file=sys.stderr,
                  flush=True)

    peaks = measured_peaks(torch, device)
    print(f"# measured peaks: {json.dumps(peaks)}", file=sys.stderr, flush=True)
    digest = source_digest()
    traffic = load_traffic(digest, head["workload"], head["main_kernel"])
    mean_us = head["us_per_call_timed_mean"]
    k_us, k_bytes = head["main_kernel_cold_us_mean"], head["main_kernel_bytes"]
    achieved = k_bytes / (k_us * 1e-6) / 1e9
    call_gbs = head["compulsory_bytes"] / (mean_us * 1e-6) / 1e9
    roofline = {
        "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
        "traffic": traffic, "kernel": head["main_kernel"],
        "scope": "the dominant kernel alone, cold (caches flushed before each call): its algorithmic bytes (q, "
                 "index row, positions, distinct pool rows and scales; the FP8 output is written by the split "
                 "combine) over its mean span between the library's profiling events, recorded on its stream "
                 "just before and just after it (the span includes the event overhead, timing_overheads)",
        "bytes_per_launch": k_bytes, "mean_us": k_us,
        "whole_call": {"kernels": head["kernels"], "bytes": head["compulsory_bytes"], "mean_us": mean_us,
                       "achieved_GBs": call_gbs, "frac": call_gbs / HBM_PEAK_GBS,
                       "traffic": load_traffic(digest, head["workload"])},
        "peak_measured_copy_GBs": peaks.get("copy_GBs"),
        "frac_of_measured_copy": achieved / peaks["copy_GBs"] if peaks.get("copy_GBs") else None,
    }
    cpu, cpu_cfg = None, None
    if not args.no_cpu_baseline:
        cpu, cpu_cfg = cpu_baseline(args.workload, [c["workload"] for c in configs[1:4]], torch, device,
                                    args.cpu_seconds)
    value = head["s_q"] / (mean_us * 1e-6)
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": wall / n * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": value / (1e6 / PAGES_US_SQ1),
        "vs_baseline_note": "value / (1 / 22.7 us): the pages' fused kernel at s_q=1 on GB200 TP4 (context, "
                            "another machine)",
        "value_note": "s_q / the mean span of the K timed steps; each step flushes the caches and synchronizes "
                      "outside the span, then launches one call directly behind a GPU spin (ms_per_step is the "
                      "wall time of a whole step, flush included); a one-call graph replay reads more, by the "
                      "runtime's graph-launch overhead (timing_overheads, us_per_call_graph_cold_median)",
        "timing_overheads": overheads,
        "dtype": "e4m3+bf16", "data": "synthetic",
        "dtype_note": "QK^T on E4M3 MFMAs (q split into two E4M3 terms with UE8M0 scales), P.V on bf16 "
                      "MFMAs, f32 accumulation and softmax",
        "config": {"workload": head["description"], "name": head["workload"], "s_q": head["s_q"],
                   "num_splits": head["num_splits"], "graph": True, "timing": "cold"},
        "roofline": roofline, "cpu_baseline": cpu, "cpu_oracle_configs": cpu_cfg, "measured_peaks": peaks,
        "configs": configs,
        "two_pool_nvfp4": two_pool,
        "two_pool_note": "the same workloads over the nvfp4_ds_mla cache: SWA rows E4M3 + UE8M0 (528 B), "
                         "compressed rows NVFP4 (256 B of E2M1 pairs + 32 E4M3 scales = 288 B), one smla_nv "
                         "launch (bf16 MFMAs) plus the split combine",
        "kv_insert": inserts, "build_index": builds, "wo_a": projs,
        "device": torch.cuda.get_device_name(device), "host": host_info(), "source_digest": digest,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
