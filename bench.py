"""Benchmark of the paged K/V-cache path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads prefill,fp8prefill,shared,fp8,commit]
                    [--no-cpu-baseline]

Prints ONE JSON line.  The headline workload is the bf16 GQA decode (64
sequences, lengths uniform in [512, 4096], 32 q / 8 kv heads of 128, 32-token
pages in a 16384-page pool): one step = one ``pkv_attn_decode_append`` call,
whose decode kernel writes the step's 64 new tokens into their slots and then
attends, inputs resident in HBM.  ``value`` is the step's algorithmic bytes
(K/V of every valid token once per kv head, Q, O, the table entries and
lengths read, the new tokens read and written) over the measured step time.

The other workloads (block-causal prefill, shared-prefix n-sample decode,
long fp8 decode) are measured in the same run and reported under
``"workloads"``; each timed step there is bracketed by HIP events on the
launch stream with a 512 MiB read between steps (outside the events) so
their working sets cannot stay in the 256 MiB Infinity Cache.

``roofline`` describes the dominant call of the headline (the decode), timed
with HIP events on the launch stream around each call of a second run of
``--steps`` steps after the timed region (events inside it would add their own
cost to the wall-clock step); ``cpu_baseline``
times the float64 CPU oracle on whole steps of the same headline batch.

Every timed workload is first checked against the float64 oracle on its own
output (the whole output, every row), within the tolerances the path is held
to (bf16: 2e-2 abs + 2e-2 rel on outputs; fp8 K/V: 6e-2 + 6e-2; LSE 2e-2 /
6e-2 absolute; integer and byte results bit-exact).  A workload that fails is
reported with its error and no figures; a failing headline prints no value and
exits with status 1.  Each workload entry carries ``parity_max_err``, the
oracle's own seconds on that workload (``oracle_s``) and the host cores it was
given (``cores``: BLAS threads = the process's CPU affinity).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
ORACLE_CORES = len(os.sched_getaffinity(0))   # BLAS threads given to the oracle
# output tolerances |gpu - ref| <= atol + rtol |ref|, and the absolute LSE bound
OUT_TOL = {"bf16": (2e-2, 2e-2), "fp8": (6e-2, 6e-2)}
LSE_TOL = {"bf16": 2e-2, "fp8": 6e-2}
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense fp8

# HBM byte counters of the decode call, taken by separate rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE) and scaled by what the same counters read for a
# copy of known size.  Valid only while the decode sources hash to the value
# recorded with them; otherwise ``roofline.traffic`` is null.
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_gqa_bf16_hbm_counters.txt")
DECODE_SOURCES = ["paged_kv_cache_slots_amd/csrc/decode.hip", "paged_kv_cache_slots_amd/csrc/pkv_device.hpp",
                  "paged_kv_cache_slots_amd/csrc/pkv_internal.hpp", "paged_kv_cache_slots_amd/csrc/pkv_api.hip"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workloads", default="prefill,fp8prefill,shared,fp8,commit",
                    help="secondary workloads to run: comma list of prefill, fp8prefill, shared, fp8, commit (or none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device copies of MIB MiB (calibrates the HBM byte counters) and exit")
    return ap.parse_args()


# ----------------------------------------------------------------------------- helpers

def decode_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per decode call from the committed counter summary, or None
    when it is missing or was taken on other decode sources."""
    try:
        kv = {}
        with open(COUNTERS_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != decode_sources_sha256():
            return None
        return int(kv["traffic_bytes_per_call"])
    except (OSError, KeyError, ValueError):
        return None


class ParityError(RuntimeError):
    pass


def oracle_threads():
    """Context in which numpy's BLAS uses every core of this process's affinity."""
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=ORACLE_CORES)


def bf16_to_f64(t):
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
            np.float64)
    return t.numpy().astype(np.float64)


def check_out(got, ref, tol, what):
    """Max |got - ref| after checking every element against the tolerance."""
    atol, rtol = OUT_TOL[tol]
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if got.shape != ref.shape:
        raise ParityError(f"{what}: shape {got.shape} != {ref.shape}")
    if not np.all(np.isfinite(got)):
        raise ParityError(f"{what}: non-finite values in the GPU output")
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if np.any(bad):
        raise ParityError(f"{what}: {int(bad.sum())} of {err.size} values outside tolerance (max err "
                          f"{err.max():.3g})")
    return float(err.max()) if err.size else 0.0


def check_lse(got, ref, tol, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    inf = np.isinf(ref)
    if not (np.array_equal(np.isinf(got), inf) and np.array_equal(got[inf], ref[inf])):
        raise ParityError(f"{what}: infinities differ")
    err = np.abs(got[~inf] - ref[~inf])
    if err.size and (np.isnan(err).any() or err.max() > LSE_TOL[tol]):
        raise ParityError(f"{what}: LSE off by {np.nanmax(err):.3g} > {LSE_TOL[tol]}")
    return float(err.max()) if err.size else 0.0


def timed_oracle(fn):
    """Run an oracle computation on every core; returns (result, seconds)."""
    with oracle_threads():
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0


def to_dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda:0")


def decode_bytes(kv_lens, page_size, hkv, d, kv_esize, n_rows_q, hq, q_esize, out_esize, with_lse, fp8_scales):
    """Algorithmic bytes of one decode call: every valid K/V element once per kv
    head, the used fp8 scales, Q, O, LSE, the table entries and lengths."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    pages = np.ceil(kv_lens / page_size).astype(np.int64)
    b = 2 * int(kv_lens.sum()) * hkv * d * kv_esize
    if fp8_scales:
        b += 2 * int(pages.sum()) * hkv * 4
    b += n_rows_q * hq * d * (q_esize + out_esize)
    if with_lse:
        b += n_rows_q * hq * 4
    b += int(pages.sum()) * 4 + len(kv_lens) * 4
    return b


def prefill_flops(seq_len, n_ctx, causal_block_size, d, hq):
    """Algorithmic flops of one batch entry of the block-causal prefill: QK^T
    and PV, 2 flops per multiply-add each, over the keys every real query
    sees (n_ctx + the end of its causal block; padding rows count nothing)."""
    cbs = causal_block_size or seq_len
    vis = sum(n_ctx + min((i // cbs + 1) * cbs, seq_len) for i in range(seq_len))
    return 4.0 * d * hq * vis


class Flusher:
    """Reads 512 MiB between steps (a read, so no dirty lines are left to write
    back) so the next step finds none of its inputs in the 256 MiB Infinity Cache."""

    def __init__(self, torch):
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")

    def __call__(self):
        self.buf.sum()


def time_kernel_events(torch, pkv, step, reps, flush=None):
    """Median (ms) of a call's main kernel alone: the library launches it with
    a start / stop event pair (hipExtLaunchKernel), which take the kernel's own
    start and end times."""
    times = []
    for _ in range(reps):
        if flush:
            flush()
        ks, ke = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ks.record()     # creates the events; the launch sets them again
        ke.record()
        pkv.pkv_set_timing_events(ks, ke)
        try:
            step()
        finally:
            pkv.pkv_set_timing_events(None, None)
        torch.cuda.synchronize()
        times.append(ks.elapsed_time(ke))
    return float(np.median(times))


def time_events(torch, step, reps, flush=None):
    """Median/p10/p90 of per-step times (ms) from HIP events on the current stream."""
    times = []
    for _ in range(reps):
        if flush:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    t = np.array(times)
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


# ----------------------------------------------------------------------------- headline: bf16 GQA paged decode

def setup_decode_case(case, torch, pkv):
    pool = pkv.Pool(to_dev(case.pool.k, torch), to_dev(case.pool.v, torch),
                    None if case.pool.k_scale is None else to_dev(case.pool.k_scale, torch),
                    None if case.pool.v_scale is None else to_dev(case.pool.v_scale, torch))
    t, n, hq, d = case.q.shape
    dev = dict(
        pool=pool, q=to_dev(case.q, torch), tables=to_dev(case.tables, torch), lens=to_dev(case.kv_lens, torch),
        out=torch.empty((t, n, hq, d), dtype=torch.bfloat16, device="cuda:0"),
        ws=torch.empty(max(16, pkv.pkv_attn_decode_workspace_bytes(t, n, hq, case.pool.num_kv_heads, d,
                                                                    case.max_kv_len)),
                       dtype=torch.uint8, device="cuda:0"))
    if case.slots is not None:
        dev.update(new_k=to_dev(case.new_k, torch), new_v=to_dev(case.new_v, torch), slots=to_dev(case.slots, torch))
    return dev


def run_headline(args, torch, pkv, W):
    case = W.gqa_bf16_decode()
    dev = setup_decode_case(case, torch, pkv)
    hkv, d = case.pool.num_kv_heads, case.pool.head_dim
    t, n, hq, _ = case.q.shape
    # the step is one pkv_attn_decode_append call: its decode kernel reads the
    # 64 new tokens' K and V and writes them into their slots, then attends
    append_bytes = 2 * 2 * len(case.slots) * hkv * d * 2
    dec_bytes = decode_bytes(case.kv_lens, case.pool.page_size, hkv, d, 2, t * n, hq, 2, 2, False, False)
    kern_bytes = dec_bytes + append_bytes
    step_bytes = kern_bytes
    ev = []

    def step(record=False, kernel=False):
        if record:
            # a: before the call; b: after it.  With `kernel`, the library
            # launches the decode kernel with the pair (ks, ke), which take
            # that kernel's own start and end (not the merge kernel of the
            # split units); calls and kernels are timed in steps of their own.
            a, ks, ke, b = (torch.cuda.Event(enable_timing=True) for _ in range(4))
            if kernel:
                ks.record()     # creates the events; the launch sets them again
                ke.record()
            a.record()
            if kernel:
                pkv.pkv_set_timing_events(ks, ke)
        pkv.pkv_attn_decode_append(dev["pool"], dev["new_k"], dev["new_v"], dev["q"], dev["tables"], dev["lens"],
                                   case.max_kv_len, case.sm_scale, dev["out"], None, dev["ws"])
        if record:
            if kernel:
                pkv.pkv_set_timing_events(None, None)
            b.record()
            ev.append((a, (ks, ke) if kernel else None, b))

    # parity gate: the first step's output against the oracle (whole batch)
    import oracle as orc
    step()
    torch.cuda.synchronize()
    got = bf16_to_f64(dev["out"])

    def ref_step():
        kp = orc.scatter_slots(case.pool.k, case.new_k, case.slots)
        vp = orc.scatter_slots(case.pool.v, case.new_v, case.slots)
        return orc.attn_decode(kp, vp, case.q, case.tables, case.kv_lens, case.sm_scale)

    (ref, _), oracle_s = timed_oracle(ref_step)
    parity = {"parity_max_err": check_out(got, ref, "bf16", "headline decode"), "oracle_s": round(oracle_s, 3),
              "cores": ORACLE_CORES, "parity_rows": int(ref.shape[0] * ref.shape[1] * ref.shape[2])}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps: wall clock only (HIP events between the launches would
    # lengthen every step, by ~5 us for the pair around the decode call)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    # the decode call's own duration: the same number of steps again, with HIP
    # events on the launch stream around every call; then as many steps with
    # the decode kernel's own end recorded by the library
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    dec_ms = float(np.mean([a.elapsed_time(b) for a, _, b in ev]))
    ev.clear()
    for _ in range(args.steps):
        step(record=True, kernel=True)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([ks.elapsed_time(ke) for _, (ks, ke), _ in ev]))
    flushed = time_events(torch, lambda: step(), 20, Flusher(torch))
    return case, dict(step_bytes=step_bytes, dec_bytes=kern_bytes, ms_per_step=wall * 1e3, decode_ms=dec_ms,
                      decode_kernel_ms=kern_ms, append_bytes=append_bytes, flushed_step_ms=flushed, parity=parity)


# ----------------------------------------------------------------------------- secondary workloads

def run_prefill(torch, pkv, W, flush):
    case = W.block_causal_prefill()
    pool = pkv.Pool(to_dev(case.pool.k, torch), to_dev(case.pool.v, torch))
    qkv = to_dev(case.qkv, torch)                       # [1, S, Hq + 2 Hkv, D]
    hq, hkv, d = case.num_q_heads, case.num_kv_heads, qkv.shape[-1]
    s_q = case.s_q
    flat = qkv.view(s_q, hq + 2 * hkv, d)
    k_src, v_src = flat[:, hq:hq + hkv], flat[:, hq + hkv:]
    slots = to_dev(case.slots, torch)
    tables, n_ctx, seq = to_dev(case.tables, torch), to_dev(case.n_ctx, torch), to_dev(case.seq_len, torch)
    out = torch.empty((1, s_q, hq, d), dtype=torch.bfloat16, device="cuda:0")
    q = qkv[:, :, :hq]
    # workspace for the split leftover query tiles (contents ignored)
    ws = torch.empty(max(16, pkv.pkv_attn_prefill_workspace_bytes(1, s_q, hq, hkv, d, case.max_keys)),
                     dtype=torch.uint8, device="cuda:0")

    def scatter():
        pkv.pkv_scatter_slots(pool, k_src, v_src, slots)

    def prefill():
        pkv.pkv_attn_prefill_block_causal(pool, q, tables, n_ctx, seq, case.causal_block_size, case.max_keys,
                                          case.sm_scale, out, None, ws)

    try:
        scatter()
        prefill()
        torch.cuda.synchronize()
        got = bf16_to_f64(out)
        lse = torch.empty((1, s_q, hq), dtype=torch.float32, device="cuda:0")
        pkv.pkv_attn_prefill_block_causal(pool, q, tables, n_ctx, seq, case.causal_block_size, case.max_keys,
                                          case.sm_scale, out, lse, ws)
        torch.cuda.synchronize()
        got_lse = lse.cpu().numpy()
    except pkv.PkvError as e:
        return {"error": str(e)}
    import oracle as orc

    def ref_step():
        k_np, v_np = case.qkv.reshape(s_q, hq + 2 * hkv, d)[:, hq:hq + hkv], case.qkv.reshape(
            s_q, hq + 2 * hkv, d)[:, hq + hkv:]
        kp = orc.scatter_slots(case.pool.k, k_np, case.slots)
        vp = orc.scatter_slots(case.pool.v, v_np, case.slots)
        return orc.attn_prefill_block_causal(kp, vp, case.qkv[:, :, :hq], case.tables, case.n_ctx, case.seq_len,
                                             case.causal_block_size, case.sm_scale)

    (ref, ref_lse), oracle_s = timed_oracle(ref_step)
    try:
        parity = {"parity_max_err": check_out(got, ref, "bf16", "prefill out"),
                  "parity_max_lse_err": check_lse(got_lse, ref_lse, "bf16", "prefill lse"),
                  "oracle_s": round(oracle_s, 3), "cores": ORACLE_CORES}
    except ParityError as e:
        return {"error": f"parity failed: {e}"}
    for _ in range(5):
        prefill()
    seq_len, ctx = int(case.seq_len[0]), int(case.n_ctx[0])
    flops = prefill_flops(seq_len, ctx, case.causal_block_size, d, hq)
    parity["oracle_gflops"] = round(flops / oracle_s / 1e9, 2)
    med, p10, p90 = time_events(torch, prefill, 30, flush)
    kmed = time_kernel_events(torch, pkv, prefill, 30, flush)
    smed, _, _ = time_events(torch, scatter, 30, flush)
    both, _, _ = time_events(torch, lambda: (scatter(), prefill()), 30, flush)
    tflops = flops / (med * 1e-3) / 1e12
    scat_bytes = 2 * 2 * seq_len * hkv * d * 2 + seq_len * 8
    return {"workload": "bf16 block-causal prefill: 24 heads x 128, 1560 real queries (1568 rows) over a 1024 "
                        "prefix + 4096 history + own block, 32-token pages",
            "gflop": flops / 1e9, "prefill_ms": med, "prefill_ms_p10_p90": [p10, p90], "tflops": tflops,
            "frac_bf16_mfma_peak": tflops / BF16_MFMA_PEAK_TFLOPS,
            "prefill_kernel_ms": kmed, "kernel_frac_bf16_mfma_peak": flops / (kmed * 1e-3) / 1e12 /
            BF16_MFMA_PEAK_TFLOPS, "scatter_ms": smed,
            "scatter_gbs": scat_bytes / (smed * 1e-3) / 1e9, "scatter_plus_prefill_ms": both, **parity}


def run_fp8_prefill(torch, pkv, W, flush):
    """The block-causal prefill's geometry over an fp8 e4m3fn K/V pool (scale
    per page and kv head; every key resident), bf16 queries and output."""
    case = W.make_fp8_prefill_case("fp8_prefill", 3, 1003, 1, 1568, [1560], [5120], 24, 24, 128, 32, 1560,
                                   num_pool_pages=512)
    pool = pkv.Pool(to_dev(case.pool.k, torch), to_dev(case.pool.v, torch), to_dev(case.pool.k_scale, torch),
                    to_dev(case.pool.v_scale, torch))
    qkv = to_dev(case.qkv, torch)
    hq, hkv, d, s_q = case.num_q_heads, case.num_kv_heads, qkv.shape[-1], case.s_q
    tables, n_ctx, seq = to_dev(case.tables, torch), to_dev(case.n_ctx, torch), to_dev(case.seq_len, torch)
    out = torch.empty((1, s_q, hq, d), dtype=torch.bfloat16, device="cuda:0")
    q = qkv[:, :, :hq]
    ws = torch.empty(max(16, pkv.pkv_attn_prefill_workspace_bytes(1, s_q, hq, hkv, d, case.max_keys)),
                     dtype=torch.uint8, device="cuda:0")

    def prefill():
        pkv.pkv_attn_prefill_block_causal(pool, q, tables, n_ctx, seq, case.causal_block_size, case.max_keys,
                                          case.sm_scale, out, None, ws)

    try:
        prefill()
        torch.cuda.synchronize()
        got = bf16_to_f64(out)
        lse = torch.empty((1, s_q, hq), dtype=torch.float32, device="cuda:0")
        pkv.pkv_attn_prefill_block_causal(pool, q, tables, n_ctx, seq, case.causal_block_size, case.max_keys,
                                          case.sm_scale, out, lse, ws)
        torch.cuda.synchronize()
        got_lse = lse.cpu().numpy()
    except pkv.PkvError as e:
        return {"error": str(e)}
    import oracle as orc
    (ref, ref_lse), oracle_s = timed_oracle(lambda: orc.attn_prefill_block_causal(
        case.pool.k, case.pool.v, case.qkv[:, :, :hq], case.tables, case.n_ctx, case.seq_len,
        case.causal_block_size, case.sm_scale, kv_dtype="fp8", q_dtype="bf16", k_scale=case.pool.k_scale,
        v_scale=case.pool.v_scale))
    try:
        parity = {"parity_max_err": check_out(got, ref, "fp8", "fp8 prefill out"),
                  "parity_max_lse_err": check_lse(got_lse, ref_lse, "fp8", "fp8 prefill lse"),
                  "oracle_s": round(oracle_s, 3), "cores": ORACLE_CORES}
    except ParityError as e:
        return {"error": f"parity failed: {e}"}
    for _ in range(5):
        prefill()
    seq_len, ctx = int(case.seq_len[0]), int(case.n_ctx[0])
    flops = prefill_flops(seq_len, ctx, case.causal_block_size, d, hq)
    parity["oracle_gflops"] = round(flops / oracle_s / 1e9, 2)
    med, p10, p90 = time_events(torch, prefill, 30, flush)
    tflops = flops / (med * 1e-3) / 1e12
    # half the flops (QK^T) run on fp8 MFMA, half (PV) on bf16 MFMA: at both peaks
    # the mix would take F/2/5.0 + F/2/2.5 PFLOP-seconds, i.e. 3.33 PFLOP/s overall
    mixed_peak = 1.0 / (0.5 / FP8_MFMA_PEAK_TFLOPS + 0.5 / BF16_MFMA_PEAK_TFLOPS)
    return {"workload": "fp8 e4m3fn K/V block-causal prefill: 24 heads x 128, 1560 real queries (1568 rows) over "
                        "5120 cached keys + own block, 32-token pages; QK^T on fp8 MFMA from the raw K tile "
                        "(Q as hi + lo e4m3 codes), PV on bf16 MFMA over V widened in LDS",
            "gflop": flops / 1e9, "prefill_ms": med, "prefill_ms_p10_p90": [p10, p90], "tflops": tflops,
            "frac_bf16_mfma_peak": tflops / BF16_MFMA_PEAK_TFLOPS,
            "frac_mixed_mfma_peak": tflops / mixed_peak, **parity}


def run_shared_prefix(torch, pkv, W, flush):
    c = W.shared_prefix_decode()
    pool = pkv.Pool(to_dev(c.pool.k, torch), to_dev(c.pool.v, torch))
    new_k, new_v, slots = to_dev(c.new_k, torch), to_dev(c.new_v, torch), to_dev(c.slots, torch)
    n_rows, hq, d, hkv = c.q.shape[0], c.num_q_heads, c.pool.head_dim, c.pool.num_kv_heads
    g, s = c.num_groups, c.samples
    q = to_dev(c.q, torch)
    po = torch.empty((2, n_rows, hq, d), dtype=torch.float32, device="cuda:0")
    pl = torch.empty((2, n_rows, hq), dtype=torch.float32, device="cuda:0")
    out = torch.empty((n_rows, hq, d), dtype=torch.bfloat16, device="cuda:0")
    mp, mt = int(c.prefix_lens.max()), int(c.tail_lens.max())
    ws = torch.empty(max(16, pkv.pkv_attn_decode_workspace_bytes(g, s, hq, hkv, d, mp),
                         pkv.pkv_attn_decode_workspace_bytes(n_rows, 1, hq, hkv, d, mt)),
                     dtype=torch.uint8, device="cuda:0")
    pt, plen = to_dev(c.prefix_tables, torch), to_dev(c.prefix_lens, torch)
    tt, tlen = to_dev(c.tail_tables, torch), to_dev(c.tail_lens, torch)
    ft, flen = to_dev(c.full_tables, torch), to_dev(c.full_lens, torch)
    uout = torch.empty((n_rows, 1, hq, d), dtype=torch.bfloat16, device="cuda:0")
    mf = int(c.full_lens.max())
    ws2 = torch.empty(max(16, pkv.pkv_attn_decode_workspace_bytes(n_rows, 1, hq, hkv, d, mf)), dtype=torch.uint8,
                      device="cuda:0")

    def shared():
        pkv.pkv_scatter_slots(pool, new_k, new_v, slots)
        pkv.pkv_attn_decode(pool, q.view(g, s, hq, d), pt, plen, mp, c.sm_scale, po[0].view(g, s, hq, d),
                            pl[0].view(g, s, hq), ws)
        pkv.pkv_attn_decode(pool, q, tt, tlen, mt, c.sm_scale, po[1].view(n_rows, 1, hq, d),
                            pl[1].view(n_rows, 1, hq), ws)
        pkv.pkv_merge_states(po, pl, out)

    def unshared():
        pkv.pkv_scatter_slots(pool, new_k, new_v, slots)
        pkv.pkv_attn_decode(pool, q, ft, flen, mf, c.sm_scale, uout, None, ws2)

    fout = torch.empty((n_rows, 1, hq, d), dtype=torch.bfloat16, device="cuda:0")
    ws3 = torch.empty(pkv.pkv_attn_decode_shared_prefix_workspace_bytes(g, s, 1, hq, d, mp), dtype=torch.uint8,
                      device="cuda:0")

    # one call: the tail workgroups write the step's tokens (one per sample,
    # the tail's last key), then prefix + tail + merge
    def fused():
        pkv.pkv_attn_decode_shared_prefix_append(pool, new_k, new_v, q, s, pt, plen, mp, tt, tlen, mt, c.sm_scale,
                                                 fout, ws3)

    # parity gate: the merged, unshared and fused outputs of one step each
    # against the oracle's attention over the full (prefix + tail) tables
    import oracle as orc
    fused()     # first, on the pool whose step slots still hold poison
    shared()
    unshared()
    torch.cuda.synchronize()
    got_m, got_u, got_f = bf16_to_f64(out), bf16_to_f64(uout)[:, 0], bf16_to_f64(fout)[:, 0]

    def ref_step():
        kp = orc.scatter_slots(c.pool.k, c.new_k, c.slots)
        vp = orc.scatter_slots(c.pool.v, c.new_v, c.slots)
        return orc.attn_decode(kp, vp, c.q, c.full_tables, c.full_lens, c.sm_scale)

    (ref, _), oracle_s = timed_oracle(ref_step)
    try:
        parity = {"parity_max_err": max(check_out(got_m, ref[:, 0], "bf16", "prefix + tail + merge"),
                                        check_out(got_u, ref[:, 0], "bf16", "unshared decode"),
                                        check_out(got_f, ref[:, 0], "bf16", "fused n-sample step")),
                  "oracle_s": round(oracle_s, 3), "cores": ORACLE_CORES}
    except ParityError as e:
        return {"error": f"parity failed: {e}"}
    for _ in range(5):
        shared()
        unshared()
        fused()
    med, p10, p90 = time_events(torch, shared, 30, flush)
    umed, _, _ = time_events(torch, unshared, 30, flush)
    fmed, fp10, fp90 = time_events(torch, fused, 30, flush)
    pre = decode_bytes(c.prefix_lens, 32, hkv, d, 2, n_rows, hq, 2, 4, True, False)
    tail = decode_bytes(c.tail_lens, 32, hkv, d, 2, n_rows, hq, 2, 4, True, False)
    merge = 2 * n_rows * hq * (d + 1) * 4 + n_rows * hq * d * 2
    scat = 2 * 2 * n_rows * hkv * d * 2 + n_rows * 8
    total = pre + tail + merge + scat
    gbs = total / (med * 1e-3) / 1e9
    return {"workload": "shared-prefix n-sample decode: 8 prompts x 16 samples, 2048-token shared prefix, tails "
                        "U[1,512], 32/8 heads x 128, bf16 (scatter + prefix decode + tail decode + merge)",
            "algorithmic_mb": total / 1e6, "step_ms": med, "step_ms_p10_p90": [p10, p90], "gbs": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS,
            "fused_step_ms": fmed, "fused_step_ms_p10_p90": [fp10, fp90],
            "fused_gbs": total / (fmed * 1e-3) / 1e9, "fused_frac_hbm_peak": total / (fmed * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "fused_launches": 2, "unfused_launches": 6, "unshared_step_ms": umed,
            "unshared_mb": (decode_bytes(c.full_lens, 32, hkv, d, 2, n_rows, hq, 2, 2, False, False) + scat) / 1e6,
            "oracle_gbs": round(total / oracle_s / 1e9, 3), **parity}


def run_long_fp8(torch, pkv, W, flush):
    c = W.long_fp8_decode()
    dev = setup_decode_case(c, torch, pkv)
    t, n, hq, d = c.q.shape
    hkv = c.pool.num_kv_heads

    def step():
        pkv.pkv_attn_decode(dev["pool"], dev["q"], dev["tables"], dev["lens"], c.max_kv_len, c.sm_scale,
                            dev["out"], None, dev["ws"])

    # parity gate: every row against the oracle (which streams one sequence
    # at a time, so host memory stays bounded)
    import oracle as orc
    step()
    torch.cuda.synchronize()
    got = bf16_to_f64(dev["out"])
    (ref, _), oracle_s = timed_oracle(lambda: orc.attn_decode(
        c.pool.k, c.pool.v, c.q, c.tables, c.kv_lens, c.sm_scale, kv_dtype="fp8", q_dtype="bf16",
        k_scale=c.pool.k_scale, v_scale=c.pool.v_scale))
    try:
        parity = {"parity_max_err": check_out(got, ref, "fp8", "fp8 decode"), "oracle_s": round(oracle_s, 3),
                  "cores": ORACLE_CORES}
    except ParityError as e:
        return {"error": f"parity failed: {e}"}
    for _ in range(3):
        step()
    med, p10, p90 = time_events(torch, step, 20, flush)
    nbytes = decode_bytes(c.kv_lens, 32, hkv, d, 1, t * n, hq, 2, 2, False, True)
    parity["oracle_gbs"] = round(nbytes / oracle_s / 1e9, 3)
    gbs = nbytes / (med * 1e-3) / 1e9
    return {"workload": "fp8 decode: 256 sequences, lengths log-uniform in [1024, 32768], 64/8 heads x 128, "
                        "e4m3fn K/V with per-(page, kv head) scales, bf16 q/out",
            "algorithmic_gb": nbytes / 1e9, "decode_ms": med, "decode_ms_p10_p90": [p10, p90], "gbs": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS, **parity}


def commit_sequence(torch, pkv, flush):
    """One exact-window commit and one layer's forward-side writes at the
    block-causal prefill's geometry: fixed region 1024, window 4096, a
    1560-token chunk cut into three 520-token causal blocks, 32-token pages,
    24 kv heads x 128 bf16, 30 layers.  Commit = rotate the rolling table +
    lay out the blocks + copy committed keys into private pages (every
    layer); forward writes = scatter the chunk to its slots and private copies
    + copy earlier blocks' keys (one layer)."""
    ps, pin, window, sizes, layers, hkv, d = 32, 1024, 4096, [520, 520, 520], 30, 24, 128
    lay = pkv.CausalLayout(ps, pin, window, sizes, device="cuda:0")
    b = lay.bounds
    n_tab = b["fixed_pages"] + b["rolling_pages"]
    n_pages = n_tab + len(sizes) * b["private_pages"]
    ids = torch.randperm(n_pages, generator=torch.Generator().manual_seed(9)).to(torch.int32)
    table = ids[:n_tab].to("cuda:0")
    priv = ids[n_tab:].view(len(sizes), -1).to("cuda:0")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(10)
    k = torch.randn((layers, n_pages, ps, hkv, d), generator=g, device="cuda:0").to(torch.bfloat16)
    v = torch.randn((layers, n_pages, ps, hkv, d), generator=g, device="cuda:0").to(torch.bfloat16)
    pool = pkv.Pool(k[0], v[0])
    layer_stride = n_pages * ps * hkv * d
    committed = pin + window + 3 * 1560 + 17          # steady state, chunk start off a page boundary
    evicted = pkv.pkv_window_evicted_tokens(ps, pin, window, committed)
    shift = (evicted - pkv.pkv_window_evicted_tokens(ps, pin, window, committed - 1560)) // ps
    total = sum(sizes)
    new_k = torch.randn((total, hkv, d), generator=g, device="cuda:0").to(torch.bfloat16)
    new_v = torch.randn((total, hkv, d), generator=g, device="cuda:0").to(torch.bfloat16)

    def commit():
        pkv.pkv_rotate_rows(table[b["fixed_pages"]:], shift)
        pkv.pkv_causal_layout(lay, table, priv, committed, evicted)
        pkv.pkv_copy_slots(pool, lay.commit_src, lay.commit_dst, layers, layer_stride)

    def forward_writes():
        pkv.pkv_scatter_slots(pool, new_k, new_v, lay.stage_slots, slots2=lay.stage_slots2)
        pkv.pkv_copy_slots(pool, lay.current_src, lay.current_dst)

    # parity gate on the first commit and forward: the rotated table, every
    # layout tensor and the copied pool rows bit-exact against the oracle
    import oracle as orc

    def host(t):
        return t.cpu().view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.cpu().numpy()

    table0, priv0, k0, v0 = host(table), host(priv), host(k), host(v)
    commit()
    torch.cuda.synchronize()
    fp = b["fixed_pages"]
    t0 = time.perf_counter()
    with oracle_threads():
        want_table = table0.copy()
        want_table[fp:] = orc.rotate_rows(table0[None, fp:], shift)[0]
        want = orc.causal_layout(want_table, priv0, ps, pin, window, committed, evicted, sizes, b["table_width"],
                                 b["list_stride"])
        ok = np.array_equal(host(table), want_table)
        for name in ("block_tables", "n_ctx", "seq_len", "stage_slots", "stage_slots2", "commit_src", "commit_dst",
                     "current_src", "current_dst"):
            ok = ok and np.array_equal(host(getattr(lay, name)), want[name])
        k1 = orc.copy_slots(k0, want["commit_src"], want["commit_dst"])
        v1 = orc.copy_slots(v0, want["commit_src"], want["commit_dst"])
        ok = ok and np.array_equal(host(k), k1) and np.array_equal(host(v), v1)
        oracle_s = time.perf_counter() - t0
    forward_writes()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with oracle_threads():
        # one layer: scatter of the staged tokens to one or two slots, then the current copies
        k_l = orc.scatter_slots(k1[0], host(new_k), want["stage_slots"], slots2=want["stage_slots2"])
        v_l = orc.scatter_slots(v1[0], host(new_v), want["stage_slots"], slots2=want["stage_slots2"])
        k_l = orc.copy_slots(k_l[None], want["current_src"], want["current_dst"])[0]
        v_l = orc.copy_slots(v_l[None], want["current_src"], want["current_dst"])[0]
        ok = ok and np.array_equal(host(k[0]), k_l) and np.array_equal(host(v[0]), v_l)
        oracle_s += time.perf_counter() - t0
    del k0, v0, k1, v1, k_l, v_l
    if not ok:
        raise ParityError("exact-window commit or forward writes differ from the oracle")
    for _ in range(3):
        commit()
        forward_writes()
    cmed, cp10, cp90 = time_events(torch, commit, 30, flush)
    fmed, fp10, fp90 = time_events(torch, forward_writes, 30, flush)
    n_commit = int((lay.commit_src >= 0).sum())
    n_current = int((lay.current_src >= 0).sum())
    return {"commit_ms": cmed, "commit_ms_p10_p90": [cp10, cp90], "commit_copied_keys": n_commit,
            "forward_writes_ms": fmed, "forward_writes_ms_p10_p90": [fp10, fp90],
            "forward_current_copied_keys": n_current, "launches_per_commit": 3, "launches_per_forward_layer": 2,
            "parity": "bit-exact", "oracle_s": round(oracle_s, 3), "cores": ORACLE_CORES}


def run_commit(torch, pkv, W, flush):
    """Exact-window commit ops at the block-causal prefill's geometry (24 kv
    heads x 128, bf16, 32-token pages, 512-page pool): a private-page fill of
    2048 slots in each of 8 layers, and the rotation of the page-table row."""
    layers, pages, ps, hkv, d = 8, 512, 32, 24, 128
    g = torch.Generator(device="cuda:0")
    g.manual_seed(7)
    k = torch.randn((layers, pages, ps, hkv, d), generator=g, device="cuda:0").to(torch.bfloat16)
    v = torch.randn((layers, pages, ps, hkv, d), generator=g, device="cuda:0").to(torch.bfloat16)
    pool = pkv.Pool(k[0], v[0])
    perm = torch.randperm(pages * ps, generator=torch.Generator().manual_seed(8))
    src = perm[:2048].to("cuda:0", torch.int64)
    dst = perm[2048:4096].to("cuda:0", torch.int64)
    layer_stride = pages * ps * hkv * d

    def copy():
        pkv.pkv_copy_slots(pool, src, dst, layers, layer_stride)

    import oracle as orc

    def host(t):
        return t.cpu().view(torch.int16).numpy().view(np.uint16)

    k0, v0 = host(k), host(v)
    copy()
    torch.cuda.synchronize()
    (k1, v1), oracle_s = timed_oracle(lambda: (orc.copy_slots(k0, src.cpu().numpy(), dst.cpu().numpy()),
                                               orc.copy_slots(v0, src.cpu().numpy(), dst.cpu().numpy())))
    if not (np.array_equal(host(k), k1) and np.array_equal(host(v), v1)):
        return {"error": "parity failed: slot copy differs from the oracle"}
    del k0, v0, k1, v1
    for _ in range(3):
        copy()
    med, p10, p90 = time_events(torch, copy, 30, flush)
    nbytes = 2 * 2 * 2048 * layers * hkv * d * 2 + 2 * 2048 * 8     # K and V rows read + written, slot ids
    table = torch.arange(209, dtype=torch.int32, device="cuda:0")

    def rot():
        pkv.pkv_rotate_rows(table, 32)

    rot()
    if not np.array_equal(table.cpu().numpy(), orc.rotate_rows(np.arange(209, dtype=np.int32)[None], 32)[0]):
        return {"error": "parity failed: row rotation differs from the oracle"}
    for _ in range(3):
        rot()
    rmed, _, _ = time_events(torch, rot, 30, flush)
    try:
        seq = commit_sequence(torch, pkv, flush)
    except ParityError as e:
        return {"error": f"parity failed: {e}"}
    return {"workload": "exact-window commit: private-page fill of 2048 slots x 8 layers (24 kv heads x 128, bf16, "
                        "32-token pages) and the rotation of a 209-page table row",
            "commit_sequence": seq,
            "copy_slots_mb": nbytes / 1e6, "copy_slots_ms": med, "copy_slots_ms_p10_p90": [p10, p90],
            "copy_slots_gbs": nbytes / (med * 1e-3) / 1e9, "copy_slots_frac_hbm_peak": nbytes / (med * 1e-3) / 1e9 /
            HBM_PEAK_GBS, "rotate_rows_ms": rmed, "parity": "bit-exact", "oracle_s": round(oracle_s, 3),
            "cores": ORACLE_CORES}


# ----------------------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(case, seconds):
    """Time the float64 oracle on whole headline steps (scatter of the new
    tokens + decode of all 64 sequences), with numpy's BLAS on every core of
    this process's affinity, repeated until about ``seconds`` of work; report
    the same algorithmic bytes per second as the GPU figure."""
    import oracle as orc

    hkv, d = case.pool.num_kv_heads, case.pool.head_dim
    t_rows, n, hq, _ = case.q.shape
    step_bytes = (decode_bytes(case.kv_lens, case.pool.page_size, hkv, d, 2, t_rows * n, hq, 2, 2, False, False)
                  + 2 * 2 * len(case.slots) * hkv * d * 2 + len(case.slots) * 8)
    steps, spent = 0, 0.0
    with oracle_threads():
        while spent < seconds:
            t0 = time.perf_counter()
            kp = orc.scatter_slots(case.pool.k, case.new_k, case.slots)
            vp = orc.scatter_slots(case.pool.v, case.new_v, case.slots)
            orc.attn_decode(kp, vp, case.q, case.tables, case.kv_lens, case.sm_scale)
            spent += time.perf_counter() - t0
            steps += 1
    return {"value": steps * step_bytes / spent / 1e9, "unit": "GB/s", "cores": ORACLE_CORES, "kind": "oracle",
            "sample": f"{steps} whole steps of the headline batch (scatter of 64 new tokens + float64 decode of "
                      f"all 64 sequences, {int(case.kv_lens.sum())} keys, {step_bytes / 1e6:.1f} MB algorithmic "
                      f"per step) in {spent:.1f} s, numpy BLAS on {ORACLE_CORES} threads (the process's CPU "
                      f"affinity)"}


# ----------------------------------------------------------------------------- main

def device_info(torch, pkv):
    """The GPU as the runtime reports it, and the peaks derived from it beside
    the published ones: bf16 dense MFMA = CUs x clock x 4096 flop per clock."""
    import ctypes
    props = torch.cuda.get_device_properties(0)
    clock_khz = None
    # the HIP runtime libpkv is linked to (the process's only one), through libpkv's handle
    get_attr = getattr(pkv.load_library(), "hipDeviceGetAttribute", None)
    if get_attr is not None:
        v = ctypes.c_int(0)
        if get_attr(ctypes.byref(v), 5, 0) == 0:   # hipDeviceAttributeClockRate, kHz
            clock_khz = v.value
    cus = int(props.multi_processor_count)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "compute_units": cus,
            "max_clock_mhz": None if clock_khz is None else clock_khz / 1000.0,
            "memory_gib": round(props.total_memory / 2**30, 1),
            "spec_peaks": {"hbm_gbs": HBM_PEAK_GBS, "bf16_mfma_tflops": BF16_MFMA_PEAK_TFLOPS}}
    if clock_khz:
        info["derived_bf16_mfma_tflops"] = round(cus * clock_khz * 1e3 * 4096 / 1e12, 1)
    return info


def copy_ceiling(torch, mib=1024):
    """Achievable streaming bandwidth: a device copy of MIB MiB (read + write),
    median of 10; reported against the HBM peak, which stays the roofline."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    med, _, _ = time_events(torch, lambda: dst.copy_(src), 10)
    gbs = 2 * (mib << 20) / (med * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"what": f"device copy of {mib} MiB (read + write)", "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_slots_amd as pkv
    import workloads as W

    pkv.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe > 0:
        # a copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch against
        # MIB MiB each give the counters' scale on this chip
        src = torch.empty(args.copy_probe << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        ms = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dst.copy_(src)
            b.record()
            b.synchronize()
            ms.append(a.elapsed_time(b))
        print(json.dumps({"copy_probe_mib": args.copy_probe, "median_ms": float(np.median(ms)),
                          "gbs_read_plus_write": 2 * (args.copy_probe << 20) / (float(np.median(ms)) * 1e-3) / 1e9}))
        return
    try:
        case, h = run_headline(args, torch, pkv, W)
    except ParityError as e:
        # no figure for an output that does not match the oracle
        print(json.dumps({"metric": "paged decode K/V GB/s (% HBM peak) + block-causal prefill TFLOP/s (% MFMA)",
                          "value": None, "error": f"headline parity failed: {e}"}))
        sys.exit(1)
    value = h["step_bytes"] / (h["ms_per_step"] * 1e-3) / 1e9
    achieved = h["dec_bytes"] / (h["decode_kernel_ms"] * 1e-3) / 1e9
    call_gbs = h["dec_bytes"] / (h["decode_ms"] * 1e-3) / 1e9
    result = {
        "metric": "paged decode K/V GB/s (% HBM peak) + block-causal prefill TFLOP/s (% MFMA)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(h["ms_per_step"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "bf16 GQA paged decode: 64 sequences, lengths U[512,4096], 32 q / 8 kv heads x 128, "
                               "32-token pages shuffled over a 16384-page pool; step = one "
                               "pkv_attn_decode_append call (the decode kernel writes the 64 new tokens into their "
                               "slots, then attends)",
                   "global_batch": 64, "seq_len": int(case.max_kv_len), "total_keys": int(case.kv_lens.sum()),
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "kernel": "decode_skh_kernel (the dominant kernel of the pkv_attn_decode_append call; it also "
                               "writes the step's 64 tokens)",
                     "timing": "HIP events on the launch stream over --steps further steps (not inside the "
                               "wall-clock loop): the library launches the decode kernel through "
                               "hipExtLaunchKernel with a start / stop event pair, which take that kernel's own "
                               "start and end times (the merge kernel of the split units is outside the span)",
                     "bytes_per_launch": h["dec_bytes"], "avg_launch_ms": round(h["decode_kernel_ms"], 5),
                     "call": {"what": "the whole pkv_attn_decode_append call: decode kernel (with the token writes) + "
                                      "merge kernel of the split units + the gap between them",
                              "avg_ms": round(h["decode_ms"], 5), "achieved": round(call_gbs, 1),
                              "frac": round(call_gbs / HBM_PEAK_GBS, 4)}},
        "parity": h["parity"],
        "append": {"what": "the step's 64 new tokens (K and V, 8 kv heads x 128): read and written into their "
                           "slots by the decode kernel itself, before its own walk reads them (no scatter launch)",
                   "bytes": h["append_bytes"]},
        "flushed_step_ms_median_p10_p90": [round(x, 5) for x in h["flushed_step_ms"]],
        "device": device_info(torch, pkv),
        "copy_ceiling": copy_ceiling(torch),
    }
    workloads = {}
    flush = Flusher(torch)
    runners = {"prefill": ("block_causal_prefill", run_prefill),
               "fp8prefill": ("fp8_block_causal_prefill", run_fp8_prefill),
               "shared": ("shared_prefix_decode", run_shared_prefix),
               "fp8": ("long_fp8_decode", run_long_fp8), "commit": ("exact_window_commit", run_commit)}
    for name in [w.strip() for w in args.workloads.split(",") if w.strip() and w.strip() != "none"]:
        key, fn = runners[name]
        workloads[key] = fn(torch, pkv, W, flush)
        torch.cuda.empty_cache()
    if workloads:
        result["workloads"] = workloads
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
