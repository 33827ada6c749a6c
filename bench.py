#!/usr/bin/env python3
"""Benchmark of split-KV decode on one MI355X.

One step = one decode() call through the C ABI: plan (partition count + tile size, host),
split kernel, LSE-merge reducer, on one stream, inputs already resident in HBM.

Prints ONE JSON line (rank 0): the headline workload's KV-read GB/s (KV payload bytes of the
call / wall time per call), the split kernel's roofline against the 8 TB/s HBM peak (HIP events
on the launch stream), a per-workload table (us/call, GB/s, % of peak for every workload), and
the CPU oracle timed on a bounded sample of the headline workload (with the sampled parity
errors of the GPU result against it).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
LOG2E = 1.4426950408889634


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mla_h64_b16_s131072_q1")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload (no per-workload table)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sparse-sweep", action="store_true",
                    help="only time the sparse top-k split sweep and print it")
    ap.add_argument("--proportional-sweep", action="store_true",
                    help="only the equal-split vs length-proportional sweep over skewed batches")
    ap.add_argument("--branch-sweep", action="store_true",
                    help="only the planner-branch sweep (MLA 32/128 heads, GQA one kv head)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--table-steps", type=int, default=50)
    ap.add_argument("--sweep-steps", type=int, default=20,
                    help="timed calls per point of the planner sweeps")
    ap.add_argument("--oracle-seconds", type=float, default=1.0,
                    help="target CPU time of each workload's oracle sample in the per-workload table")
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed run of each workload's step before its warmup, so clocks settle")
    ap.add_argument("--block-k", type=int, default=0,
                    help="force the split kernel's key tile (0: the CTA-keyed tile rule)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times): the reference kernel "
                         "that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes")
    return ap.parse_args()


def make_workloads():
    import workloads as w
    items = [
        ("mla_tiny_b1_h16_s4096_np1", lambda d: w.mla_tiny(d), 1),
        ("mla_tiny_b1_h16_s4096_np4", lambda d: w.mla_tiny(d), 4),
        ("mla_tiny_b1_h16_s4096_np16", lambda d: w.mla_tiny(d), 16),
        ("mla_h64_b2_s65536", lambda d: w.mla_b2_s65536(d), 0),
        ("mla_h64_b8_s131072_q1", lambda d: w.mla_long(8, 1, d), 0),
        ("mla_h64_b16_s131072_q1", lambda d: w.mla_long(16, 1, d), 0),
        ("mla_h64_b8_s131072_q4", lambda d: w.mla_long(8, 4, d), 0),
        ("mla_h64_b16_s131072_q4", lambda d: w.mla_long(16, 4, d), 0),
        ("gqa_b32_hq64_hkv8_d128_p16", lambda d: w.gqa_paged(d), 0),
        ("gqa_b32_hq64_hkv1_d128_p16", lambda d: w.gqa_mqa(d), 0),
        # not one of the quoted configurations: a skewed batch, where the equal split leaves the
        # long request's few partitions to carry most of the keys
        ("mla_h64_b32_skewed_1x131072_31x2048", lambda d: w.mla_skewed(d), 0),
    ]
    for nq in w.SPARSE_QUERY_COUNTS:
        items.append(("sparse_mla_h64_topk2048_nq%d" % nq, (lambda n: lambda d: w.sparse_topk(n, d))(nq), 0))
    # the same rows stored as bf16 (twice the bytes per key)
    items += [
        ("mla_h64_b16_s131072_q1_bf16", lambda d: w.mla_long_bf16(16, 1, d), 0),
        ("mla_h64_b8_s131072_q4_bf16", lambda d: w.mla_long_bf16(8, 4, d), 0),
        ("sparse_mla_h64_topk2048_nq256_bf16", lambda d: w.sparse_topk(256, d, kv_dtype="bf16"), 0),
    ]
    return items


class Case:
    """One workload bound to the C ABI: problem, output and workspace buffers."""

    def __init__(self, inp, np_fixed, stream, block_k=0):
        import torch
        import gqa_plan_splits_amd as g
        self.g = g
        self.inp = inp
        self.is_mla = hasattr(inp, "pool")
        if self.is_mla:
            self.p = g.mla_problem(inp.q_lat, inp.q_pe, inp.pool, inp.kv_indices, inp.kv_indptr,
                                   inp.seq_lens, batch=inp.B, q_len=inp.q_len, num_heads=inp.H,
                                   max_num_keys=inp.max_num_keys, scale=inp.scale,
                                   kv_scale=inp.kv_scale, d_v=inp.d_v)
            self.d_v = inp.d_v
        else:
            self.p = g.gqa_problem(inp.q, inp.k_cache, inp.v_cache, inp.kv_page_indices,
                                   inp.kv_indptr, inp.seq_lens, batch=inp.B, q_len=inp.q_len,
                                   max_num_keys=inp.max_num_keys, scale=inp.scale)
            self.d_v = inp.D
        self.np_arg = np_fixed
        self.bk_arg = block_k
        self.np, self.bk = g.decode_plan(self.p, np_fixed, block_k)
        rows = self.p.rows
        dev = torch.device("cuda")
        self.out = torch.empty((rows, self.d_v), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((rows,), dtype=torch.float32, device=dev)
        ws = g.decode_workspace_bytes(self.p, self.np)
        self.ws = torch.empty((max(ws, 256) // 4 + 64,), dtype=torch.float32, device=dev)
        self.po = torch.empty((rows, self.np, self.d_v), dtype=torch.float32, device=dev)
        self.pl = torch.empty((rows, self.np), dtype=torch.float32, device=dev)
        self.stream = stream
        self.rows = rows

    def step(self):
        # the whole hot path: plan (np=0 / block_k=0 -> planner and tile rule) + split + reduce
        self.g.decode(self.p, self.out, self.lse, np=self.np_arg, block_k=self.bk_arg,
                      workspace=self.ws, stream=self.stream)

    def split_only(self):
        self.g.decode_split(self.p, self.np, self.bk, self.po, self.pl, stream=self.stream)

    def alloc_proportional(self):
        import torch
        if not hasattr(self, "ws_prop"):
            n = self.g.decode_proportional_workspace_bytes(self.p, self.np)
            self.ws_prop = torch.empty((n // 4 + 64,), dtype=torch.float32, device="cuda")

    def proportional_step(self):
        # the same budget of np partitions per request, planned on the device in proportion to
        # the lengths (at most 256 partitions per request: cap 0)
        self.alloc_proportional()
        self.g.decode_proportional(self.p, self.out, self.lse, np=self.np, block_k=self.bk,
                                   workspace=self.ws_prop, stream=self.stream)

    def reduce_only(self):
        self.g.splitk_reduce(self.rows, self.np, self.d_v, self.po, self.pl, self.out, self.lse,
                             stream=self.stream)

    def kv_bytes(self):
        return self.inp.kv_bytes

    def split_algorithmic_bytes(self):
        """Compulsory HBM bytes of one split launch: each key's payload and index once, Q once,
        the fp32 partial outputs and LSEs written once (np == 1 writes bf16 output directly)."""
        inp = self.inp
        keys = int(inp.seq_lens.sum().item())
        if self.is_mla:
            q_bytes = self.rows * inp.d_qk * 2
            idx = keys * 4
        else:
            q_bytes = self.rows * inp.D * 2
            idx = sum((int(x) + inp.page_size - 1) // inp.page_size for x in inp.seq_lens.tolist()) * 4
        if self.np == 1:
            writes = self.rows * (self.d_v * 2 + 4)
        else:
            writes = self.rows * self.np * (self.d_v + 1) * 4
        return self.kv_bytes() + idx + q_bytes + writes


# Counter summaries under profiles/, per timed workload: the file and the sources its kernel is
# compiled from (hashed in this order).
MLA_SOURCES = ("mla_split.hip", "mla_common.hpp", "device_common.hpp", "kernels.hpp")
WIDE_SOURCES = ("mla_wide.hip", "mla_common.hpp", "device_common.hpp", "kernels.hpp")
COUNTER_PROFILES = {
    "mla_h64_b16_s131072_q1": ("mla_split_b16_s131072_counters.txt", MLA_SOURCES),
    "mla_h64_b16_s131072_q4": ("mla_split_b16_s131072_q4_counters.txt", MLA_SOURCES),
    "sparse_mla_h64_topk2048_nq256": ("mla_wide_sparse_nq256_counters.txt", WIDE_SOURCES),
    "mla_h64_b16_s131072_q1_bf16": ("mla_split_b16_s131072_bf16_counters.txt", MLA_SOURCES),
    "gqa_b32_hq64_hkv8_d128_p16": ("gqa_pair_b32_hq64_hkv8_counters.txt",
                                   ("gqa_split.hip", "device_common.hpp", "kernels.hpp")),
}


def split_kernel_name(inp):
    """The split kernel a workload's decode launches: 512-byte fp8 rows of one cache (the sparse
    top-k layout) run on mla_wide_kernel, other MLA rows on mla_split_kernel; GQA with an even
    number of kv heads and at most 16 query rows per head group on gqa_pair_kernel, other GQA
    shapes on gqa_split_kernel."""
    if not hasattr(inp, "pool"):
        rows = inp.q_len * (inp.Hq // inp.Hkv)
        return "gqa_pair_kernel" if inp.Hkv % 2 == 0 and rows <= 16 else "gqa_split_kernel"
    if inp.d_qk == 512 and not inp.kv_bf16 and inp.pool2 is None:
        return "mla_wide_kernel"
    return "mla_split_kernel"


def source_sha256(names):
    """sha256 over kernel sources under the package's csrc/, in the given order."""
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "gqa_plan_splits_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_counters(workload):
    """HBM bytes per split launch and the MFMA busy fraction, from the committed rocprofv3 counter
    summary of this workload; FETCH_SIZE / WRITE_SIZE are scaled by the plain-copy calibration
    recorded beside them. None unless the summary was taken on the current kernel sources (their
    sha256 must match)."""
    if workload not in COUNTER_PROFILES:
        return None
    fname, sources = COUNTER_PROFILES[workload]
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = (x.strip() for x in line.split("=", 1))
            vals[k] = v
    if vals.get("kernel_source_sha256") != source_sha256(sources):
        return None
    fetch = float(vals["fetch_kib_per_dispatch"]) * float(vals["copy_bytes"]) / float(vals["copy_fetch_kib"])
    write = float(vals["write_kib_per_dispatch"]) * float(vals["copy_bytes"]) / float(vals["copy_write_kib"])
    # SQ_VALU_MFMA_BUSY_CYCLES is summed over every SIMD; GRBM_GUI_ACTIVE over the XCDs.
    busy = float(vals["mfma_busy_cycles"]) / (
        float(vals["grbm_gui_active"]) / float(vals["xcds"]) * float(vals["simds"]))
    out = {"traffic": int(fetch + write), "mfma_busy": round(busy, 4)}
    if "valu_active_inst" in vals:
        # SQ_ACTIVE_INST_VALU counts issue quads (4 cycles) summed over every wave
        out["valu_busy"] = round(float(vals["valu_active_inst"]) * 4 / (
            float(vals["valu_grbm_gui_active"]) / float(vals["xcds"]) * float(vals["simds"])), 4)
    return out


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), and the logical CPUs this process may use."""
    name = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return name


def oracle_sample(case, target_s, n_threads=0):
    """The oracle on a bounded sample of this workload's rows (doubling the sample until it takes
    about target_s / 2), extrapolated to the whole call; also the sampled rows' parity of the GPU
    output against it."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from gpu_util import compare, oracle_gqa, oracle_mla, sample_rows
    inp = case.inp
    H = inp.H if case.is_mla else inp.Hq
    total = case.rows
    threads = n_threads or oracle.default_threads()
    n = min(total, max(threads, 4))
    while True:
        rows = sample_rows(inp.B, inp.q_len, H, n, seed=n) if n < total else list(range(total))
        t0 = time.perf_counter()
        ref_o, ref_l = (oracle_mla if case.is_mla else oracle_gqa)(inp, rows, n_threads=threads)
        dt = time.perf_counter() - t0
        if dt * 2.2 > target_s or n >= total:
            break
        n = min(total, n * 2)
    max_abs, rel, lse_err = compare(case.out[rows], case.lse[rows], ref_o, ref_l, inp.name + " oracle sample")
    return {"s_per_call": round(dt * total / len(rows), 4), "rows": len(rows), "of_rows": total,
            "threads": threads, "sample_s": round(dt, 3),
            "parity": {"max_abs": max_abs, "rel": rel, "lse2_rel": lse_err}}


def planner_ns_per_call(reps=20000):
    """Host planner and tile rule through the C ABI (ctypes call included), ns per call."""
    import gqa_plan_splits_amd as g
    t0 = time.perf_counter()
    for _ in range(reps):
        g.plan_splits(16, 131072, 64, 256, 1)
    t_plan = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    for _ in range(reps):
        g.block_k_for(512, 256)
    t_bk = (time.perf_counter() - t0) / reps
    return {"plan_splits_ns": round(t_plan * 1e9, 1), "block_k_for_ns": round(t_bk * 1e9, 1),
            "note": "ctypes call from Python included"}


def ceilings(stream, case):
    """Streaming-read and row-gather ceilings of this GPU with the split kernels' copy instruction
    (the library's bw_stream_read and bw_gather_rows): a 2 GiB contiguous read, and a gather of
    the headline workload's own shuffled slot list over its pool, in the MLA kernel's copy
    pattern (128-byte lines of 8 rows per copy instruction) and with whole-row requests (512
    bytes of 2 rows per instruction).  Median of 5 timed launches after 2 untimed ones, HIP
    events on the stream."""
    import torch
    import gqa_plan_splits_amd as g
    inp = case.inp
    buf = torch.ones(2 << 30, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def timed(fn):
        for _ in range(2):
            fn()
        ts = sorted(time_events(fn, 1, stream) for _ in range(5))
        return ts[2]
    ms_stream = timed(lambda: g.bw_stream_read(buf, buf.numel(), 1024, stream=stream))
    del buf
    torch.cuda.empty_cache()
    stream_gbs = (2 << 30) / (ms_stream * 1e-3) / 1e9
    if not case.is_mla:   # a paged GQA headline: no slot list of rows to gather
        return {"stream_read_gbs": round(stream_gbs, 1), "stream_read_pct_peak": round(100 * stream_gbs / HBM_PEAK_GBS, 1),
                "method": "bw_stream_read (2 GiB, 1024 CTAs); global_load_lds_dwordx4 nt into LDS; median of 5 "
                          "launches, HIP events"}
    n = (inp.kv_indices.numel() // 64) * 64
    row_bytes = inp.pool.shape[1]
    ms_gather = timed(lambda: g.bw_gather_rows(inp.pool, row_bytes, inp.kv_indices, n, 256, stream=stream))
    gather_gbs = n * row_bytes / (ms_gather * 1e-3) / 1e9
    ms_whole = timed(lambda: g.bw_gather_whole_rows(inp.pool, row_bytes, inp.kv_indices, n, 256, stream=stream))
    whole_gbs = n * row_bytes / (ms_whole * 1e-3) / 1e9
    return {"stream_read_gbs": round(stream_gbs, 1), "stream_read_pct_peak": round(100 * stream_gbs / HBM_PEAK_GBS, 1),
            "gather_rows_gbs": round(gather_gbs, 1), "gather_rows_pct_peak": round(100 * gather_gbs / HBM_PEAK_GBS, 1),
            "gather_whole_rows_gbs": round(whole_gbs, 1), "gather_whole_rows_pct_peak": round(100 * whole_gbs / HBM_PEAK_GBS, 1),
            "gather_rows": n, "row_bytes": row_bytes,
            "method": "bw_stream_read (2 GiB, 1024 CTAs), bw_gather_rows and bw_gather_whole_rows (the headline's slot list, 256 CTAs); "
                      "global_load_lds_dwordx4 nt into LDS; median of 5 launches, HIP events"}


def mla_flops(inp):
    """Algorithmic flops of one MLA decode: per (row, visible key) 2 * (d_qk + d_v) (QK^T and PV)."""
    lens = inp.seq_lens.tolist()
    q, H = inp.q_len, inp.H
    keys = sum(sum(max(0, L - q + t + 1) for t in range(q)) for L in lens)
    return keys * H * 2 * (inp.d_qk + inp.d_v)


def settle(fn, ms):
    """Untimed: repeat fn for about `ms` milliseconds of wall time so that the GPU clocks reach
    their steady state under this load before the counted warmup and timed steps."""
    import torch
    if ms <= 0:
        return
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def check_slots(inp):
    """Host check of the device-data contract before a launch: every MLA slot id is a pool row
    (or negative, a skipped key).  The kernels trust the ids."""
    hi = int(inp.kv_indices.max()) if inp.kv_indices.numel() else -1
    if hi >= inp.pool.shape[0]:
        raise RuntimeError("%s: slot id %d outside a pool of %d rows" % (inp.name, hi, inp.pool.shape[0]))


def time_events(fn, n, stream):
    """Average ms per call of fn over n calls, HIP events recorded on `stream`."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n


def time_graph(fn, n, stream):
    """Average ms per replay of a HIP graph holding one call of fn (captured on `stream`), so
    that host launch work is out of the timing; None if capture fails."""
    import torch
    try:
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            fn()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):   # a replay runs on the current stream
            for _ in range(3):
                graph.replay()
            return time_events(graph.replay, n, stream)
    except RuntimeError:
        torch.cuda.synchronize()
        return None


def time_interleaved(fns, n, stream):
    """Average ms per call of each fn over n calls each, timed in five interleaved rounds of
    n / 5 calls (when 5 divides n) so that slow drifts of the clock weigh on all of them alike."""
    rounds = 5 if n % 5 == 0 and n >= 5 else 1
    k = n // rounds
    tot = [0.0] * len(fns)
    for _ in range(rounds):
        for i, fn in enumerate(fns):
            if fn is not None:
                tot[i] += time_events(fn, k, stream) * k
    return [t / n for t in tot]


def time_cold(fn, n, stream, flush):
    """Average ms per call of fn with the caches cold: before each call, outside its event pair,
    a 512 MiB buffer is written, which evicts L2 and the 256 MB MALL."""
    import torch
    total = 0.0
    for _ in range(n):
        with torch.cuda.stream(stream):
            flush.fill_(1.0)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        fn()
        end.record(stream)
        end.synchronize()
        total += start.elapsed_time(end)
    return total / n


def dcp_line(stream, steps, world=8):
    """Decode context parallelism at the headline shape, one GPU: rank 0 of `world` ranks (every
    `world`-th position of each 131072-key request: its split and its fp32 merge), and the merge
    of `world` rank outputs (the ranks' copies of rank 0's output stand in for the others)."""
    import torch
    import gqa_plan_splits_amd as g
    import workloads as w
    with torch.cuda.stream(stream):
        inp = w.mla_long(16, 1, "cuda")
        B, S = inp.B, int(inp.max_num_keys)
        idx = inp.kv_indices.view(B, S)[:, 0::world].contiguous().view(-1)
        local = S // world
        indptr = torch.arange(B + 1, dtype=torch.int32, device="cuda") * local
        lens = torch.full((B,), local, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()   # the inputs exist before any kernel on `stream` reads them
    check_slots(inp)
    p = g.mla_problem(inp.q_lat, inp.q_pe, inp.pool, idx, indptr, lens, batch=B, q_len=1,
                      num_heads=inp.H, max_num_keys=local, scale=inp.scale, kv_scale=inp.kv_scale,
                      d_v=512, glen=inp.seq_lens, cp_rank=0, cp_world=world)
    np_, bk = g.decode_plan(p)
    rows = p.rows
    po = torch.empty((rows, np_, 512), dtype=torch.float32, device="cuda")
    pl = torch.empty((rows, np_), dtype=torch.float32, device="cuda")
    parts = torch.empty((world, rows, 512), dtype=torch.float32, device="cuda")
    lses = torch.empty((world, rows), dtype=torch.float32, device="cuda")
    out = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")

    def rank():
        g.decode_split(p, np_, bk, po, pl, stream=stream)
        g.splitk_reduce_f32(rows, np_, 512, po, pl, parts[0], lses[0], stream=stream)

    def merge():
        g.merge_ranks(world, rows, 512, parts, lses, out, lse, stream=stream)

    for _ in range(5):
        rank()
    torch.cuda.synchronize()
    for r in range(1, world):
        parts[r].copy_(parts[0])
        lses[r].copy_(lses[0])
    rank_ms = time_events(rank, steps, stream)
    merge_ms = time_events(merge, steps, stream)
    kv = B * local * 576
    return {"world": world, "rank_keys_per_request": local, "np": np_, "block_k": bk,
            "rank_us": round(rank_ms * 1e3, 2), "rank_kv_gbs": round(kv / (rank_ms * 1e-3) / 1e9, 1),
            "merge_us": round(merge_ms * 1e3, 2)}


def wave_sweep(stream, steps):
    """The planner's one-wave / two-wave choice for MLA with 16 heads (the page's exception,
    where the two-wave count is the planner's), timed at both counts and at the count of
    plan_mla_splits_measured (this kernel's own CTAs, one wave): batch 4 over 32K-128K keys and
    batches 8 and 16 at short context."""
    import torch
    import gqa_plan_splits_amd as g
    import workloads as w
    sm = g.device_sm_count()
    res = {}
    for B, S in ((4, 32768), (4, 65536), (4, 131072), (8, 16384), (16, 16384)):
        with torch.cuda.stream(stream):
            inp = w.mla_inputs(B=B, q_len=1, H=16, seq_lens=[S] * B, pool_rows=B * S, seed=5000,
                               device="cuda", name="h16")
        torch.cuda.synchronize()   # the inputs exist before any kernel on `stream` reads them
        check_slots(inp)
        p = g.mla_problem(inp.q_lat, inp.q_pe, inp.pool, inp.kv_indices, inp.kv_indptr,
                          inp.seq_lens, batch=B, q_len=1, num_heads=16, max_num_keys=S,
                          scale=inp.scale, kv_scale=inp.kv_scale, d_v=512)
        ctas = B   # one 32-row head block per request at 16 heads
        pages = -(-S // 256)
        counts = {"one_wave": max(1, min(sm // ctas, pages, 256)),
                  "two_wave": max(1, min(2 * sm // ctas, pages, 256)),
                  "planner": g.decode_plan(p)[0],
                  "measured": g.plan_mla_splits_measured(B, S, 16, sm)}
        row = {}
        for name, n in counts.items():
            bk = g.block_k_for(B * n, sm)
            ws = torch.empty((g.decode_workspace_bytes(p, n) // 4 + 64,), dtype=torch.float32, device="cuda")
            out = torch.empty((p.rows, 512), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((p.rows,), dtype=torch.float32, device="cuda")
            fn = (lambda n=n, bk=bk, ws=ws, out=out, lse=lse:
                  g.decode(p, out, lse, np=n, block_k=bk, workspace=ws, stream=stream))
            for _ in range(5):
                fn()
            ms = time_graph(fn, steps, stream) or time_events(fn, steps, stream)
            row[name] = {"np": n, "us_per_call": round(ms * 1e3, 2)}
        row["two_wave_speedup"] = round(row["one_wave"]["us_per_call"] / row["two_wave"]["us_per_call"], 3)
        best = min(row[k]["us_per_call"] for k in counts)
        row["measured_vs_best"] = round(row["measured"]["us_per_call"] / best, 3)
        res["mla_h16_b%d_s%d" % (B, S)] = row
        del inp, p
        torch.cuda.empty_cache()
    return res


def branch_sweep(stream, steps):
    """The planner's other branches on this library's kernels: MLA with 16 heads (the page's
    two-wave exception), 32, 64 (two requests of 65536 keys) and 128 heads, and
    GQA with one kv head (16 query heads) and with 4 query heads per kv head, each timed at every
    power-of-two partition count up to 256 (graph-replayed decode calls) beside the planner's
    choice."""
    import torch
    import gqa_plan_splits_amd as g
    import workloads as w
    cases = [("mla_h16_b4_s65536", "mla", 4, 16, 1, 65536), ("mla_h16_b16_s16384", "mla", 16, 16, 1, 16384),
             ("mla_h64_b2_s65536", "mla", 2, 64, 1, 65536),
             ("mla_h32_b4_s65536", "mla", 4, 32, 1, 65536), ("mla_h32_b16_s16384", "mla", 16, 32, 1, 16384),
             ("mla_h128_b4_s65536", "mla", 4, 128, 1, 65536), ("mla_h128_b16_s16384", "mla", 16, 128, 1, 16384),
             ("gqa_hq16_hkv1_b8_s32768", "gqa", 8, 16, 1, 32768), ("gqa_hq16_hkv1_b64_s8192", "gqa", 64, 16, 1, 8192),
             ("gqa_hq32_hkv8_b8_s32768", "gqa", 8, 32, 8, 32768), ("gqa_hq32_hkv8_b64_s8192", "gqa", 64, 32, 8, 8192)]
    res = {}
    for name, kind, B, H, Hkv, S in cases:
        with torch.cuda.stream(stream):
            if kind == "mla":
                inp = w.mla_inputs(B=B, q_len=1, H=H, seq_lens=[S] * B, pool_rows=B * S, seed=5100,
                                   device="cuda", name=name)
            else:
                inp = w.gqa_inputs(B=B, Hq=H, Hkv=Hkv, D=128, page_size=16, seq_lens=[S] * B,
                                   num_pages=B * S // 16, seed=5200, device="cuda", name=name)
        torch.cuda.synchronize()   # the inputs exist before any kernel on `stream` reads them
        if kind == "mla":
            check_slots(inp)
            p = g.mla_problem(inp.q_lat, inp.q_pe, inp.pool, inp.kv_indices, inp.kv_indptr,
                              inp.seq_lens, batch=B, q_len=1, num_heads=H, max_num_keys=S,
                              scale=inp.scale, kv_scale=inp.kv_scale, d_v=512)
            d_v = 512
        else:
            p = g.gqa_problem(inp.q, inp.k_cache, inp.v_cache, inp.kv_page_indices, inp.kv_indptr,
                              inp.seq_lens, batch=B, q_len=1, max_num_keys=S, scale=inp.scale)
            d_v = 128
        planner = g.decode_plan(p)[0]
        out = torch.empty((p.rows, d_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((p.rows,), dtype=torch.float32, device="cuda")
        times = {}
        for n in sorted({1, 2, 4, 8, 16, 32, 64, 128, 256, planner}):
            ws = torch.empty((g.decode_workspace_bytes(p, n) // 4 + 64,), dtype=torch.float32,
                             device="cuda")
            fn = (lambda n=n, ws=ws: g.decode(p, out, lse, np=n, workspace=ws, stream=stream))
            for _ in range(3):
                fn()
            times[n] = (time_graph(fn, steps, stream) or time_events(fn, steps, stream)) * 1e3
            del ws
        best = min(times, key=times.get)
        res[name] = {"us_by_np": {str(k): round(v, 2) for k, v in times.items()}, "best_np": best,
                     "planner_np": planner, "planner_vs_best": round(times[planner] / times[best], 3)}
        # the MI355X-measured variants (a power of two, or the planner's np)
        m = g.plan_gqa_splits_measured(B, S, Hkv) if kind == "gqa" else g.plan_mla_splits_measured(B, S, H)
        if m in times:
            res[name].update(measured_np=m, measured_vs_best=round(times[m] / times[best], 3))
        print("# branch %s %s" % (name, json.dumps(res[name])), file=sys.stderr, flush=True)
        del inp, p, out, lse
        torch.cuda.empty_cache()
    return res


def proportional_sweep(stream, steps):
    """decode (np equal partitions per request) against decode_proportional (the same budget
    spread by length on the device) as one long request of 131072 keys stands among shorter
    ones: MLA, H = 64, batches of 8 and 32, graph-replayed calls."""
    import torch
    import gqa_plan_splits_amd as g
    import workloads as w
    res = {}
    for B in (8, 32):
        for short in (131072, 32768, 8192, 2048, 256):
            lens = [131072] + [short] * (B - 1)
            name = "mla_h64_b%d_1x131072_%dx%d" % (B, B - 1, short)
            with torch.cuda.stream(stream):
                inp = w.mla_inputs(B=B, q_len=1, H=64, seq_lens=lens, pool_rows=sum(lens), seed=5300,
                                   device="cuda", name=name)
            torch.cuda.synchronize()   # the inputs exist before any kernel on `stream` reads them
            check_slots(inp)
            p = g.mla_problem(inp.q_lat, inp.q_pe, inp.pool, inp.kv_indices, inp.kv_indptr,
                              inp.seq_lens, batch=B, q_len=1, num_heads=64, max_num_keys=131072,
                              scale=inp.scale, kv_scale=inp.kv_scale, d_v=512)
            np_, bk = g.decode_plan(p)
            out = torch.empty((p.rows, 512), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((p.rows,), dtype=torch.float32, device="cuda")
            ws = torch.empty((g.decode_workspace_bytes(p, np_) // 4 + 64,), dtype=torch.float32,
                             device="cuda")
            wsp = torch.empty((g.decode_proportional_workspace_bytes(p, np_) // 4 + 64,),
                              dtype=torch.float32, device="cuda")
            eq = lambda: g.decode(p, out, lse, np=np_, block_k=bk, workspace=ws, stream=stream)
            prop = lambda: g.decode_proportional(p, out, lse, np=np_, block_k=bk, workspace=wsp,
                                                 stream=stream)
            # both captured, then replayed in five alternating rounds after a settling phase, so
            # that clock drift weighs on both alike
            graphs = []
            for fn in (eq, prop):
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=stream):
                    fn()
                torch.cuda.synchronize()
                graphs.append(gr)
            with torch.cuda.stream(stream):
                settle(graphs[0].replay, 150.0)
                t_eq, t_prop = time_interleaved([graphs[0].replay, graphs[1].replay],
                                                max(5, steps // 5 * 5), stream)
            times = {"equal": t_eq * 1e3, "proportional": t_prop * 1e3}
            res[name] = {"np": np_, "equal_us": round(times["equal"], 2),
                         "proportional_us": round(times["proportional"], 2),
                         "proportional_vs_equal": round(times["proportional"] / times["equal"], 3)}
            print("# proportional %s %s" % (name, json.dumps(res[name])), file=sys.stderr, flush=True)
            del inp, p, out, lse, ws, wsp, graphs
            torch.cuda.empty_cache()
    return res


def sparse_sweep(stream, steps):
    """Sparse top-k MLA (64 heads, 2048 candidates per query) at every split count from 1 to 32
    per query count, beside the choices of the two planners: the wave-aligned one decode uses
    and the sparse page's rules (plan_sparse_splits, CTAs of 64 heads = head_tiles 4)."""
    import torch
    import gqa_plan_splits_amd as g
    import workloads as w
    sm = g.device_sm_count()
    res = {}
    for nq in (1, 2, 4, 8, 16, 24, 32, 64, 128, 256):
        with torch.cuda.stream(stream):
            inp = w.sparse_topk(nq, "cuda")
        torch.cuda.synchronize()   # the inputs exist before any kernel on `stream` reads them
        check_slots(inp)
        p = g.mla_problem(inp.q_lat, inp.q_pe, inp.pool, inp.kv_indices, inp.kv_indptr,
                          inp.seq_lens, batch=inp.B, q_len=1, num_heads=inp.H,
                          max_num_keys=inp.max_num_keys, scale=inp.scale, kv_scale=inp.kv_scale,
                          d_v=inp.d_v)
        out = torch.empty((p.rows, inp.d_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((p.rows,), dtype=torch.float32, device="cuda")
        times = {}
        for n in (1, 2, 4, 8, 16, 32):
            bk = g.block_k_for(nq * n, sm)
            ws = torch.empty((g.decode_workspace_bytes(p, n) // 4 + 64,), dtype=torch.float32, device="cuda")
            fn = (lambda n=n, bk=bk, ws=ws:
                  g.decode(p, out, lse, np=n, block_k=bk, workspace=ws, stream=stream))
            for _ in range(3):
                fn()
            ms = time_graph(fn, steps, stream) or time_events(fn, steps, stream)
            times[n] = round(ms * 1e3, 2)
        best = min(times, key=times.get)
        wave_np = g.decode_plan(p)[0]
        page_np, cpb = g.plan_sparse_splits(nq, inp.H, int(inp.max_num_keys), num_sms=sm, head_tiles=4)
        meas_np = g.plan_sparse_splits_measured(nq, inp.H, int(inp.max_num_keys), sm_count=sm, max_splits=32)
        res["nq%d" % nq] = {"us_by_np": times, "best_np": best, "wave_planner_np": wave_np,
                            "sparse_planner_np": page_np, "sparse_chunks_per_block": cpb,
                            "measured_rule_np": meas_np,
                            "wave_planner_vs_best": round(times[wave_np] / times[best], 3),
                            "sparse_planner_vs_best": round(times[page_np] / times[best], 3),
                            "measured_rule_vs_best": round(times[meas_np] / times[best], 3)}
        print("# sparse nq%d %s" % (nq, json.dumps(res["nq%d" % nq])), file=sys.stderr, flush=True)
        del inp, p
        torch.cuda.empty_cache()
    return res


def cpu_baseline(case, target_s):
    """The oracle as it stands, on a bounded sample of rows of the headline workload, with the
    sampled parity of the GPU output against it."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from gpu_util import compare, oracle_gqa, oracle_mla, sample_rows

    inp = case.inp
    H = inp.H if case.is_mla else inp.Hq
    total_rows = case.rows
    cores = oracle.default_threads()
    n = max(cores, 8)
    t_used = 0.0
    while True:
        rows = sample_rows(inp.B, inp.q_len, H, n, seed=n)
        t0 = time.perf_counter()
        ref_o, ref_l = (oracle_mla if case.is_mla else oracle_gqa)(inp, rows, n_threads=cores)
        dt = time.perf_counter() - t0
        t_used += dt
        if dt * 2.2 > target_s or n * 2 > total_rows or t_used > 2 * target_s:
            break
        n *= 2
    max_abs, rel, lse_err = compare(case.out[rows], case.lse[rows], ref_o, ref_l, "bench parity")
    full_s = dt * total_rows / len(rows)
    return {
        "value": round(case.kv_bytes() / full_s / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d of %d output rows of %s (fp64 unsplit attention, %d threads, %.2f s); "
                  "value = KV bytes / (sample time x rows / sampled rows)"
                  % (len(rows), total_rows, inp.name, cores, dt),
        "cpu_model": cpu_model(),
        "parity": {"max_abs": max_abs, "rel": rel, "lse2_rel": lse_err, "rows": len(rows)},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import gqa_plan_splits_amd as g
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return
    # All of the process's GPU work (inputs, launches, copies, graph capture) goes to this one
    # stream: once a second stream has run work, the hardware serves more than one queue, and
    # splits of more than about a thousand CTAs measured 4-5 % slower on MI355X (the paged GQA
    # split, 4096 CTAs: 374 against 355 us; the MLA split's 256 CTAs: unchanged).
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    sm = g.device_sm_count()
    if args.sparse_sweep:
        print(json.dumps({"sparse_planner": sparse_sweep(stream, args.sweep_steps)}), flush=True)
        return
    if args.proportional_sweep:
        print(json.dumps({"proportional": proportional_sweep(stream, args.sweep_steps)}), flush=True)
        return
    if args.branch_sweep:
        print(json.dumps({"planner_branches": branch_sweep(stream, args.sweep_steps)}), flush=True)
        return
    flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device="cuda")

    table = {}
    headline = None
    graph_todo = []
    # Every row's inputs, workspaces and outputs are allocated before any timing (about 19 GB for
    # the whole table), as a serving process allocates its KV cache and workspaces once: buffers
    # allocated into memory that earlier rows freed measured up to 4 % slower (the paged GQA split,
    # 353-356 us with fresh buffers, 364 us with only its partial-output buffer allocated after
    # assorted buffers were freed, 366 us with everything allocated after that).
    made = []
    for name, make, np_fixed in make_workloads():
        if args.headline_only and name != args.workload:
            continue
        with torch.cuda.stream(stream):
            inp = make("cuda")
        made.append((name, inp, np_fixed))
    torch.cuda.synchronize()
    for row, (name, inp, np_fixed) in enumerate(made):
        if hasattr(inp, "pool"):
            check_slots(inp)
        case = Case(inp, np_fixed, stream, args.block_k)
        if not args.headline_only:
            case.alloc_proportional()
        made[row] = (name, case)
    torch.cuda.synchronize()
    for row in range(len(made)):
        name, case = made[row]
        made[row] = None
        inp = case.inp
        is_head = name == args.workload
        steps = args.steps if is_head else args.table_steps
        warm = args.warmup if is_head else max(3, args.warmup // 2)
        settle(case.step, args.settle_ms)
        for _ in range(warm):
            case.step()
        torch.cuda.synchronize()
        ms, ms_split, ms_red = time_interleaved(
            [case.step, case.split_only, case.reduce_only if case.np > 1 else None], steps, stream)
        ms_cold = time_cold(case.step, max(5, steps // 4), stream, flush)
        ms_eq = ms_prop = None
        if not args.headline_only:   # keeps a profiled headline run to the headline's launches
            case.proportional_step()
            ms_eq, ms_prop = time_interleaved([case.step, case.proportional_step],
                                              max(5, steps // 10 * 5), stream)
        case.step()
        torch.cuda.synchronize()
        entry = {
            "us_per_call": round(ms * 1e3, 2),
            "kv_gbs": round(case.kv_bytes() / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * case.kv_bytes() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
            "us_per_call_cold": round(ms_cold * 1e3, 2),
            "pct_hbm_peak_cold": round(100 * case.kv_bytes() / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
            "us_per_call_graph": None,   # second pass, below
            "split_us": round(ms_split * 1e3, 2),
            "reduce_us": round(ms_red * 1e3, 2),
            "np": case.np, "block_k": case.bk, "kv_bytes": case.kv_bytes(),
            "kv_dtype": ("bf16" if inp.kv_bf16 else "fp8_e4m3fn") if case.is_mla else "bf16",
            # decode_proportional with the same budget, timed against decode in one interleave
            "us_per_call_proportional": round(ms_prop * 1e3, 2) if ms_prop else None,
            "proportional_vs_equal": round(ms_prop / ms_eq, 3) if ms_prop else None,
        }
        if not args.headline_only and not args.no_cpu_baseline:
            entry["oracle"] = oracle_sample(case, args.oracle_seconds)
            if name == "mla_tiny_b1_h16_s4096_np1":   # the tiny call on one host thread
                entry["oracle_single_thread"] = oracle_sample(case, 60.0, n_threads=1)
        if case.is_mla and inp.q_len == 4:
            entry["mfma_tflops"] = round(mla_flops(inp) / (ms_split * 1e-3) / 1e12, 1)
        table[name] = entry
        print("# %-36s %s" % (name, json.dumps(entry)), file=sys.stderr, flush=True)
        if is_head:
            headline = (case, ms, ms_split, steps)
        graph_todo.append((name, case, steps))
        del case, inp


    if headline is None:
        print("unknown workload %s" % args.workload, file=sys.stderr)
        sys.exit(2)
    case, ms, ms_split, steps = headline
    alg = case.split_algorithmic_bytes()
    kv = case.kv_bytes()
    achieved = kv / (ms_split * 1e-3) / 1e9
    counters = measured_counters(args.workload)
    inp = case.inp
    result = {
        "metric": "split-KV decode KV-read GB/s (% of HBM peak) and us/call per config",
        "value": round(case.kv_bytes() / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 KV: bf16 QK^T and fp16 PV MFMA, fp32 accumulate" if case.is_mla and inp.kv_bf16
                  else "fp8e4m3 KV decoded exactly: bf16 QK^T and fp16 PV MFMA, fp32 accumulate" if case.is_mla
                  else "bf16 QK^T and PV MFMA, fp32 accumulate"),
        "data": ("synthetic (seeded N(0,1) bf16 queries, bf16 KV = N(0,1), shuffled slots)" if case.is_mla and inp.kv_bf16
                 else "synthetic (seeded N(0,1) bf16 queries, fp8 e4m3fn KV = N(0,1)*32, shuffled slots)" if case.is_mla
                 else "synthetic (seeded N(0,1) bf16 queries and K/V pages, random page placement)"),
        "config": {
            "workload": args.workload,
            "batch": inp.B, "q_len": inp.q_len,
            "heads": inp.H if case.is_mla else inp.Hq,
            "seq_len": int(inp.max_num_keys),
            "kv_dtype": ("bf16" if inp.kv_bf16 else "fp8_e4m3fn") if case.is_mla else "bf16",
            "np": case.np, "block_k": case.bk, "sm_count": sm,
            "us_per_call": round(ms * 1e3, 2),
            "pct_hbm_peak": round(100 * case.kv_bytes() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": split_kernel_name(inp),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counters["traffic"] if counters else None,
            "mfma_busy": counters["mfma_busy"] if counters else None,
            "valu_busy": counters.get("valu_busy") if counters else None,
            "algorithmic_bytes": kv,
            "algorithmic_bytes_what": ("KV payload: every key's row once (%d B per key)" % (inp.d_qk * inp.pool.element_size())
                                       if case.is_mla else "KV payload: every token's K and V rows once per kv head (512 B)"),
            "bytes_with_ids_q_partials": alg,
            "avg_launch_us": round(ms_split * 1e3, 2),
            "timer": "HIP events on the launch stream around the split-only launches of the timed "
                     "interleaved rounds (average per launch)",
        },
        "per_config": table,
    }
    q4 = table.get("mla_h64_b16_s131072_q4")
    if q4 and "mfma_tflops" in q4:
        result["roofline_q4"] = {
            "kernel": "mla_split_kernel", "workload": "mla_h64_b16_s131072_q4", "bound": "mfma",
            "achieved": q4["mfma_tflops"], "peak": 2500.0, "unit": "TFLOP/s",
            "frac": round(q4["mfma_tflops"] / 2500.0, 4), "avg_launch_us": q4["split_us"],
            "flops_what": "per (row, visible key) 2 x (576 + 512): QK^T on bf16 MFMA and PV on fp16 MFMA, "
                          "both at the 2.5 PFLOP/s dense bf16/fp16 peak"}
        q4_counters = measured_counters("mla_h64_b16_s131072_q4")
        if q4_counters:
            result["roofline_q4"].update({k: q4_counters.get(k) for k in ("traffic", "mfma_busy", "valu_busy")})
    gq = table.get("gqa_b32_hq64_hkv8_d128_p16")
    if gq and args.workload != "gqa_b32_hq64_hkv8_d128_p16":
        # the paged GQA workload's split kernel against the HBM peak (its table row's split-only time)
        gq_counters = measured_counters("gqa_b32_hq64_hkv8_d128_p16")
        gq_gbs = gq["kv_bytes"] / (gq["split_us"] * 1e-6) / 1e9
        result["roofline_gqa"] = {
            "kernel": "gqa_pair_kernel", "workload": "gqa_b32_hq64_hkv8_d128_p16", "bound": "hbm",
            "achieved": round(gq_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gq_gbs / HBM_PEAK_GBS, 4), "avg_launch_us": gq["split_us"],
            "traffic": gq_counters["traffic"] if gq_counters else None,
            "mfma_busy": gq_counters["mfma_busy"] if gq_counters else None,
            "bytes_what": "KV payload: every token's K and V rows once per kv head (512 B)",
            "timer": "HIP events around the table row's split-only launches (50 per row)"}
    if not args.headline_only:
        result["ceilings"] = ceilings(stream, case)
        if "gather_rows_gbs" in result["ceilings"]:
            result["ceilings"]["headline_split_pct_of_gather"] = round(
                100 * achieved / result["ceilings"]["gather_rows_gbs"], 1)
        print("# ceilings %s" % json.dumps(result["ceilings"]), file=sys.stderr, flush=True)
        result["planner_ns"] = planner_ns_per_call()
        result["dcp"] = dcp_line(stream, args.sweep_steps)
        print("# dcp %s" % json.dumps(result["dcp"]), file=sys.stderr, flush=True)
        result["planner_waves"] = wave_sweep(stream, args.sweep_steps)
        print("# planner_waves %s" % json.dumps(result["planner_waves"]), file=sys.stderr, flush=True)
        result["sparse_planner"] = sparse_sweep(stream, args.sweep_steps)
        print("# sparse_planner %s" % json.dumps(result["sparse_planner"]), file=sys.stderr, flush=True)
        result["planner_branches"] = branch_sweep(stream, args.sweep_steps)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    # HIP graph timings last, after every other timing (the sweeps too): a graph capture switches
    # the process to serving several hardware queues, in which splits of more than about a
    # thousand CTAs measured 4-5 % slower on MI355X (the paged GQA split: 356 us before the first
    # capture, 375 us after; launches on one stream, copies to the host and other kernels before
    # it changed nothing).
    for name, gcase, gsteps in graph_todo:
        ms_graph = time_graph(gcase.step, gsteps, stream)
        table[name]["us_per_call_graph"] = round(ms_graph * 1e3, 2) if ms_graph else None
        print("# graph %-30s %s" % (name, table[name]["us_per_call_graph"]), file=sys.stderr, flush=True)
    del graph_todo
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
