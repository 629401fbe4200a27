#!/usr/bin/env python3
"""Benchmark of the paged MLA decode hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--interleave I]
                [--varlen | --fp8] [--no-cpu-baseline]

A step is one pass of the hot path over one batch of synthetic input:
  * slot mapping of the step's new tokens (cp_local_slot),
  * each rank's decode (mla_decode: row bounds, paged gather, QK^T, online
    softmax, PV, split combine, finalise),
  * and, for a sharded workload, the LSE merge of the ranks' partials.
Without --config every workload runs, one after another in one process:
  1 tiny (B=2, H=16, q_len 1), 2 single-token decode (B=64, H=16),
  3 causal spec decode (B=32, H=128, q_len 4), 4 DCP-8 shards + merge
  (B=16, H=128, q_len 4), 5 the non-causal draft block under DCP 2
  (B=16, H=128, q_len 16, rank 1), the largest, which is the headline
  (the line's top-level value, roofline and cpu_baseline); and 6, spec
  decode with 16 heads (B=64, H=16, q_len 4: the 64-row tile).  Every
  workload's own figures are under "configs".  --config N runs workload N alone as the
  headline.  --fp8 stores the cache as E4M3 codes with one scale
  (mla_decode_fp8); --varlen draws a query length per request
  (mla_decode_varlen); --interleave deals positions to the ranks in
  segments of I.
Inputs are resident in HBM before timing starts.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode TFLOP/s + KV GB/s and % of binding roofline, 1×MI355X"
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2516.6    # 256 CU x 4096 flop/clk x 2.4 GHz, dense bf16
FLOP_PER_KEY_ROW = 2 * 576 + 2 * 512   # QK^T (576-wide) + PV (512-wide) per (row, key)
KV_ROW_BYTES = 576 * 2
FP8_KV_SCALE = 1.0 / 64           # --fp8: codes of N(0,1) values / this scale (|value| < 7 stays below 448)
HEADLINE = 5                      # the largest workload
MEM_BOUND = (1, 2, 6)             # 16-head workloads (64 rows and fewer): HBM is the binding roof
MAX_CPU_WORKERS = 16              # host share of one GPU on the measurement boxes


def kv_row_bytes(s):
    return 576 if s.kv_dtype == "fp8" else KV_ROW_BYTES


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ HIP events
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b):
        assert self.lib.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


# ------------------------------------------------------------------ algorithmic work
def row_keys(seq, tot, Q, j, W, r, causal, I=1):
    """Rank-local visible keys of row j (the same bound the kernel applies):
    of the global prefix g, rank r holds the positions of the segments of I
    dealt to it."""
    if not causal:
        return seq
    g = max(tot - (Q - 1 - j), 0)
    return min(seq, g // (I * W) * I + min(max(g % (I * W) - r * I, 0), I))


def q_lens_of(s):
    return [int(x) for x in s.q_lens] if s.q_lens is not None else [s.Q] * s.B


def request_work(wl, r, b):
    """Algorithmic flops and KV bytes of request b on rank r."""
    s = wl.spec
    ql = q_lens_of(s)[b]
    seq = int(wl.seq_lens[r][b])
    tot = int(wl.tot[b]) if not s.global_is_null else seq
    nmax = row_keys(seq, tot, ql, ql - 1, s.W, r, s.causal, s.interleave) if ql else 0
    flops = sum(row_keys(seq, tot, ql, j, s.W, r, s.causal, s.interleave) for j in range(ql)) * s.H * FLOP_PER_KEY_ROW
    return flops, nmax * kv_row_bytes(s), nmax


def rank_work(wl, r):
    s = wl.spec
    flops = kv = bt = 0
    for b in range(s.B):
        f, k, nmax = request_work(wl, r, b)
        flops += f
        kv += k
        bt += -(-nmax // s.block_size) * 4
    rows = sum(q_lens_of(s)) * s.H
    return dict(flops=flops, kv_bytes=kv, q_bytes=rows * KV_ROW_BYTES, bt_bytes=bt,
                out_bytes=rows * 512 * 2, lse_bytes=rows * 4)


def source_hash():
    """Hash of the sources the attention kernels are built from (traffic
    figures taken on other sources are not reported)."""
    h = hashlib.sha256()
    for name in ("mla_decode.hip", "mla_device.h"):
        h.update(open(os.path.join(ROOT, "decode_attention_11_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def make_spec(n, args):
    import numpy as np
    import workloads as WL
    kv_kw = dict(kv_dtype="fp8", kv_scale=FP8_KV_SCALE) if args.fp8 else {}
    spec = WL.config(n, interleave=args.interleave, **kv_kw)
    if args.varlen:
        ql = np.random.default_rng([spec.seed, 31337]).integers(1, spec.Q, size=spec.B, endpoint=True)
        ql[0] = spec.Q  # the largest length stays the workload's q_len
        spec = WL.config(n, interleave=args.interleave, q_lens=[int(x) for x in ql])
    return spec


def workload_name(s):
    return s.name + ("_varlen" if s.q_lens is not None else "") + ("_fp8kv" if s.kv_dtype == "fp8" else "")


# ------------------------------------------------------------------ CPU baseline (oracle)
_CPU_JOB = {}


def _oracle_item(item):
    """One (request, rank) of the workload through the float64 oracle: all
    query rows and heads of request b on rank r.  Runs in a forked worker."""
    import numpy as np
    import oracle
    b, r = item
    wl = _CPU_JOB["wl"]
    s = wl.spec
    kvs = s.kv_scale if s.kv_dtype == "fp8" else None
    seq = wl.seq_lens[r][b:b + 1]
    tot = None if (s.global_is_null and s.W == 1) else wl.tot[b:b + 1]
    rows_of = lambda _b, pos: wl.global_rows(b, pos)  # noqa: E731
    if s.q_lens is not None:
        qsl = wl.query_start_loc
        one = np.array([0, qsl[b + 1] - qsl[b]], dtype=np.int32)
        out, lse = oracle.mla_decode_varlen(wl.q_tok[qsl[b]:qsl[b + 1]], one, rows_of, seq, tot, s.W, r, s.causal,
                                            s.scale, s.lse_base, interleave=s.interleave)
    else:
        out, lse = oracle.mla_decode(wl.q_bits[b:b + 1], rows_of, seq, tot, s.W, r, s.causal, s.scale, s.lse_base,
                                     interleave=s.interleave, kv_scale=kvs)
    flops, kv, _ = request_work(wl, r, b)
    return b, r, flops, kv, out, lse


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, ranks, unit, budget_s=25.0, workers=None):
    """The float64 oracle on the host cores: a fork pool of worker processes
    over (request, rank) items, longest first, stopped once budget_s of wall
    time has passed.  A sharded workload whose every rank ran also merges
    each finished request's partials (oracle.merge_lse); the draft-block
    workload also maps its slots (oracle.cp_local_slot).  The calling process
    must not have touched the GPU, and its BLAS must be single-threaded (set
    before numpy is imported), or every worker runs a thread pool of its own:
    cpu_baseline_child() arranges both."""
    import multiprocessing as mp
    import numpy as np
    import oracle
    import workloads as WL
    s = wl.spec
    n_aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    workers = max(1, min(MAX_CPU_WORKERS, n_aff) if workers is None else workers)
    items = sorted(((b, r) for b in range(s.B) for r in ranks), key=lambda it: -request_work(wl, it[1], it[0])[0])
    _CPU_JOB["wl"] = wl
    ctx = mp.get_context("fork")
    done = {}
    flops = kv = 0
    t0 = time.perf_counter()
    pool = ctx.Pool(workers)
    try:
        for b, r, f, k, out, lse in pool.imap_unordered(_oracle_item, items):
            done.setdefault(b, {})[r] = (out, lse)
            flops += f
            kv += k
            log(f"cpu baseline: request {b} rank {r} done ({time.perf_counter() - t0:.1f} s)")
            if len(done[b]) == len(ranks) and s.W > 1 and len(ranks) == s.W:
                oracle.merge_lse([done[b][x][0] for x in ranks], [done[b][x][1] for x in ranks], s.lse_base)
            if time.perf_counter() - t0 > budget_s:
                break
    finally:
        pool.terminate()
        pool.join()
    if s.W > 1 and not s.causal:
        si = WL.draft_slot_inputs(wl)
        for r in ranks:
            oracle.cp_local_slot(si["ctx_positions"], wl.block_table, s.block_size, s.W, r, s.interleave,
                                 si["ctx_num_valid"])
            oracle.cp_local_slot(si["query_positions"], wl.block_table, s.block_size, s.W, r, s.interleave)
    dt = time.perf_counter() - t0
    _CPU_JOB.clear()
    n_items = sum(len(v) for v in done.values())
    value = kv / dt / 1e9 if unit == "GB/s" else flops / dt / 1e12
    extra = ("; with the LSE merge of each request whose ranks all finished" if s.W > 1 and len(ranks) == s.W
             else "") + ("; with both slot mappings" if s.W > 1 and not s.causal else "")
    return {"value": round(value, 6), "unit": unit, "cores": int(workers), "kind": "oracle",
            "sample": f"{n_items} of {len(items)} (request, rank) items of {workload_name(s)}, every query row and "
                      f"head of each{extra}; float64 numpy oracle in {workers} single-threaded worker processes "
                      f"(of {n_aff} host CPUs, {cpu_model()}), {dt:.1f} s wall"}


BLAS_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def cpu_baseline_child(n, args, budget_s):
    """Runs cpu_baseline for workload n in a child process of its own (GPU-
    free, single-threaded BLAS in every worker), which rebuilds the seeded
    inputs, and returns its record (None if it failed)."""
    import subprocess
    env = dict(os.environ)
    for v in BLAS_THREAD_VARS:
        env[v] = "1"
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-only", str(n), "--cpu-budget", str(budget_s),
           "--interleave", str(args.interleave)] + (["--fp8"] if args.fp8 else []) + (["--varlen"] if args.varlen else [])
    proc = subprocess.run(cmd, env=env, stdout=subprocess.PIPE, text=True)
    if proc.returncode != 0:
        log(f"cpu baseline of workload {n} failed ({proc.returncode})")
        return None
    return json.loads(proc.stdout.strip().splitlines()[-1])


# ------------------------------------------------------------------ achievable peaks
def measured_peaks(torch, mla, hip, stream, dev, reps=5):
    """Achievable HBM and bf16 matrix rates on this GPU, measured with torch
    (not this library): a 1 GiB device copy (bytes read + written), row sums
    over 1 GiB (bytes read: the memory-bound kernels' bytes are nearly all
    reads) and an 8192^3 bf16 GEMM (hipBLASLt); and the library's bare bf16
    MFMA loop (mla_probe_mfma: 1024 workgroups, 2000 steps of four
    32x32x16 MFMAs per wave).  Reported beside the published peaks."""
    out = {}
    x = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    a_, b_ = hip.event(), hip.event()
    y.copy_(x)
    torch.cuda.synchronize()
    hip.record(a_, stream)
    for _ in range(reps):
        y.copy_(x)
    hip.record(b_, stream)
    out["hbm_copy_GBps"] = round((2 << 30) * reps / (hip.elapsed_ms(a_, b_) * 1e-3) / 1e9, 1)
    # row sums of 4 KiB rows: 1 GiB read, 1 MiB written (a full reduction
    # reads far slower in torch)
    rows = x.view(-1, 1024)
    acc = torch.empty(rows.shape[0], dtype=torch.float32, device=dev)
    torch.sum(rows, 1, out=acc)
    torch.cuda.synchronize()
    hip.record(a_, stream)
    for _ in range(reps):
        torch.sum(rows, 1, out=acc)
    hip.record(b_, stream)
    out["hbm_read_GBps"] = round(((1 << 30) + acc.numel() * 4) * reps / (hip.elapsed_ms(a_, b_) * 1e-3) / 1e9, 1)
    del x, y, rows, acc
    n = 8192
    g = torch.Generator(device=dev).manual_seed(0)
    m1 = torch.randn((n, n), dtype=torch.bfloat16, device=dev, generator=g).contiguous()
    m2 = torch.randn((n, n), dtype=torch.bfloat16, device=dev, generator=g).contiguous()
    torch.matmul(m1, m2)
    torch.cuda.synchronize()
    hip.record(a_, stream)
    for _ in range(reps):
        torch.matmul(m1, m2)
    hip.record(b_, stream)
    out["bf16_gemm_TFLOPs"] = round(2.0 * n ** 3 * reps / (hip.elapsed_ms(a_, b_) * 1e-3) / 1e12, 1)
    del m1, m2
    wg, iters = 1024, 2000
    probe = mla.probe_mfma(wg, iters)
    torch.cuda.synchronize()
    hip.record(a_, stream)
    for _ in range(reps):
        mla.probe_mfma(wg, iters, out=probe)
    hip.record(b_, stream)
    out["mfma_loop_TFLOPs"] = round(wg * 4 * iters * 4 * 32768.0 * reps / (hip.elapsed_ms(a_, b_) * 1e-3) / 1e12, 1)
    del probe
    hip.destroy(a_)
    hip.destroy(b_)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------------ KV write
def kv_write_rates(torch, mla, hip, stream, dev, step_job, reps=20, bulk_rows=1 << 18, kv_scale=None):
    """Times mla_kv_write (mla_kv_write_fp8 with kv_scale) twice: storing the
    step's new-token rows at their slots (quantised, for FP8), and a bulk
    scatter of bulk_rows random rows to a permutation of a scratch cache's
    rows (bytes = rows x 1152 read + rows x 1152 written, or x 576 for FP8,
    + 8 per slot)."""
    rows, slots, cache = step_job
    kw = {} if kv_scale is None else {"kv_scale": kv_scale}
    a_, b_ = hip.event(), hip.event()
    mla.kv_write(rows, slots, cache, **kw)
    torch.cuda.synchronize()
    step_us = 0.0
    for _ in range(reps):  # one launch between each event pair: the host enqueues slower than it runs
        hip.record(a_, stream)
        mla.kv_write(rows, slots, cache, **kw)
        hip.record(b_, stream)
        step_us += hip.elapsed_ms(a_, b_) * 1e3 / reps
    g = torch.Generator(device=dev).manual_seed(1)
    big_rows = torch.randint(-32768, 32767, (bulk_rows, 576), dtype=torch.int16, device=dev,
                             generator=g).view(torch.bfloat16)
    big_cache = torch.empty((bulk_rows // 64, 64, 576), dtype=torch.bfloat16 if kv_scale is None else torch.uint8,
                            device=dev)
    big_slots = torch.randperm(bulk_rows, device=dev, generator=g)
    mla.kv_write(big_rows, big_slots, big_cache, **kw)
    torch.cuda.synchronize()
    hip.record(a_, stream)
    for _ in range(5):
        mla.kv_write(big_rows, big_slots, big_cache, **kw)
    hip.record(b_, stream)
    bulk_us = hip.elapsed_ms(a_, b_) * 1e3 / 5
    nbytes = bulk_rows * (1152 + (1152 if kv_scale is None else 576) + 8)
    hip.destroy(a_)
    hip.destroy(b_)
    del big_rows, big_cache, big_slots
    gbps = nbytes / (bulk_us * 1e-6) / 1e9
    return {"step_rows": int(rows.numel() // 576), "step_us": round(step_us, 2), "bulk_rows": bulk_rows,
            "bulk_us": round(bulk_us, 1), "bulk_GBps": round(gbps, 1), "bulk_frac": round(gbps / HBM_PEAK_GBPS, 4)}


# ------------------------------------------------------------------ one workload on the GPU
class GpuRun:
    """Device copies of one workload and the step that runs it."""

    def __init__(self, torch, mla, wl, dev, replicas):
        import numpy as np
        import workloads as WL
        s = wl.spec
        self.wl, self.s, self.torch, self.mla = wl, s, torch, mla
        self.ranks = sorted(wl.pools)
        self.replicas = replicas

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

        def kv_dev(pool):
            if pool.dtype == np.uint8:  # E4M3 codes
                return torch.from_numpy(np.ascontiguousarray(pool)).to(dev)
            return bf16(pool)

        self.bf16 = bf16
        self.q = bf16(wl.q_tok if s.q_lens is not None else wl.q_bits)
        self.qsl = torch.from_numpy(wl.query_start_loc).to(dev) if s.q_lens is not None else None
        self.T = sum(q_lens_of(s))
        self.bt = torch.from_numpy(wl.block_table).to(dev)
        tot = torch.from_numpy(wl.tot.astype(np.int32)).to(dev)
        self.fp8_kw = dict(kv_scale=s.kv_scale) if s.kv_dtype == "fp8" else {}
        self.pools = {r: [kv_dev(wl.pools[r])] for r in self.ranks}
        for r in self.ranks:
            for _ in range(replicas - 1):
                self.pools[r].append(self.pools[r][0].clone())
        self.seq = {r: torch.from_numpy(wl.seq_lens[r]).to(dev) for r in self.ranks}
        self.glob = None if s.global_is_null else tot
        if s.W > 1 and not s.causal:
            si = WL.draft_slot_inputs(wl)
            self.slot_jobs = [(torch.from_numpy(si["ctx_positions"]).to(dev),
                               torch.from_numpy(si["ctx_num_valid"]).to(dev)),
                              (torch.from_numpy(si["query_positions"]).to(dev), None)]
        else:
            qls = np.asarray(q_lens_of(s))
            newpos = (wl.tot[:, None] - qls[:, None] + np.arange(s.Q)[None, :]).astype(np.int64)
            newpos[np.arange(s.Q)[None, :] >= qls[:, None]] = -1  # shorter requests: pad positions
            self.slot_jobs = [(torch.from_numpy(newpos).to(dev), None)]
        self.max_seq = {r: int(wl.seq_lens[r].max()) for r in self.ranks}
        self.outs = {r: torch.empty((self.T, s.H, 512), dtype=torch.bfloat16, device=dev) for r in self.ranks}
        self.lses = {r: torch.empty((self.T, s.H), dtype=torch.float32, device=dev) for r in self.ranks}
        self.ws = {r: torch.empty((max(mla.mla_decode_workspace_size(s.B, s.Q, s.H, self.max_seq[r]), 1),),
                                  dtype=torch.uint8, device=dev) for r in self.ranks}
        self.merged = (torch.empty((self.T, s.H, 512), dtype=torch.bfloat16, device=dev),
                       torch.empty((self.T, s.H), dtype=torch.float32, device=dev))

    def step(self, i, evs=None):
        s, mla = self.s, self.mla
        rep = i % self.replicas
        for r in self.ranks:
            for pos, nv in self.slot_jobs:
                mla.cp_local_slot(pos, self.bt, s.block_size, s.W, r, nv, cp_interleave=s.interleave)
            if evs is not None:
                a, b_ = evs.pop()
                mla.profile_attention_events(a, b_)
            if self.qsl is not None:
                mla.mla_decode_varlen(self.q, self.qsl, self.pools[r][rep], self.bt, self.seq[r], self.glob, s.W, r,
                                      s.causal, s.scale, s.lse_base, max_q_len=s.Q, max_seq_len=self.max_seq[r],
                                      out=self.outs[r], lse=self.lses[r], workspace=self.ws[r],
                                      cp_interleave=s.interleave)
            else:
                mla.mla_decode(self.q, self.pools[r][rep], self.bt, self.seq[r], self.glob, s.W, r, None, s.causal,
                               s.scale, s.lse_base, max_seq_len=self.max_seq[r], out=self.outs[r], lse=self.lses[r],
                               workspace=self.ws[r], cp_interleave=s.interleave, **self.fp8_kw)
        if evs is not None:
            mla.profile_attention_events(None, None)
        if s.W > 1 and len(self.ranks) == s.W:
            mla.mla_merge_lse([self.outs[r] for r in self.ranks], [self.lses[r] for r in self.ranks], s.lse_base,
                              out=self.merged[0], lse=self.merged[1])

    def parts(self, hip, stream, n):
        """The step's parts timed apart with HIP events, n repetitions each: the
        slot mapping of the step's tokens (every rank), and for a sharded step
        the LSE merge, whose bytes (the ranks' bf16 partials and fp32 LSEs read,
        the merged pair written) give its HBM rate."""
        torch, s, mla = self.torch, self.s, self.mla

        def timed(fn):
            # a device-side spin first, so that the n calls are all queued before
            # the first runs and the events see GPU time, not Python launch time
            a, b = hip.event(), hip.event()
            torch.cuda._sleep(4_000_000)
            hip.record(a, stream)
            for _ in range(n):
                fn()
            hip.record(b, stream)
            ms = hip.elapsed_ms(a, b) / n
            hip.destroy(a)
            hip.destroy(b)
            return ms

        def slots():
            for r in self.ranks:
                for pos, nv in self.slot_jobs:
                    mla.cp_local_slot(pos, self.bt, s.block_size, s.W, r, nv, cp_interleave=s.interleave)

        out = {"slot_calls_per_step": len(self.ranks) * len(self.slot_jobs),
               "slot_us_per_step": round(timed(slots) * 1e3, 2)}
        if s.W > 1 and len(self.ranks) == s.W:
            def merge():
                mla.mla_merge_lse([self.outs[r] for r in self.ranks], [self.lses[r] for r in self.ranks],
                                  s.lse_base, out=self.merged[0], lse=self.merged[1])
            ms = timed(merge)
            nbytes = (len(self.ranks) + 1) * self.T * s.H * (512 * 2 + 4)
            out.update({"merge_us": round(ms * 1e3, 2), "merge_bytes": nbytes,
                        "merge_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "merge_frac_of_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)})
        return out


def graph_steps(torch, hip, stream, run, steps, warmup):
    """The same steps replayed from HIP graphs (torch.cuda.CUDAGraph), one
    captured per KV replica, as a serving loop replays its captured decode
    step (PR #52188 page, risks: the captured step replayed every decode
    step): ms per step, launch overheads excluded.  Nothing in a step
    allocates, synchronises with the host or clears memory.  None if the
    capture fails."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(run.replicas):
                run.step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for i in range(run.replicas):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run.step(i)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(max(warmup, run.replicas)):
            graphs[i % run.replicas].replay()
        torch.cuda.synchronize()
        g_start, g_stop = hip.event(), hip.event()
        hip.record(g_start, stream)
        for i in range(steps):
            graphs[i % run.replicas].replay()
        hip.record(g_stop, stream)
        torch.cuda.synchronize()
        ms = hip.elapsed_ms(g_start, g_stop) / steps
        hip.destroy(g_start)
        hip.destroy(g_stop)
        del graphs
        return ms
    except Exception as e:  # reported as null; the eager figures stand
        log(f"graph replay not measured: {e}")
        return None


def measure(torch, hip, stream, run, n, args):
    """Warm-up, then exactly args.steps timed steps of one workload with the
    attention kernel's own events, then the same steps without those events;
    returns the workload's figures."""
    import numpy as np
    s, wl, ranks = run.s, run.wl, run.ranks
    log(f"{s.name}: warmup {args.warmup} steps")
    for i in range(args.warmup):
        run.step(i)
    torch.cuda.synchronize()
    pairs = [(hip.event(), hip.event()) for _ in range(args.steps * len(ranks))]
    todo = list(reversed(pairs))
    t_start, t_stop = hip.event(), hip.event()
    log(f"{s.name}: timing {args.steps} steps")
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    hip.record(t_start, stream)
    for i in range(args.steps):
        run.step(i, todo)
    hip.record(t_stop, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = hip.elapsed_ms(t_start, t_stop)
    attn_ms = [hip.elapsed_ms(a, b_) for a, b_ in pairs]
    for e in (t_start, t_stop):
        hip.destroy(e)
    for a, b_ in pairs:
        hip.destroy(a)
        hip.destroy(b_)
    # the same steps once more without the events around the attention
    # launches (reported beside the instrumented figure, not as the value)
    u_start, u_stop = hip.event(), hip.event()
    hip.record(u_start, stream)
    for i in range(args.steps):
        run.step(i)
    hip.record(u_stop, stream)
    plain_ms_per_step = hip.elapsed_ms(u_start, u_stop) / args.steps
    hip.destroy(u_start)
    hip.destroy(u_stop)
    graph_ms_per_step = graph_steps(torch, hip, stream, run, args.steps, args.warmup)
    ms_per_step = total_ms / args.steps
    avg_attn_ms = sum(attn_ms) / len(attn_ms)
    log(f"{s.name}: {ms_per_step:.4f} ms/step (wall {wall / args.steps * 1e3:.4f}), "
        f"attention kernel avg {avg_attn_ms:.4f} ms")

    work = [rank_work(wl, r) for r in ranks]
    step_flops = sum(w["flops"] for w in work)
    step_kv = sum(w["kv_bytes"] for w in work)
    step_alg_bytes = sum(w["kv_bytes"] + w["q_bytes"] + w["bt_bytes"] + w["out_bytes"] + w["lse_bytes"] for w in work)
    tflops = step_flops / (ms_per_step * 1e-3) / 1e12
    kv_gbps = step_kv / (ms_per_step * 1e-3) / 1e9
    # per launch of the attention kernel: it reads KV, Q and the block table
    launch_bytes = sum(w["kv_bytes"] + w["q_bytes"] + w["bt_bytes"] for w in work) / len(ranks)
    launch_flops = step_flops / len(ranks)
    if n in MEM_BOUND:
        achieved = launch_bytes / (avg_attn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
        unit, value = "GB/s", kv_gbps
    else:
        achieved = launch_flops / (avg_attn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
        unit, value = "TFLOP/s", tflops
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["algorithmic_per_launch"] = int(launch_bytes) if n in MEM_BOUND else int(launch_flops)
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_config{n}{'_fp8' if args.fp8 else ''}.json")
    if os.path.exists(tfile) and not args.varlen and args.interleave == 1:
        t = json.load(open(tfile))
        if t.get("source_hash") == source_hash():
            traffic = t.get("bytes_per_launch")
    roof["traffic"] = traffic
    parts = run.parts(hip, stream, args.steps)
    parts["attention_ms_per_step"] = round(avg_attn_ms * len(ranks), 5)
    return {
        "workload": workload_name(s), "value": round(value, 3), "unit": unit, "ms_per_step": round(ms_per_step, 5),
        "tflops": round(tflops, 3), "kv_gbps": round(kv_gbps, 1),
        "alg_bytes_per_step": int(step_alg_bytes), "flops_per_step": int(step_flops),
        "attention_kernel_ms": round(avg_attn_ms, 5),
        "attention_kernel_ms_median": round(float(np.median(attn_ms)), 5),
        "attention_kernel_ms_min": round(float(min(attn_ms)), 5),
        "attention_launches_per_step": len(ranks),
        "ms_per_step_without_kernel_events": round(plain_ms_per_step, 5),
        "ms_per_step_graph": None if graph_ms_per_step is None else round(graph_ms_per_step, 5),
        "roofline": roof, "parts": parts,
        "shape": {"batch": s.B, "heads": s.H, "q_len": s.Q if s.q_lens is None else f"1..{s.Q} per request",
                  "causal": s.causal, "cp_world": s.W, "cp_interleave": s.interleave, "ranks": ranks,
                  "block_size": s.block_size, "kv_replicas": run.replicas,
                  "kv_cache": "fp8_e4m3" if s.kv_dtype == "fp8" else "bf16"},
    }


def kv_write_step_job(run):
    """The headline step's new-token rows of rank 0 with their slots."""
    import numpy as np
    s, wl, mla = run.s, run.wl, run.mla
    r0 = run.ranks[0]
    pos0, nv0 = run.slot_jobs[0]
    slots0 = mla.cp_local_slot(pos0, run.bt, s.block_size, s.W, r0, nv0, cp_interleave=s.interleave)
    pos_np = pos0.cpu().numpy()
    rows_np = np.zeros(pos_np.shape + (576,), dtype=np.uint16)  # rows of positions other ranks own stay zero
    I = s.interleave
    for b in range(s.B):
        for i, p in enumerate(pos_np[b]):
            t = (p // (I * s.W)) * I + p % I  # the rank's local row of p
            if p >= 0 and (p // I) % s.W == r0 and t < len(wl.shards[r0][b]):
                rows_np[b, i] = wl.shards[r0][b][t] if s.kv_dtype != "fp8" else 0
    return run.bf16(rows_np), slots0, run.pools[r0][0]


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", type=int, default=0, choices=[0, 1, 2, 3, 4, 5, 6],
                    help="run only this workload (0: all six, the largest as the headline)")
    ap.add_argument("--replicas", type=int, default=0, help="KV replicas rotated per step (0: auto)")
    ap.add_argument("--varlen", action="store_true",
                    help="per-request query lengths uniform in [1, q_len] (seeded), through mla_decode_varlen")
    ap.add_argument("--interleave", type=int, default=1,
                    help="DCP interleave: ranks hold segments of this many positions (sharded workloads)")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 (E4M3) latent cache with one dequantisation scale, through mla_decode_fp8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=25.0, help="seconds of oracle time for the headline")
    ap.add_argument("--cpu-baseline-only", type=int, default=0, help=argparse.SUPPRESS)
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("this benchmark runs on one GPU only: decode-context-parallel shards are computed one after "
               "another on a single MI355X and merged locally; run with --gpus 1")
        print(msg, file=sys.stderr)
        if int(os.environ.get("RANK", "0")) == 0:
            print(json.dumps({"metric": METRIC, "error": msg, "n_gpus": args.gpus}))
        sys.exit(2)
    if args.fp8 and args.varlen:
        print("--fp8 and --varlen are separate entry points; pick one", file=sys.stderr)
        sys.exit(2)

    import workloads as WL
    if args.cpu_baseline_only:
        # the child process of cpu_baseline_child: the oracle only, one JSON line
        n = args.cpu_baseline_only
        wl = WL.build(make_spec(n, args))
        unit = "GB/s" if n in MEM_BOUND else "TFLOP/s"
        print(json.dumps(cpu_baseline(wl, sorted(wl.pools), unit, args.cpu_budget)), flush=True)
        return
    order = [args.config] if args.config else [1, 2, 6, 3, 4, 5]
    headline = args.config or HEADLINE

    # the CPU baselines first, each in a child process of its own, so that
    # the GPU timings below run on a quiet host
    cpu = {}
    if not args.no_cpu_baseline:
        for n in order:
            budget = args.cpu_budget if n == headline else min(args.cpu_budget, 10.0)
            log(f"workload {n}: cpu baseline, oracle worker pool, budget {budget:.0f} s")
            cpu[n] = cpu_baseline_child(n, args, budget)
            if cpu[n]:
                log(f"workload {n}: cpu baseline {cpu[n]['value']} {cpu[n]['unit']}")
    wls = {}
    for n in order:
        spec = make_spec(n, args)
        log(f"workload {spec.name}: generating inputs")
        t0 = time.perf_counter()
        wls[n] = WL.build(spec)
        log(f"generated in {time.perf_counter() - t0:.1f} s")

    import torch
    import decode_attention_11_amd as mla
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    mla.load_library()
    dev = torch.device("cuda:0")
    hip = Hip()
    stream = torch.cuda.current_stream(dev).cuda_stream

    results = {}
    kvw = None
    for n in order:
        wl = wls[n]
        replicas = args.replicas or (3 if n in MEM_BOUND else 1)
        run = GpuRun(torch, mla, wl, dev, replicas)
        torch.cuda.synchronize()
        results[n] = measure(torch, hip, stream, run, n, args)
        results[n]["cpu_baseline"] = cpu.get(n)
        if n == headline:
            log("kv write: the step's new-token rows, and a bulk scatter")
            kvw = kv_write_rates(torch, mla, hip, stream, dev, kv_write_step_job(run),
                                 kv_scale=wl.spec.kv_scale if wl.spec.kv_dtype == "fp8" else None)
        del run
        wls[n] = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    log("achievable peaks: 1 GiB copy, 1 GiB of row sums, 8192^3 bf16 GEMM (torch), bare MFMA loop")
    peaks = measured_peaks(torch, mla, hip, stream, dev)
    for n, res in results.items():
        meas = peaks["hbm_read_GBps"] if n in MEM_BOUND else peaks["mfma_loop_TFLOPs"]
        res["roofline"]["frac_of_measured_peak"] = round(res["roofline"]["achieved"] / meas, 4) if meas > 0 else None

    h = results[headline]
    line = {
        "metric": METRIC, "value": h["value"], "unit": h["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": h["workload"], **h["shape"]},
        "tflops": h["tflops"], "kv_gbps": h["kv_gbps"],
        "alg_bytes_per_step": h["alg_bytes_per_step"], "flops_per_step": h["flops_per_step"],
        "attention_kernel_ms": h["attention_kernel_ms"],
        "attention_kernel_ms_median": h["attention_kernel_ms_median"],
        "attention_kernel_ms_min": h["attention_kernel_ms_min"],
        "ms_per_step_without_kernel_events": h["ms_per_step_without_kernel_events"],
        "ms_per_step_graph": h["ms_per_step_graph"],
        "source_hash": source_hash(),
        "roofline": h["roofline"], "cpu_baseline": h["cpu_baseline"],
        "measured_peaks": peaks, "kv_write": kvw, "parts": h["parts"],
        "configs": {f"C{n}": {k: v for k, v in r.items() if k != "shape"} | {"shape": r["shape"]}
                    for n, r in results.items()},
    }
    txt = json.dumps(line)
    print(txt, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(txt + "\n")


if __name__ == "__main__":
    main()
