"""The float64 oracle over every element of a full-size workload, in a pool
of worker processes (test infrastructure for the full-size GPU parity tests).

python -m tests.oracle_full --config N --out DIR [--workers K] [--unsharded] [--fp8]

Runs in a process of its own that never touches the GPU: it builds the
workload from its seed (the same inputs the test uploads), forks single-
threaded workers over (request, rank) items, and writes for every rank r of
the workload DIR/out_r{r}.npy [B*Q, H, 512] and DIR/lse_r{r}.npy [B*Q, H]
(float64, the oracle's own precision).  With --unsharded it also writes
DIR/out_u.npy and DIR/lse_u.npy: the attention of every row over its whole
global causal prefix (W = 1 over the contiguous global KV), which the
LSE-merged shards must equal.  With --fp8 the workload's cache holds E4M3
codes with the scale FP8_KV_SCALE, as bench.py --fp8 builds it.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_JOB = {}
FP8_KV_SCALE = 1.0 / 64  # codes of N(0,1) values / this scale, as in bench.py --fp8


def spec_of(config, fp8=False):
    import workloads as WL
    return WL.config(config, kv_dtype="fp8", kv_scale=FP8_KV_SCALE) if fp8 else WL.config(config)


def _item(it):
    import numpy as np
    import oracle
    b, r = it
    wl = _JOB["wl"]
    s = wl.spec
    rows_of = lambda _b, pos: wl.global_rows(b, pos)  # noqa: E731
    kvs = s.kv_scale if s.kv_dtype == "fp8" else None
    if r == "u":
        tot = wl.tot[b:b + 1]
        out, lse = oracle.mla_decode(wl.q_bits[b:b + 1], rows_of, tot.astype(np.int64), tot, 1, 0, True, s.scale,
                                     s.lse_base, interleave=1, kv_scale=kvs)
    else:
        tot = None if (s.global_is_null and s.W == 1) else wl.tot[b:b + 1]
        out, lse = oracle.mla_decode(wl.q_bits[b:b + 1], rows_of, wl.seq_lens[r][b:b + 1], tot, s.W, r, s.causal,
                                     s.scale, s.lse_base, interleave=s.interleave, kv_scale=kvs)
    return b, r, out, lse


def run(spec, out_dir, workers, unsharded=False):
    import multiprocessing as mp
    import numpy as np
    import workloads as WL
    wl = WL.build(spec)
    s = wl.spec
    ranks = sorted(wl.pools)
    keys = list(ranks) + (["u"] if unsharded else [])
    res = {k: (np.full((s.B * s.Q, s.H, 512), np.nan), np.full((s.B * s.Q, s.H), np.nan)) for k in keys}
    items = [(b, k) for b in range(s.B) for k in keys]
    # longest requests first, so the pool's tail is short
    items.sort(key=lambda it: -int(wl.tot[it[0]]))
    _JOB["wl"] = wl
    with mp.get_context("fork").Pool(workers) as pool:
        for b, k, out, lse in pool.imap_unordered(_item, items):
            res[k][0][b * s.Q:(b + 1) * s.Q] = out
            res[k][1][b * s.Q:(b + 1) * s.Q] = lse
    for k, (out, lse) in res.items():
        tag = f"r{k}" if k != "u" else "u"
        np.save(os.path.join(out_dir, f"out_{tag}.npy"), out)
        np.save(os.path.join(out_dir, f"lse_{tag}.npy"), lse)


def default_workers():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def start(config, out_dir, unsharded=False, fp8=False):
    """Start the oracle for workload `config` in a child process (single-
    threaded BLAS in every worker); returns the Popen."""
    import subprocess
    env = dict(os.environ)
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        env[v] = "1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    cmd = [sys.executable, "-m", "tests.oracle_full", "--config", str(config), "--out", str(out_dir),
           "--workers", str(default_workers())]
    if unsharded:
        cmd.append("--unsharded")
    if fp8:
        cmd.append("--fp8")
    return subprocess.Popen(cmd, cwd=ROOT, env=env)


def load(out_dir, key):
    import numpy as np
    tag = f"r{key}" if key != "u" else "u"
    return np.load(os.path.join(out_dir, f"out_{tag}.npy")), np.load(os.path.join(out_dir, f"lse_{tag}.npy"))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--workers", type=int, default=0)
    ap.add_argument("--unsharded", action="store_true")
    ap.add_argument("--fp8", action="store_true")
    args = ap.parse_args()
    sys.path.insert(0, ROOT)
    t0 = time.perf_counter()
    run(spec_of(args.config, args.fp8), args.out, args.workers or default_workers(), args.unsharded)
    print(f"[oracle_full] workload {args.config}: {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
