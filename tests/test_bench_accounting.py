"""The benchmark's algorithmic work (the numerator of every roofline figure)
against the oracle's own enumeration of what each row sees.

bench.rank_work counts flops as (visible keys) x heads x (2*576 + 2*512) per
row and KV bytes as the keys of a request's widest row x the row width; the
visible keys come from a closed-form bound.  Here the same quantities are
recounted from oracle.visible_positions, which enumerates the positions a
rank holds and filters them by the causal prefix (PR #52188 page, key source
snippets; PR #54012 page, implementation breakdown).  CPU only.
"""
import numpy as np
import pytest

import bench
import oracle
import workloads as WL

SPECS = [
    WL.Spec(name="acct_w1_causal", B=3, H=16, Q=4, causal=True, seed=11, lengths=[5, 70, 257]),
    WL.Spec(name="acct_w4_causal", B=3, H=8, Q=3, causal=True, seed=12, lengths=[2, 9, 300], W=4, ranks=(0, 1, 2, 3)),
    WL.Spec(name="acct_w4_i2", B=2, H=8, Q=5, causal=True, seed=13, lengths=[17, 203], W=4, ranks=(0, 3), interleave=2),
    WL.Spec(name="acct_w2_draft", B=2, H=16, Q=16, causal=False, seed=14, lengths=[40, 333], W=2, ranks=(0, 1)),
    WL.Spec(name="acct_varlen", B=3, H=24, Q=4, causal=True, seed=15, lengths=[60, 129, 7], W=2, ranks=(1,),
            q_lens=[4, 1, 3]),
    WL.Spec(name="acct_fp8", B=2, H=16, Q=1, causal=True, seed=16, lengths=[100, 64], kv_dtype="fp8", kv_scale=0.5),
]


@pytest.mark.parametrize("spec", SPECS, ids=[s.name for s in SPECS])
def test_rank_work_matches_the_oracle_enumeration(spec):
    wl = WL.build(spec)
    q_lens = bench.q_lens_of(spec)
    row_bytes = 576 if spec.kv_dtype == "fp8" else 1152
    for r in spec.ranks:
        flops = kv = 0
        for b in range(spec.B):
            seq = int(wl.seq_lens[r][b])
            tot = int(wl.tot[b])
            counts = [len(oracle.visible_positions(seq, tot, q_lens[b], j, spec.W, r, spec.causal, spec.interleave))
                      for j in range(q_lens[b])]
            flops += sum(counts) * spec.H * (2 * 576 + 2 * 512)
            kv += (max(counts) if counts else 0) * row_bytes
        w = bench.rank_work(wl, r)
        assert w["flops"] == flops, (r, w["flops"], flops)
        assert w["kv_bytes"] == kv, (r, w["kv_bytes"], kv)


def test_flop_count_of_one_row_and_key():
    # one visible key for one head of one row: QK^T over 576 dims and PV over
    # 512, a multiply and an add each
    assert bench.FLOP_PER_KEY_ROW == 2176
    spec = WL.Spec(name="acct_one", B=1, H=1, Q=1, causal=True, seed=17, lengths=[1])
    w = bench.rank_work(WL.build(spec), 0)
    assert w["flops"] == 2176 and w["kv_bytes"] == 1152
    assert np.isclose(w["q_bytes"], 1152) and w["out_bytes"] == 1024 and w["lse_bytes"] == 4


@pytest.mark.parametrize("spec", SPECS, ids=[s.name for s in SPECS])
def test_cpu_baseline_runs_every_item_of_a_tiny_workload(spec):
    """The benchmark's CPU-baseline leg (the oracle in a pool of worker
    processes) on each kind of workload, varlen and FP8 included: every
    (request, rank) item finishes inside the budget, the reported work equals
    the accounting above, and the record names its worker count."""
    wl = WL.build(spec)
    ranks = sorted(wl.pools)
    unit = "TFLOP/s" if spec.H * spec.Q > 16 else "GB/s"
    res = bench.cpu_baseline(wl, ranks, unit, budget_s=120.0, workers=2)
    assert res["kind"] == "oracle" and res["cores"] == 2 and res["unit"] == unit
    assert res["value"] > 0
    assert res["sample"].startswith(f"{spec.B * len(ranks)} of {spec.B * len(ranks)} (request, rank) items")
