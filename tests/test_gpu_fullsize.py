"""GPU parity at the benchmark's full sizes, in the launch configuration
bench.py times (max_seq_len = the rank's longest local length, the same
workspace sizing), on sampled rows the oracle computes one by one; every row
is also checked for the properties that hold at any size (finite outputs,
the empty-row contract), and slot mappings are compared bit-exactly in full.
"""
import numpy as np
import pytest
import torch

import decode_attention_11_amd as mla
import oracle
import workloads as WL
from tests.gpu_util import Uploaded, compare, say, i32_dev, i64_dev

pytestmark = pytest.mark.gpu


def sample_rows(wl, n, seed):
    """(b, j, h) triples: the longest and shortest requests at their first and
    last query rows and heads, then seeded random ones."""
    s = wl.spec
    rng = np.random.default_rng(seed)
    rows = set()
    for b in (int(np.argmax(wl.tot)), int(np.argmin(wl.tot))):
        rows.add((b, s.Q - 1, s.H - 1))
        rows.add((b, 0, 0))
    while len(rows) < n:
        rows.add((int(rng.integers(s.B)), int(rng.integers(s.Q)), int(rng.integers(s.H))))
    return sorted(rows)


def run_rank(up, wl, r):
    msl = max(int(wl.seq_lens[r].max()), 1)
    return up.run(r, wl.spec.lse_base, max_seq_len=msl)


def every_row_properties(out, lse, label):
    o = out.float()
    l = lse
    assert bool(torch.isfinite(o).all()), f"{label}: non-finite output"
    empty = ~torch.isfinite(l)
    assert bool((l[empty] == -float("inf")).all()), f"{label}: non-finite LSE that is not -inf"
    if bool(empty.any()):
        assert bool((o[empty] == 0).all()), f"{label}: empty rows must be zero"


def oracle_rows(wl, r, rows):
    s = wl.spec
    tot = None if (s.global_is_null and s.W == 1) else wl.tot
    return oracle.mla_decode(wl.q_bits, wl.global_rows, wl.seq_lens[r], tot, s.W, r, s.causal, s.scale,
                             s.lse_base, rows=rows)


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_full_size_rank_matches_oracle_on_sampled_rows(cfg):
    spec = WL.config(cfg)
    say(f"{spec.name}: generating")
    wl = WL.build(spec)
    up = Uploaded(wl)
    rows = sample_rows(wl, 24, 7000 + cfg)
    for r in sorted(wl.pools):
        say(f"{spec.name} rank {r}: {len(rows)} sampled rows")
        out, lse = run_rank(up, wl, r)
        torch.cuda.synchronize()
        every_row_properties(out, lse, f"{spec.name} r{r}")
        ro, rl = oracle_rows(wl, r, rows)
        compare(out, lse, ro, rl, f"{spec.name} r{r}", rows=[(b * spec.Q + j, h) for (b, j, h) in rows])


def test_full_size_dcp8_shards_merge_to_the_unsharded_attention():
    spec = WL.config(4)
    say(f"{spec.name}: generating")
    wl = WL.build(spec)
    up = Uploaded(wl)
    rows = sample_rows(wl, 16, 7004)
    flat = [(b * spec.Q + j, h) for (b, j, h) in rows]
    outs, lses = [], []
    for r in range(spec.W):
        say(f"{spec.name} rank {r}")
        out, lse = run_rank(up, wl, r)
        torch.cuda.synchronize()
        every_row_properties(out, lse, f"{spec.name} r{r}")
        if r in (0, spec.W - 1):
            ro, rl = oracle_rows(wl, r, rows)
            compare(out, lse, ro, rl, f"{spec.name} r{r}", rows=flat)
        outs.append(out)
        lses.append(lse)
    mo, ml = mla.mla_merge_lse(outs, lses, spec.lse_base)
    torch.cuda.synchronize()
    every_row_properties(mo, ml, f"{spec.name} merged")
    # the unsharded attention over the contiguous global KV (W = 1, every row
    # sees its global causal prefix)
    ro, rl = oracle.mla_decode(wl.q_bits, wl.global_rows, wl.tot.astype(np.int32), wl.tot, 1, 0, True, spec.scale,
                               spec.lse_base, rows=rows)
    compare(mo, ml, ro, rl, f"{spec.name} merged vs unsharded", rows=flat)


def test_full_size_draft_block_slots_bit_exact():
    spec = WL.config(5)
    wl = WL.build(spec)
    si = WL.draft_slot_inputs(wl)
    bt = i32_dev(wl.block_table)
    for r in range(spec.W):
        for key, nv in (("ctx_positions", si["ctx_num_valid"]), ("query_positions", None)):
            pos = si[key]
            got = mla.cp_local_slot(i64_dev(pos), bt, spec.block_size, spec.W, r,
                                    i32_dev(nv) if nv is not None else None).cpu().numpy()
            exp = oracle.cp_local_slot(pos, wl.block_table, spec.block_size, spec.W, r, 1, nv)
            assert np.array_equal(got, np.asarray(exp, dtype=np.int64)), f"rank {r} {key}"
            if nv is not None:
                # the rejected suffix of the context window maps to the pad slot
                for b in range(spec.B):
                    assert np.all(got[b, int(nv[b]):] == mla.PAD_SLOT_ID)


def test_full_size_new_token_slots_bit_exact():
    for cfg in (3, 4):
        spec = WL.config(cfg)
        wl = WL.build(spec)
        newpos = (wl.tot[:, None] - spec.Q + np.arange(spec.Q)[None, :]).astype(np.int64)
        bt = i32_dev(wl.block_table)
        for r in range(spec.W):
            got = mla.cp_local_slot(i64_dev(newpos), bt, spec.block_size, spec.W, r).cpu().numpy()
            exp = oracle.cp_local_slot(newpos, wl.block_table, spec.block_size, spec.W, r, 1, None)
            assert np.array_equal(got, np.asarray(exp, dtype=np.int64)), f"{spec.name} rank {r}"
