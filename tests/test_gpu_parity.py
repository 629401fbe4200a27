"""GPU parity of the HIP path against the CPU oracle on small seeded inputs.

Sizes are small enough for the full oracle but span several key subtiles,
row tiles and workgroup ranges, with ragged tails, empty shards and the
degenerate cases of the method.  Bar: slots bit-exact; attention output
max-abs <= 2e-2 and mean-abs <= 2e-3 against float64; LSE within 1e-3;
rows with nothing visible exactly (0, -inf).
"""
import json
import math
import os
import zlib

import numpy as np
import pytest
import torch

import decode_attention_11_amd as mla
import oracle
import workloads as WL
from tests.gpu_util import Uploaded, compare, say, bf16_dev, i32_dev, i64_dev, dev

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def oracle_rank(wl, r, base="e", causal=None):
    s = wl.spec
    causal = s.causal if causal is None else causal
    tot = None if (s.global_is_null and s.W == 1) else wl.tot
    return oracle.mla_decode(wl.q_bits, wl.global_rows, wl.seq_lens[r], tot, s.W, r, causal, s.scale, base,
                             interleave=s.interleave)


def spec(name, B, H, Q, causal, lengths, W=1, ranks=None, bs=64, seed=None, **kw):
    return WL.Spec(name=name, B=B, H=H, Q=Q, causal=causal, seed=seed if seed is not None else zlib.crc32(name.encode()) % 10000,
                   lengths=list(lengths), W=W, ranks=tuple(range(W)) if ranks is None else tuple(ranks),
                   block_size=bs, **kw)


CASES = [
    spec("c1_tiny", 2, 16, 1, True, [37, 100], pool_blocks=4, global_is_null=True, seed=1001),
    spec("h16_q1_ragged", 5, 16, 1, True, [1, 63, 64, 65, 3000], global_is_null=True),
    spec("h8_q2_two_rows_per_tile", 3, 8, 2, True, [2, 700, 1290], global_is_null=True),
    spec("h16_q4_dcp2", 3, 16, 4, True, [5, 333, 2049], W=2),
    spec("h24_q3_dcp8_rank3_bs128", 2, 24, 3, True, [31, 35], W=8, ranks=[3], bs=128),
    spec("h24_q3_dcp8_all_bs128", 2, 24, 3, True, [200, 1111], W=8, bs=128),
    spec("h128_q4_causal", 2, 128, 4, True, [4, 900], global_is_null=True),
    spec("h128_q4_dcp8_short", 2, 128, 4, True, [3, 77], W=8),
    spec("h16_q16_noncausal_dcp2", 2, 16, 16, False, [100, 2500], W=2),
    spec("h128_q16_noncausal_dcp2_rank1", 2, 128, 16, False, [64, 1000], W=2, ranks=[1]),
    spec("bs1", 2, 16, 1, True, [17, 90], bs=1, global_is_null=True),
    spec("bs16_dcp4", 3, 16, 2, True, [9, 130, 515], W=4, bs=16),
    spec("nan_fill", 3, 16, 4, True, [70, 130, 1000], W=2, fill="nan"),
    spec("nan_fill_h128", 2, 128, 4, True, [70, 600], W=2, fill="nan"),
    spec("zero_query", 2, 16, 4, True, [50, 700], W=3, q_zero=True),
    spec("peaky_query", 3, 16, 1, True, [100, 1500, 4000], q_mult=8.0, global_is_null=True),
    spec("peaky_h128", 2, 128, 4, True, [100, 1500], q_mult=8.0, global_is_null=True),
    spec("h1_q1", 3, 1, 1, True, [5, 64, 300], global_is_null=True),
    spec("h3_q5", 2, 3, 5, True, [10, 400], W=3),
    # 300 requests of 0..4 keys: more than 256 requests (several scan chunks)
    # and far more pieces per workgroup range than one batch of segments holds
    spec("many_tiny_requests", 300, 16, 1, True, [(7 * i) % 5 for i in range(300)], global_is_null=True),
    spec("many_tiny_requests_h128", 40, 128, 2, True, [(3 * i) % 4 for i in range(40)], W=2),
    # one request over every bundle: dozens of partial slots per group, merged
    # by the combine several batches at a time
    spec("one_request_all_bundles_h128", 1, 128, 4, True, [12000], global_is_null=True),
    # ranks holding segments of several positions (interleave > 1)
    spec("h16_q4_dcp2_interleave4", 3, 16, 4, True, [5, 333, 2049], W=2, interleave=4),
    spec("h128_q4_dcp4_interleave16", 2, 128, 4, True, [70, 1500], W=4, interleave=16, bs=64),
    spec("h16_q16_noncausal_dcp3_interleave2", 2, 16, 16, False, [100, 900], W=3, interleave=2),
    spec("h24_q3_dcp8_interleave8_bs128", 2, 24, 3, True, [200, 1111], W=8, interleave=8, bs=128),
    # block sizes that are not powers of two: both kernel families divide
    # instead of shifting
    spec("bs48_h128_q4", 3, 128, 4, True, [47, 1000, 2401], global_is_null=True, bs=48),
    # 128-row pieces start on 32-key boundaries when 32 divides the block
    # size: ranges that hold under 32 keys of a request lose them to the next
    # range, and the combine skips the emptied ones
    spec("h128_q2_piece_bounds_bs64", 5, 128, 2, True, [31, 33, 95, 290, 1700], global_is_null=True),
    spec("h128_q4_bs32_dcp2", 3, 128, 4, True, [40, 777, 2050], W=2, bs=32),
    spec("bs80_h128_q4_dcp2", 2, 128, 4, True, [161, 3000], W=2, bs=80),
    spec("bs48_h16_q1", 4, 16, 1, True, [1, 48, 49, 3000], global_is_null=True, bs=48),
    spec("bs80_h16_q1_dcp3", 3, 16, 1, True, [79, 800, 2500], W=3, bs=80),
    # 17-32 and 33-64 rows per request: the 32- and 64-row tiles (one or two
    # score waves), full and partly filled
    spec("rows24_h24_q1", 3, 24, 1, True, [40, 1000, 3000], global_is_null=True),
    spec("rows32_h16_q2_dcp2", 3, 16, 2, True, [5, 700, 2600], W=2),
    spec("rows48_h48_q1", 2, 48, 1, True, [900, 4100], global_is_null=True),
    spec("rows64_h16_q4_spec", 4, 16, 4, True, [3, 64, 1500, 5000], global_is_null=True),
    spec("rows48_h16_q3_dcp2_bs48", 2, 16, 3, True, [500, 3000], W=2, bs=48),
    spec("rows64_h16_q4_noncausal_dcp4_interleave2", 2, 16, 4, False, [100, 2100], W=4, interleave=2),
    # more than 128 rows: a full 128-row tile and a partial one (its rows past
    # the request's read the zero row and are never stored)
    spec("rows160_h40_q4_partial_tile", 3, 40, 4, True, [50, 900, 2500], global_is_null=True),
    spec("rows140_h20_q7_dcp2", 2, 20, 7, True, [300, 2049], W=2),
    spec("rows200_h25_q8_noncausal_bs128", 2, 25, 8, False, [129, 1700], bs=128, global_is_null=True),
]


@pytest.mark.parametrize("sp", CASES, ids=[c.name for c in CASES])
def test_decode_matches_oracle(sp):
    wl = WL.build(sp)
    up = Uploaded(wl)
    for r in sorted(wl.pools):
        for base in ("e", "2"):
            say(f"{sp.name} rank {r} base {base} B={sp.B} H={sp.H} Q={sp.Q} W={sp.W} bs={sp.block_size}")
            out, lse = up.run(r, base)
            torch.cuda.synchronize()
            ro, rl = oracle_rank(wl, r, base)
            compare(out, lse, ro, rl, f"{sp.name} r{r} {base}")


@pytest.mark.parametrize("name", ["many_tiny_requests", "many_tiny_requests_h128"])
def test_tight_max_seq_len_packs_many_pieces_per_workgroup(name):
    # max_seq_len = the longest local length: few workgroups, each covering
    # dozens of (request, row tile) pieces
    sp = next(c for c in CASES if c.name == name)
    wl = WL.build(sp)
    up = Uploaded(wl)
    for r in sorted(wl.pools):
        msl = max(int(wl.seq_lens[r].max()), 1)
        say(f"{sp.name} rank {r} max_seq_len {msl}")
        out, lse = up.run(r, "e", max_seq_len=msl)
        torch.cuda.synchronize()
        ro, rl = oracle_rank(wl, r, "e")
        compare(out, lse, ro, rl, f"{sp.name} r{r} tight")


@pytest.mark.parametrize("H", [16, 128])
def test_fewer_work_units_than_workgroups(H):
    # a loose max_seq_len plans a full grid for requests that hold fewer work
    # units than there are ranges: most ranges are empty, some of them between
    # two ranges that hold keys of the same request.  The combine must read
    # only the slots written by this call: the workspace first holds NaN bytes,
    # then the partials of a call on longer requests.
    msl = 1 << 20
    small = spec(f"few_units_h{H}", 2, H, 1, True, [5, 20], global_is_null=True, seed=515)
    big = spec(f"many_units_h{H}", 2, H, 1, True, [3000, 900], global_is_null=True, seed=516)
    ws = torch.full((mla.mla_decode_workspace_size(2, 1, H, msl),), 0xFF, dtype=torch.uint8, device=dev())
    for sp in (small, big, small):
        wl = WL.build(sp)
        say(f"{sp.name} max_seq_len {msl}")
        out, lse = Uploaded(wl).run(0, "e", max_seq_len=msl, workspace=ws)
        torch.cuda.synchronize()
        ro, rl = oracle_rank(wl, 0, "e")
        compare(out, lse, ro, rl, f"{sp.name} loose max_seq_len")


def test_long_piece_spans_several_block_table_windows():
    # block size 1 and 270k keys: each workgroup range covers more block-table
    # entries than one LDS window holds, so a piece continues across batches;
    # sampled rows against the oracle
    sp = spec("bs1_270k", 1, 2, 1, True, [270000], bs=1, global_is_null=True, seed=4242)
    say(f"{sp.name}: generating")
    wl = WL.build(sp)
    up = Uploaded(wl)
    out, lse = up.run(0, "e")
    torch.cuda.synchronize()
    rows = [(0, 0, 0), (0, 0, 1)]
    ro, rl = oracle.mla_decode(wl.q_bits, wl.global_rows, wl.seq_lens[0], None, 1, 0, True, sp.scale, "e", rows=rows)
    compare(out, lse, ro, rl, sp.name, rows=[(0, 0), (0, 1)])


def test_zero_query_lse_is_log_of_visible_count():
    sp = spec("zero_q_counts", 3, 16, 4, True, [3, 50, 700], W=3, q_zero=True)
    wl = WL.build(sp)
    up = Uploaded(wl)
    for r in range(3):
        out, lse = up.run(r)
        gl = lse.cpu().numpy()
        for b in range(3):
            for j in range(4):
                n = oracle.visible_positions(int(wl.seq_lens[r][b]), int(wl.tot[b]), 4, j, 3, r, True).size
                row = gl[b * 4 + j]
                if n == 0:
                    assert np.all(row == -np.inf)
                else:
                    np.testing.assert_allclose(row, math.log(n), atol=1e-5)


def test_single_rank_global_equals_null_global_bitwise():
    sp = spec("w1_global_vs_null", 3, 16, 4, True, [10, 500, 3000])
    wl = WL.build(sp)
    up = Uploaded(wl)
    o1, l1 = up.run(0, global_null=False)
    o0, l0 = up.run(0, global_null=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)


def test_base2_lse_is_base_e_over_ln2():
    sp = spec("bases", 2, 16, 2, True, [100, 900], W=2)
    wl = WL.build(sp)
    up = Uploaded(wl)
    for r in range(2):
        oe, le = up.run(r, "e")
        o2, l2 = up.run(r, "2")
        assert torch.equal(oe, o2)
        le, l2 = le.cpu().double().numpy(), l2.cpu().double().numpy()
        fin = np.isfinite(le)
        np.testing.assert_allclose(le[fin], l2[fin] * math.log(2.0), rtol=1e-5, atol=1e-6)


def test_flattened_rows_equal_native_multi_token():
    # B*Q single-token calls with per-row rank-local lengths and a repeated
    # block table give the native per-row-bounded result (the legacy flattened path)
    sp = spec("flattened", 3, 16, 4, True, [40, 700, 1999], W=4)
    wl = WL.build(sp)
    up = Uploaded(wl)
    B, Q, H, W = 3, 4, 16, 4
    for r in range(W):
        native_o, native_l = up.run(r)
        n = np.array([[oracle.visible_positions(int(wl.seq_lens[r][b]), int(wl.tot[b]), Q, j, W, r, True).size
                       for j in range(Q)] for b in range(B)], dtype=np.int32).reshape(-1)
        qf = up.q.view(B * Q, 1, H, 576)
        btf = up.bt.repeat_interleave(Q, dim=0).contiguous()
        fo, fl = mla.mla_decode(qf, up.pools[r], btf, i32_dev(n), None, cp_world=1, cp_rank=0, causal=False,
                                scale=sp.scale)
        torch.cuda.synchronize()
        # both are separate bf16 results: each must meet the bar against the oracle
        ro, rl = oracle_rank(wl, r)
        compare(native_o, native_l, ro, rl, f"native r{r}")
        compare(fo, fl, ro, rl, f"flattened r{r}")
        nl, fl_ = native_l.cpu().numpy(), fl.cpu().numpy()
        assert np.array_equal(np.isfinite(nl), np.isfinite(fl_))


def test_end_aligned_mask_is_not_what_the_kernel_does():
    # W=8, r=0, tot=32, Q=4: every row must see all 4 local keys (an
    # end-aligned local mask would give 1, 2, 3, 4)
    sp = spec("end_aligned", 1, 16, 4, True, [32], W=8, ranks=[0], q_zero=True)
    wl = WL.build(sp)
    up = Uploaded(wl)
    _, lse = up.run(0)
    np.testing.assert_allclose(lse.cpu().numpy(), math.log(4.0), atol=1e-5)


@pytest.mark.parametrize("W,base,I", [(2, "e", 1), (8, "e", 1), (8, "2", 1), (3, "2", 1), (2, "e", 16), (8, "e", 4)])
def test_sharded_then_merged_equals_unsharded(W, base, I):
    sp = spec(f"shard_merge_w{W}_i{I}", 3, 128 if W == 8 else 16, 4, True, [7, 800, 2600], W=W, interleave=I)
    wl = WL.build(sp)
    up = Uploaded(wl)
    parts = [up.run(r, base) for r in range(W)]
    mo, ml = mla.mla_merge_lse([p[0] for p in parts], [p[1] for p in parts], base)
    un = WL.unsharded(wl)
    uu = Uploaded(un)
    uo, ul = uu.run(0, base, global_null=True)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode(un.q_bits, un.global_rows, un.seq_lens[0], None, 1, 0, True, sp.scale, base)
    compare(mo, ml, ro, rl, f"merged W={W}")
    compare(uo, ul, ro, rl, f"unsharded W={W}")


def test_merge_matches_oracle_with_empty_partials():
    rng = np.random.default_rng(5)
    n, rows, H = 5, 7, 3
    outs = [WL.bf16_bits(rng.standard_normal((rows, H, 512), dtype=np.float32)) for _ in range(n)]
    lses = [rng.standard_normal((rows, H)).astype(np.float32) * 3 for _ in range(n)]
    lses[1][2, :] = -np.inf
    for i in range(n):
        lses[i][4, 1] = -np.inf        # one item empty in every partial
    for base in ("e", "2"):
        mo, ml = mla.mla_merge_lse([bf16_dev(o) for o in outs], [torch.from_numpy(l).to(dev()) for l in lses], base)
        torch.cuda.synchronize()
        ro, rl = oracle.merge_lse([oracle.bf16_bits_to_f64(o) for o in outs], [l.astype(np.float64) for l in lses],
                                  base)
        compare(mo, ml, ro, rl, f"merge {base}")


# ---------------------------------------------------------------- slots

@pytest.mark.parametrize("fname", ["cp_local_slot_hand_example.json", "cp_local_slot_interleave2_hand_example.json"])
def test_slot_hand_examples(fname):
    g = json.load(open(os.path.join(GOLDEN, fname)))
    for r, exp in g["expected"].items():
        got = mla.cp_local_slot(i64_dev(g["positions"]), i32_dev(g["block_table"]), g["block_size"],
                                g["cp_world"], int(r), cp_interleave=g["interleave"])
        assert got.cpu().tolist() == exp


@pytest.mark.parametrize("W,I,bs", [(1, 1, 64), (2, 1, 1), (2, 1, 4), (3, 1, 16), (4, 2, 16), (8, 1, 64),
                                    (8, 4, 128), (16, 1, 64), (16, 2, 2), (5, 1, 128)])
def test_slots_bit_exact_against_oracle(W, I, bs):
    rng = np.random.default_rng(W * 100 + I * 10 + bs)
    B, n, maxb = 5, 97, 9
    bt = rng.integers(0, 1 << 20, size=(B, maxb)).astype(np.int32)
    pos = rng.integers(-5, maxb * bs * W + 40, size=(B, n)).astype(np.int64)
    pos[0, :5] = [0, 1, bs * W - 1, bs * W, maxb * bs * W - 1]
    nv = rng.integers(0, n + 1, size=B).astype(np.int32)
    for r in range(W):
        for use_nv in (False, True):
            got = mla.cp_local_slot(i64_dev(pos), i32_dev(bt), bs, W, r, i32_dev(nv) if use_nv else None, I)
            exp = oracle.cp_local_slot(pos, bt, bs, W, r, I, nv if use_nv else None)
            np.testing.assert_array_equal(got.cpu().numpy(), exp)


@pytest.mark.parametrize("bs,W,I", [(1 << 20, 1 << 10, 1), (1 << 20, 6, 1 << 18), (1 << 30, 1 << 23, 1)])
def test_slots_exact_at_block_and_segment_boundaries(bs, W, I):
    # positions on and next to virtual-block and segment edges, below 2^52
    # (quotients through one double division) and, with a 2^53-position
    # virtual block, above it (64-bit integer division); checked for the
    # rank that owns each position and for the first and last rank
    span = bs * W
    edges = [0, 1, I - 1, I, I + 1, span - 1, span, span + 1, 2 * span + 5 * I, 2 * span + 5 * I - 1, 4 * span - 1,
             (1 << 52) - 1, 1 << 52, (1 << 52) + 1, (1 << 53) - 1, 1 << 53, (1 << 53) + 1]
    pos = np.array([sorted({p for p in edges if 0 <= p < 4 * span})], dtype=np.int64)
    bt = np.array([[11, 3, 1 << 20, 9]], dtype=np.int32)
    ranks = sorted({(int(p) % span) // I % W for p in pos[0]} | {0, W - 1})
    for rank in ranks:
        got = mla.cp_local_slot(i64_dev(pos), i32_dev(bt), bs, W, rank, cp_interleave=I).cpu().numpy()
        exp = np.asarray(oracle.cp_local_slot(pos, bt, bs, W, rank, I, None), dtype=np.int64)
        assert np.array_equal(got, exp), (rank, pos, got, exp)


def test_slots_large_positions_int64():
    bt = np.array([[2_000_000_000, 7]], dtype=np.int32)
    pos = np.array([[0, 1, 2, 3, 130, 131]], dtype=np.int64)
    got = mla.cp_local_slot(i64_dev(pos), i32_dev(bt), 64, 2, 1)
    exp = oracle.cp_local_slot(pos, bt, 64, 2, 1)
    np.testing.assert_array_equal(got.cpu().numpy(), exp)
    assert exp[0, 1] == 2_000_000_000 * 64


PROFILED = [
    WL.Spec(name="profiled_m16", B=3, H=16, Q=1, causal=True, seed=71, lengths=[50, 700, 2100]),
    WL.Spec(name="profiled_r128", B=2, H=128, Q=4, causal=True, seed=72, lengths=[90, 1500]),
    WL.Spec(name="profiled_m16_fp8", B=2, H=16, Q=1, causal=True, seed=73, lengths=[300, 1000], kv_dtype="fp8",
            kv_scale=0.5),
]


@pytest.mark.parametrize("sp", PROFILED, ids=[s.name for s in PROFILED])
def test_profiling_events_leave_results_unchanged(sp):
    """With profiling events set, the attention kernel is launched through
    the path that records them at its start and end; the results must be
    the same bits, and the events must bracket a positive duration."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    say(sp.name)
    up = Uploaded(WL.build(sp))
    o1, l1 = up.run(0)
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    try:
        mla.profile_attention_events(ev[0].value, ev[1].value)
        try:
            o2, l2 = up.run(0)
        finally:
            mla.profile_attention_events(None, None)
        torch.cuda.synchronize()
        assert hip.hipEventSynchronize(ev[1]) == 0
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert ms.value > 0.0
    finally:
        for e in ev:
            hip.hipEventDestroy(e)
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("name,H,Q,bs,kv", [("h128_q4", 128, 4, 64, "bf16"), ("h16_q1", 16, 1, 64, "bf16"),
                                            ("h16_q4", 16, 4, 32, "bf16"), ("h128_q4_bs48", 128, 4, 48, "bf16"),
                                            ("h128_q4_fp8", 128, 4, 64, "fp8")])
def test_unused_block_table_entries_are_never_read(name, H, Q, bs, kv):
    """Block-table entries past a request's last block may hold anything (a
    serving loop leaves them stale or -1): poisoning them with -1, huge ids
    and ids past the pool changes no bit of the result."""
    kw = dict(kv_dtype="fp8", kv_scale=1.0 / 64) if kv == "fp8" else {}
    sp = spec(f"unused_bt_{name}", 4, H, Q, True, [40, 333, 1030, 2900], W=2, bs=bs, **kw)
    wl = WL.build(sp)
    up = Uploaded(wl)
    for r in sorted(wl.pools):
        say(f"{sp.name} rank {r}")
        out0, lse0 = up.run(r)
        bt = wl.block_table.copy()
        nblocks = wl.pools[r].shape[0]
        poison = np.array([-1, 2**31 - 1, nblocks, nblocks + 7], dtype=np.int32)
        for b in range(sp.B):
            used = -(-int(wl.seq_lens[r][b]) // bs)
            if used < bt.shape[1]:
                bt[b, used:] = poison[np.arange(bt.shape[1] - used) % poison.size]
        saved = up.bt
        up.bt = i32_dev(bt)
        out1, lse1 = up.run(r)
        up.bt = saved
        torch.cuda.synchronize()
        assert torch.equal(out0, out1) and torch.equal(lse0, lse1), f"{sp.name} rank {r}"
