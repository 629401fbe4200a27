"""GPU parity of the FP8 (E4M3) latent cache path (mla_decode_fp8) against the
oracle: every E4M3 code's conversion, small seeded workloads over the shapes
the bf16 tests cover, a full-size sampled check, and agreement with the bf16
path on a cache holding the same values (bitwise where both run the same
single workgroup).  Bar as for bf16: output max-abs <= 2e-2 and mean-abs <=
2e-3 against float64, LSE within 1e-3.
"""
import zlib

import numpy as np
import pytest
import torch

import decode_attention_11_amd as mla
import oracle
import workloads as WL
from tests import oracle_full
from tests.gpu_util import Uploaded, compare, say, bf16_dev, u8_dev, i32_dev

pytestmark = pytest.mark.gpu


def spec(name, B, H, Q, causal, lengths, W=1, ranks=None, bs=64, kv_scale=1.0 / 64, **kw):
    return WL.Spec(name=name, B=B, H=H, Q=Q, causal=causal, seed=zlib.crc32(name.encode()) % 10000,
                   lengths=list(lengths), W=W, ranks=tuple(range(W)) if ranks is None else tuple(ranks),
                   block_size=bs, kv_dtype="fp8", kv_scale=kv_scale, **kw)


CASES = [
    spec("fp8_h16_q1_ragged", 5, 16, 1, True, [1, 63, 64, 65, 3000], global_is_null=True),
    spec("fp8_h16_q1_scale1", 3, 16, 1, True, [40, 700, 2100], global_is_null=True, kv_scale=1.0),
    spec("fp8_h8_q2", 3, 8, 2, True, [2, 700, 1290], global_is_null=True, kv_scale=0.0123),
    spec("fp8_h16_q4_dcp2", 3, 16, 4, True, [5, 333, 2049], W=2),
    spec("fp8_h24_q3_dcp8_bs128", 2, 24, 3, True, [200, 1111], W=8, bs=128),
    spec("fp8_h128_q4_causal", 2, 128, 4, True, [4, 900], global_is_null=True),
    spec("fp8_h128_q16_noncausal_dcp2_rank1", 2, 128, 16, False, [64, 1000], W=2, ranks=[1]),
    spec("fp8_bs1", 2, 16, 1, True, [17, 90], bs=1, global_is_null=True),
    spec("fp8_bs16_dcp4", 3, 16, 2, True, [9, 130, 515], W=4, bs=16),
    spec("fp8_nan_fill", 3, 16, 4, True, [70, 130, 1000], W=2, fill="nan"),
    spec("fp8_peaky", 3, 16, 1, True, [100, 1500, 4000], q_mult=8.0, global_is_null=True),
    spec("fp8_h16_q4_dcp2_interleave4", 3, 16, 4, True, [5, 333, 2049], W=2, interleave=4),
    spec("fp8_many_tiny_requests", 300, 16, 1, True, [(7 * i) % 5 for i in range(300)], global_is_null=True),
    spec("fp8_bs48_h128_q4", 2, 128, 4, True, [47, 2401], global_is_null=True, bs=48),
    spec("fp8_bs80_h128_q4_dcp2", 2, 128, 4, True, [161, 3000], W=2, bs=80),
    spec("fp8_bs48_h16_q1", 3, 16, 1, True, [48, 49, 3000], global_is_null=True, bs=48),
    spec("fp8_bs80_h16_q1", 3, 16, 1, True, [79, 800, 2500], global_is_null=True, bs=80),
    spec("fp8_rows24_h24_q1", 2, 24, 1, True, [40, 3000], global_is_null=True),
    spec("fp8_rows48_h16_q3_dcp2", 2, 16, 3, True, [500, 3000], W=2),
    # blocks under 32 keys in the 128- and 64-row tiles (a row lookup per lane)
    spec("fp8_bs1_h128_q4", 2, 128, 4, True, [17, 300], global_is_null=True, bs=1),
    spec("fp8_bs16_h32_q2_dcp2", 2, 32, 2, True, [40, 900], W=2, bs=16),
    spec("fp8_rows160_h40_q4_partial_tile", 2, 40, 4, True, [50, 2500], global_is_null=True),
]


def oracle_rank(wl, r):
    s = wl.spec
    tot = None if (s.global_is_null and s.W == 1) else wl.tot
    return oracle.mla_decode(wl.q_bits, wl.global_rows, wl.seq_lens[r], tot, s.W, r, s.causal, s.scale, s.lse_base,
                             interleave=s.interleave, kv_scale=s.kv_scale)


@pytest.mark.parametrize("sp", CASES, ids=[c.name for c in CASES])
def test_fp8_decode_matches_oracle(sp):
    wl = WL.build(sp)
    up = Uploaded(wl)
    for r in sorted(wl.pools):
        say(f"{sp.name} rank {r}")
        out, lse = up.run(r)
        torch.cuda.synchronize()
        ro, rl = oracle_rank(wl, r)
        compare(out, lse, ro, rl, f"{sp.name} r{r}")


@pytest.mark.parametrize("kv_scale", [1.0, 0.25])
def test_every_e4m3_code_converts_exactly(kv_scale):
    """One visible key per request, so the output is that key's value row,
    which is exactly representable in bf16: every finite code is compared
    bit for bit with the oracle's decoding."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)  # the two NaN codes
    B, H, bs, D = 4, 16, 16, oracle.D_QK
    rows = np.zeros((B, D), dtype=np.uint8)
    for b in range(B):
        # every finite code lands in the value columns of two requests, at
        # different columns
        rows[b, :512] = np.roll(np.resize(codes, 512), 37 * b)
        rows[b, 512:] = codes[(np.arange(64) * 5 + b) % codes.size]
    pool = np.zeros((B, bs, D), dtype=np.uint8)
    pool[:, 0, :] = rows
    bt = np.arange(B, dtype=np.int32).reshape(B, 1)
    seq = np.ones(B, dtype=np.int32)
    q = torch.zeros((B, 1, H, D), dtype=torch.bfloat16, device="cuda:0")
    say(f"all codes, kv_scale {kv_scale}")
    out, lse = mla.mla_decode(q, u8_dev(pool), i32_dev(bt), i32_dev(seq), None, kv_scale=kv_scale)
    torch.cuda.synchronize()
    want = oracle.e4m3_to_f64(rows[:, :512]) * kv_scale  # exactly representable in bf16
    got = out.float().cpu().numpy().astype(np.float64)
    for b in range(B):
        assert np.array_equal(got[b], np.broadcast_to(want[b], (H, 512))), f"request {b}"
    assert np.all(lse.cpu().numpy() == 0.0)  # a zero query: one key with score 0


def fp8_and_bf16_runs(sp):
    """The FP8 call, and the bf16 call on a bf16 cache of the decoded codes
    (kv_scale 1: the same values, exactly)."""
    wl = WL.build(sp)
    up = Uploaded(wl)
    codes = wl.pools[0]
    vals = oracle.e4m3_to_f64(codes).astype(np.float32)  # exact: E4M3 values fit in bf16
    bf = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bf), oracle.e4m3_to_f64(codes))
    o8, l8 = up.run(0)
    o16, l16 = mla.mla_decode(up.q, bf16_dev(bf), up.bt, up.seq[0], None, scale=sp.scale)
    torch.cuda.synchronize()
    return o8, l8, o16, l16


def test_fp8_equals_bf16_path_bitwise_in_one_workgroup():
    # 100 keys: fewer units than one workgroup's minimum for either cache
    # type, so both calls run one workgroup over the same single piece
    o8, l8, o16, l16 = fp8_and_bf16_runs(spec("fp8_vs_bf16_one_wg", 1, 16, 1, True, [100], global_is_null=True,
                                              kv_scale=1.0))
    assert torch.equal(o8, o16)
    assert torch.equal(l8, l16)


def test_fp8_equals_bf16_path_to_rounding():
    """Longer requests: the two calls split the keys at different points (an
    FP8 piece is charged more), and each piece rounds P to bf16 against its
    own running maximum, so outputs agree to two bf16 units of |out| < 1
    and LSEs to float32 rounding."""
    o8, l8, o16, l16 = fp8_and_bf16_runs(spec("fp8_vs_bf16", 4, 16, 1, True, [30, 500, 1500, 4100],
                                              global_is_null=True, kv_scale=1.0))
    d = (o8.float() - o16.float()).abs()
    assert float(d.max()) <= 2.0 ** -6 and float(d.mean()) <= 2e-4
    assert float((l8 - l16).abs().max()) <= 1e-5


def test_fp8_equals_bf16_path_bitwise_in_the_128_row_kernel():
    # more than 16 rows per request: both calls take the 128-row kernel with
    # the same plan, and its k-steps are summed in the same order whatever
    # the cache type, so the results are identical
    o8, l8, o16, l16 = fp8_and_bf16_runs(spec("fp8_vs_bf16_h128", 3, 128, 4, True, [70, 900, 2600],
                                              global_is_null=True, kv_scale=1.0))
    assert torch.equal(o8, o16)
    assert torch.equal(l8, l16)


def test_fp8_cache_scale_scales_scores_and_values():
    """Codes c with scale s against codes c with scale 2s: the second equals
    the first with the query doubled (scores) and the output doubled."""
    sp = spec("fp8_scale_rel", 3, 16, 1, True, [100, 900, 2500], global_is_null=True, kv_scale=1.0 / 32)
    wl = WL.build(sp)
    up = Uploaded(wl)
    o1, l1 = up.run(0)
    o2, l2 = up.run(0, kv_scale=2.0 / 32)
    q2 = (up.q.float() * 2).to(torch.bfloat16)  # exact: doubling a bf16 value
    o3, l3 = mla.mla_decode(q2, up.pools[0], up.bt, up.seq[0], None, scale=sp.scale, kv_scale=1.0 / 32)
    torch.cuda.synchronize()
    assert torch.equal(o2.float(), (o3.float() * 2))
    assert torch.equal(l2, l3)
    assert not torch.equal(l1, l2)


@pytest.mark.parametrize("cfg", [2, 6, 3, 5])
def test_fp8_full_size_matches_oracle_on_every_element(cfg, tmp_path):
    """The benchmark's workloads with the FP8 cache of bench.py --fp8, at full
    size in the launch configuration bench.py times, every (row, head,
    column) against the float64 oracle on the same E4M3 codes (computed in a
    GPU-free worker pool while the GPU runs).  The single-token workload
    uses the weighted ranges of the two workgroups per CU."""
    sp = oracle_full.spec_of(cfg, fp8=True)
    say(f"{sp.name} fp8: oracle started in a worker pool; generating")
    proc = oracle_full.start(cfg, tmp_path, fp8=True)
    try:
        wl = WL.build(sp)
        up = Uploaded(wl)
        r = min(wl.pools)
        say(f"{sp.name} fp8 rank {r}: GPU")
        out, lse = up.run(r, sp.lse_base, max_seq_len=int(wl.seq_lens[r].max()))
        torch.cuda.synchronize()
        out, lse = out.cpu(), lse.cpu()
        del up
        say(f"{sp.name} fp8: waiting for the oracle")
        rc = proc.wait(timeout=900)
        assert rc == 0, f"{sp.name} fp8: the oracle process failed ({rc})"
    finally:
        if proc.poll() is None:
            proc.kill()
            proc.wait()
    ro, rl = oracle_full.load(tmp_path, r)
    assert not np.isnan(ro).any() and not np.isnan(rl).any(), "the oracle left rows uncomputed"
    compare(out, lse, ro, rl, f"{sp.name} fp8, all {ro.size} outputs")
