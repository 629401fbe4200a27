"""GPU parity of mla_decode_varlen (a query length per request) against the
oracle: both kernel families, requests without tokens, shorter requests
whose upper row tiles have nothing to compute, causal and non-causal,
sharded ranks with and without interleave, and the merged result."""
import numpy as np
import pytest
import torch

import decode_attention_11_amd as mla
import oracle
import workloads as WL
from tests.gpu_util import compare, say, bf16_dev, i32_dev

pytestmark = pytest.mark.gpu

CASES = [
    # (name, H, q_lens, lengths, W, causal, interleave)
    ("h8_m16_family", 8, [1, 2, 0, 2], [40, 700, 90, 1500], 1, True, 1),
    ("h16_one_row_tile", 16, [1, 4, 3, 0, 2], [5, 333, 2049, 64, 700], 2, True, 1),
    ("h128_skipped_row_tiles", 128, [4, 1, 2], [70, 900, 1600], 2, True, 1),
    ("h16_noncausal_dcp2", 16, [16, 3, 0, 9], [100, 2500, 40, 800], 2, False, 1),
    ("h24_interleave2_dcp3", 24, [3, 1, 2, 3], [31, 400, 1111, 90], 3, True, 2),
    ("h16_rows64_tile", 16, [4, 1, 3, 0], [700, 30, 2500, 90], 1, True, 1),
    # 70 requests of up to 4 row tiles: 280 (request, row tile) work items,
    # more than one chunk of the in-kernel plan's scan
    ("h128_280_items", 128, [1 + (3 * i) % 4 if i % 7 else 0 for i in range(70)],
     [33 + (97 * i) % 600 for i in range(70)], 2, True, 1),
]


def run_rank(wl, r, base="e"):
    s = wl.spec
    q = bf16_dev(wl.q_tok)
    qsl = i32_dev(wl.query_start_loc)
    g = i32_dev(wl.tot) if (s.W > 1 or not s.global_is_null) else None
    return mla.mla_decode_varlen(q, qsl, bf16_dev(wl.pools[r]), i32_dev(wl.block_table), i32_dev(wl.seq_lens[r]), g,
                                 s.W, r, s.causal, s.scale, base, max_q_len=s.Q, cp_interleave=s.interleave)


def oracle_rank(wl, r, base="e"):
    s = wl.spec
    return oracle.mla_decode_varlen(wl.q_tok, wl.query_start_loc, wl.global_rows, wl.seq_lens[r], wl.tot, s.W, r,
                                    s.causal, s.scale, base, interleave=s.interleave)


@pytest.mark.parametrize("name,H,q_lens,lengths,W,causal,I", CASES, ids=[c[0] for c in CASES])
def test_varlen_matches_oracle(name, H, q_lens, lengths, W, causal, I):
    spec = WL.Spec(name=name, B=len(q_lens), H=H, Q=max(q_lens), causal=causal, seed=2024 + H, lengths=lengths,
                   W=W, ranks=tuple(range(W)), interleave=I, q_lens=q_lens)
    wl = WL.build(spec)
    outs, lses = [], []
    for r in range(W):
        for base in ("e", "2"):
            say(f"{name} rank {r} base {base}")
            out, lse = run_rank(wl, r, base)
            torch.cuda.synchronize()
            ro, rl = oracle_rank(wl, r, base)
            compare(out, lse, ro, rl, f"{name} r{r} {base}")
            if base == "e":
                outs.append(out)
                lses.append(lse)
    if W > 1:
        mo, ml = mla.mla_merge_lse(outs, lses, "e")
        torch.cuda.synchronize()
        ro, rl = oracle.mla_decode_varlen(wl.q_tok, wl.query_start_loc, wl.global_rows, wl.tot.astype(np.int32),
                                          wl.tot, 1, 0, causal, spec.scale, "e")
        compare(mo, ml, ro, rl, f"{name} merged vs unsharded")


def test_varlen_with_equal_lengths_is_the_uniform_call_bitwise():
    spec = WL.Spec(name="varlen_equal", B=3, H=16, Q=4, causal=True, seed=77, lengths=[50, 900, 2000], W=2,
                   ranks=(0, 1), q_lens=[4, 4, 4])
    wl = WL.build(spec)
    for r in range(2):
        out, lse = run_rank(wl, r)
        q = bf16_dev(wl.q_tok.reshape(3, 4, 16, oracle.D_QK))
        uo, ul = mla.mla_decode(q, bf16_dev(wl.pools[r]), i32_dev(wl.block_table), i32_dev(wl.seq_lens[r]),
                                i32_dev(wl.tot), 2, r, None, True, spec.scale, "e")
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), uo.view(torch.int16))
        assert torch.equal(lse, ul)
