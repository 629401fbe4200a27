"""mla_decode_noalloc (the decode with its workspace in the library's fixed
per-GPU array) against mla_decode with a caller workspace, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input (fewer
requests, heads and rows, so a different plan over the same array, whose
first bytes still hold the first call's partials): each output must equal
mla_decode's bit for bit (same kernels, same plan) and meet the usual bars
against the oracle.  A third call repeats the first, after the array has
held the second call's partials.
"""
import pytest
import torch

import decode_attention_11_amd as mla
import oracle
import workloads as WL
from tests.gpu_util import Uploaded, compare, say

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, Q, causal, lengths, W, rank: a 128-row DCP shard first, then a smaller 16-row call
    ("big_h128_q4_dcp2", 3, 128, 4, True, [900, 4000, 2500], 2, 1),
    ("small_h16_q1", 2, 16, 1, True, [70, 1500], 1, 0),
    ("big_h128_q4_dcp2", 3, 128, 4, True, [900, 4000, 2500], 2, 1),
]


def test_noalloc_matches_the_workspace_call_on_consecutive_calls():
    for name, B, H, Q, causal, lengths, W, r in CASES:
        spec = WL.Spec(name=name, B=B, H=H, Q=Q, causal=causal, seed=6100 + H, lengths=lengths, W=W,
                       ranks=(r,), global_is_null=(W == 1))
        wl = WL.build(spec)
        up = Uploaded(wl)
        say(f"{name}: B={B} H={H} Q={Q} W={W} rank {r}")
        msl = int(wl.seq_lens[r].max())
        ref_out, ref_lse = up.run(r, "e", max_seq_len=msl)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        g = None if spec.global_is_null else up.tot
        mla.mla_decode_noalloc(up.q, up.pools[r], up.bt, up.seq[r], g, W, r, causal, spec.scale, "e",
                               out=out, lse=lse, max_seq_len=msl)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"{name}: out differs from mla_decode"
        assert torch.equal(lse, ref_lse), f"{name}: lse differs from mla_decode"
        tot = None if spec.global_is_null else wl.tot
        ro, rl = oracle.mla_decode(wl.q_bits, wl.global_rows, wl.seq_lens[r], tot, W, r, causal, spec.scale)
        compare(out, lse, ro, rl, f"{name} no-alloc vs oracle")


def test_noalloc_refuses_sizes_beyond_its_array_without_launching():
    # 3000 single-token requests of 16 heads: 3256 partial slots of 33 KB,
    # more than the array holds; refused on the host before any launch
    dev = torch.device("cuda:0")
    B = 3000
    q = torch.zeros((B, 1, 16, 576), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((4, 64, 576), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, 1), dtype=torch.int32, device=dev)
    sl = torch.ones((B,), dtype=torch.int32, device=dev)
    out = torch.full((B, 16, 512), 7.0, dtype=torch.bfloat16, device=dev)
    assert mla.mla_decode_workspace_size(B, 1, 16, 64) > mla.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ValueError):
        mla.mla_decode_noalloc(q, kv, bt, sl, None, out=out, max_seq_len=64)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call must not write its output"
