"""A whole DCP decode step captured once in a HIP graph (torch.cuda.CUDAGraph)
and replayed on new inputs.

The slot layout has to stay stable while the draft metadata is captured in a
graph, and the decode runs once per step under graph replay (PR #52188 page,
key source snippets: cp_local_slot runs inside the captured draft step;
risks: replaying the captured step every decode step).  The step here is the
DCP-8 one: the slot mapping of the step's new tokens for every rank, the
eight ranks' decodes over their shards, and the LSE merge.  Nothing in it may
allocate, synchronise with the host or leave a memset node in the graph.

The graph is replayed on two input sets in turn (other values, lengths and
block tables copied into the captured buffers), with the program's own eager
calls and synchronisations between the replays.  Every replay is compared
with the eager step on the same inputs (bit for bit: the same kernels and the
same plan) and with the oracle: the merged result against the attention over
each row's whole global causal prefix, the slots exactly.
"""
import numpy as np
import pytest
import torch

import decode_attention_11_amd as mla
import oracle
import workloads as WL
from tests.gpu_util import bf16_dev, compare, i32_dev, i64_dev, say

pytestmark = pytest.mark.gpu

W, H, Q, B, BS = 8, 128, 4, 3, 64


def make_inputs(seed, lengths):
    spec = WL.Spec(name=f"graph_{seed}", B=B, H=H, Q=Q, causal=True, seed=seed, lengths=lengths, W=W,
                   ranks=tuple(range(W)))
    wl = WL.build(spec)
    newpos = (wl.tot[:, None] - Q + np.arange(Q)[None, :]).astype(np.int64)
    ro, rl = oracle.mla_decode(wl.q_bits, wl.global_rows, wl.tot.astype(np.int64), wl.tot, 1, 0, True, spec.scale)
    slots = {r: oracle.cp_local_slot(newpos, wl.block_table, BS, W, r) for r in range(W)}
    return wl, newpos, (ro, rl), slots


def test_captured_dcp_step_replays_on_new_inputs():
    sets = [make_inputs(4101, [3000, 5100, 4077]), make_inputs(4102, [2999, 4100, 5203])]
    mb = max(s[0].block_table.shape[1] for s in sets)
    nblk = max(s[0].pools[0].shape[0] for s in sets)
    msl = {r: max(int(s[0].seq_lens[r].max()) for s in sets) for r in range(W)}
    dev = torch.device("cuda:0")

    # the captured buffers: every input, output and workspace of the step
    q = torch.empty((B, Q, H, 576), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, mb), dtype=torch.int32, device=dev)
    tot = torch.empty((B,), dtype=torch.int32, device=dev)
    newpos = torch.empty((B, Q), dtype=torch.int64, device=dev)
    pools = {r: torch.empty((nblk, BS, 576), dtype=torch.bfloat16, device=dev) for r in range(W)}
    seq = {r: torch.empty((B,), dtype=torch.int32, device=dev) for r in range(W)}
    slots = {r: torch.empty((B, Q), dtype=torch.int64, device=dev) for r in range(W)}
    outs = {r: torch.empty((B * Q, H, 512), dtype=torch.bfloat16, device=dev) for r in range(W)}
    lses = {r: torch.empty((B * Q, H), dtype=torch.float32, device=dev) for r in range(W)}
    ws = {r: torch.empty((mla.mla_decode_workspace_size(B, Q, H, msl[r]),), dtype=torch.uint8, device=dev)
          for r in range(W)}
    merged = (torch.empty((B * Q, H, 512), dtype=torch.bfloat16, device=dev),
              torch.empty((B * Q, H), dtype=torch.float32, device=dev))

    def load(i):
        wl, pos, _, _ = sets[i]
        q.copy_(bf16_dev(wl.q_bits))
        bt.zero_()
        bt[:, :wl.block_table.shape[1]].copy_(i32_dev(wl.block_table))
        tot.copy_(i32_dev(wl.tot))
        newpos.copy_(i64_dev(pos))
        for r in range(W):
            pools[r][:wl.pools[r].shape[0]].copy_(bf16_dev(wl.pools[r]))
            seq[r].copy_(i32_dev(wl.seq_lens[r]))

    def step(out_slots, out_o, out_l, out_m):
        for r in range(W):
            mla.cp_local_slot(newpos, bt, BS, W, r, out=out_slots[r])
            mla.mla_decode(q, pools[r], bt, seq[r], tot, W, r, causal=True, scale=sets[0][0].spec.scale,
                           lse_base="e", max_seq_len=msl[r], out=out_o[r], lse=out_l[r], workspace=ws[r])
        mla.mla_merge_lse([out_o[r] for r in range(W)], [out_l[r] for r in range(W)], "e",
                          out=out_m[0], lse=out_m[1])

    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(slots, outs, lses, merged)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(slots, outs, lses, merged)
    torch.cuda.synchronize()

    e_slots = {r: torch.empty_like(slots[r]) for r in range(W)}
    e_outs = {r: torch.empty_like(outs[r]) for r in range(W)}
    e_lses = {r: torch.empty_like(lses[r]) for r in range(W)}
    e_merged = (torch.empty_like(merged[0]), torch.empty_like(merged[1]))
    for rep, i in enumerate([0, 1, 1, 0, 1]):
        say(f"replay {rep} on input set {i}")
        load(i)
        merged[0].fill_(float("nan"))  # stale results must not survive a replay
        graph.replay()
        torch.cuda.synchronize()
        # the eager step on the same inputs, between the replays
        step(e_slots, e_outs, e_lses, e_merged)
        torch.cuda.synchronize()
        _, _, (ro, rl), exp_slots = sets[i]
        for r in range(W):
            assert torch.equal(slots[r], e_slots[r]), f"replay {rep} rank {r}: slots differ from the eager call"
            assert np.array_equal(slots[r].cpu().numpy(), np.asarray(exp_slots[r], dtype=np.int64)), \
                f"replay {rep} rank {r}: slots differ from the oracle"
            assert torch.equal(outs[r].view(torch.int16), e_outs[r].view(torch.int16)), f"replay {rep} rank {r}: out"
            assert torch.equal(lses[r], e_lses[r]), f"replay {rep} rank {r}: lse"
        assert torch.equal(merged[0].view(torch.int16), e_merged[0].view(torch.int16))
        assert torch.equal(merged[1], e_merged[1])
        compare(merged[0], merged[1], ro, rl, f"replay {rep} (inputs {i}) merged vs unsharded oracle")
