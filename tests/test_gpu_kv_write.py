"""GPU parity of the paged KV write (mla_kv_write) against the oracle, and a
write-then-attend pass: the new tokens' KV rows are stored through
cp_local_slot's slots, then every rank decodes and the merged result is
compared with the oracle's attention over the contiguous global KV."""
import numpy as np
import pytest
import torch

import decode_attention_11_amd as mla
import oracle
import workloads as WL
from tests.gpu_util import Uploaded, compare, say, bf16_dev, i32_dev, i64_dev, dev

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,P,bs", [(1, 2, 64), (300, 16, 64), (4099, 80, 64), (77, 9, 16), (50, 200, 1)])
def test_kv_write_matches_oracle(n, P, bs):
    rng = np.random.default_rng(n * 7 + bs)
    cache = rng.integers(0, 1 << 16, size=(P, bs, oracle.D_QK), dtype=np.uint16)
    rows = rng.integers(0, 1 << 16, size=(n, oracle.D_QK), dtype=np.uint16)
    # distinct in-range slots for most rows; pad, negative and past-the-end ones mixed in
    assert n <= P * bs
    slots = rng.permutation(P * bs)[:n].astype(np.int64)
    kinds = rng.integers(0, 10, n)
    slots = np.where(kinds == 0, oracle.PAD_SLOT_ID, slots)
    slots = np.where(kinds == 1, -(1 << 40), slots)
    slots = np.where(kinds == 2, P * bs + rng.integers(0, 1 << 20, n), slots)
    slots = slots.astype(np.int64)
    exp = oracle.kv_write(cache, rows, slots)
    c = bf16_dev(cache)
    say(f"kv_write n={n} P={P} bs={bs}")
    mla.kv_write(bf16_dev(rows), i64_dev(slots), c)
    torch.cuda.synchronize()
    assert np.array_equal(bits(c), exp)


@pytest.mark.parametrize("H,Q,W,causal,I", [(16, 4, 2, True, 1), (128, 4, 4, True, 1), (16, 16, 2, False, 1),
                                             (16, 4, 2, True, 8), (128, 4, 4, True, 2)])
def test_write_new_tokens_then_attend(H, Q, W, causal, I):
    spec = WL.Spec(name=f"write_then_attend_h{H}_w{W}_i{I}", B=3, H=H, Q=Q, causal=causal, seed=808 + H + W + I,
                   lengths=[Q + 1, 700, 2500], W=W, ranks=tuple(range(W)), interleave=I)
    wl = WL.build(spec)
    up = Uploaded(wl)
    bt = i32_dev(wl.block_table)
    bs = spec.block_size
    new_pos = (wl.tot[:, None] - Q + np.arange(Q)[None, :]).astype(np.int64)  # the step's new tokens
    new_rows = np.stack([wl.global_rows(b, new_pos[b]) for b in range(spec.B)])  # [B, Q, 576]
    for r in range(W):
        # the cache before the step: the new tokens' rows hold garbage
        pool = wl.pools[r].copy()
        for b in range(spec.B):
            for p in new_pos[b]:
                p = int(p)
                if (p // I) % W == r:
                    t = (p // (I * W)) * I + p % I  # the rank's local row of p
                    pool[wl.block_table[b, t // bs], t % bs] = 0x7FC0
        up.pools[r] = bf16_dev(pool)
        say(f"{spec.name} rank {r}: slots and write of {spec.B}x{Q} new rows")
        slots = mla.cp_local_slot(i64_dev(new_pos), bt, bs, W, r, cp_interleave=I)
        mla.kv_write(bf16_dev(new_rows), slots, up.pools[r])
        torch.cuda.synchronize()
        assert np.array_equal(bits(up.pools[r]), wl.pools[r]), f"rank {r} pool after the write"
    outs, lses = [], []
    for r in range(W):
        o, l = up.run(r, "e")
        outs.append(o)
        lses.append(l)
    mo, ml = mla.mla_merge_lse(outs, lses, "e")
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode(wl.q_bits, wl.global_rows, wl.tot.astype(np.int32), wl.tot, 1, 0, causal,
                               spec.scale, "e")
    compare(mo, ml, ro, rl, f"{spec.name} merged after the write")


def test_rejected_context_suffix_is_not_written():
    # the draft's context window: its rejected suffix maps to the pad slot,
    # so those rows leave the cache untouched on every rank
    spec = WL.Spec(name="draft_ctx_write", B=4, H=16, Q=16, causal=False, seed=919, lengths=[200, 333, 64, 1000],
                   W=2, ranks=(0, 1))
    wl = WL.build(spec)
    si = WL.draft_slot_inputs(wl)
    pos, nv = si["ctx_positions"], si["ctx_num_valid"]
    rng = np.random.default_rng(3)
    rows = rng.integers(0, 1 << 16, size=pos.shape + (oracle.D_QK,), dtype=np.uint16)
    bt = i32_dev(wl.block_table)
    for r in range(2):
        slots = mla.cp_local_slot(i64_dev(pos), bt, spec.block_size, 2, r, i32_dev(nv))
        exp_slots = oracle.cp_local_slot(pos, wl.block_table, spec.block_size, 2, r, 1, nv)
        assert np.array_equal(slots.cpu().numpy(), exp_slots)
        c = bf16_dev(wl.pools[r])
        mla.kv_write(bf16_dev(rows), slots, c)
        torch.cuda.synchronize()
        exp = oracle.kv_write(wl.pools[r], rows.reshape(-1, oracle.D_QK), np.asarray(exp_slots).reshape(-1))
        assert np.array_equal(bits(c), exp), f"rank {r}"


# ---------------------------------------------------------------- FP8 cache

def special_rows(rng, n):
    """bf16 rows mixing magnitudes from 2^-20 to 2^20 with zeros of both
    signs, infinities, NaN and values near the saturation bound."""
    mag = np.exp2(rng.uniform(-20, 20, size=(n, oracle.D_QK))).astype(np.float32)
    v = (mag * rng.choice([-1, 1], size=mag.shape)).astype(np.float32)
    flat = v.reshape(-1)
    k = rng.integers(0, flat.size, 64)
    flat[k[:8]] = 0.0
    flat[k[8:16]] = -0.0
    flat[k[16:20]] = np.inf
    flat[k[20:24]] = -np.inf
    flat[k[24:28]] = np.nan
    flat[k[28:64]] = rng.uniform(-520, 520, 36)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("n,P,bs,scale", [(1, 2, 64, 1.0), (300, 16, 64, 1 / 64), (4099, 80, 64, 0.0123),
                                          (77, 9, 16, 3.7), (50, 200, 1, 2.0 ** -10)])
def test_kv_write_fp8_matches_oracle(n, P, bs, scale):
    rng = np.random.default_rng(n * 11 + bs)
    cache = rng.integers(0, 256, size=(P, bs, oracle.D_QK), dtype=np.uint8)
    rows = special_rows(rng, n)
    slots = rng.permutation(P * bs)[:n].astype(np.int64)
    kinds = rng.integers(0, 10, n)
    slots = np.where(kinds == 0, oracle.PAD_SLOT_ID, slots)
    slots = np.where(kinds == 1, -(1 << 40), slots)
    slots = np.where(kinds == 2, P * bs + rng.integers(0, 1 << 20, n), slots).astype(np.int64)
    exp = oracle.kv_write_fp8(cache, rows, slots, scale)
    c = torch.from_numpy(cache).to(dev())
    say(f"kv_write_fp8 n={n} P={P} bs={bs} scale={scale}")
    mla.kv_write(bf16_dev(rows), i64_dev(slots), c, kv_scale=scale)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), exp)


@pytest.mark.parametrize("H,Q,W,causal,I", [(16, 1, 1, True, 1), (16, 4, 2, True, 1), (128, 4, 4, True, 2),
                                             (16, 16, 2, False, 1)])
def test_fp8_write_new_tokens_then_attend(H, Q, W, causal, I):
    spec = WL.Spec(name=f"fp8_write_then_attend_h{H}_w{W}_i{I}", B=3, H=H, Q=Q, causal=causal, seed=909 + H + W + I,
                   lengths=[Q + 1, 700, 2500], W=W, ranks=tuple(range(W)), interleave=I, kv_dtype="fp8",
                   kv_scale=1 / 64, global_is_null=(W == 1))
    wl = WL.build(spec)
    up = Uploaded(wl)
    bt = i32_dev(wl.block_table)
    bs, s = spec.block_size, spec.kv_scale
    rng = np.random.default_rng(spec.seed)
    new_pos = (wl.tot[:, None] - Q + np.arange(Q)[None, :]).astype(np.int64)  # the step's new tokens
    # N(0,1) like the rest of the cache (the absolute tolerance assumes unit-scale values)
    new_vals = rng.standard_normal((spec.B, Q, oracle.D_QK)).astype(np.float32)
    new_rows = (new_vals.view(np.uint32) >> 16).astype(np.uint16)  # bf16 rows to quantise
    new_codes = oracle.e4m3_encode((oracle.bf16_bits_to_f64(new_rows).astype(np.float32) / np.float32(s)))
    new_codes = new_codes.reshape(spec.B, Q, oracle.D_QK)
    for r in range(W):
        pool = wl.pools[r].copy()
        slots_np = oracle.cp_local_slot(new_pos, wl.block_table, bs, W, r, I, None)
        pool_garbage = pool.copy()
        for b in range(spec.B):
            for i, sl in enumerate(np.asarray(slots_np)[b]):
                if sl >= 0:
                    pool_garbage[sl // bs, sl % bs] = 0x7F  # NaN codes until written
        up.pools[r] = torch.from_numpy(pool_garbage).to(dev())
        say(f"{spec.name} rank {r}: quantising write of {spec.B}x{Q} new rows")
        slots = mla.cp_local_slot(i64_dev(new_pos), bt, bs, W, r, cp_interleave=I)
        mla.kv_write(bf16_dev(new_rows), slots, up.pools[r], kv_scale=s)
        torch.cuda.synchronize()
        exp = oracle.kv_write_fp8(pool_garbage, new_rows.reshape(-1, oracle.D_QK), np.asarray(slots_np).reshape(-1), s)
        assert np.array_equal(up.pools[r].cpu().numpy(), exp), f"rank {r} pool after the write"

    def rows_after(b, pos):
        out = wl.global_rows(b, pos).copy()
        for i, p in enumerate(np.asarray(pos)):
            j = int(p) - int(new_pos[b, 0])
            if 0 <= j < Q:
                out[i] = new_codes[b, j]
        return out

    outs, lses = [], []
    for r in range(W):
        o, l = up.run(r, "e")
        outs.append(o)
        lses.append(l)
    if W > 1:
        mo, ml = mla.mla_merge_lse(outs, lses, "e")
    else:
        mo, ml = outs[0], lses[0]
    torch.cuda.synchronize()
    # the unsharded attention over the contiguous global KV
    ro, rl = oracle.mla_decode(wl.q_bits, rows_after, wl.tot.astype(np.int32), wl.tot, 1, 0, causal, spec.scale, "e",
                               kv_scale=s)
    compare(mo, ml, ro, rl, f"{spec.name} after the quantising write")
