"""Pins of the CPU oracle against facts it does not compute itself.

Each test fixes a part of the oracle by something other than its own code:
the pages' printed integer formulas, closed forms of softmax attention,
torch's float64 scaled-dot-product attention with an explicit mask, a pure
Python brute force, algebraic identities of the LSE merge, and hand-worked
slot examples.  A plausible slip in the oracle (a dropped rope term, a wrong
causal offset or rank, a transposed operand, a wrong LSE base, an off-by-one
slot) breaks at least one of them; test_mutations_are_caught checks that.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_oracle as O
import workloads as WL
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(B=2, H=3, Q=3, W=2, causal=True, lengths=(9, 14), seed=11, ranks=None, **kw):
    spec = WL.Spec(name="tiny", B=B, H=H, Q=Q, causal=causal, seed=seed, lengths=list(lengths), W=W,
                   ranks=tuple(range(W)) if ranks is None else ranks, block_size=4, **kw)
    return WL.build(spec)


def oracle_rank(wl, r, base="e", causal=None):
    s = wl.spec
    causal = s.causal if causal is None else causal
    return oracle.mla_decode(wl.q_bits, wl.global_rows, wl.seq_lens[r], wl.tot, s.W, r, causal, s.scale, base,
                             interleave=s.interleave)


# ---------------------------------------------------------------- lengths

def page_local_len(G, W, r, I):
    """Rank-local length as printed on the PR #52188 page (key source snippets)."""
    span = W * I
    rem = min(max(G % span - r * I, 0), I)
    return G // span * I + rem


def test_local_count_matches_page_formula_and_ceil():
    for W in range(1, 17):
        for r in range(W):
            for G in range(0, 2000):
                n = oracle.local_count(G, W, r)
                assert n == page_local_len(G, W, r, 1), (G, W, r)
                assert n == -(-max(G - r, 0) // W), (G, W, r)


def test_page_formula_with_interleave_matches_enumeration():
    # ownership with interleave I: segment index (p // I) mod W picks the rank
    for I in (1, 2, 4):
        for W in (1, 2, 3, 8):
            for r in range(W):
                for G in range(0, 300):
                    enum = sum(1 for p in range(G) if (p // I) % W == r)
                    assert enum == page_local_len(G, W, r, I)


def test_held_positions_with_interleave_match_the_slot_ownership():
    # the positions a rank holds, in order, are the positions cp_local_slot
    # gives it a slot for, and local row t of them gets the t-th slot of the
    # rank's paging (table entry t // bs, offset t % bs)
    bs = 8
    for I in (1, 2, 4, 8):
        for W in (1, 2, 3, 4):
            for r in range(W):
                L = 157
                held = oracle.held_positions(oracle.local_count(L, W, r, I), W, r, I)
                pos = np.arange(L, dtype=np.int64)[None, :]
                bt = np.arange(100, dtype=np.int32)[None, :] * 3 + 1
                slots = oracle.cp_local_slot(pos, bt, bs, W, r, I)[0]
                owned = np.nonzero(slots != oracle.PAD_SLOT_ID)[0]
                assert owned.tolist() == held.tolist(), (I, W, r)
                t = np.arange(held.size)
                assert slots[owned].tolist() == (bt[0, t // bs].astype(np.int64) * bs + t % bs).tolist()


def test_visible_positions_with_interleave_match_bruteforce_predicate():
    for I in (2, 4):
        for W in (2, 3):
            for r in range(W):
                for tot in range(0, 60, 5):
                    seq = oracle.local_count(tot, W, r, I)
                    assert seq == page_local_len(tot, W, r, I)
                    for Q in (1, 4):
                        for j in range(Q):
                            for causal in (True, False):
                                got = oracle.visible_positions(seq, tot, Q, j, W, r, causal, I).tolist()
                                exp = [p for p in range(tot + W * I)
                                       if brute.is_visible(p, j, Q, tot, seq, W, r, causal, I)]
                                assert got == exp, (I, W, r, tot, Q, j, causal)


def test_visible_count_textbook_causal_w1():
    # the token at global position tot-Q+j sees positions 0..tot-Q+j
    for tot in range(0, 40):
        for Q in range(1, 6):
            for j in range(Q):
                pos = oracle.visible_positions(tot, tot, Q, j, 1, 0, True)
                expect = max(tot - Q + j + 1, 0)
                assert pos.tolist() == list(range(expect))


def test_visible_positions_match_bruteforce_predicate():
    for W in (1, 2, 3, 8):
        for r in range(W):
            for tot in range(0, 45, 3):
                seq = oracle.local_count(tot, W, r)
                for Q in (1, 3, 4):
                    for j in range(Q):
                        for causal in (True, False):
                            got = oracle.visible_positions(seq, tot, Q, j, W, r, causal).tolist()
                            exp = [p for p in range(tot + W) if brute.is_visible(p, j, Q, tot, seq, W, r, causal)]
                            assert got == exp


def test_end_aligned_local_mask_differs_under_dcp():
    # PR #48180 page, review highlights: a local end-aligned causal mask is
    # wrong under DCP when q_len > 1.  W=8, r=0, tot=32, Q=4.
    W, r, tot, Q = 8, 0, 32, 4
    n_local = oracle.local_count(tot, W, r)
    correct = [oracle.visible_positions(n_local, tot, Q, j, W, r, True).size for j in range(Q)]
    end_aligned = [n_local - (Q - 1 - j) for j in range(Q)]
    assert correct == [4, 4, 4, 4]
    assert end_aligned == [1, 2, 3, 4]
    assert correct != end_aligned


# ---------------------------------------------------------------- attention values

def sdpa_reference(wl, r, base="e"):
    """torch float64 SDPA over the *full global* KV with a visibility mask."""
    s = wl.spec
    B, Q, H = s.B, s.Q, s.H
    outs = np.zeros((B * Q, H, 512))
    lses = np.zeros((B * Q, H))
    for b in range(B):
        kv = O.bf16_bits_to_f64(wl.global_kv(b))
        L = kv.shape[0]
        q = O.bf16_bits_to_f64(wl.q_bits[b])            # [Q, H, 576]
        mask = np.zeros((Q, L), dtype=bool)
        for j in range(Q):
            for p in range(L):
                mask[j, p] = brute.is_visible(p, j, Q, int(wl.tot[b]), int(wl.seq_lens[r][b]), s.W, r, s.causal)
        qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)          # [1, H, Q, 576]
        kt = torch.from_numpy(kv).unsqueeze(0).unsqueeze(0).expand(1, H, L, 576)
        vt = torch.from_numpy(np.ascontiguousarray(kv[:, :512])).unsqueeze(0).unsqueeze(0).expand(1, H, L, 512)
        mt = torch.from_numpy(mask)
        for j in range(Q):
            if not mask[j].any():
                outs[b * Q + j] = 0.0
                lses[b * Q + j] = -np.inf
                continue
            o = torch.nn.functional.scaled_dot_product_attention(
                qt[:, :, j:j + 1], kt, vt, attn_mask=mt[j:j + 1], scale=s.scale)
            outs[b * Q + j] = o[0, :, 0].numpy()
            sc = s.scale * (qt[0, :, j].unsqueeze(1) @ kt[0].transpose(-1, -2)).squeeze(1)   # [H, L]
            sc = sc.masked_fill(~mt[j], -math.inf)
            l = torch.logsumexp(sc, dim=-1).numpy()
            lses[b * Q + j] = l / math.log(2.0) if base == "2" else l
    return outs, lses


@pytest.mark.parametrize("W,causal", [(1, True), (2, True), (3, True), (2, False), (4, False)])
def test_oracle_matches_torch_sdpa(W, causal):
    wl = tiny(B=2, H=3, Q=3, W=W, causal=causal, lengths=(9, 23), seed=100 + W)
    for r in range(W):
        o, l = oracle_rank(wl, r)
        ro, rl = sdpa_reference(wl, r)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, rl, rtol=0, atol=1e-12)


def test_oracle_matches_pure_python_bruteforce():
    wl = tiny(B=2, H=2, Q=3, W=3, causal=True, lengths=(7, 11), seed=5)
    s = wl.spec
    for r in range(3):
        for base in ("e", "2"):
            o, l = oracle_rank(wl, r, base)
            for b in range(2):
                kv = [[brute.bf16_to_float(x) for x in row] for row in wl.global_kv(b)]
                for j in range(s.Q):
                    for h in range(s.H):
                        q = [brute.bf16_to_float(x) for x in wl.q_bits[b, j, h]]
                        bo, bl = brute.attend_row(q, kv, j, s.Q, int(wl.tot[b]), int(wl.seq_lens[r][b]),
                                                  s.W, r, True, s.scale, base)
                        assert abs(l[b * s.Q + j, h] - bl) <= 1e-12 or (bl == -math.inf and l[b * s.Q + j, h] == -math.inf)
                        np.testing.assert_allclose(o[b * s.Q + j, h], bo, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- FP8 cache

def test_e4m3_decode_matches_torch_and_closed_forms():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert got[0x38] == 1.0 and got[0xB8] == -1.0 and got[0x7E] == 448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


@pytest.mark.parametrize("kv_scale", [1.0, 0.25, 3.0])
def test_fp8_cache_is_the_bf16_path_on_its_values(kv_scale):
    # the oracle's FP8 branch equals its bf16 branch on the cache's values
    # (torch decodes the codes; values times kv_scale are exact in bf16 for
    # these scales), which pins the decoding and where the scale applies
    wl8 = tiny(B=2, H=3, Q=3, W=2, causal=True, lengths=(9, 14), seed=23, kv_dtype="fp8", kv_scale=kv_scale)
    s = wl8.spec

    def rows_bf16(b, pos):
        v = torch.from_numpy(wl8.global_rows(b, pos)).view(torch.float8_e4m3fn).float() * kv_scale
        return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    for r in range(2):
        o8, l8 = oracle.mla_decode(wl8.q_bits, wl8.global_rows, wl8.seq_lens[r], wl8.tot, s.W, r, True, s.scale,
                                   "e", kv_scale=kv_scale)
        ob, lb = oracle.mla_decode(wl8.q_bits, rows_bf16, wl8.seq_lens[r], wl8.tot, s.W, r, True, s.scale, "e")
        np.testing.assert_array_equal(o8, ob)
        np.testing.assert_array_equal(l8, lb)


def test_e4m3_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_to_f64(codes)), codes)


def test_e4m3_encode_matches_torch_below_saturation():
    # torch rounds to nearest even but turns magnitudes from 464 up into NaN;
    # below that the two must agree bit for bit
    rng = np.random.default_rng(5)
    mag = np.exp2(rng.uniform(-14, np.log2(463.9), 20000)).astype(np.float32)
    x = np.concatenate([mag * rng.choice([-1, 1], mag.size), np.float32([0.0, -0.0, 2.0 ** -10, -2.0 ** -10,
                                                                         1.5 * 2.0 ** -10, 448.0, 463.0])])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


def test_e4m3_encode_ties_go_to_the_even_code():
    # the midpoint between two neighbouring codes of one sign (exact in
    # float32) encodes to whichever of them has an even mantissa field
    for c in list(range(0, 0x7E)) + list(range(0x80, 0xFE)):
        lo, hi = oracle.e4m3_to_f64(np.uint8([c, c + 1]))
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2
        got = int(oracle.e4m3_encode(np.float32([mid]))[0])
        assert got == (c if c % 2 == 0 else c + 1), hex(c)


def test_e4m3_encode_saturates_and_keeps_nan():
    x = np.float32([448.0, 449.0, 464.0, 500.0, 3e38, np.inf, -448.0, -1e9, -np.inf, np.nan])
    assert list(oracle.e4m3_encode(x)) == [0x7E] * 6 + [0xFE] * 3 + [0x7F]
    # smallest subnormal and the half-way points below and above it
    assert list(oracle.e4m3_encode(np.float32([2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -9, -2.0 ** -11]))) == [1, 0, 2, 0x80]


def test_kv_write_fp8_stores_the_nearest_codes_of_value_over_scale():
    rng = np.random.default_rng(9)
    n, P, bs, s = 40, 3, 16, 0.0123
    vals = (rng.standard_normal((n, oracle.D_QK)) * 3).astype(np.float32)
    rows = (vals.view(np.uint32) >> 16).astype(np.uint16)  # bf16 bits (truncated; any bf16 values do)
    cache = rng.integers(0, 256, size=(P, bs, oracle.D_QK), dtype=np.uint8)
    slots = rng.permutation(P * bs)[:n].astype(np.int64)
    slots[::7] = oracle.PAD_SLOT_ID
    out = oracle.kv_write_fp8(cache, rows, slots, s)
    x = oracle.bf16_bits_to_f64(rows)
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        got = oracle.e4m3_to_f64(out[sl // bs, sl % bs])
        q = (x[i].astype(np.float32) / np.float32(s)).astype(np.float64)
        # nearest: no E4M3 value is closer to the float32 quotient
        allv = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
        allv = allv[np.isfinite(allv)]
        best = np.min(np.abs(q[:, None] - allv[None, :]), axis=1)
        assert np.all(np.abs(q - got) == best)
    untouched = np.ones(P * bs, bool)
    untouched[slots[slots >= 0]] = False
    assert np.array_equal(out.reshape(P * bs, -1)[untouched], cache.reshape(P * bs, -1)[untouched])


# ---------------------------------------------------------------- varlen

def tiny_varlen(q_lens, W=2, causal=True, lengths=(9, 14, 6), seed=17, I=1):
    spec = WL.Spec(name="tiny_varlen", B=len(q_lens), H=2, Q=max(q_lens), causal=causal, seed=seed,
                   lengths=list(lengths), W=W, ranks=tuple(range(W)), block_size=4, interleave=I, q_lens=list(q_lens))
    return WL.build(spec)


def varlen_rank(wl, r, base="e"):
    s = wl.spec
    return oracle.mla_decode_varlen(wl.q_tok, wl.query_start_loc, wl.global_rows, wl.seq_lens[r], wl.tot, s.W, r,
                                    s.causal, s.scale, base, interleave=s.interleave)


@pytest.mark.parametrize("causal,I", [(True, 1), (False, 1), (True, 2)])
def test_varlen_oracle_matches_pure_python_bruteforce(causal, I):
    wl = tiny_varlen([3, 0, 1], W=2, causal=causal, lengths=(9, 5, 12), I=I)
    s, qsl = wl.spec, wl.query_start_loc
    for r in range(2):
        o, l = varlen_rank(wl, r)
        for b in range(s.B):
            kv = [[brute.bf16_to_float(x) for x in row] for row in wl.global_kv(b)]
            ql = int(qsl[b + 1] - qsl[b])
            for j in range(ql):
                for h in range(s.H):
                    q = [brute.bf16_to_float(x) for x in wl.q_tok[qsl[b] + j, h]]
                    bo, bl = brute.attend_row(q, kv, j, ql, int(wl.tot[b]), int(wl.seq_lens[r][b]), s.W, r, causal,
                                              s.scale, "e", I)
                    got = l[qsl[b] + j, h]
                    assert abs(got - bl) <= 1e-12 or (bl == -math.inf and got == -math.inf)
                    np.testing.assert_allclose(o[qsl[b] + j, h], bo, rtol=0, atol=1e-12)


def test_varlen_equals_one_uniform_call_per_request():
    # each request alone is a uniform call with its own query length
    wl = tiny_varlen([4, 1, 2], W=3, lengths=(17, 8, 23))
    s, qsl = wl.spec, wl.query_start_loc
    for r in range(3):
        o, l = varlen_rank(wl, r)
        for b in range(s.B):
            ql = int(qsl[b + 1] - qsl[b])
            q1 = wl.q_tok[qsl[b]:qsl[b + 1]][None]  # [1, ql, H, 576]
            uo, ul = oracle.mla_decode(q1, lambda _b, pos: wl.global_rows(b, pos), wl.seq_lens[r][b:b + 1],
                                       wl.tot[b:b + 1], s.W, r, True, s.scale, "e")
            np.testing.assert_array_equal(o[qsl[b]:qsl[b + 1]], uo)
            np.testing.assert_array_equal(l[qsl[b]:qsl[b + 1]], ul)


def test_varlen_with_equal_lengths_is_the_uniform_call():
    wl = tiny_varlen([3, 3, 3], W=2, lengths=(9, 14, 6))
    s = wl.spec
    for r in range(2):
        o, l = varlen_rank(wl, r)
        q = wl.q_tok.reshape(s.B, 3, s.H, oracle.D_QK)
        uo, ul = oracle.mla_decode(q, wl.global_rows, wl.seq_lens[r], wl.tot, s.W, r, True, s.scale, "e")
        np.testing.assert_array_equal(o, uo)
        np.testing.assert_array_equal(l, ul)


def test_zero_query_gives_uniform_mean_and_log_count():
    # q = 0: every visible score is 0, softmax is uniform: lse = ln(count), out = mean of V
    wl = tiny(B=2, H=2, Q=4, W=3, causal=True, lengths=(17, 30), seed=9, q_zero=True)
    s = wl.spec
    for r in range(3):
        o, l = oracle_rank(wl, r)
        for b in range(2):
            kv = O.bf16_bits_to_f64(wl.global_kv(b))
            for j in range(s.Q):
                vis = [p for p in range(kv.shape[0]) if brute.is_visible(p, j, s.Q, int(wl.tot[b]),
                                                                        int(wl.seq_lens[r][b]), 3, r, True)]
                if not vis:
                    assert np.all(l[b * s.Q + j] == -np.inf) and np.all(o[b * s.Q + j] == 0)
                    continue
                np.testing.assert_allclose(l[b * s.Q + j], math.log(len(vis)), atol=1e-14)
                np.testing.assert_allclose(o[b * s.Q + j], np.broadcast_to(kv[vis, :512].mean(0), (s.H, 512)), atol=1e-13)


def test_single_visible_key_and_identical_keys_closed_forms():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 576))
    k = rng.standard_normal((1, 576))
    out, lse = oracle.attend(q, k, 0.37)
    np.testing.assert_allclose(out, np.broadcast_to(k[0, :512], (4, 512)), atol=1e-15)
    np.testing.assert_allclose(lse, 0.37 * (q @ k[0]), atol=1e-13)
    kk = np.repeat(k, 7, axis=0)
    out, lse = oracle.attend(q, kk, 0.37)
    np.testing.assert_allclose(out, np.broadcast_to(k[0, :512], (4, 512)), atol=1e-14)
    np.testing.assert_allclose(lse, 0.37 * (q @ k[0]) + math.log(7), atol=1e-13)
    # nothing visible
    out, lse = oracle.attend(q, np.zeros((0, 576)), 0.37)
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_lse_base_two_is_base_e_over_ln2():
    wl = tiny(B=2, H=3, Q=2, W=2, causal=True, lengths=(10, 13), seed=21)
    for r in range(2):
        oe, le = oracle_rank(wl, r, "e")
        o2, l2 = oracle_rank(wl, r, "2")
        np.testing.assert_array_equal(oe, o2)
        fin = np.isfinite(le)
        np.testing.assert_allclose(le[fin], math.log(2.0) * l2[fin], rtol=1e-14)


def test_single_rank_equals_non_dcp():
    wl = tiny(B=2, H=3, Q=3, W=1, causal=True, lengths=(12, 19), seed=31)
    o1, l1 = oracle.mla_decode(wl.q_bits, wl.global_rows, wl.seq_lens[0], wl.tot, 1, 0, True, wl.spec.scale)
    o0, l0 = oracle.mla_decode(wl.q_bits, wl.global_rows, wl.seq_lens[0], None, 1, 0, True, wl.spec.scale)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(l1, l0)


@pytest.mark.parametrize("W,causal,base,I", [(2, True, "e", 1), (8, True, "e", 1), (3, False, "2", 1),
                                           (8, True, "2", 1), (2, True, "e", 4), (3, True, "2", 2),
                                           (4, False, "e", 2)])
def test_sharded_then_merged_equals_unsharded(W, causal, base, I):
    wl = tiny(B=3, H=2, Q=4, W=W, causal=causal, lengths=(5, 29, 40), seed=41 + W + I, interleave=I)
    parts = [oracle_rank(wl, r, base) for r in range(W)]
    mo, ml = oracle.merge_lse([p[0] for p in parts], [p[1] for p in parts], base)
    un = WL.unsharded(wl)
    uo, ul = oracle.mla_decode(un.q_bits, un.global_rows, un.seq_lens[0], un.tot, 1, 0, causal, wl.spec.scale, base)
    np.testing.assert_allclose(mo, uo, atol=1e-12)
    np.testing.assert_allclose(ml, ul, atol=1e-12)


def test_merge_special_cases():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((3, 2, 512))
    l = rng.standard_normal((3, 2))
    mo, ml = oracle.merge_lse([o], [l])
    np.testing.assert_allclose(mo, o, atol=1e-15)
    np.testing.assert_allclose(ml, l, atol=1e-15)
    # a -inf partial has weight 0
    mo, ml = oracle.merge_lse([o, np.zeros_like(o)], [l, np.full_like(l, -np.inf)])
    np.testing.assert_allclose(mo, o, atol=1e-15)
    np.testing.assert_allclose(ml, l, atol=1e-15)
    # every partial empty
    mo, ml = oracle.merge_lse([np.zeros_like(o)] * 3, [np.full_like(l, -np.inf)] * 3)
    assert np.all(mo == 0) and np.all(ml == -np.inf)
    # two equal partials: same out, lse + ln 2 (base e) / + 1 (base 2)
    mo, ml = oracle.merge_lse([o, o], [l, l], "e")
    np.testing.assert_allclose(mo, o, atol=1e-15)
    np.testing.assert_allclose(ml, l + math.log(2), atol=1e-14)
    mo, ml = oracle.merge_lse([o, o], [l, l], "2")
    np.testing.assert_allclose(ml, l + 1.0, atol=1e-14)


# ---------------------------------------------------------------- slots

@pytest.mark.parametrize("fname", ["cp_local_slot_hand_example.json", "cp_local_slot_interleave2_hand_example.json"])
def test_slot_hand_examples(fname):
    g = json.load(open(os.path.join(GOLDEN, fname)))
    bt = np.array(g["block_table"], dtype=np.int32)
    pos = np.array(g["positions"], dtype=np.int64)
    for r, exp in g["expected"].items():
        got = oracle.cp_local_slot(pos, bt, g["block_size"], g["cp_world"], int(r), g["interleave"])
        assert got.tolist() == exp


def test_slot_single_rank_is_textbook_paging():
    rng = np.random.default_rng(1)
    bt = rng.permutation(50).astype(np.int32)[:40].reshape(4, 10)
    pos = rng.integers(0, 10 * 16, size=(4, 33))
    got = oracle.cp_local_slot(pos, bt, 16, 1, 0)
    exp = np.array([[bt[b, p // 16] * 16 + p % 16 for p in pos[b]] for b in range(4)])
    np.testing.assert_array_equal(got, exp)


@pytest.mark.parametrize("W,I,bs", [(2, 1, 4), (4, 1, 16), (8, 1, 64), (3, 2, 4), (4, 4, 16)])
def test_slot_ownership_and_local_layout(W, I, bs):
    # exactly one rank owns each position; rank r's slots are its local rows
    # t = 0, 1, ... laid out by plain paging inside the shared table
    rng = np.random.default_rng(W * 10 + I)
    nb = 6
    bt = rng.permutation(3 * nb).astype(np.int32)[:nb].reshape(1, nb)
    L = nb * bs * W
    pos = np.arange(L, dtype=np.int64).reshape(1, L)
    slots = np.stack([oracle.cp_local_slot(pos, bt, bs, W, r, I)[0] for r in range(W)])
    owners = (slots != oracle.PAD_SLOT_ID).sum(0)
    assert np.all(owners == 1)
    for r in range(W):
        mine = slots[r][slots[r] != oracle.PAD_SLOT_ID]
        n = mine.size
        exp = [bt[0, t // bs] * bs + t % bs for t in range(n)]
        assert mine.tolist() == exp


def test_slot_pad_cases():
    bt = np.array([[2, 5], [1, 0]], dtype=np.int32)
    pos = np.array([[0, 1, 2, -3, 40, 9], [3, 4, 5, 6, 7, 8]], dtype=np.int64)
    nv = np.array([4, 2], dtype=np.int32)
    got = oracle.cp_local_slot(pos, bt, 4, 2, 0, 1, nv)
    # request 0: index >= 4 is the rejected suffix; -3 is negative
    assert got[0].tolist() == [8, -1, 9, -1, -1, -1]
    # request 1: only the first 2 entries are valid
    assert got[1].tolist() == [-1, 6, -1, -1, -1, -1]
    # virtual block past the table width
    got = oracle.cp_local_slot(np.array([[16, 15]]), np.array([[3, 4]], dtype=np.int32), 4, 2, 1)
    assert got.tolist() == [[-1, 19]]


def test_draft_rejected_suffix_maps_to_pad():
    # PR #52188 page: at cp_rank=1, cp_size=2 the rejected context suffix maps to the pad slot
    spec = WL.Spec(name="draft", B=4, H=2, Q=16, causal=False, seed=77, lengths=[300, 517, 1000, 1601],
                   W=2, ranks=(1,), block_size=8)
    wl = WL.build(spec)
    si = WL.draft_slot_inputs(wl)
    got = oracle.cp_local_slot(si["ctx_positions"], wl.block_table, 8, 2, 1, 1, si["ctx_num_valid"])
    for b in range(4):
        nv = int(si["ctx_num_valid"][b])
        assert np.all(got[b, nv:] == oracle.PAD_SLOT_ID)
        for i in range(nv):
            p = int(si["ctx_positions"][b, i])
            if p % 2 == 1:
                t = p // 2
                assert got[b, i] == wl.block_table[b, t // 8] * 8 + t % 8
            else:
                assert got[b, i] == oracle.PAD_SLOT_ID


# ---------------------------------------------------------------- generator consistency

def test_paged_pool_holds_the_shards():
    wl = tiny(B=3, H=2, Q=2, W=3, causal=True, lengths=(1, 30, 47), seed=61)
    bs = wl.spec.block_size
    for r in range(3):
        for b in range(3):
            n = int(wl.seq_lens[r][b])
            for t in range(n):
                np.testing.assert_array_equal(wl.pools[r][wl.block_table[b, t // bs], t % bs], wl.shards[r][b][t])


# ---------------------------------------------------------------- KV write

@pytest.mark.parametrize("I", [1, 2, 4])
def test_kv_write_rebuilds_every_rank_pool_from_the_global_kv(I):
    """Writing each global position's row at the slot cp_local_slot gives it,
    for every rank, rebuilds the rank pools the generator laid out by its own
    paging code (the rows requests use; the others keep their filler)."""
    wl = tiny(B=3, H=2, Q=2, W=3, causal=True, lengths=(1, 70, 131), seed=63, interleave=I)
    bs, W = wl.spec.block_size, wl.spec.W
    for r in range(W):
        cache = wl.pools[r].copy()
        used = np.zeros(cache.shape[:2], dtype=bool)
        for b in range(wl.spec.B):
            n = int(wl.seq_lens[r][b])
            for t in range(n):
                used[wl.block_table[b, t // bs], t % bs] = True
        cache[used] = 0xFFFF  # forget what the generator put there
        for b in range(wl.spec.B):
            L = int(wl.tot[b])
            pos = np.arange(L, dtype=np.int64)[None, :]
            slots = oracle.cp_local_slot(pos, wl.block_table[b:b + 1], bs, W, r, I)
            cache = oracle.kv_write(cache, wl.global_kv(b), slots[0])
        np.testing.assert_array_equal(cache, wl.pools[r])


def test_kv_write_scatter_invariants():
    """Distinct in-range slots: the cache row at each slot is the row written
    there and every other row is unchanged; pad, negative and past-the-end
    slots write nothing; of two rows with one slot the later one stays."""
    rng = np.random.default_rng(5)
    P, bs, n = 5, 4, 9
    cache = rng.integers(0, 1 << 16, size=(P, bs, oracle.D_QK), dtype=np.uint16)
    rows = rng.integers(0, 1 << 16, size=(n, oracle.D_QK), dtype=np.uint16)
    slots = np.array([7, oracle.PAD_SLOT_ID, 0, 19, -5, 20, 1 << 40, 3, 12], dtype=np.int64)
    got = oracle.kv_write(cache, rows, slots)
    expect = cache.copy().reshape(P * bs, oracle.D_QK)
    for i, s in enumerate(slots):
        if 0 <= s < P * bs:
            expect[s] = rows[i]
    np.testing.assert_array_equal(got.reshape(P * bs, -1), expect)
    assert np.array_equal(cache, oracle.kv_write(cache, rows[:0], slots[:0]))  # nothing to write
    dup = oracle.kv_write(cache, rows[:2], np.array([6, 6], dtype=np.int64))
    np.testing.assert_array_equal(dup[1, 2], rows[1])


# ---------------------------------------------------------------- planted mistakes

def test_mutations_are_caught(monkeypatch):
    """Plant plausible slips in the oracle (CPU only) and check a pin catches each."""
    wl = tiny(B=2, H=2, Q=3, W=2, causal=True, lengths=(9, 16), seed=7)

    def pins_pass():
        try:
            for r in range(2):
                o, l = oracle_rank(wl, r)
                ro, rl = sdpa_reference(wl, r)
                np.testing.assert_allclose(o, ro, atol=1e-9)
                np.testing.assert_allclose(l, rl, atol=1e-9)
            return True
        except AssertionError:
            return False

    assert pins_pass()
    real_attend = O.attend
    real_vis = O.visible_positions

    muts = {
        "drop rope part of the score": lambda q, kv, sc, base="e": real_attend(
            np.concatenate([q[:, :512], 0 * q[:, 512:]], 1), kv, sc, base),
        "wrong scale": lambda q, kv, sc, base="e": real_attend(q, kv, sc * 1.01, base),
        "lse in base 2": lambda q, kv, sc, base="e": real_attend(q, kv, sc, "2"),
    }
    for name, fn in muts.items():
        monkeypatch.setattr(O, "attend", fn)
        assert not pins_pass(), name
        monkeypatch.setattr(O, "attend", real_attend)

    vis_muts = {
        "causal offset off by one": lambda s, t, Q, j, W, r, c, i=1: real_vis(s, t + 1, Q, j, W, r, c, i),
        "wrong rank": lambda s, t, Q, j, W, r, c, i=1: real_vis(s, t, Q, j, W, (r + 1) % W, c, i),
        "end-aligned local mask": lambda s, t, Q, j, W, r, c, i=1: real_vis(s, t, Q, j, W, r, False, i)[
            : max(s - (Q - 1 - j), 0)],
    }
    for name, fn in vis_muts.items():
        monkeypatch.setattr(O, "visible_positions", fn)
        assert not pins_pass(), name
        monkeypatch.setattr(O, "visible_positions", real_vis)
    assert pins_pass()
