"""fp64 reference for absorbed MLA decode with round-robin KV sharding.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and plain on
purpose: exact two-pass softmax over an explicitly enumerated set of global
positions, read from the *contiguous global* KV of each request (no block
tables, no online softmax, no splitting).

Sources (three vLLM PR digest pages):
  * PR #52188 page ("support Kimi-K3 DSpark speculative decoding with DCP"),
    key source snippets: the per-query causal prefix of a multi-token query
    (row j of a q_len block sees the global prefix tot - (q_len - 1 - j),
    clamped at 0); the round-robin rank-local length; the non-causal draft
    block where every row sees the same context; and the `cp_local_slot`
    kernel (ownership of a position by rank, rank-local offset, pad slot).
  * PR #54012 page ("MLA decode with DCP uses FlashInfer's native CP mask"),
    implementation breakdown and key source snippets: the kernel takes the
    rank-local seq_lens plus the *global* causal lengths, cp_world and cp_rank
    and masks per row itself; interleave must be 1; the returned LSE is a
    natural log; partial results of all ranks are merged across ranks.
  * PR #48180 page ("TokenSpeed MLA with DCP and Eagle"), implementation
    breakdown: the same kernel contract with a base-2 LSE, and review
    highlights: an end-aligned local causal mask is wrong under DCP when
    q_len > 1.

Readings where the pages are silent (each is also listed in the design notes):
  * LSE is the log-normaliser of the softmax over *scaled* scores; base 2 is
    the base-e value divided by ln 2.
  * The query at row j of a causal block is the token at global position
    tot - q_len + j and sees every global position p <= itself.
  * Rank r holds local rows t < seq_lens[b] that are the global positions
    p = t*W + r (interleave 1).  A row sees the positions it holds that its
    causal bound admits; a non-causal row sees every position it holds.
  * A row with nothing visible yields out = 0 and lse = -inf.
  * The merge weights each partial by base**(lse_r - max lse); partials with
    lse = -inf get weight 0; if every partial is -inf the result is (0, -inf).
  * The pad slot id is -1; a position whose index in its request is at or
    past num_valid[b] (the rejected suffix), a negative position and a
    virtual block past the table width all map to the pad slot.
"""
from __future__ import annotations

import math
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

D_QK = 576   # absorbed query / latent KV width: 512 latent + 64 rope
D_V = 512    # value width: the latent part of the KV row
PAD_SLOT_ID = -1


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def owns(p: np.ndarray, W: int, r: int, interleave: int = 1) -> np.ndarray:
    """Whether rank r holds global position p: positions are dealt to the
    ranks in segments of `interleave`, segment k going to rank k mod W
    (PR #52188 page, key source snippets, cp_local_slot)."""
    return (np.asarray(p) // interleave) % W == r


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode 8-bit floats with 1 sign, 4 exponent (bias 7) and 3 mantissa bits
    (the OCP E4M3 format, no infinities): exponent 0 is subnormal
    (m/8 * 2^-6), the code with all exponent and mantissa bits set is NaN,
    the largest value is 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, out)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """8-bit E4M3 code of each float32 value: the nearest E4M3 value, ties
    to the even code (mantissa field even); finite magnitudes at or above
    448 and infinities saturate to +-448 (0x7E/0xFE); NaN gives 0x7F; the
    sign of zero and of values that round to zero is kept.

    Written from the format (1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals m/8 * 2^-6): below 2^-6 the code is the number of 2^-9
    steps, rounded half to even; above, with |x| = (1 + f) 2^e, the exponent
    field is e + 7 and the mantissa field is 8f rounded half to even, a
    carry moving to the next exponent.  All steps are exact in float64.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64).reshape(-1)
    out = np.empty(x.size, dtype=np.uint8)
    for i, v in enumerate(x):
        sign = 0x80 if math.copysign(1.0, v) < 0 else 0
        if math.isnan(v):
            out[i] = 0x7F
            continue
        a = abs(v)
        if a >= 448.0:
            out[i] = sign | 0x7E
            continue
        if a < 2.0 ** -6:
            out[i] = sign | int(np.rint(a * 2.0 ** 9))  # 0..8; 8 is the smallest normal, code 0x08
            continue
        fr, k = math.frexp(a)  # a = fr 2^k, fr in [0.5, 1)
        e = k - 1
        mant = np.rint((a / 2.0 ** e - 1.0) * 8.0)
        if mant == 8.0:
            e, mant = e + 1, 0.0
        out[i] = sign | ((e + 7) << 3) | int(mant)
    return out


def kv_write_fp8(cache_codes: np.ndarray, rows_bits: np.ndarray, slots: np.ndarray, kv_scale: float) -> np.ndarray:
    """kv_write into an FP8 cache: each bf16 row is divided by kv_scale in
    float32 (the correctly rounded quotient) and stored as the E4M3 codes of
    e4m3_encode, at the same slots and with the same skips as kv_write (the
    cache then holds value / kv_scale, which mla_decode multiplies back by
    kv_scale; PR #54012 page, key source snippets: the cache dtype and its
    scales).  cache_codes [num_blocks, block_size, 576] uint8."""
    rows = bf16_bits_to_f64(np.asarray(rows_bits)).astype(np.float32)
    q = (rows / np.float32(kv_scale)).astype(np.float32)
    codes = e4m3_encode(q).reshape(rows.shape)
    return kv_write(cache_codes, codes, slots)


def held_positions(seq_len: int, W: int, r: int, interleave: int = 1) -> np.ndarray:
    """Global positions of the local rows a rank holds, in order: the first
    seq_len positions it owns (local row t is the t-th of them).  By
    enumeration; with interleave 1 these are t*W + r."""
    n = int(seq_len)
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    span = (n // interleave + 2) * interleave * W  # enough positions to hold n owned ones
    p = np.arange(span, dtype=np.int64)
    return p[owns(p, W, r, interleave)][:n]


def local_count(g: int, W: int, r: int, interleave: int = 1) -> int:
    """How many of the global positions 0..g-1 rank r holds, by enumeration."""
    if g <= 0:
        return 0
    p = np.arange(int(g), dtype=np.int64)
    return int(np.count_nonzero(owns(p, W, r, interleave)))


def visible_positions(seq_len: int, tot: Optional[int], q_len: int, j: int,
                      W: int, r: int, causal: bool, interleave: int = 1) -> np.ndarray:
    """Global positions row j of a request attends to on rank r.

    Causal: the row is the token at global position tot - q_len + j, so it
    sees the global prefix of length tot - (q_len - 1 - j) (PR #52188 page,
    key source snippets, flattened decode metadata: offsets q_len-1 .. 0
    subtracted from the global length, clamped at 0).  Of those, the rank
    sees the ones it holds.  Non-causal: every held position (the draft block
    repeats the same context length for each row).
    """
    held = held_positions(seq_len, W, r, interleave)
    if not causal:
        return held
    g = max(int(tot) - (q_len - 1 - j), 0)
    return held[held < g]


def attend(q_rows: np.ndarray, kv_rows: np.ndarray, scale: float, base: str = "e"
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of query rows [n, 576] over KV rows [m, 576], in float64.

    Scores use all 576 columns (latent and rope parts); values are the first
    512 columns of the same rows (absorbed MLA: the latent is also the value).
    Returns out [n, 512] and lse [n] in the requested base.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    n = q_rows.shape[0]
    if kv_rows.shape[0] == 0:
        return np.zeros((n, D_V)), np.full((n,), -np.inf)
    kv_rows = np.asarray(kv_rows, dtype=np.float64)
    s = scale * (q_rows @ kv_rows.T)                  # [n, m]
    m = s.max(axis=1, keepdims=True)                  # pass 1: row max
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)                  # pass 2: normaliser
    out = (e @ kv_rows[:, :D_V]) / z
    lse = (m + np.log(z))[:, 0]
    if base == "2":
        lse = lse / math.log(2.0)
    return out, lse


def mla_decode(q_bits: np.ndarray, kv_rows: Callable[[int, np.ndarray], np.ndarray],
               seq_lens: Sequence[int], tot: Optional[Sequence[int]], W: int, r: int,
               causal: bool, scale: float, base: str = "e",
               rows: Optional[Sequence[Tuple[int, int, int]]] = None, interleave: int = 1,
               kv_scale: Optional[float] = None):
    """Oracle for one rank's decode call.

    q_bits:   [B, Q, H, 576] bf16 bits.
    kv_rows:  kv_rows(b, positions) -> bf16 bits [len(positions), 576] from the
              contiguous global KV of request b.
    seq_lens: rank-local lengths; tot: global causal lengths (None: equal to
              seq_lens, the single-rank case).
    rows:     optional list of (b, j, h) to compute; default all.
    interleave: the rank holds positions in segments of this many (1: every
              W-th position).
    kv_scale: None for a bf16 cache; otherwise kv_rows returns 8-bit E4M3
              codes and the key/value rows are their values times kv_scale
              (one dequantisation scale for the latent cache, which is both
              key and value).
    Returns (out [B*Q, H, 512], lse [B*Q, H]) as float64; rows not asked for
    are NaN.
    """
    B, Q, H, D = q_bits.shape
    assert D == D_QK
    out = np.full((B * Q, H, D_V), np.nan)
    lse = np.full((B * Q, H), np.nan)
    want = {}
    if rows is None:
        for b in range(B):
            for j in range(Q):
                want[(b, j)] = list(range(H))
    else:
        for (b, j, h) in rows:
            want.setdefault((b, j), []).append(h)
    cache = {}
    for (b, j), heads in sorted(want.items()):
        t = None if tot is None else int(tot[b])
        if t is None:
            t = int(seq_lens[b])
        pos = visible_positions(int(seq_lens[b]), t, Q, j, W, r, causal, interleave)
        key = (b, pos.size, int(pos[-1]) if pos.size else -1)
        if key not in cache:
            cache.clear()
            raw = kv_rows(b, pos)
            cache[key] = bf16_bits_to_f64(raw) if kv_scale is None else e4m3_to_f64(raw) * float(kv_scale)
        kv = cache[key]
        qr = bf16_bits_to_f64(q_bits[b, j, heads, :])
        o, l = attend(qr, kv, scale, base)
        out[b * Q + j, heads] = o
        lse[b * Q + j, heads] = l
    return out, lse


def mla_decode_varlen(q_tok: np.ndarray, query_start_loc: Sequence[int],
                      kv_rows: Callable[[int, np.ndarray], np.ndarray],
                      seq_lens: Sequence[int], tot: Optional[Sequence[int]], W: int, r: int,
                      causal: bool, scale: float, base: str = "e", interleave: int = 1):
    """Oracle for one rank's decode call with a query length per request.

    q_tok:  [T, H, 576] bf16 bits, the query tokens of all requests packed;
            request b owns tokens query_start_loc[b] .. query_start_loc[b+1]-1.
    Reading (PR #52188 page, key source snippets: the per-row causal prefix
    tot - (query_len - 1 - j); summary: the builder declares support for
    batches of different query lengths): each request applies the per-row
    prefix with its own query length; a request with no tokens has no rows.
    Returns (out [T, H, 512], lse [T, H]) as float64.
    """
    T, H, D = q_tok.shape
    assert D == D_QK
    qsl = [int(x) for x in query_start_loc]
    out = np.full((T, H, D_V), np.nan)
    lse = np.full((T, H), np.nan)
    for b in range(len(qsl) - 1):
        q_len = qsl[b + 1] - qsl[b]
        t = int(seq_lens[b]) if tot is None else int(tot[b])
        for j in range(q_len):
            pos = visible_positions(int(seq_lens[b]), t, q_len, j, W, r, causal, interleave)
            kv = bf16_bits_to_f64(kv_rows(b, pos))
            o, l = attend(bf16_bits_to_f64(q_tok[qsl[b] + j]), kv, scale, base)
            out[qsl[b] + j] = o
            lse[qsl[b] + j] = l
    return out, lse


def merge_lse(outs: List[np.ndarray], lses: List[np.ndarray], base: str = "e"
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Combine partial (out, lse) pairs of disjoint key sets into the full result.

    The pages name the cross-rank merge of partial outputs by their LSE
    (PR #54012 page, implementation breakdown: the LSE base must agree across
    ranks before merging) without printing it; this is the standard
    log-sum-exp combine: weights base**(lse_r - M) with M = max_r lse_r.
    """
    beta = math.e if base == "e" else 2.0
    o = np.stack([np.asarray(x, dtype=np.float64) for x in outs])     # [n, rows, H, 512]
    lam = np.stack([np.asarray(x, dtype=np.float64) for x in lses])   # [n, rows, H]
    M = lam.max(axis=0)
    empty = ~np.isfinite(M)
    Msafe = np.where(empty, 0.0, M)
    w = np.where(np.isfinite(lam), np.power(beta, lam - Msafe[None]), 0.0)
    wsum = w.sum(axis=0)
    num = (w[..., None] * o).sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(empty[..., None], 0.0, num / np.where(empty, 1.0, wsum)[..., None])
        lse = np.where(empty, -np.inf, Msafe + np.log(np.where(empty, 1.0, wsum)) / math.log(beta))
    return out, lse


def cp_local_slot(positions: np.ndarray, block_table: np.ndarray, block_size: int,
                  W: int, r: int, interleave: int = 1,
                  num_valid: Optional[np.ndarray] = None) -> np.ndarray:
    """Rank-local KV slot of each position, or PAD_SLOT_ID, with plain Python ints.

    PR #52188 page, key source snippets (cp_local_slot): a block-table entry
    covers block_size * W consecutive global positions (the virtual block,
    index pos // (block_size * W), as the DFlash input preparation computes
    it); inside it, segments of `interleave` positions go to ranks in turn;
    a rank's local offset counts its whole rounds of segments and then the
    offset inside the current segment; positions the rank does not own get
    the pad slot.  With W == 1 the slot is the plain paged slot.
    The rejected context suffix (index >= num_valid[b]), negative positions
    and virtual blocks past the table width also get the pad slot.
    """
    positions = np.asarray(positions)
    B, n = positions.shape
    out = np.empty((B, n), dtype=np.int64)
    nb = block_table.shape[1]
    for b in range(B):
        for i in range(n):
            pos = int(positions[b, i])
            if (num_valid is not None and i >= int(num_valid[b])) or pos < 0:
                out[b, i] = PAD_SLOT_ID
                continue
            span = block_size * W
            v = pos // span
            off = pos % span
            if v >= nb:
                out[b, i] = PAD_SLOT_ID
                continue
            blk = int(block_table[b, v])
            if W == 1:
                out[b, i] = blk * block_size + off
                continue
            if (off // interleave) % W != r:
                out[b, i] = PAD_SLOT_ID
                continue
            local = (off // (interleave * W)) * interleave + off % interleave
            out[b, i] = blk * block_size + local
    return out


def kv_write(cache_bits: np.ndarray, rows_bits: np.ndarray, slots: np.ndarray) -> np.ndarray:
    """A copy of the paged cache with each new KV row stored at its slot.

    PR #52188 page, key source snippets (cp_local_slot) and risks: the draft's
    KV is written at the rank-local slot of its position, and a position the
    rank does not own gets the pad slot so that nothing is written for it
    (writing there would overwrite another rank's data).  Slot s names row
    s % block_size of block s // block_size of the cache.  Reading: a slot
    that is negative (the pad slot) or past the cache's rows writes nothing.

    cache_bits [num_blocks, block_size, 576] and rows_bits [n, 576] are bf16
    bit patterns; slots [n] int64.  Rows are stored one after another in
    index order, so of several rows with one slot the last one stays (the
    GPU kernel leaves that case unspecified; cp_local_slot never gives two
    positions one slot).
    """
    out = np.array(cache_bits, copy=True)
    num_blocks, block_size = out.shape[0], out.shape[1]
    rows_bits = np.asarray(rows_bits)
    for i, s in enumerate(np.asarray(slots).reshape(-1)):
        s = int(s)
        if s < 0 or s >= num_blocks * block_size:
            continue
        out[s // block_size, s % block_size, :] = rows_bits[i]
    return out

