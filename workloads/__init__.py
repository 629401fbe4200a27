"""Seeded synthetic inputs for paged MLA decode, shared by the oracle and the GPU path.

This module only *builds inputs*: bf16 query and latent-KV values, lengths,
rank shards, paged pools with block tables, and the position lists fed to the
slot mapping.  It holds none of the attention, merge or slot arithmetic.

Shapes follow the pages: per-head 576-wide absorbed queries (512 latent + 64
rope) against 576-wide latent KV rows (vLLM PR #54012 digest, key source
snippets, the native-DCP forward test: query [tokens, heads, 576], kv cache
[blocks, block_size, 576], out [tokens, heads, 512], lse [tokens, heads]).

Layout conventions (all little-endian numpy, values are bf16 bit patterns):
  q_bits     [B, Q, H, 576] uint16
  shard[r][b]  [n_{b,r}, 576] uint16   rank r's rows of request b, in local order
  pool[r]    [P, block_size, 576] uint16   rank r's paged cache
  block_table [B, max_blocks] int32     shared by every rank
Under decode context parallelism with interleave 1 the global position p of a
request lives on rank p % W as that rank's local row p // W (vLLM PR #52188
digest, key source snippets, cp_local_slot: positions are dealt out to ranks
round-robin in interleave-sized segments).  Every shard is generated directly
from its own seeded stream, and the contiguous global view is the interleave of
the shards.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

D_QK = 576
D_V = 512
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)

_THREADS = 8


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


BF16_NAN = np.uint16(0x7FC0)


def _normal_bits(seed_key: Sequence[int], shape) -> np.ndarray:
    rng = np.random.default_rng(list(seed_key))
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


# the 127 non-negative finite values of the 8-bit E4M3 format (codes 0..126)
_E4M3_POS = np.array([(m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
                      for e in range(16) for m in range(8)][:127])


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round float values to 8-bit E4M3 codes: nearest value, ties to the even
    code, magnitudes past 448 saturate to 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a), 1, 126)
    lo = hi - 1
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return (pick | np.where(x < 0, 0x80, 0)).astype(np.uint8)


def _normal_kv(spec, seed_key: Sequence[int], shape) -> np.ndarray:
    """N(0,1) latent rows: bf16 bits, or E4M3 codes of value / kv_scale."""
    if spec.kv_dtype == "fp8":
        rng = np.random.default_rng(list(seed_key))
        return e4m3_codes(rng.standard_normal(shape, dtype=np.float32) / spec.kv_scale)
    return _normal_bits(seed_key, shape)


@dataclass
class Spec:
    """A synthetic workload.

    tot: global KV length of each request.  For causal multi-token queries it
    includes the request's own q_len new tokens (the last query row sees all
    of it); for a non-causal draft block every row sees the whole context.
    """
    name: str
    B: int
    H: int
    Q: int
    causal: bool
    seed: int
    lengths: object  # ("uniform", lo, hi) or explicit list of global lengths
    W: int = 1
    ranks: Sequence[int] = (0,)
    interleave: int = 1   # ranks hold segments of this many consecutive positions
    q_lens: Optional[Sequence[int]] = None  # per-request query lengths (varlen); Q is then their maximum
    kv_dtype: str = "bf16"  # "bf16" or "fp8" (8-bit E4M3 codes of value / kv_scale)
    kv_scale: float = 1.0
    block_size: int = 64
    scale: float = DEFAULT_SCALE
    lse_base: str = "e"
    pool_factor: float = 1.5
    pool_blocks: Optional[int] = None
    fill: str = "normal"  # "normal" or "nan": spare blocks and block tails
    q_mult: float = 1.0   # scales q before bf16 rounding ("peaky" variants)
    q_zero: bool = False
    global_is_null: bool = False  # causal W=1: pass no global lengths


@dataclass
class Workload:
    spec: Spec
    tot: np.ndarray                     # [B] int64 global lengths
    q_bits: np.ndarray                  # [B, Q, H, 576] uint16
    seq_lens: Dict[int, np.ndarray]     # rank -> [B] int32 local lengths
    shards: Dict[int, List[np.ndarray]]  # rank -> per request [n, 576] uint16
    block_table: np.ndarray             # [B, max_blocks] int32
    pools: Dict[int, np.ndarray]        # rank -> [P, bs, 576] uint16
    slot_inputs: Optional[dict] = None
    q_tok: Optional[np.ndarray] = None  # varlen: [T, H, 576] uint16, requests' tokens packed
    query_start_loc: Optional[np.ndarray] = None  # varlen: [B+1] int32

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def global_rows(self, b: int, positions: np.ndarray) -> np.ndarray:
        """bf16 rows of request b at the given global positions (contiguous global view)."""
        W, I = self.spec.W, self.spec.interleave
        positions = np.asarray(positions, dtype=np.int64)
        out = np.empty((positions.size, D_QK), dtype=np.uint8 if self.spec.kv_dtype == "fp8" else np.uint16)
        owner = (positions // I) % W
        local = (positions // (I * W)) * I + positions % I
        for r in np.unique(owner) if positions.size else []:
            sel = owner == r
            if int(r) not in self.shards:
                raise KeyError(f"rank {int(r)} shard of request {b} was not generated")
            out[sel] = self.shards[int(r)][b][local[sel]]
        return out

    def global_kv(self, b: int) -> np.ndarray:
        """Whole contiguous global KV of request b (every rank's shard interleaved)."""
        W, I = self.spec.W, self.spec.interleave
        L = int(self.tot[b])
        g = np.empty((L, D_QK), dtype=np.uint8 if self.spec.kv_dtype == "fp8" else np.uint16)
        for r in range(W):
            g[_owned(L, W, r, I)] = self.shards[r][b]
        return g


def _owned(L: int, W: int, r: int, I: int) -> np.ndarray:
    """The global positions 0..L-1 that rank r holds, in order: positions go
    to the ranks in segments of I, segment k to rank k mod W."""
    p = np.arange(int(L), dtype=np.int64)
    return p[(p // I) % W == r]


def _lengths(spec: Spec) -> np.ndarray:
    if isinstance(spec.lengths, tuple) and spec.lengths and spec.lengths[0] == "uniform":
        _, lo, hi = spec.lengths
        rng = np.random.default_rng([spec.seed, 9999])
        return rng.integers(lo, hi, size=spec.B, endpoint=True).astype(np.int64)
    arr = np.asarray(spec.lengths, dtype=np.int64)
    assert arr.shape == (spec.B,)
    return arr


def _fill_rows(spec: Spec, r: int, n_rows: int) -> np.ndarray:
    if spec.fill == "nan":
        if spec.kv_dtype == "fp8":
            return np.full((n_rows, D_QK), 0x7F, dtype=np.uint8)
        return np.full((n_rows, D_QK), BF16_NAN, dtype=np.uint16)
    # a fixed random pattern, tiled: N(0,1)-distributed filler for unused rows
    pat = _normal_kv(spec, [spec.seed, 7777, r], (min(n_rows, 4096), D_QK))
    reps = -(-n_rows // pat.shape[0])
    return np.ascontiguousarray(np.tile(pat, (reps, 1))[:n_rows])


def build(spec: Spec, ranks: Optional[Sequence[int]] = None) -> Workload:
    ranks = tuple(spec.ranks if ranks is None else ranks)
    B, H, Q, W, bs = spec.B, spec.H, spec.Q, spec.W, spec.block_size
    tot = _lengths(spec)

    # query (varlen: request b's q_lens[b] tokens, packed)
    q_tok = qsl = None
    if spec.q_lens is not None:
        ql = [int(x) for x in spec.q_lens]
        assert len(ql) == B and max(ql) == Q, "Q must be the largest per-request query length"
        qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)

        def mkq_var(b):
            rng = np.random.default_rng([spec.seed, b, 1])
            return bf16_bits(rng.standard_normal((ql[b], H, D_QK), dtype=np.float32) * np.float32(spec.q_mult))
        q_tok = np.concatenate([mkq_var(b) for b in range(B)]) if qsl[-1] else np.zeros((0, H, D_QK), np.uint16)
    if spec.q_zero:
        q_bits = np.zeros((B, Q, H, D_QK), dtype=np.uint16)
    else:
        def mkq(b):
            rng = np.random.default_rng([spec.seed, b, 1])
            return bf16_bits(rng.standard_normal((Q, H, D_QK), dtype=np.float32) * np.float32(spec.q_mult))
        with ThreadPoolExecutor(_THREADS) as ex:
            q_bits = np.stack(list(ex.map(mkq, range(B))))

    # rank shards: rank r holds the positions of the segments dealt to it
    # (with interleave 1: r, r+W, r+2W, ...) of each request, in order
    I = spec.interleave
    shards: Dict[int, List[np.ndarray]] = {}
    seq_lens: Dict[int, np.ndarray] = {}
    for r in ranks:
        counts = [len(_owned(int(tot[b]), W, r, I)) for b in range(B)]
        with ThreadPoolExecutor(_THREADS) as ex:
            shards[r] = list(ex.map(lambda b: _normal_kv(spec, [spec.seed, b, r, 0], (counts[b], D_QK)), range(B)))
        seq_lens[r] = np.asarray(counts, dtype=np.int32)

    # one block table shared by all ranks; sized for rank 0's (largest) shard
    need = [max(1, -(-len(_owned(int(tot[b]), W, 0, I)) // bs)) for b in range(B)]
    used = int(sum(need))
    P = spec.pool_blocks if spec.pool_blocks is not None else max(used + 1, int(math.ceil(spec.pool_factor * used)))
    assert P >= used
    rng = np.random.default_rng([spec.seed, 4242])
    perm = rng.permutation(P).astype(np.int32)
    max_blocks = max(need)
    spare = perm[used:] if P > used else perm[:1]
    bt = np.empty((B, max_blocks), dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :need[b]] = perm[off:off + need[b]]
        if need[b] < max_blocks:
            bt[b, need[b]:] = spare[np.arange(max_blocks - need[b]) % len(spare)]
        off += need[b]

    pools: Dict[int, np.ndarray] = {}
    for r in ranks:
        pool = _fill_rows(spec, r, P * bs).reshape(P, bs, D_QK)
        for b in range(B):
            rows = shards[r][b]
            n = rows.shape[0]
            nb = -(-n // bs)
            if nb == 0:
                continue
            full = n // bs
            if full:
                pool[bt[b, :full]] = rows[:full * bs].reshape(full, bs, D_QK)
            if n % bs:
                pool[bt[b, full], :n % bs] = rows[full * bs:]
        pools[r] = pool

    return Workload(spec=spec, tot=tot, q_bits=q_bits, seq_lens=seq_lens, shards=shards,
                    block_table=bt, pools=pools, q_tok=q_tok, query_start_loc=qsl)


def unsharded(wl: Workload) -> Workload:
    """The same global KV held by a single rank (W = 1), with its own paged pool."""
    s = wl.spec
    assert set(wl.shards) == set(range(s.W)), "every rank's shard is needed"
    g = [wl.global_kv(b) for b in range(s.B)]
    bs = s.block_size
    need = [max(1, -(-int(wl.tot[b]) // bs)) for b in range(s.B)]
    used = int(sum(need))
    P = max(used + 1, int(math.ceil(s.pool_factor * used)))
    rng = np.random.default_rng([s.seed, 4343])
    perm = rng.permutation(P).astype(np.int32)
    max_blocks = max(need)
    bt = np.empty((s.B, max_blocks), dtype=np.int32)
    spare = perm[used:]
    off = 0
    for b in range(s.B):
        bt[b, :need[b]] = perm[off:off + need[b]]
        if need[b] < max_blocks:
            bt[b, need[b]:] = spare[np.arange(max_blocks - need[b]) % len(spare)]
        off += need[b]
    pool = _fill_rows(s, 0, P * bs).reshape(P, bs, D_QK)
    for b in range(s.B):
        rows = g[b]
        n = rows.shape[0]
        full = n // bs
        if full:
            pool[bt[b, :full]] = rows[:full * bs].reshape(full, bs, D_QK)
        if n % bs:
            pool[bt[b, full], :n % bs] = rows[full * bs:]
    spec1 = Spec(**{**s.__dict__, "W": 1, "ranks": (0,)})
    return Workload(spec=spec1, tot=wl.tot.copy(), q_bits=wl.q_bits, seq_lens={0: wl.tot.astype(np.int32)},
                    shards={0: g}, block_table=bt, pools={0: pool})


def draft_slot_inputs(wl: Workload, n_draft: int = 16) -> dict:
    """Positions for the KV writes of a draft step under DCP.

    Per request: a context window of n_draft positions whose last rej_b entries
    are a rejected suffix (they must map to the pad slot and are excluded via
    num_valid), and the n_draft positions of the new draft block itself
    (vLLM PR #52188 digest, implementation breakdown: the DFlash input
    preparation applies the rank-local slot mapping to context and query
    slots; its test covers a rejected context suffix at cp_rank=1, cp_size=2).
    """
    s = wl.spec
    rng = np.random.default_rng([s.seed, 5151])
    rej = rng.integers(0, n_draft - 1, size=s.B, endpoint=True).astype(np.int32)
    L = wl.tot
    ctx_start = L - n_draft - (n_draft - rej)
    ctx = ctx_start[:, None] + np.arange(n_draft)[None, :]
    qry = (L - n_draft)[:, None] + np.arange(n_draft)[None, :]
    return {
        "rejected": rej,
        "ctx_positions": ctx.astype(np.int64),
        "ctx_num_valid": (n_draft - rej).astype(np.int32),
        "query_positions": qry.astype(np.int64),
    }


# --- the five workloads the measurements use -------------------------------

def config(n: int, **overrides) -> Spec:
    """Workload n in 1..6 (sizes of the single- and multi-token MLA decode cases)."""
    base = {
        1: dict(name="tiny_b2_h16_q1", B=2, H=16, Q=1, causal=True, seed=1001, lengths=[37, 100],
                pool_blocks=4, global_is_null=True),
        2: dict(name="decode_b64_h16_q1_len1k-8k", B=64, H=16, Q=1, causal=True, seed=1002,
                lengths=("uniform", 1024, 8192), global_is_null=True),
        3: dict(name="spec_b32_h128_q4_causal_len4k-32k", B=32, H=128, Q=4, causal=True, seed=1003,
                lengths=("uniform", 4096, 32768), global_is_null=True),
        4: dict(name="dcp8_b16_h128_q4_causal_len32k-128k", B=16, H=128, Q=4, causal=True, seed=1004,
                lengths=("uniform", 32768, 131072), W=8, ranks=tuple(range(8))),
        5: dict(name="dcp2r1_b16_h128_q16_noncausal_len64k-256k", B=16, H=128, Q=16, causal=False, seed=1005,
                lengths=("uniform", 65536, 262144), W=2, ranks=(1,)),
        # beyond the five: speculative decode with 16 heads (a tensor-parallel
        # shard of the heads) and q_len 4, 64 rows per request
        6: dict(name="spec_b64_h16_q4_causal_len1k-8k", B=64, H=16, Q=4, causal=True, seed=1006,
                lengths=("uniform", 1024, 8192), global_is_null=True),
    }[n]
    base.update(overrides)
    return Spec(**base)
