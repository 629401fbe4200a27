"""Helpers for GPU parity tests: upload generated inputs, call the C ABI
through the binding, compare with the oracle at the stated tolerances."""
import sys

import numpy as np
import torch

import decode_attention_11_amd as mla

OUT_MAX_ABS = 2e-2
OUT_MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def dev():
    return torch.device("cuda:0")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def u8_dev(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(dev())


def kv_dev(pool: np.ndarray) -> torch.Tensor:
    """A cache pool: bf16 bits (uint16) or E4M3 codes (uint8)."""
    return u8_dev(pool) if pool.dtype == np.uint8 else bf16_dev(pool)


def i32_dev(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).to(dev())


def i64_dev(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int64))).to(dev())


class Uploaded:
    """Device copies of one workload (query, block table, per-rank pools and lengths)."""

    def __init__(self, wl):
        self.wl = wl
        self.q = bf16_dev(wl.q_bits)
        self.bt = i32_dev(wl.block_table)
        self.tot = i32_dev(wl.tot)
        self.pools = {r: kv_dev(p) for r, p in wl.pools.items()}
        self.seq = {r: i32_dev(s) for r, s in wl.seq_lens.items()}

    def run(self, r, base="e", causal=None, global_null=None, **kw):
        s = self.wl.spec
        causal = s.causal if causal is None else causal
        gnull = s.global_is_null if global_null is None else global_null
        g = None if gnull else self.tot
        if s.kv_dtype == "fp8":
            kw.setdefault("kv_scale", s.kv_scale)
        return mla.mla_decode(self.q, self.pools[r], self.bt, self.seq[r], g, cp_world=s.W, cp_rank=r,
                              causal=causal, scale=s.scale, lse_base=base, cp_interleave=s.interleave, **kw)


def compare(out, lse, ro, rl, label="", rows=None):
    """out/lse: device results [B*Q, H, 512] / [B*Q, H]; ro/rl: oracle float64 arrays.
    rows: optional list of (flat_row, h) pairs to compare (sampled outputs)."""
    go = out.float().cpu().numpy()
    gl = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        idx = tuple(np.array(rows).T)
        go, gl, ro, rl = go[idx], gl[idx], ro[idx], rl[idx]
    assert np.all(np.isfinite(go)), f"{label}: non-finite output"
    empty = ~np.isfinite(rl)
    assert np.array_equal(empty, ~np.isfinite(gl)), f"{label}: empty-row pattern differs"
    if empty.any():
        assert np.all(gl[empty] == -np.inf), f"{label}: empty rows must have lse -inf"
        assert np.all(go[empty] == 0), f"{label}: empty rows must have out 0"
    err = np.abs(go - ro)
    lerr = np.abs(gl[~empty] - rl[~empty]) if (~empty).any() else np.zeros(1)
    msg = f"{label}: out max {err.max():.3e} mean {err.mean():.3e}, lse max {lerr.max():.3e}"
    say(msg)
    assert err.max() <= OUT_MAX_ABS, msg
    assert err.mean() <= OUT_MEAN_ABS, msg
    assert lerr.max() <= LSE_ABS, msg
    return err.max(), err.mean(), lerr.max()
