"""Latent values of any bf16 magnitude through both kernel families.

The latent row is both key and value (PR #54012 page, key source snippets:
the 576-wide cache row whose first 512 entries are the 512-wide output's
source).  Scaling every cache value by 2^s and every query value by 2^-s
(both exact in bf16) leaves the scores unchanged and scales the output by
exactly 2^s, so the output divided by 2^s must meet the usual bars against
the oracle on the scaled inputs, and the LSE must not move.  At 2^17 the
values pass fp16's largest finite value (65504) and at 2^-20 they sit below
its smallest normal (6.1e-5): the split-KV partials must keep them anyway.
"""
import numpy as np
import pytest

import oracle
import workloads as WL
from tests.gpu_util import Uploaded, compare, say

pytestmark = pytest.mark.gpu


def scaled_bits(bits, e):
    f = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    out = WL.bf16_bits(f * np.float32(2.0 ** e))
    assert np.array_equal((out.astype(np.uint32) << 16).view(np.float32), f * np.float32(2.0 ** e)), "not exact"
    return out


def scale_workload(wl, e):
    """The same workload with every cache value times 2^e and every query value times 2^-e."""
    wl.q_bits = scaled_bits(wl.q_bits, -e)
    for r in wl.shards:
        wl.shards[r] = [scaled_bits(x, e) for x in wl.shards[r]]
        wl.pools[r] = scaled_bits(wl.pools[r], e)
    return wl


CASES = [
    # name, H, Q, causal, lengths: 128-row kernel (multi-token, 128 heads) and 16-row kernel
    ("r128_h128_q4", 128, 4, True, [700, 3000, 129]),
    ("r128_h64_q16_draft", 64, 16, False, [2500, 333]),
    ("m16_h16_q1", 16, 1, True, [1500, 4000, 65]),
]


@pytest.mark.parametrize("e", [17, -20])
@pytest.mark.parametrize("name,H,Q,causal,lengths", CASES, ids=[c[0] for c in CASES])
def test_extreme_value_magnitudes_keep_the_bars(name, H, Q, causal, lengths, e):
    spec = WL.Spec(name=name, B=len(lengths), H=H, Q=Q, causal=causal, seed=3300 + H + Q, lengths=lengths)
    wl = scale_workload(WL.build(spec), e)
    say(f"{name}: cache x 2^{e}, query x 2^{-e}")
    up = Uploaded(wl)
    out, lse = up.run(0, "e")
    ro, rl = oracle.mla_decode(wl.q_bits, wl.global_rows, wl.seq_lens[0], wl.tot, 1, 0, causal, spec.scale)
    assert np.abs(ro).max() > 2.0 ** e * 0.5, "the scaled outputs must reach the scale being tested"
    o = out.float() * float(2.0 ** -e)
    compare(o, lse, ro * 2.0 ** -e, rl, f"{name} at 2^{e}")
