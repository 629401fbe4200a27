"""Independent pure-Python brute force used to pin the oracle on tiny inputs.

Scalar loops over every global position with an explicit visibility
predicate, math.exp without max-subtraction (inputs are tiny), math.fsum.
Shares nothing with oracle/ beyond reading the same generated inputs.
"""
import math


def bf16_to_float(bits: int) -> float:
    import struct
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def is_visible(p, j, q_len, tot, seq_len, W, r, causal, interleave=1):
    """Global position p is visible to query row j of the request on rank r."""
    I = interleave
    if (p // I) % W != r:    # rank r holds the segments of I positions dealt to it
        return False
    # ... and only its first seq_len positions: p is its local row
    # (whole rounds of W segments before p) * I + offset inside the segment
    if (p // (I * W)) * I + p % I >= seq_len:
        return False
    if causal:
        query_pos = tot - q_len + j   # the row's own global position
        return p <= query_pos
    return True


def attend_row(q, kv_global, j, q_len, tot, seq_len, W, r, causal, scale, base="e", interleave=1):
    """q: list of 576 floats; kv_global: list of rows (list of 576 floats) indexed by global position."""
    weights = []
    vals = []
    for p in range(len(kv_global)):
        if not is_visible(p, j, q_len, tot, seq_len, W, r, causal, interleave):
            continue
        s = scale * math.fsum(q[d] * kv_global[p][d] for d in range(576))
        weights.append(math.exp(s))
        vals.append(kv_global[p][:512])
    if not weights:
        return [0.0] * 512, -math.inf
    z = math.fsum(weights)
    out = [math.fsum(w * v[c] for w, v in zip(weights, vals)) / z for c in range(512)]
    lse = math.log(z)
    if base == "2":
        lse = lse / math.log(2.0)
    return out, lse
