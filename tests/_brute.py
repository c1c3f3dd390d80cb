"""Pure-Python brute force used to pin the oracle on tiny inputs.

Written independently of ``oracle/``: scalar loops, math.exp / math.fsum,
the raw e4m3fn bit layout decoded with integer arithmetic, and the page
lookup done token by token.
"""

from __future__ import annotations

import math


def bf16_bits_to_float(bits: int) -> float:
    import struct

    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def brute_attention_row(q, keys, values, scale, key_bias=None):
    """softmax(scale * q.k_j + bias_j) weighted sum of values; returns (out list, lse).

    A key with bias -inf has weight e^-inf = 0 and is left out; with no key left
    the result is (zeros, -inf)."""
    if key_bias is not None:
        kept = [j for j in range(len(keys)) if key_bias[j] != -math.inf]
        keys = [keys[j] for j in kept]
        values = [values[j] for j in kept]
        key_bias = [key_bias[j] for j in kept]
    n = len(keys)
    if n == 0:
        return [0.0] * (len(values[0]) if values else len(q)), -math.inf
    logits = []
    for j in range(n):
        dot = math.fsum(qa * ka for qa, ka in zip(q, keys[j]))
        logits.append(scale * dot + (key_bias[j] if key_bias is not None else 0.0))
    m = max(logits)
    tot = math.fsum(math.exp(s - m) for s in logits)
    lse = m + math.log(tot)
    dv = len(values[0])
    out = [math.fsum(math.exp(logits[j] - lse) * values[j][d] for j in range(n)) for d in range(dv)]
    return out, lse


def brute_paged(q, cache, table, lens, *, Hkv, P, D, scale, window=0, dec=float,
                k_scale=1.0, v_scale=1.0, causal=False):
    """Paged attention by brute force over nested Python lists / numpy arrays.

    q[b][t][h][d]; cache[page][kvh][slot][0..2D); table[b][col]; dec decodes
    one stored element.  Returns dict (b, t, h) -> (out, lse).
    """
    res = {}
    B = len(q)
    for b in range(B):
        sq = len(q[b])
        Hq = len(q[b][0])
        G = Hq // Hkv
        L = int(lens[b])
        start = 0
        if window > 0 and not causal:
            # smallest page-aligned start that keeps the last window+sq-1 tokens
            first_needed = L - (window + sq - 1)
            while start + P <= first_needed:
                start += P
        for t in range(sq):
            for h in range(Hq):
                kvh = h // G
                keys, vals = [], []
                for j in range(start, L):
                    if causal:
                        pos = L - sq + t  # the token's own position
                        if j > pos or (window > 0 and pos - j >= window):
                            continue
                    page = int(table[b][j // P])
                    row = cache[page][kvh][j % P]
                    keys.append([dec(row[d]) * k_scale for d in range(D)])
                    vals.append([dec(row[D + d]) * v_scale for d in range(D)])
                qrow = [dec(x) for x in q[b][t][h]]
                res[(b, t, h)] = brute_attention_row(qrow, keys, vals, scale)
    return res
