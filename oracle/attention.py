"""fp64 softmax attention over paged K/V, Split-KV partials and DASH segments (oracle).

Test infrastructure only: a plain statement of the definitions, with no
blocking, online softmax or fusion.

Conventions taken from the pages:
  * The query block of a request sees every visible key (dense, non-causal
    mask): vllm.v1.attention.backends.flashinfer_ts, module docstring.
  * K and V are the two halves of each cache row ``[pages, Hkv, P, 2*D]``:
    K = ``[..., :D]``, V = ``[..., D:]`` (same page, ``_kv_views``).
  * The pre-softmax scale is ``scale * k_scale`` and V is multiplied by
    ``v_scale`` (same page, ``FlashInferTSImpl.forward``: bmm1_scale /
    bmm2_scale), with q_scale = 1 because the query stays bf16/fp16.
  * LSE is a natural logarithm, one value per (row, head)
    (vllm.v1.attention.ops.dash_attention, ``flash_dash_attention``:
    ``lse_base="ln"``, layout rows x heads).
  * Query head h reads kv head h // (Hq / Hkv) (consecutive query heads
    share a kv head; the pages give only the head counts, this is the
    reading taken).
  * A row with no visible key has O = 0 and LSE = -inf.
"""

from __future__ import annotations

import numpy as np

from .formats import decode
from .paging import split_page_ranges, window_start_page


# ----------------------------------------------------------------------------
# The definition
# ----------------------------------------------------------------------------
def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, key_bias=None):
    """O, LSE of softmax(scale * q K^T + key_bias) V for q [R, D], K [n, D], V [n, Dv].

    LSE_r = ln sum_j exp(s_rj); O_r = sum_j exp(s_rj - LSE_r) V_j.  With no
    keys, O = 0 and LSE = -inf.  A key whose bias is -inf has weight 0; a row
    whose every logit is -inf is treated like a row with no keys (the softmax
    of such a row is NaN, which the DASH combine turns into zero weights).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    R = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((R, V.shape[1])), np.full(R, -np.inf)
    s = scale * (q @ K.T)
    if key_bias is not None:
        s = s + np.asarray(key_bias, dtype=np.float64)[None, :]
    m = s.max(axis=1)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    tot = np.exp(s - m_safe[:, None]).sum(axis=1)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
    w = np.where(empty[:, None], 0.0, np.exp(s - np.where(empty, 0.0, lse)[:, None]))
    return w @ V, lse


def attention_weights(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """The softmax weights softmax(scale * q K^T) of ``softmax_attention`` (rows sum to 1)."""
    s = scale * (np.asarray(q, np.float64) @ np.asarray(K, np.float64).T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------
# Paged K/V
# ----------------------------------------------------------------------------
def kv_halves(cache: np.ndarray, D: int):
    """K and V views of a ``[pages, Hkv, P, 2*D]`` cache (flashinfer_ts ``_kv_views``)."""
    return cache[..., :D], cache[..., D:]


def _gather_request(k_pages, v_pages, kv_dtype, table_row, kvh, start, L, P, k_scale, v_scale):
    j = np.arange(start, L, dtype=np.int64)
    pages = np.asarray(table_row, dtype=np.int64)[j // P]
    off = j % P
    K = decode(k_pages[pages, kvh, off, :], kv_dtype) * k_scale
    V = decode(v_pages[pages, kvh, off, :], kv_dtype) * v_scale
    return K, V


def paged_attention(
    q,
    q_dtype,
    k_pages,
    v_pages,
    kv_dtype,
    block_table,
    seq_lens,
    *,
    scale: float,
    window: int = 0,
    k_scale: float = 1.0,
    v_scale: float = 1.0,
    requests=None,
    kv_heads=None,
    token_range=None,
    causal: bool = False,
    q_scale: float = 1.0,
):
    """Attention of a uniform query block over a paged cache.

    q: stored [B, sq, Hq, D]; k_pages, v_pages: stored [pool, Hkv, P, D]
    (views of one [pool, Hkv, P, 2D] cache or two compact planes);
    block_table [B, W] int; seq_lens [B] (each L includes the query block).
    Request b sees keys [start, L) with start = window_start_page * P
    (the page-aligned window suffix; start = 0 without a window), key j
    living at slot j % P of page block_table[b, j // P].
    ``token_range(b, start, L) -> (lo, hi)`` optionally narrows the keys
    (used for Split-KV partials).  Returns O [B, sq, Hq, D] and LSE
    [B, sq, Hq] in fp64; entries of requests / kv heads not asked for are NaN.

    causal (flashinfer_ts ``_get_plan``: ``mask_type="causal"`` with
    ``window_left = window - 1``; ``build`` skips the page restriction then):
    the block's tokens sit at positions L - sq + t, token t sees keys
    j <= L - sq + t and, with a window, j >= L - sq + t - (window - 1): an
    exact per-token window of ``window`` keys ending at the token itself.

    q_scale: the real query is q_scale times the stored one (an fp8 query
    arrives quantized; flashinfer_ts ``forward`` folds its scale into
    bmm1_scale together with k_scale).
    """
    qv = decode(q, q_dtype) * q_scale
    B, sq, Hq, D = qv.shape
    pool, Hkv, P, Dk = k_pages.shape
    if Dk != D or Hq % Hkv:
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    O = np.full((B, sq, Hq, v_pages.shape[-1]), np.nan)
    LSE = np.full((B, sq, Hq), np.nan)
    reqs = range(B) if requests is None else requests
    heads = range(Hkv) if kv_heads is None else kv_heads
    for b in reqs:
        L = int(seq_lens[b])
        start = 0 if causal else window_start_page(L, window, sq, P) * P
        lo, hi = (start, L) if token_range is None else token_range(b, start, L)
        for kvh in heads:
            K, V = _gather_request(k_pages, v_pages, kv_dtype, block_table[b], kvh, lo, hi, P,
                                   k_scale, v_scale)
            hs = slice(kvh * G, (kvh + 1) * G)
            if not causal:
                rows = qv[b, :, hs, :].reshape(sq * G, D)
                o, lse = softmax_attention(rows, K, V, scale)
                O[b, :, hs, :] = o.reshape(sq, G, -1)
                LSE[b, :, hs] = lse.reshape(sq, G)
                continue
            j = np.arange(lo, hi)
            for t in range(sq):
                pos = L - sq + t
                keep = j <= pos
                if window > 0:
                    keep &= j >= pos - (window - 1)
                o, lse = softmax_attention(qv[b, t, hs, :], K[keep], V[keep], scale)
                O[b, t, hs, :] = o
                LSE[b, t, hs] = lse
    return O, LSE


# ----------------------------------------------------------------------------
# Split-KV
# ----------------------------------------------------------------------------
def split_partials(q, q_dtype, k_pages, v_pages, kv_dtype, block_table, seq_lens, *,
                   scale, num_splits, window=0, k_scale=1.0, v_scale=1.0,
                   requests=None, kv_heads=None):
    """Per-split (O_s, LSE_s): attention restricted to split s's keys.

    Visible pages [sp, ceil(L/P)) are cut by ``split_page_ranges``; split s
    keeps the visible keys on its pages.  An empty split gives (0, -inf).
    Returns part_o [S, B, sq, Hq, D], part_lse [S, B, sq, Hq].
    """
    P = k_pages.shape[2]
    parts_o, parts_l = [], []
    for s in range(num_splits):
        def tr(b, start, L, s=s):
            sp = start // P
            n_pages = -(-L // P) - sp if L > 0 else 0
            first, count = split_page_ranges(max(n_pages, 0), num_splits)[s]
            lo = max(start, (sp + first) * P)
            hi = min(L, (sp + first + count) * P)
            return (lo, max(lo, hi))
        o, lse = paged_attention(q, q_dtype, k_pages, v_pages, kv_dtype, block_table, seq_lens,
                                 scale=scale, window=window, k_scale=k_scale, v_scale=v_scale,
                                 requests=requests, kv_heads=kv_heads, token_range=tr)
        parts_o.append(o)
        parts_l.append(lse)
    return np.stack(parts_o), np.stack(parts_l)


def _weighted_combine(part_o, logits, live):
    """sum_g w_g O_g with w = softmax over the live g of ``logits``; no live g -> w = 0.

    Mirrors the combine of vllm.v1.attention.ops.dash_attention
    ``flash_dash_attention``: dead entries get logit -inf and O = 0, and the
    NaN softmax of an all-dead set becomes 0 (``nan_to_num``).  The combined
    LSE is logsumexp over the live logits (-inf when none is live).
    part_o [G, ..., D], logits [G, ...], live [G, ...] (bool).
    """
    logits = np.where(live, np.asarray(logits, np.float64), -np.inf)
    # a live partial with logit -inf (a -inf bias) gets weight 0 like a dead one; if no
    # finite logit is left the page's softmax is NaN everywhere and nan_to_num makes it 0
    live = live & (logits > -np.inf)
    m = logits.max(axis=0)
    any_live = live.any(axis=0)
    m_safe = np.where(any_live, m, 0.0)
    e = np.where(live, np.exp(logits - m_safe[None]), 0.0)
    tot = e.sum(axis=0)
    w = np.where(any_live[None], e / np.where(any_live, tot, 1.0)[None], 0.0)
    o = np.where(live[..., None], np.asarray(part_o, np.float64), 0.0)
    out = (w[..., None] * o).sum(axis=0)
    lse = np.where(any_live, m_safe + np.log(np.where(any_live, tot, 1.0)), -np.inf)
    return out, lse


def combine_splits(part_o, part_lse):
    """Merge Split-KV partials: LSE = ln sum_live e^{LSE_s}; O = sum_live e^{LSE_s - LSE} O_s.

    The segment combine with zero bias, live meaning LSE_s > -inf.
    part_o [S, ..., D], part_lse [S, ...].
    """
    part_lse = np.asarray(part_lse, np.float64)
    return _weighted_combine(part_o, part_lse, part_lse > -np.inf)


# ----------------------------------------------------------------------------
# DASH gathered segments
# ----------------------------------------------------------------------------
def segment_base(n: int, g: int, topk: int, bs: int, local: int) -> int:
    """First token row of segment g of query n in the contiguous segment buffer.

    Per query the buffer holds topk remote segments of bs rows then one local
    segment of ``local`` rows (dash_attention ``flash_dash_attention``
    docstring [N*(topk*bs+local), Hkv, D]; the mask it builds lists the
    remote segments first and the local one last).
    """
    per = topk * bs + local
    return n * per + (g * bs if g < topk else topk * bs)


def segment_partials(q, k, v, used, *, topk, bs, local, scale, q_dtype="bf16", kv_dtype="bf16",
                     queries=None):
    """(O_g, LSE_g) of each query over the first used[n, g] rows of each segment.

    q [N, Hq, D]; k, v [T, Hkv, D] stored; used [N, topk+1].  One query token
    per segment, non-causal, scale as given (the page uses D**-0.5).
    Returns O [N, G, Hq, D], LSE [N, G, Hq] (NaN for queries not asked for).
    """
    qv = decode(q, q_dtype)
    N, Hq, D = qv.shape
    Hkv = k.shape[1]
    G = topk + 1
    grp = Hq // Hkv
    O = np.full((N, G, Hq, v.shape[-1]), np.nan)
    LSE = np.full((N, G, Hq), np.nan)
    for n in (range(N) if queries is None else queries):
        for g in range(G):
            base = segment_base(n, g, topk, bs, local)
            u = int(used[n, g])
            for kvh in range(Hkv):
                K = decode(k[base:base + u, kvh, :], kv_dtype)
                V = decode(v[base:base + u, kvh, :], kv_dtype)
                hs = slice(kvh * grp, (kvh + 1) * grp)
                o, lse = softmax_attention(qv[n, hs, :], K, V, scale)
                O[n, g, hs, :] = o
                LSE[n, g, hs] = lse
    return O, LSE


def combine_segments(part_o, part_lse, used, bias):
    """LSE + bias combine of segment partials (dash_attention ``flash_dash_attention``).

    live = used > 0; the prior is the per-segment bias with 0 for the local
    (last) segment; weights are the softmax over segments of LSE + prior,
    dead segments excluded, all-dead giving zero weights; the output is the
    weighted sum of the live partial outputs.  Also returns the combined
    LSE = logsumexp over live segments of (LSE_g + prior_g), -inf if none
    (an extension: the page returns only the output).
    part_o [N, G, Hq, D], part_lse [N, G, Hq], used [N, G], bias [N, G-1].
    """
    part_o = np.asarray(part_o, np.float64)
    part_lse = np.asarray(part_lse, np.float64)
    used = np.asarray(used)
    bias = np.asarray(bias, np.float64)
    N, G, Hq, D = part_o.shape
    prior = np.concatenate([bias, np.zeros((N, 1))], axis=1)  # [N, G]
    logits = part_lse + prior[:, :, None]  # [N, G, Hq]
    live = np.broadcast_to((used > 0)[:, :, None], logits.shape)
    out, lse = _weighted_combine(np.moveaxis(part_o, 1, 0), np.moveaxis(logits, 1, 0),
                                 np.moveaxis(live, 1, 0))
    return out, lse


def segment_attention(q, k, v, used, bias, *, topk, bs, local, scale, q_dtype="bf16",
                      kv_dtype="bf16", queries=None):
    """Two-stage DASH result: per-segment attention, then the LSE + bias combine."""
    O, LSE = segment_partials(q, k, v, used, topk=topk, bs=bs, local=local, scale=scale,
                              q_dtype=q_dtype, kv_dtype=kv_dtype, queries=queries)
    if queries is not None:
        sel = list(queries)
        out, lse = combine_segments(O[sel], LSE[sel], np.asarray(used)[sel], np.asarray(bias)[sel])
        full_o = np.full((O.shape[0],) + out.shape[1:], np.nan)
        full_l = np.full((O.shape[0],) + lse.shape[1:], np.nan)
        full_o[sel] = out
        full_l[sel] = lse
        return full_o, full_l
    return combine_segments(O, LSE, used, bias)


def segment_attention_union(q, k, v, used, bias, *, topk, bs, local, scale, q_dtype="bf16",
                            kv_dtype="bf16"):
    """Closed form of the two-stage DASH result: ONE softmax over the union of live prefixes.

    Key j of segment g gets logit scale * q.k_j + b_g (b = bias, 0 for the
    local segment).  Since sum_g w_g O_g = sum_g e^{b_g} sum_{j in g} e^{s_j} V_j
    / sum_g e^{LSE_g + b_g}, this equals ``segment_attention`` exactly.
    """
    qv = decode(q, q_dtype)
    N, Hq, D = qv.shape
    Hkv = k.shape[1]
    G = topk + 1
    grp = Hq // Hkv
    out = np.zeros((N, Hq, v.shape[-1]))
    lse_out = np.full((N, Hq), -np.inf)
    for n in range(N):
        rows, biases = [], []
        for g in range(G):
            base = segment_base(n, g, topk, bs, local)
            u = int(used[n, g])
            rows.append(np.arange(base, base + u))
            biases.append(np.full(u, float(bias[n, g]) if g < topk else 0.0))
        idx = np.concatenate(rows).astype(np.int64)
        kb = np.concatenate(biases)
        for kvh in range(Hkv):
            K = decode(k[idx, kvh, :], kv_dtype)
            V = decode(v[idx, kvh, :], kv_dtype)
            hs = slice(kvh * grp, (kvh + 1) * grp)
            o, lse = softmax_attention(qv[n, hs, :], K, V, scale, key_bias=kb)
            out[n, hs, :] = o
            lse_out[n, hs] = lse
    return out, lse_out
