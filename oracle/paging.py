"""Integer side of the path: window restriction, visible keys, Split-KV ranges (oracle).

Test infrastructure only.  All results are Python ints / int64 arrays and are
compared bit-exactly with the GPU path.
"""

from __future__ import annotations

import numpy as np


def window_start_page(L: int, window: int, query_len: int, page_size: int) -> int:
    """First page a page-aligned sliding window can reach.

    Page vllm.v1.attention.backends.flashinfer_ts, module docstring
    "Sliding window" and ``_restrict_to_window``.  Every query token of the
    block sits at the end of its request, so the keys any of them can reach
    through a window of ``window`` keys begin ``window + query_len - 1`` keys
    before the end of the sequence.  The start page is that key index
    divided by the page size with the floor taken, never below page 0.
    ``window <= 0`` means no window (every key visible).
    """
    if window <= 0:
        return 0
    span = window + query_len - 1
    return max(0, (int(L) - span) // page_size)  # Python // floors negative values


def window_table_width(window: int, query_len: int, page_size: int, width: int) -> int:
    """Columns of the restricted block table.

    Page vllm.v1.attention.backends.flashinfer_ts, ``_window_pages``: with a
    window the table needs ceil((w + query_len - 1) / P) + 1 columns;
    without one the caller's table is used unchanged (``width``).
    """
    if window <= 0:
        return width
    span = window + query_len - 1
    return -(-span // page_size) + 1


def restrict_to_window(seq_lens, block_table, window: int, query_len: int, page_size: int):
    """Window-restricted (lengths, block table), as ``_restrict_to_window`` states it.

    lengths'  = L - start_page * P              (renumbered from the new first page)
    table'[j] = table[min(start_page + j, W - 1)] for j < window_table_width
    Without a window both are returned unchanged (as int64 / int32 copies).
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    table = np.asarray(block_table, dtype=np.int64)
    B, W = table.shape
    if window <= 0:
        return lens.copy(), table.astype(np.int32)
    width = window_table_width(window, query_len, page_size, W)
    out_lens = np.empty(B, dtype=np.int64)
    out_table = np.empty((B, width), dtype=np.int32)
    for b in range(B):
        sp = window_start_page(int(lens[b]), window, query_len, page_size)
        out_lens[b] = lens[b] - sp * page_size
        for j in range(width):
            out_table[b, j] = table[b, min(sp + j, W - 1)]
    return out_lens, out_table


def visible_range(L: int, window: int, query_len: int, page_size: int) -> tuple[int, int]:
    """Token interval [start, L) of the original sequence that every query token sees.

    Dense (non-causal) mask: every token of the query block sees the same keys
    (flashinfer_ts module docstring: mask_type="dense" makes the draft block
    non-causal, and the page-aligned window gives all query tokens one start).
    """
    sp = window_start_page(L, window, query_len, page_size)
    return sp * page_size, int(L)


def split_page_ranges(n_pages: int, num_splits: int) -> list[tuple[int, int]]:
    """Split-KV partition of ``n_pages`` visible pages into ``num_splits`` chunks.

    The pages name Split-KV and ``num_splits`` (vllm.v1.attention.backends.fa_utils,
    ``FlashAttentionCuTeDSLCompileSpec``) but fix no boundary rule.  Reading
    taken here: equal page-granular chunks of ceil(n_pages / S) pages, in
    order; trailing chunks may be empty.  Returns (first_page, page_count)
    relative to the first visible page.  Among all in-order cuts into
    num_splits chunks this is the one with the smallest largest chunk, filled
    front to back (the brute-force pin in the tests).  The combined result
    does not depend on the rule.
    """
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    per = -(-n_pages // num_splits) if n_pages > 0 else 0
    out = []
    for s in range(num_splits):
        first = min(s * per, n_pages)
        last = min((s + 1) * per, n_pages)
        out.append((first, last - first))
    return out
