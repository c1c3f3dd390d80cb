"""Oracle: a plain, slow, fp64 CPU statement of what the paged-attention path computes.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
bench's CPU-baseline leg may import this package.  The GPU path never calls
it, never links it, and shares no code, tables or constants with it.

Sources (vLLM API documentation pages):
  * vllm.v1.attention.backends.flashinfer_ts -- uniform query-block paged
    decode over the K/V-halves page, ``_restrict_to_window``, ``forward``
    scale folding, ``_kv_kernel_dtype`` (fp8 cache bytes read as e4m3).
  * vllm.v1.attention.ops.dash_attention -- ``flash_dash_attention``:
    gathered segments, natural-log LSE, LSE + bias combine.
  * vllm.v1.attention.backends.fa_utils -- ``FlashAttentionCuTeDSLCompileSpec``
    (``return_softmax_lse``, ``num_splits``: Split-KV).

Every attention result here is the plain softmax definition evaluated in
fp64 over the visible keys; paging, window restriction, splitting and
combining only decide WHICH keys are visible or how exact partial results
are merged.

Pinning status of each function (the pins live in tests/test_oracle_*.py):
  formats.bf16_to_f64, formats.e4m3fn_to_f64 ..... pinned (format definition
      points, torch float8_e4m3fn on all 256 bytes)
  paging.window_start_page, restrict_to_window ... pinned (hand-worked page
      examples, covering-suffix property, brute force)
  paging.split_page_ranges ........................ pinned (brute force over
      every in-order cut of up to 12 pages into up to 5 chunks: the cut with
      the smallest largest chunk, filled front to back; partition invariants).
      The pages fix no boundary rule: that selection is a reading, and results
      downstream are rule-independent (split-then-combine == unsplit)
  attention.softmax_attention ..................... pinned (closed forms,
      brute force, torch SDPA in fp64, logaddexp)
  attention.paged_attention ....................... pinned (page permutation,
      GQA repeat, window suffix, strided vs compact planes, fp8 scale folding;
      causal mode: brute force, torch SDPA with a boolean mask in fp64, each
      token == dense decode of the truncated sequence)
  attention.split_partials / combine_splits ....... pinned (identity with
      unsplit attention)
  attention.segment_partials / combine_segments ... pinned (union closed form,
      dead-segment invariance, plain attention when every segment is full)
  cache_write.e4m3fn_encode ....................... pinned (torch float8_e4m3fn
      cast on finite in-range values, round trip of every finite code, hand
      ties and saturation points)
  cache_write.write_kv_cache ...................... pinned (write then paged
      attention == plain attention over the written rows, padding and
      out-of-pool slots write nothing, order independence); the readings it
      follows where the page is silent are listed in its module docstring
"""

from .formats import bf16_to_f64, fp16_to_f64, e4m3fn_to_f64, e4m3fn_value, E4M3FN_TABLE  # noqa: F401
from .paging import (  # noqa: F401
    window_start_page,
    window_table_width,
    restrict_to_window,
    split_page_ranges,
    visible_range,
)
from .attention import (  # noqa: F401
    softmax_attention,
    attention_weights,
    paged_attention,
    split_partials,
    combine_splits,
    segment_partials,
    combine_segments,
    segment_attention,
    segment_attention_union,
)
from .cache_write import convert_row, e4m3fn_encode, quantize_e4m3fn, write_kv_cache  # noqa: F401
