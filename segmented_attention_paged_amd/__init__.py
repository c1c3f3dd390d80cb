"""MI355X (gfx950) paged-KV attention: uniform query block, GQA, page-aligned window,
Split-KV and DASH-style segment combine, behind a C ABI (include/paged_attn.h).

The HIP library ``libsapaged.so`` is built in-tree by
``python -m segmented_attention_paged_amd.build``; the functions below load it
on first use and raise if it is missing.
"""

from .api import (  # noqa: F401
    PagedAttnError,
    pa_last_error,
    pa_version,
    paged_attn_plan,
    paged_attn_resolve_splits,
    paged_attn_window_width,
    paged_attn_workspace_size,
    dtype_code,
    kv_desc,
    kv_halves,
    paged_attn_describe,
    paged_attn_describe_host,
    paged_attn_partial,
    paged_attn_run,
    paged_attn_run_causal,
    paged_attn_run_noalloc,
    paged_kv_write,
    plan,
    resolve_splits,
    segment_attn_combine,
    segment_attn_run,
    segment_attn_workspace_size,
    split_kv_combine,
    window_width,
    workspace_size,
    new_workspace,
)
from ._lib import LIB_PATH, load  # noqa: F401
