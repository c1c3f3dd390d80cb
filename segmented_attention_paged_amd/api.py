"""Torch-facing wrappers of the C ABI, with the same names as the C entry points.

These functions only marshal arguments: they take device pointers, shapes and
strides from torch tensors, allocate outputs / workspace with torch when the
caller does not pass them, pass the current torch stream, and raise
``PagedAttnError`` on a non-zero status.  No step of the attention runs here.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import PA_BF16, PA_F32, PA_FP16, PA_FP8_E4M3, PaKvDesc, check, load

_DT = {torch.bfloat16: PA_BF16, torch.float16: PA_FP16, torch.float32: PA_F32,
       torch.uint8: PA_FP8_E4M3}
if hasattr(torch, "float8_e4m3fn"):
    _DT[torch.float8_e4m3fn] = PA_FP8_E4M3
_TORCH = {PA_BF16: torch.bfloat16, PA_FP16: torch.float16, PA_F32: torch.float32}


def dtype_code(dt: torch.dtype) -> int:
    try:
        return _DT[dt]
    except KeyError:
        raise TypeError(f"unsupported dtype {dt}") from None


def _stream(dev: torch.device) -> ctypes.c_void_p:
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: Optional[torch.Tensor], name: str, shape=None, dtype=None, contiguous: bool = True):
    """Raise ValueError / TypeError unless t (skipped when None) has this shape, dtype and a
    dense row-major layout.  The kernels index these buffers from their shapes alone, so a
    smaller or strided tensor would be read or written out of bounds."""
    if t is None:
        return
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(dev: torch.device, **tensors):
    """Every given tensor must live on the GPU `dev` (a host pointer reaching a kernel faults)."""
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def kv_desc(k: torch.Tensor, v: torch.Tensor, *, k_scale: float = 1.0, v_scale: float = 1.0,
            num_pages: Optional[int] = None) -> PaKvDesc:
    """Descriptor of paged K/V views shaped [pages, Hkv, page_size, D] with any strides
    (head_dim contiguous), e.g. the two halves of a [pages, Hkv, P, 2*D] cache."""
    if k.shape != v.shape or k.dim() != 4:
        raise ValueError("k and v must both be [pages, Hkv, page_size, D]")
    if k.stride() != v.stride() or k.stride(-1) != 1:
        raise ValueError("k and v need equal strides and a contiguous head_dim")
    pages, hkv, P, _ = k.shape
    return PaKvDesc(k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1), k.stride(2), P, hkv,
                    int(num_pages if num_pages is not None else pages), dtype_code(k.dtype),
                    float(k_scale), float(v_scale))


def kv_halves(kv_cache: torch.Tensor, head_dim: int):
    """K and V views of a [pages, Hkv, page_size, 2*head_dim] cache (no copy)."""
    return kv_cache[..., :head_dim], kv_cache[..., head_dim:]


def resolve_splits(B, query_len, Hq, Hkv, D, page_size, bt_width, window=0, num_splits=0) -> int:
    return int(load().paged_attn_resolve_splits(B, query_len, Hq, Hkv, D, page_size, bt_width,
                                                window, num_splits))


def plan(B, query_len, Hq, Hkv, D, page_size, bt_width, window=0, num_splits=0) -> dict:
    """Launch plan of paged_attn_run for this shape (see paged_attn_plan in the header)."""
    buf = (ctypes.c_int32 * 6)()
    check(load().paged_attn_plan(B, query_len, Hq, Hkv, D, page_size, bt_width, window, num_splits,
                                 buf))
    S, chunk, rt, nw, rg, grid = list(buf)
    return dict(splits=S, chunk_pages=chunk, row_tiles=rt, waves=nw, row_groups=rg, grid=grid,
                partial_num_splits=(-chunk if chunk > 0 else S))


def workspace_size(B, query_len, Hq, Hkv, D, page_size, bt_width, window=0, num_splits=0) -> int:
    return int(load().paged_attn_workspace_size(B, query_len, Hq, Hkv, D, page_size, bt_width,
                                                window, num_splits))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A device workspace of at least nbytes (no initialization needed)."""
    return torch.empty(((max(int(nbytes), 16) + 15) // 16) * 16, dtype=torch.uint8, device=device)


def _check_paged_inputs(q, k, v, block_table, seq_lens):
    if q.dim() != 4:
        raise ValueError("q must be [B, query_len, Hq, D]")
    _need(q, "q")
    # the kernels step through K and V rows by the token stride and read D values of
    # each; a view narrower than q's head_dim would run into the next row or past the pool
    if k.dim() != 4 or v.dim() != 4 or k.shape[3] != q.shape[3] or v.shape[3] != q.shape[3]:
        raise ValueError(f"k and v must be [pages, Hkv, page_size, D] views with q's head_dim "
                         f"D={q.shape[3]} (got k {tuple(k.shape)}, v {tuple(v.shape)})")
    B = q.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != B or block_table.stride(1) != 1:
        raise ValueError("block_table must be [B, W] with unit column stride")
    _need(block_table, "block_table", dtype=torch.int32, contiguous=False)
    _need(seq_lens, "seq_lens", (B,), torch.int32)


def paged_attn_run(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_table: torch.Tensor,
                   seq_lens: torch.Tensor, *, scale: float, window: int = 0, num_splits: int = 0,
                   k_scale: float = 1.0, v_scale: float = 1.0, out: Optional[torch.Tensor] = None,
                   out_dtype: Optional[torch.dtype] = None, return_lse: bool = True,
                   lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   causal: bool = False):
    """Attention of q [B, sq, Hq, D] over paged K/V views [pages, Hkv, P, D].

    causal=True: bottom-right causal block with an exact per-token window
    (paged_attn_run_causal); otherwise the dense block with the page-aligned window.
    Returns (out [B, sq, Hq, D], lse [B, sq, Hq] fp32 natural log, or None)."""
    B, sq, Hq, D = q.shape
    _check_paged_inputs(q, k, v, block_table, seq_lens)
    desc = kv_desc(k, v, k_scale=k_scale, v_scale=v_scale)
    if out is None:
        default = q.dtype if q.dtype in (torch.bfloat16, torch.float16) else torch.bfloat16
        out = torch.empty((B, sq, Hq, D), dtype=out_dtype or default, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, sq, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", (B, sq, Hq, D))
    _need(lse, "lse", (B, sq, Hq), torch.float32)
    _need(workspace, "workspace")
    _same_device(q.device, k=k, v=v, block_table=block_table, seq_lens=seq_lens, out=out, lse=lse,
                 workspace=workspace)
    W = block_table.shape[1]
    need = workspace_size(B, sq, Hq, desc.num_kv_heads, D, desc.page_size, W, window, num_splits)
    if need and workspace is None:
        workspace = new_workspace(need, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = load().paged_attn_run_causal if causal else load().paged_attn_run
    check(fn(
        q.data_ptr(), dtype_code(q.dtype), ctypes.byref(desc), block_table.data_ptr(),
        block_table.stride(0), W, seq_lens.data_ptr(), B, sq, Hq, D, float(scale), int(window),
        int(num_splits), out.data_ptr(), dtype_code(out.dtype), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(q.device)))
    return out, lse


def paged_attn_run_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           block_table: torch.Tensor, seq_lens: torch.Tensor, *, scale: float,
                           out: torch.Tensor, lse: Optional[torch.Tensor] = None, window: int = 0,
                           num_splits: int = 0, k_scale: float = 1.0, v_scale: float = 1.0):
    """paged_attn_run with no workspace: the Split-KV partials go to the library's static
    per-GPU scratch (the C entry point paged_attn_run_noalloc).  Nothing is allocated here
    either, so `out` (and `lse`, if wanted) must be passed.  Calls that overlap in time on
    one GPU share the scratch and race.  Returns (out, lse)."""
    B, sq, Hq, D = q.shape
    _check_paged_inputs(q, k, v, block_table, seq_lens)
    desc = kv_desc(k, v, k_scale=k_scale, v_scale=v_scale)
    _need(out, "out", (B, sq, Hq, D))
    _need(lse, "lse", (B, sq, Hq), torch.float32)
    _same_device(q.device, k=k, v=v, block_table=block_table, seq_lens=seq_lens, out=out, lse=lse)
    W = block_table.shape[1]
    check(load().paged_attn_run_noalloc(
        q.data_ptr(), dtype_code(q.dtype), ctypes.byref(desc), block_table.data_ptr(),
        block_table.stride(0), W, seq_lens.data_ptr(), B, sq, Hq, D, float(scale), int(window),
        int(num_splits), out.data_ptr(), dtype_code(out.dtype), _ptr(lse), _stream(q.device)))
    return out, lse


def paged_attn_run_causal(q, k, v, block_table, seq_lens, **kw):
    """paged_attn_run with the bottom-right causal mask and an exact per-token window
    (the C entry point paged_attn_run_causal); same arguments and results."""
    return paged_attn_run(q, k, v, block_table, seq_lens, causal=True, **kw)


def paged_attn_partial(q, k, v, block_table, seq_lens, *, scale: float, num_splits: int,
                       window: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
                       part_o: Optional[torch.Tensor] = None, part_lse: Optional[torch.Tensor] = None):
    """Split-KV partials: (part_o [S, B*sq, Hq, D] fp32, part_lse [S, B*sq, Hq] fp32)."""
    B, sq, Hq, D = q.shape
    _check_paged_inputs(q, k, v, block_table, seq_lens)
    desc = kv_desc(k, v, k_scale=k_scale, v_scale=v_scale)
    W = block_table.shape[1]
    S = resolve_splits(B, sq, Hq, desc.num_kv_heads, D, desc.page_size, W, window, num_splits)
    if part_o is None:
        part_o = torch.empty((S, B * sq, Hq, D), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((S, B * sq, Hq), dtype=torch.float32, device=q.device)
    _need(part_o, "part_o", (S, B * sq, Hq, D), torch.float32)
    _need(part_lse, "part_lse", (S, B * sq, Hq), torch.float32)
    _same_device(q.device, k=k, v=v, block_table=block_table, seq_lens=seq_lens, part_o=part_o,
                 part_lse=part_lse)
    check(load().paged_attn_partial(
        q.data_ptr(), dtype_code(q.dtype), ctypes.byref(desc), block_table.data_ptr(),
        block_table.stride(0), W, seq_lens.data_ptr(), B, sq, Hq, D, float(scale), int(window),
        int(num_splits), part_o.data_ptr(), part_lse.data_ptr(), _stream(q.device)))
    return part_o, part_lse


def split_kv_combine(part_o: torch.Tensor, part_lse: torch.Tensor, *, out_dtype=torch.bfloat16,
                     out: Optional[torch.Tensor] = None, return_lse: bool = True):
    """LSE-weighted merge of Split-KV partials [S, rows, Hq, D] -> (out [rows, Hq, D], lse)."""
    S, rows, Hq, D = part_o.shape
    _need(part_o, "part_o", dtype=torch.float32)
    _need(part_lse, "part_lse", (S, rows, Hq), torch.float32)
    if out is None:
        out = torch.empty((rows, Hq, D), dtype=out_dtype, device=part_o.device)
    _need(out, "out", (rows, Hq, D))
    lse = torch.empty((rows, Hq), dtype=torch.float32, device=part_o.device) if return_lse else None
    _same_device(part_o.device, part_lse=part_lse, out=out)
    check(load().split_kv_combine(part_o.data_ptr(), part_lse.data_ptr(), S, rows, Hq, D,
                                  out.data_ptr(), dtype_code(out.dtype), _ptr(lse),
                                  _stream(part_o.device)))
    return out, lse


def segment_attn_combine(part_o: torch.Tensor, part_lse: torch.Tensor, used: torch.Tensor,
                         bias: Optional[torch.Tensor], *, out_dtype=torch.bfloat16,
                         out: Optional[torch.Tensor] = None, return_lse: bool = True):
    """DASH combine of [N, G, Hq, D] partials with per-segment bias -> (out [N, Hq, D], lse)."""
    N, G, Hq, D = part_o.shape
    _need(part_o, "part_o")
    _need(part_lse, "part_lse", (N, G, Hq), torch.float32)
    _need(used, "used", (N, G), torch.int32)
    if G > 1 and bias is None:
        raise ValueError("bias [N, G-1] is needed when there is more than one segment")
    _need(bias, "bias", (N, G - 1), torch.float32)
    if out is None:
        out = torch.empty((N, Hq, D), dtype=out_dtype, device=part_o.device)
    _need(out, "out", (N, Hq, D))
    lse = torch.empty((N, Hq), dtype=torch.float32, device=part_o.device) if return_lse else None
    _same_device(part_o.device, part_lse=part_lse, used=used, bias=bias, out=out)
    check(load().segment_attn_combine(part_o.data_ptr(), dtype_code(part_o.dtype),
                                      part_lse.data_ptr(), used.data_ptr(), _ptr(bias), N, G, Hq, D,
                                      out.data_ptr(), dtype_code(out.dtype), _ptr(lse),
                                      _stream(part_o.device)))
    return out, lse


def segment_attn_workspace_size(N, topk, Hq, D) -> int:
    return int(load().segment_attn_workspace_size(N, topk, Hq, D))


def segment_attn_run(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, used: torch.Tensor,
                     bias: torch.Tensor, *, bs: int, local: int, scale: Optional[float] = None,
                     fused: bool = True, out_dtype: Optional[torch.dtype] = None,
                     return_lse: bool = True, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """DASH attention of q [N, Hq, D] over gathered segments k, v [N*(topk*bs+local), Hkv, D]."""
    if q.dim() != 3 or bias.dim() != 2 or k.dim() != 3:
        raise ValueError("q must be [N, Hq, D], bias [N, topk], k and v [tokens, Hkv, D]")
    N, Hq, D = q.shape
    topk = bias.shape[1]
    Hkv = k.shape[1]
    tokens = N * (topk * int(bs) + int(local))
    _need(q, "q")
    _need(k, "k", (tokens, Hkv, D))
    _need(v, "v", (tokens, Hkv, D), k.dtype)
    _need(used, "used", (N, topk + 1), torch.int32)
    _need(bias, "bias", (N, topk), torch.float32)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((N, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out", (N, Hq, D))
    lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    if not fused and workspace is None:
        workspace = torch.empty(segment_attn_workspace_size(N, topk, Hq, D), dtype=torch.uint8,
                                device=q.device)
    _need(workspace, "workspace")
    _same_device(q.device, k=k, v=v, used=used, bias=bias, out=out, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().segment_attn_run(
        q.data_ptr(), dtype_code(q.dtype), k.data_ptr(), v.data_ptr(), dtype_code(k.dtype),
        used.data_ptr(), _ptr(bias), N, topk, int(bs), int(local), Hq, Hkv, D, float(scale),
        1 if fused else 0, out.data_ptr(), dtype_code(out.dtype), _ptr(lse), _ptr(workspace),
        ws_bytes, _stream(q.device)))
    return out, lse


def paged_kv_write(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                   k: torch.Tensor, v: torch.Tensor, *, k_scale: float = 1.0,
                   v_scale: float = 1.0) -> None:
    """Write token rows key[t], value[t] ([T, Hkv, D]) into slot slot_mapping[t] of the
    paged cache views k, v ([pages, Hkv, page_size, D], e.g. kv_halves of the cache).
    An fp8 (uint8 / float8_e4m3fn) cache stores e4m3fn(x / k_scale), e4m3fn(x / v_scale)."""
    if key.shape != value.shape or key.dim() != 3:
        raise ValueError("key and value must both be [T, Hkv, D]")
    if key.stride(1) != key.shape[2] or key.stride(2) != 1 or value.stride(1) != value.shape[2] \
            or value.stride(2) != 1:
        raise ValueError("key and value rows must be head-contiguous")
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1 or slot_mapping.shape[0] != key.shape[0]:
        raise ValueError("slot_mapping must be int64 [T]")
    desc = kv_desc(k, v, k_scale=k_scale, v_scale=v_scale)
    T, _, D = key.shape
    if key.shape[1] != k.shape[1] or D != k.shape[3]:
        raise ValueError("key/value [T, Hkv, D] must match the cache's kv heads and head_dim")
    _same_device(key.device, value=value, slot_mapping=slot_mapping, k=k, v=v)
    check(load().paged_kv_write(key.data_ptr(), key.stride(0), value.data_ptr(), value.stride(0),
                                dtype_code(key.dtype), T, D, slot_mapping.contiguous().data_ptr(),
                                ctypes.byref(desc), _stream(key.device)))


def window_width(window: int, query_len: int, page_size: int, bt_width: int) -> int:
    return int(load().paged_attn_window_width(window, query_len, page_size, bt_width))


def _describe_shapes(block_table, query_len, Hq, Hkv, D, page_size, window, num_splits):
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [B, W] with unit column stride")
    B, W = block_table.shape
    _need(block_table, "block_table", dtype=torch.int32, contiguous=False)
    S = resolve_splits(B, query_len, Hq, Hkv, D, page_size, W, window, num_splits)
    ow = window_width(window, query_len, page_size, W)
    return B, W, S, ow


def paged_attn_describe(block_table, seq_lens, *, query_len, Hq, Hkv, D, page_size, window=0,
                        num_splits=0):
    """Device integer plan: (lens [B], table [B, width], split_ranges [B, S, 4]) int32."""
    B, W, S, ow = _describe_shapes(block_table, query_len, Hq, Hkv, D, page_size, window, num_splits)
    dev = block_table.device
    _need(seq_lens, "seq_lens", (B,), torch.int32)
    _same_device(dev, seq_lens=seq_lens)
    lens = torch.empty(B, dtype=torch.int32, device=dev)
    table = torch.empty((B, ow), dtype=torch.int32, device=dev)
    ranges = torch.empty((B, S, 4), dtype=torch.int32, device=dev)
    check(load().paged_attn_describe(block_table.data_ptr(), block_table.stride(0), W,
                                     seq_lens.data_ptr(), B, query_len, Hq, Hkv, D, page_size,
                                     window, num_splits, lens.data_ptr(), table.data_ptr(), ow,
                                     ranges.data_ptr(), _stream(dev)))
    return lens, table, ranges


def paged_attn_describe_host(block_table, seq_lens, *, query_len, Hq, Hkv, D, page_size, window=0,
                             num_splits=0):
    """Same plan computed on the host from CPU int32 tensors (no GPU needed)."""
    if block_table.device.type != "cpu" or seq_lens.device.type != "cpu":
        raise ValueError("paged_attn_describe_host reads host memory: pass CPU tensors")
    block_table = block_table.contiguous()
    seq_lens = seq_lens.contiguous()
    B, W, S, ow = _describe_shapes(block_table, query_len, Hq, Hkv, D, page_size, window, num_splits)
    _need(seq_lens, "seq_lens", (B,), torch.int32)
    lens = torch.empty(B, dtype=torch.int32)
    table = torch.empty((B, ow), dtype=torch.int32)
    ranges = torch.empty((B, S, 4), dtype=torch.int32)
    check(load().paged_attn_describe_host(block_table.data_ptr(), block_table.stride(0), W,
                                          seq_lens.data_ptr(), B, query_len, Hq, Hkv, D, page_size,
                                          window, num_splits, lens.data_ptr(), table.data_ptr(), ow,
                                          ranges.data_ptr()))
    return lens, table, ranges


def pa_last_error() -> str:
    """Message of the last failing library call on this thread."""
    return _lib.last_error()


def pa_version() -> str:
    return load().pa_version().decode()


# the C entry points' own names for the planning helpers
paged_attn_plan = plan
paged_attn_resolve_splits = resolve_splits
paged_attn_workspace_size = workspace_size
paged_attn_window_width = window_width

__all__ = [
    "PagedAttnError", "dtype_code", "kv_desc", "kv_halves", "resolve_splits", "workspace_size", "plan",
    "new_workspace",
    "paged_attn_run", "paged_attn_run_causal", "paged_attn_run_noalloc", "paged_attn_partial",
    "split_kv_combine",
    "segment_attn_combine", "paged_kv_write",
    "segment_attn_run", "segment_attn_workspace_size", "window_width", "paged_attn_describe",
    "paged_attn_describe_host", "paged_attn_plan", "paged_attn_resolve_splits",
    "paged_attn_workspace_size", "paged_attn_window_width", "pa_last_error", "pa_version",
]
PagedAttnError = _lib.PagedAttnError
