"""Seeded synthetic workloads for paged attention and DASH-style gathered segments.

Everything is drawn from one CPU ``torch.Generator`` per workload, in a fixed
order, so that the oracle and the GPU see identical bytes:

    seq_lens -> page permutation -> q -> cache (K|V rows) -> fp8 scales
    (segments: q -> K -> V -> zero mask -> used lengths -> bias)

Value recipe: bf16 values are fp32 N(0, 1) draws rounded to nearest even;
fp8 values are e4m3fn(RNE(N(0, 1))) stored as raw bytes; fp8 scales are
U[0.5, 2].  The cache layout is vLLM's ``[pages, Hkv, page_size, 2*D]`` page
with K in ``[..., :D]`` and V in ``[..., D:]`` (the K/V-halves layout described
on the vllm.v1.attention.backends.flashinfer_ts page, module docstring
"Layout").  DASH segment buffers are contiguous ``[N*(topk*bs+local), Hkv, D]``
(vllm.v1.attention.ops.dash_attention page, ``flash_dash_attention``
docstring), remote segments first and the local one last per query.

Parity runs may ask for poison: every pool page that no request owns is
filled with NaN, block-table pads point at such a page, the slots past each
request's length on its last page are NaN, and segment slots at or past
``used`` are NaN.  A correct kernel never lets those values reach a result.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Sequence

import numpy as np
import torch

NAN_E4M3_BYTE = 0x7F  # e4m3fn encodes NaN as S.1111.111
DEVICE_SEED_OFFSET = 7919  # seed offset of the on-device generator (large workloads)

# Number of random values drawn per chunk when filling large buffers.  The
# draw order (chunk by chunk along the leading dimension) is part of the recipe.
_CHUNK_VALUES = 1 << 24


@dataclass
class PagedInputs:
    name: str
    B: int
    sq: int
    Hq: int
    Hkv: int
    D: int
    P: int
    window: int
    num_splits: int
    kv_dtype: str  # "bf16" or "fp8_e4m3"
    scale: float
    k_scale: float
    v_scale: float
    q: torch.Tensor  # [B, sq, Hq, D] bfloat16
    cache: torch.Tensor  # [pool, Hkv, P, 2*D] bfloat16, or uint8 e4m3fn bytes
    block_table: torch.Tensor  # [B, W] int32
    seq_lens: torch.Tensor  # [B] int32 (includes the query block)
    poison: bool
    q_dtype: str = "bf16"  # or "fp8_e4m3": q holds e4m3fn bytes, real q = q_scale * q
    q_scale: float = 1.0

    def to(self, device) -> "PagedInputs":
        return replace(
            self,
            q=self.q.to(device),
            cache=self.cache.to(device),
            block_table=self.block_table.to(device),
            seq_lens=self.seq_lens.to(device),
        )

    @property
    def pool(self) -> int:
        return int(self.cache.shape[0])

    @property
    def width(self) -> int:
        return int(self.block_table.shape[1])


@dataclass
class SegmentInputs:
    name: str
    N: int
    Hq: int
    Hkv: int
    D: int
    topk: int
    bs: int
    local: int
    scale: float
    q: torch.Tensor  # [N, Hq, D] bfloat16
    k: torch.Tensor  # [N*(topk*bs+local), Hkv, D] bfloat16
    v: torch.Tensor  # same
    used: torch.Tensor  # [N, topk+1] int32, 0 = inactive segment
    bias: torch.Tensor  # [N, topk] float32 (the local segment has no bias)
    poison: bool

    @property
    def G(self) -> int:
        return self.topk + 1

    @property
    def per_query(self) -> int:
        return self.topk * self.bs + self.local

    def to(self, device) -> "SegmentInputs":
        return replace(
            self,
            q=self.q.to(device),
            k=self.k.to(device),
            v=self.v.to(device),
            used=self.used.to(device),
            bias=self.bias.to(device),
        )


def _randn_bf16(shape: Sequence[int], g: torch.Generator) -> torch.Tensor:
    """N(0,1) fp32 draws rounded to bf16, drawn chunk by chunk along dim 0 on g's device."""
    dev = g.device
    out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=dev)
    if out.numel() == 0:
        return out
    per_row = out[0].numel() if out.dim() > 0 else 1
    rows = max(1, _CHUNK_VALUES // max(per_row, 1))
    for r0 in range(0, out.shape[0], rows):
        r1 = min(out.shape[0], r0 + rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=dev).to(torch.bfloat16)
    return out


def _randn_e4m3_bytes(shape: Sequence[int], g: torch.Generator) -> torch.Tensor:
    """e4m3fn(RNE(N(0,1))) stored as uint8 bytes, drawn chunk by chunk along dim 0 on g's device."""
    dev = g.device
    out = torch.empty(tuple(shape), dtype=torch.uint8, device=dev)
    if out.numel() == 0:
        return out
    per_row = out[0].numel()
    rows = max(1, _CHUNK_VALUES // max(per_row, 1))
    for r0 in range(0, out.shape[0], rows):
        r1 = min(out.shape[0], r0 + rows)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=dev)
        try:
            out[r0:r1] = x.to(torch.float8_e4m3fn).view(torch.uint8)
        except RuntimeError:  # no device-side fp8 cast: round on the host instead
            out[r0:r1] = x.cpu().to(torch.float8_e4m3fn).view(torch.uint8).to(dev)
    return out


def make_paged(
    *,
    B: int,
    sq: int,
    Hq: int,
    Hkv: int,
    D: int,
    P: int,
    seq_lens,
    seed: int,
    window: int = 0,
    num_splits: int = 0,
    kv_dtype: str = "bf16",
    poison: bool = False,
    pool_pages: int = 0,
    table_width: int = 0,
    name: str = "paged",
    device=None,
    q_dtype: str = "bf16",
) -> PagedInputs:
    """Draw one paged-attention workload.

    ``seq_lens`` is either a sequence of ints or ``("uniform", lo, hi)`` for
    lengths drawn uniformly from the integers in [lo, hi].  With ``device``
    set to a GPU, q and the cache are drawn there by a second generator
    seeded with ``seed + DEVICE_SEED_OFFSET`` (same distributions, other
    bytes; lengths, permutation and scales still come from the CPU stream).
    """
    if kv_dtype not in ("bf16", "fp8_e4m3"):
        raise ValueError(kv_dtype)
    if q_dtype not in ("bf16", "fp8_e4m3") or (q_dtype == "fp8_e4m3" and kv_dtype != "fp8_e4m3"):
        raise ValueError(q_dtype)
    g = torch.Generator().manual_seed(int(seed))

    # 1. sequence lengths
    if isinstance(seq_lens, tuple) and seq_lens and seq_lens[0] == "uniform":
        lo, hi = int(seq_lens[1]), int(seq_lens[2])
        lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)
    else:
        lens = torch.tensor(list(seq_lens), dtype=torch.int64)
        if lens.numel() != B:
            raise ValueError("seq_lens must have B entries")
    lens_l = [int(x) for x in lens]
    pages_per = [-(-L // P) for L in lens_l]
    used_pages = sum(pages_per)
    pool = max(int(pool_pages), used_pages)
    if poison and pool == used_pages:
        pool += 1  # room for one NaN page that the pads can point at

    # 2. page permutation: logical page j of request b -> perm[first_b + j]
    perm = torch.randperm(pool, generator=g)
    W = int(table_width) if table_width else max(1, max(pages_per) if pages_per else 1)
    if pages_per and max(pages_per) > W:
        raise ValueError("table_width is smaller than the longest request")
    spare = perm[used_pages:]
    pad_page = int(spare[0]) if (poison and spare.numel()) else 0
    table = torch.full((B, W), pad_page, dtype=torch.int32)
    cursor = 0
    for b, n in enumerate(pages_per):
        table[b, :n] = perm[cursor : cursor + n].to(torch.int32)
        cursor += n

    # 3. queries, 4. cache rows [K | V]
    gd = g
    if device is not None and torch.device(device).type != "cpu":
        gd = torch.Generator(device=device).manual_seed(int(seed) + DEVICE_SEED_OFFSET)
    q = _randn_bf16((B, sq, Hq, D), gd) if q_dtype == "bf16" else _randn_e4m3_bytes((B, sq, Hq, D), gd)
    if kv_dtype == "bf16":
        cache = _randn_bf16((pool, Hkv, P, 2 * D), gd)
    else:
        cache = _randn_e4m3_bytes((pool, Hkv, P, 2 * D), gd)

    # 5. per-tensor fp8 scales
    if kv_dtype == "fp8_e4m3":
        sc = torch.rand(2, generator=g, dtype=torch.float64) * 1.5 + 0.5
        k_scale, v_scale = float(sc[0]), float(sc[1])
    else:
        k_scale = v_scale = 1.0
    # 6. fp8 query scale (real q = q_scale * stored q)
    q_scale = float(torch.rand((), generator=g, dtype=torch.float64) * 1.5 + 0.5) \
        if q_dtype == "fp8_e4m3" else 1.0

    if poison:
        fill_value = float("nan") if kv_dtype == "bf16" else NAN_E4M3_BYTE
        if spare.numel():
            cache.index_fill_(0, spare.to(cache.device), fill_value)
        for b, (L, n) in enumerate(zip(lens_l, pages_per)):
            if n == 0:
                continue
            last = int(table[b, n - 1])
            tail0 = L - (n - 1) * P
            if tail0 < P:
                cache[last, :, tail0:, :] = fill_value

    table = table.to(q.device)
    lens = lens.to(q.device)
    return PagedInputs(
        name=name,
        B=B,
        sq=sq,
        Hq=Hq,
        Hkv=Hkv,
        D=D,
        P=P,
        window=int(window),
        num_splits=int(num_splits),
        kv_dtype=kv_dtype,
        scale=float(D) ** -0.5,
        k_scale=k_scale,
        v_scale=v_scale,
        q=q,
        cache=cache,
        block_table=table,
        seq_lens=lens.to(torch.int32),
        poison=poison,
        q_dtype=q_dtype,
        q_scale=q_scale,
    )


def make_segments(
    *,
    N: int,
    Hq: int,
    Hkv: int,
    D: int,
    topk: int,
    bs: int,
    local: int,
    seed: int,
    zero_frac: float = 0.1,
    poison: bool = False,
    name: str = "segments",
    device=None,
) -> SegmentInputs:
    """Draw one DASH-style gathered-segment workload.

    used[n, g] is 0 with probability ``zero_frac``, otherwise uniform in
    {1..cap}, cap = bs for the topk remote segments and local for the last one.
    With ``device`` set to a GPU, q, K and V are drawn there by a second
    generator seeded with ``seed + DEVICE_SEED_OFFSET``.
    """
    g = torch.Generator().manual_seed(int(seed))
    gd = g
    if device is not None and torch.device(device).type != "cpu":
        gd = torch.Generator(device=device).manual_seed(int(seed) + DEVICE_SEED_OFFSET)
    G = topk + 1
    T = N * (topk * bs + local)
    q = _randn_bf16((N, Hq, D), gd)
    k = _randn_bf16((T, Hkv, D), gd)
    v = _randn_bf16((T, Hkv, D), gd)
    zero = torch.rand((N, G), generator=g) < zero_frac
    caps = torch.tensor([bs] * topk + [local], dtype=torch.float64)
    u = torch.rand((N, G), generator=g, dtype=torch.float64)
    vals = torch.floor(u * caps).to(torch.int64) + 1  # uniform in {1..cap}
    used = torch.where(zero, torch.zeros_like(vals), vals).to(torch.int32)
    bias = torch.randn((N, topk), generator=g, dtype=torch.float32)
    used = used.to(q.device)
    bias = bias.to(q.device)
    if poison:
        per = topk * bs + local
        nan = float("nan")
        used_host = used.cpu()
        for n in range(N):
            for s in range(G):
                base = n * per + (s * bs if s < topk else topk * bs)
                cap = bs if s < topk else local
                u_ns = int(used_host[n, s])
                if u_ns < cap:
                    k[base + u_ns : base + cap] = nan
                    v[base + u_ns : base + cap] = nan
    return SegmentInputs(
        name=name,
        N=N,
        Hq=Hq,
        Hkv=Hkv,
        D=D,
        topk=topk,
        bs=bs,
        local=local,
        scale=float(D) ** -0.5,
        q=q,
        k=k,
        v=v,
        used=used,
        bias=bias,
        poison=poison,
    )


# The five workloads the method is measured on.  Seeds are 1000 + config number.
CONFIGS = {
    "c1_tiny": dict(
        kind="paged", B=2, sq=1, Hq=4, Hkv=1, D=64, P=16, seq_lens=[37, 100],
        pool_pages=16, seed=1001,
    ),
    "c2_gqa_decode": dict(
        kind="paged", B=64, sq=1, Hq=32, Hkv=8, D=128, P=16, seq_lens=("uniform", 512, 8192),
        table_width=512, seed=1002,
    ),
    "c3_query_block": dict(
        kind="paged", B=32, sq=16, Hq=32, Hkv=8, D=128, P=16, seq_lens=("uniform", 1024, 32768),
        table_width=2048, seed=1003,
    ),
    "c3w_query_block_window": dict(
        kind="paged", B=32, sq=16, Hq=32, Hkv=8, D=128, P=16, seq_lens=("uniform", 1024, 32768),
        table_width=2048, window=4096, seed=1003,
    ),
    "c3f_query_block_fp8": dict(
        kind="paged", B=32, sq=16, Hq=32, Hkv=8, D=128, P=16, seq_lens=("uniform", 1024, 32768),
        table_width=2048, kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3", seed=1003,
    ),
    "c4_split_kv": dict(
        kind="paged", B=8, sq=1, Hq=64, Hkv=8, D=128, P=16, seq_lens=[131072] * 8,
        table_width=8192, num_splits=16, seed=1004,
    ),
    "c4f_split_kv_fp8": dict(
        kind="paged", B=8, sq=1, Hq=64, Hkv=8, D=128, P=16, seq_lens=[131072] * 8,
        table_width=8192, num_splits=16, kv_dtype="fp8_e4m3", seed=1004,
    ),
    "c5_dash_segments": dict(
        kind="segments", N=256, Hq=32, Hkv=8, D=128, topk=8, bs=64, local=128, seed=1005,
    ),
}


@dataclass
class KVWriteInputs:
    """New K/V rows of T tokens and the page cache they are written into."""

    name: str
    T: int
    Hkv: int
    D: int
    P: int
    pages: int
    in_dtype: str  # "bf16" or "fp16"
    cache_dtype: str  # in_dtype or "fp8_e4m3"
    k_scale: float
    v_scale: float
    key: torch.Tensor  # [T, Hkv, D] in_dtype
    value: torch.Tensor  # [T, Hkv, D] in_dtype
    cache: torch.Tensor  # [pages, Hkv, P, 2*D] (uint8 bytes for fp8): contents before the write
    slot_mapping: torch.Tensor  # [T] int64, distinct slots; -1 = padding token


def make_kv_write(*, T: int, Hkv: int, D: int, P: int, pages: int, seed: int,
                  in_dtype: str = "bf16", cache_dtype: str = "bf16", pad_frac: float = 0.0,
                  value_scale: float = 1.0, name: str = "kv_write",
                  device=None) -> KVWriteInputs:
    """Draw one cache-write workload.

    Order: key -> value -> prior cache contents -> slot permutation -> padding
    mask -> fp8 scales.  key and value are N(0, 1) * value_scale rounded to the
    input type; the prior cache holds N(0, 1) values (random bytes for fp8);
    the T tokens take distinct slots drawn uniformly from the pool's
    pages * P slots (T <= pages * P); a fraction pad_frac of them is -1.
    With ``device`` set to a GPU, key, value and the cache are drawn there by a
    second generator seeded with ``seed + DEVICE_SEED_OFFSET``.
    """
    if T > pages * P:
        raise ValueError("more tokens than slots")
    g = torch.Generator().manual_seed(int(seed))
    gd = g
    if device is not None and torch.device(device).type != "cpu":
        gd = torch.Generator(device=device).manual_seed(int(seed) + DEVICE_SEED_OFFSET)
    tdt = torch.float16 if in_dtype == "fp16" else torch.bfloat16

    def draw(shape):
        out = torch.empty(tuple(shape), dtype=tdt, device=gd.device)
        per_row = max(1, out[0].numel()) if out.numel() else 1
        rows = max(1, _CHUNK_VALUES // per_row)
        for r0 in range(0, out.shape[0], rows):
            r1 = min(out.shape[0], r0 + rows)
            x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gd, device=gd.device)
            out[r0:r1] = (x * value_scale).to(tdt)
        return out

    key = draw((T, Hkv, D))
    value = draw((T, Hkv, D))
    if cache_dtype == "fp8_e4m3":
        cache = torch.randint(0, 256, (pages, Hkv, P, 2 * D), generator=gd, device=gd.device,
                              dtype=torch.int32).to(torch.uint8)
    else:
        cache = draw((pages, Hkv, P, 2 * D))
    slots = torch.randperm(pages * P, generator=g)[:T].to(torch.int64)
    pad = torch.rand(T, generator=g) < pad_frac
    slots = torch.where(pad, torch.full_like(slots, -1), slots)
    k_scale = v_scale = 1.0
    if cache_dtype == "fp8_e4m3":
        k_scale = float(0.5 + 1.5 * torch.rand((), generator=g, dtype=torch.float64))
        v_scale = float(0.5 + 1.5 * torch.rand((), generator=g, dtype=torch.float64))
    return KVWriteInputs(name=name, T=T, Hkv=Hkv, D=D, P=P, pages=pages, in_dtype=in_dtype,
                         cache_dtype=cache_dtype, k_scale=k_scale, v_scale=v_scale, key=key,
                         value=value, cache=cache, slot_mapping=slots.to(gd.device))


def paged_config(name: str, poison: bool = False, device=None) -> PagedInputs:
    cfg = dict(CONFIGS[name])
    if cfg.pop("kind") != "paged":
        raise ValueError(name)
    return make_paged(name=name, poison=poison, device=device, **cfg)


def segment_config(name: str, poison: bool = False, device=None) -> SegmentInputs:
    cfg = dict(CONFIGS[name])
    if cfg.pop("kind") != "segments":
        raise ValueError(name)
    return make_segments(name=name, poison=poison, device=device, **cfg)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU tensor as numpy: bf16 -> uint16 bits, fp8 -> uint8 bytes."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    return t.numpy()
