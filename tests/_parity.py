"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on the same
bytes, compare with the tolerances the method is held to."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle.attention import kv_halves
from workloads import to_numpy_bits

# Acceptance bars (max-abs and mean-abs on the output, abs on the natural-log LSE).
TOL_BF16 = dict(max_abs=2e-2, mean_abs=2e-3, lse=1e-3)
TOL_FP8 = dict(max_abs=6e-2, mean_abs=6e-3, lse=1e-3)


def gpu_available() -> bool:
    return torch.cuda.is_available()


def run_paged(inp, *, num_splits=None, window=None, out_dtype=torch.bfloat16, causal=False):
    import segmented_attention_paged_amd as sap

    k, v = sap.kv_halves(inp.cache, inp.D)
    return sap.paged_attn_run(
        inp.q, k, v, inp.block_table, inp.seq_lens, scale=inp.scale * inp.q_scale,
        window=inp.window if window is None else window,
        num_splits=inp.num_splits if num_splits is None else num_splits,
        k_scale=inp.k_scale, v_scale=inp.v_scale, out_dtype=out_dtype, causal=causal)


def host_subset(inp, requests):
    """Host copies of just the pages the given requests reference (table remapped)."""
    bt = inp.block_table.cpu()
    lens = inp.seq_lens.cpu()
    pages = sorted({int(p) for b in requests for p in bt[b, : -(-int(lens[b]) // inp.P)].tolist()})
    remap = {p: i for i, p in enumerate(pages)}
    if pages:
        idx = torch.tensor(pages, dtype=torch.long, device=inp.cache.device)
        cache = inp.cache.index_select(0, idx).cpu()
    else:
        cache = inp.cache[:1].cpu()
    table = np.zeros(bt.shape, dtype=np.int64)
    for b in requests:
        n = -(-int(lens[b]) // inp.P)
        table[b, :n] = [remap[int(p)] for p in bt[b, :n].tolist()]
    return cache, table, lens.numpy()


def oracle_paged(inp, requests=None, kv_heads=None, window=None, causal=False):
    reqs = list(range(inp.B)) if requests is None else list(requests)
    cache, table, lens = host_subset(inp, reqs)
    k, v = kv_halves(to_numpy_bits(cache), inp.D)
    q = to_numpy_bits(inp.q.cpu())
    q_dtype = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.uint8: "fp8_e4m3"}[inp.q.dtype]
    return oracle.paged_attention(
        q, q_dtype, k, v, inp.kv_dtype, table, lens, q_scale=inp.q_scale,
        scale=inp.scale, window=inp.window if window is None else window, k_scale=inp.k_scale,
        v_scale=inp.v_scale, requests=reqs, kv_heads=kv_heads, causal=causal)


def compare(out, lse, O_ref, L_ref, tol, *, mask=None, what=""):
    """Assert GPU (out, lse) match the oracle where mask (bool over O_ref's leading dims) is set."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.float().cpu().numpy().astype(np.float64) if lse is not None else None
    if mask is None:
        mask = ~np.isnan(L_ref)
    oref = O_ref[mask]
    og = o[mask]
    assert np.all(np.isfinite(og)), f"{what}: non-finite output"
    err = np.abs(og - oref)
    assert err.max(initial=0) <= tol["max_abs"], f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= tol["mean_abs"], f"{what}: mean-abs {err.mean():.3e}"
    if l is not None:
        lr = L_ref[mask]
        lg = l[mask]
        dead = np.isneginf(lr)
        assert np.array_equal(np.isneginf(lg), dead), f"{what}: -inf LSE pattern differs"
        if (~dead).any():
            e = np.abs(lg[~dead] - lr[~dead]).max()
            assert e <= tol["lse"], f"{what}: lse err {e:.3e}"
        assert np.all(og[dead] == 0), f"{what}: rows without keys are not 0"
    return float(err.max(initial=0)), float(err.mean())
