"""GPU parity of causal query blocks (exact per-token window) against the oracle."""

import numpy as np
import pytest
import torch

from workloads import make_paged, paged_config

from _parity import TOL_BF16, TOL_FP8, compare, gpu_available, oracle_paged, run_paged

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


@pytest.fixture(scope="module")
def sap():
    import segmented_attention_paged_amd as m

    m.load()
    return m


CASES = {
    # row-split kernel (R = 64 rows)
    "sq16_g4": dict(B=4, sq=16, Hq=32, Hkv=8, D=128, P=16, seq_lens=[16, 100, 257, 640]),
    # key-split kernel (R = 16 rows), a request shorter than the block
    "sq4_g4": dict(B=4, sq=4, Hq=8, Hkv=2, D=128, P=16, seq_lens=[2, 4, 60, 300]),
    # key-split with two row tiles per wave (R = 24)
    "sq3_g8_rt2": dict(B=3, sq=3, Hq=8, Hkv=1, D=64, P=16, seq_lens=[1, 50, 333]),
    "decode_g4": dict(B=5, sq=1, Hq=16, Hkv=4, D=128, P=16, seq_lens=[1, 15, 16, 17, 700]),
    "page1_sq8": dict(B=2, sq=8, Hq=8, Hkv=2, D=64, P=1, seq_lens=[5, 40]),
    "page24_sq5": dict(B=3, sq=5, Hq=8, Hkv=4, D=128, P=24, seq_lens=[3, 25, 200]),
    "page64_sq16": dict(B=2, sq=16, Hq=16, Hkv=2, D=64, P=64, seq_lens=[70, 400]),
    "fp8_sq16": dict(B=3, sq=16, Hq=16, Hkv=2, D=128, P=16, seq_lens=[20, 129, 500],
                     kv_dtype="fp8_e4m3"),
}
WINDOWS = [0, 1, 7, 40]
SPLITS = [1, 0, 3, -2]


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("splits", SPLITS)
def test_causal_small(sap, name, window, splits):
    inp = make_paged(seed=17, poison=True, name=name, **CASES[name]).to(DEV)
    out, lse = run_paged(inp, num_splits=splits, window=window, causal=True)
    O, L = oracle_paged(inp, window=window, causal=True)
    tol = TOL_FP8 if inp.kv_dtype == "fp8_e4m3" else TOL_BF16
    compare(out, lse, O, L, tol, what=f"{name} w={window} S={splits}")


def test_causal_fp16(sap):
    inp = make_paged(seed=4, poison=True, **CASES["sq16_g4"]).to(DEV)
    inp.q = inp.q.to(torch.float16)
    inp.cache = inp.cache.to(torch.float16)
    inp.kv_dtype = "fp16"
    out, lse = run_paged(inp, num_splits=0, window=33, causal=True, out_dtype=torch.float16)
    O, L = oracle_paged(inp, window=33, causal=True)
    compare(out, lse, O, L, TOL_BF16, what="causal fp16")


def test_causal_decode_differs_from_dense_window_only_by_page_rounding(sap):
    # sq = 1: causal with window w sees exactly the last w keys; the dense
    # block sees the page-aligned suffix.  Both match their own oracle and
    # coincide when the window is a whole number of pages at a page boundary.
    inp = make_paged(B=2, sq=1, Hq=8, Hkv=2, D=128, P=16, seq_lens=[64, 160], seed=2,
                     poison=True).to(DEV)
    oc, lc = run_paged(inp, num_splits=1, window=32, causal=True)
    od, ld = run_paged(inp, num_splits=1, window=32)
    assert torch.equal(lc, ld) or torch.allclose(lc, ld, atol=1e-5)
    Oc, Lc = oracle_paged(inp, window=32, causal=True)
    compare(oc, lc, Oc, Lc, TOL_BF16, what="causal decode")


@pytest.mark.parametrize("name,window", [("c3_query_block", 0), ("c3w_query_block_window", 4096)])
def test_causal_full_size_sampled(sap, name, window):
    inp = paged_config(name, device=DEV)
    out, lse = run_paged(inp, num_splits=0, window=window, causal=True)
    rng = np.random.default_rng(5)
    reqs = sorted(rng.choice(inp.B, size=3, replace=False).tolist())
    heads = [0, inp.Hkv - 1]
    O, L = oracle_paged(inp, requests=reqs, kv_heads=heads, window=window, causal=True)
    mask = ~np.isnan(L)
    compare(out, lse, O, L, TOL_BF16, mask=mask, what=f"{name} causal")


def test_causal_entry_point_by_name(sap):
    # the binding's paged_attn_run_causal is the C entry point of that name
    inp = make_paged(B=2, sq=4, Hq=8, Hkv=2, D=128, P=16, seq_lens=[37, 90], seed=61).to(DEV)
    k, v = sap.kv_halves(inp.cache, inp.D)
    a = sap.paged_attn_run_causal(inp.q, k, v, inp.block_table, inp.seq_lens, scale=inp.scale,
                                  window=20)
    b = sap.paged_attn_run(inp.q, k, v, inp.block_table, inp.seq_lens, scale=inp.scale, window=20,
                           causal=True)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])
    O, L = oracle_paged(inp, window=20, causal=True)
    compare(*a, O, L, TOL_BF16, what="paged_attn_run_causal")
