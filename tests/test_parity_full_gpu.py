"""GPU parity at the five workloads' full sizes, in the launch configuration the bench times.

The oracle computes sampled requests / kv heads (or sampled DASH queries) one
by one from host copies of exactly the bytes the GPU read.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import paged_config, segment_config, to_numpy_bits

from _parity import TOL_BF16, TOL_FP8, compare, gpu_available, oracle_paged, run_paged

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


@pytest.fixture(scope="module")
def sap():
    import segmented_attention_paged_amd as m

    m.load()
    return m


@pytest.mark.parametrize("name,causal", [
    ("c1_tiny", False), ("c2_gqa_decode", False), ("c3_query_block", False),
    ("c3w_query_block_window", False), ("c4_split_kv", False), ("c4f_split_kv_fp8", False),
    # the blocks the bench also times with the causal mask, and with fp8 queries
    ("c3_query_block", True), ("c3w_query_block_window", True), ("c3f_query_block_fp8", False),
])
def test_full_size_sampled(sap, name, causal):
    inp = paged_config(name, poison=True, device=DEV)
    out, lse = run_paged(inp, causal=causal)  # the config's own num_splits (0 = library choice)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    lens = inp.seq_lens.cpu()
    reqs = sorted({int(torch.argmin(lens)), int(torch.argmax(lens)), inp.B // 2})
    heads = sorted({0, inp.Hkv - 1})
    O, L = oracle_paged(inp, requests=reqs, kv_heads=heads, causal=causal)
    mask = ~np.isnan(L)
    assert mask.sum() == len(reqs) * len(heads) * (inp.Hq // inp.Hkv) * inp.sq
    tol = TOL_FP8 if inp.kv_dtype == "fp8_e4m3" else TOL_BF16
    compare(out, lse, O, L, tol, mask=mask, what=f"{name} causal={causal}")


@pytest.mark.parametrize("fused", [True, False])
def test_full_size_dash_segments(sap, fused):
    s = segment_config("c5_dash_segments", poison=True, device=DEV)
    out, lse = sap.segment_attn_run(s.q, s.k, s.v, s.used, s.bias, bs=s.bs, local=s.local,
                                    fused=fused)
    torch.cuda.synchronize()
    used = s.used.cpu().numpy()
    dead_q = [int(n) for n in np.nonzero((used == 0).all(1))[0][:1]]
    queries = sorted(set([0, 1, s.N // 2, s.N - 1] + dead_q))
    O, L = oracle.segment_attention(to_numpy_bits(s.q.cpu()), to_numpy_bits(s.k.cpu()),
                                    to_numpy_bits(s.v.cpu()), used, s.bias.cpu().numpy(),
                                    topk=s.topk, bs=s.bs, local=s.local, scale=s.scale,
                                    queries=queries)
    mask = ~np.isnan(L)
    compare(out, lse, O, L, TOL_BF16, mask=mask, what=f"c5 fused={fused}")
