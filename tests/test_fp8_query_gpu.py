"""GPU parity of fp8 queries against an fp8 cache (q.k on fp8 MFMA, P.V in bf16)."""

import numpy as np
import pytest
import torch

from workloads import make_paged, paged_config

from _parity import TOL_FP8, compare, gpu_available, oracle_paged, run_paged

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


@pytest.fixture(scope="module")
def sap():
    import segmented_attention_paged_amd as m

    m.load()
    return m


CASES = {
    "decode_g8": dict(B=4, sq=1, Hq=16, Hkv=2, D=128, P=16, seq_lens=[5, 64, 300, 999]),
    "decode_d64": dict(B=3, sq=1, Hq=8, Hkv=2, D=64, P=16, seq_lens=[1, 33, 500]),
    "sq16_g4": dict(B=3, sq=16, Hq=32, Hkv=8, D=128, P=16, seq_lens=[16, 257, 640]),
    "sq16_d64_page64": dict(B=2, sq=16, Hq=8, Hkv=2, D=64, P=64, seq_lens=[20, 400]),
    "sq3_rt2": dict(B=3, sq=3, Hq=8, Hkv=1, D=128, P=16, seq_lens=[3, 50, 333]),
    # query blocks staged 32 keys at a time (two 16-slot sub-tiles): pages of 8
    # slots (one short sub-tile per page) and of 48 (three sub-tiles per page,
    # so a tile's two halves may sit in different pages), odd sub-tile counts
    "sq16_page8": dict(B=2, sq=16, Hq=8, Hkv=2, D=128, P=8, seq_lens=[17, 333]),
    "sq16_page48": dict(B=3, sq=16, Hq=8, Hkv=2, D=128, P=48, seq_lens=[16, 100, 481]),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("splits", [1, 0, 3])
@pytest.mark.parametrize("mode", ["dense", "dense_window", "causal_window"])
def test_fp8_query(sap, name, splits, mode):
    inp = make_paged(seed=29, poison=True, kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3",
                     **CASES[name]).to(DEV)
    window = 0 if mode == "dense" else 40
    causal = mode.startswith("causal")
    out, lse = run_paged(inp, num_splits=splits, window=window, causal=causal)
    assert out.dtype == torch.bfloat16
    O, L = oracle_paged(inp, window=window, causal=causal)
    compare(out, lse, O, L, TOL_FP8, what=f"{name} S={splits} {mode}")


def test_fp8_query_fp16_out(sap):
    inp = make_paged(seed=3, poison=True, kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3",
                     **CASES["sq16_g4"]).to(DEV)
    out, lse = run_paged(inp, num_splits=0, out_dtype=torch.float16)
    O, L = oracle_paged(inp)
    compare(out, lse, O, L, TOL_FP8, what="fp8 q, fp16 out")


def test_fp8_query_needs_fp8_cache(sap):
    inp = make_paged(seed=3, B=1, sq=1, Hq=4, Hkv=1, D=64, P=16, seq_lens=[10]).to(DEV)
    k, v = sap.kv_halves(inp.cache, inp.D)
    q8 = torch.zeros(inp.q.shape, dtype=torch.uint8, device=DEV)
    with pytest.raises(sap.PagedAttnError, match="PA_ENOTSUP"):
        sap.paged_attn_run(q8, k, v, inp.block_table, inp.seq_lens, scale=0.1)


def test_fp8_query_full_size_sampled(sap):
    inp = paged_config("c3f_query_block_fp8", device=DEV)
    out, lse = run_paged(inp, num_splits=0)
    rng = np.random.default_rng(6)
    reqs = sorted(rng.choice(inp.B, size=3, replace=False).tolist())
    O, L = oracle_paged(inp, requests=reqs, kv_heads=[0, inp.Hkv - 1])
    compare(out, lse, O, L, TOL_FP8, mask=~np.isnan(L), what="c3f sampled")
