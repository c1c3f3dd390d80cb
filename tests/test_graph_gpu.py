"""Graph capture and replay of the causal / fp8-query attention and of the cache write:
every replay, with eager work and synchronisations in between, equals the eager result."""

import pytest
import torch

from workloads import make_kv_write, make_paged

from _parity import TOL_FP8, compare, gpu_available, oracle_paged

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


@pytest.fixture(scope="module")
def sap():
    import segmented_attention_paged_amd as m

    m.load()
    return m


def _capture(call):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    return g


@pytest.mark.parametrize("splits", [1, 3])
def test_graph_causal_fp8_query(sap, splits):
    inp = make_paged(B=3, sq=16, Hq=16, Hkv=2, D=128, P=16, seq_lens=[20, 129, 500], seed=44,
                     poison=True, kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3").to(DEV)
    k, v = sap.kv_halves(inp.cache, inp.D)
    W = inp.block_table.shape[1]
    ws = sap.new_workspace(sap.workspace_size(inp.B, inp.sq, inp.Hq, inp.Hkv, inp.D, inp.P, W, 40,
                                              splits), DEV)
    out = torch.empty((inp.B, inp.sq, inp.Hq, inp.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((inp.B, inp.sq, inp.Hq), dtype=torch.float32, device=DEV)

    def call():
        sap.paged_attn_run(inp.q, k, v, inp.block_table, inp.seq_lens, scale=inp.scale * inp.q_scale,
                           window=40, num_splits=splits, k_scale=inp.k_scale, v_scale=inp.v_scale,
                           out=out, lse=lse, workspace=ws, causal=True)

    call()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    O, L = oracle_paged(inp, window=40, causal=True)
    compare(ref_o, ref_l, O, L, TOL_FP8, what="eager")
    g = _capture(call)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}"
        assert torch.equal(lse, ref_l), f"replay {rep}"


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8_e4m3"])
def test_graph_kv_write(sap, cache_dtype):
    w = make_kv_write(T=500, Hkv=4, D=128, P=16, pages=64, seed=45, cache_dtype=cache_dtype,
                      pad_frac=0.1, device=DEV)
    prior = w.cache.clone()
    k, v = sap.kv_halves(w.cache, w.D)

    def call():
        sap.paged_kv_write(w.key, w.value, w.slot_mapping, k, v, k_scale=w.k_scale,
                           v_scale=w.v_scale)

    call()
    torch.cuda.synchronize()
    ref = w.cache.clone()
    assert not torch.equal(ref, prior)
    w.cache.copy_(prior)
    g = _capture(call)
    for rep in range(4):
        w.cache.copy_(prior)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(w.cache, ref), f"replay {rep}"
