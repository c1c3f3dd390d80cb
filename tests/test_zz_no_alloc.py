"""paged_attn_run_noalloc (Split-KV partials in the library's static per-GPU scratch)
against paged_attn_run (partials in a caller workspace): same plan and kernels, so the
outputs agree bit for bit, and both meet the oracle's tolerances.  Called through the
C ABI by the ctypes binding."""

import pytest
import torch

from workloads import make_paged

from _parity import TOL_BF16, compare, gpu_available, oracle_paged

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


@pytest.fixture(scope="module")
def sap():
    import segmented_attention_paged_amd as m

    m.load()
    return m


def _noalloc(sap, inp, num_splits):
    k, v = sap.kv_halves(inp.cache, inp.D)
    out = torch.empty((inp.B, inp.sq, inp.Hq, inp.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((inp.B, inp.sq, inp.Hq), dtype=torch.float32, device=DEV)
    before = torch.cuda.memory_allocated()
    sap.paged_attn_run_noalloc(inp.q, k, v, inp.block_table, inp.seq_lens, scale=inp.scale,
                               window=inp.window, num_splits=num_splits, out=out, lse=lse)
    assert torch.cuda.memory_allocated() == before  # nothing allocated on the call path
    return out, lse


def _reference(sap, inp, num_splits):
    k, v = sap.kv_halves(inp.cache, inp.D)
    return sap.paged_attn_run(inp.q, k, v, inp.block_table, inp.seq_lens, scale=inp.scale,
                              window=inp.window, num_splits=num_splits)


def test_noalloc_equals_paged_attn_run_on_two_calls_in_a_row(sap):
    # a 16-token block (library split choice, several splits) then a smaller decode batch
    # with an explicit split count: the second call finds the first call's partials in
    # the scratch and must not be affected by them
    big = make_paged(B=8, sq=16, Hq=32, Hkv=8, D=128, P=16, seq_lens=("uniform", 16, 3000),
                     seed=71, poison=True, device=DEV)
    small = make_paged(B=3, sq=1, Hq=32, Hkv=8, D=128, P=16, seq_lens=[1, 200, 1500], seed=72,
                       poison=True, window=300, device=DEV)
    cases = [(big, 0), (small, 5)]
    for inp, S in cases:
        W = inp.block_table.shape[1]
        assert sap.resolve_splits(inp.B, inp.sq, inp.Hq, inp.Hkv, inp.D, inp.P, W, inp.window,
                                  S) > 1
    got = [_noalloc(sap, inp, S) for inp, S in cases]  # the two scratch calls, back to back
    torch.cuda.synchronize()
    for (inp, S), (out, lse) in zip(cases, got):
        ref_out, ref_lse = _reference(sap, inp, S)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"B={inp.B}"
        assert torch.equal(lse, ref_lse), f"B={inp.B}"
        O, L = oracle_paged(inp)
        compare(out, lse, O, L, TOL_BF16, what=f"noalloc B={inp.B} sq={inp.sq} S={S}")


def test_noalloc_single_pass_needs_no_scratch(sap):
    inp = make_paged(B=4, sq=1, Hq=16, Hkv=2, D=64, P=16, seq_lens=[0, 17, 100, 999], seed=73,
                     poison=True, device=DEV)
    out, lse = _noalloc(sap, inp, 1)
    ref_out, ref_lse = _reference(sap, inp, 1)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse, ref_lse)


def test_noalloc_rejects_partials_beyond_its_scratch(sap):
    # 64 splits of 32 x 16 tokens x 32 heads x D=128 need 512 MiB of partials
    inp = make_paged(B=32, sq=16, Hq=32, Hkv=8, D=128, P=16, seq_lens=[16] * 32, seed=74,
                     device=DEV)
    W = inp.block_table.shape[1]
    assert sap.workspace_size(inp.B, inp.sq, inp.Hq, inp.Hkv, inp.D, inp.P, W, 0, 64) > 96 << 20
    with pytest.raises(sap.PagedAttnError, match="scratch") as ei:
        _noalloc(sap, inp, 64)
    assert ei.value.code == -3  # PA_EWORKSPACE
