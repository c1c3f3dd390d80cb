"""Malformed inputs the library clamps instead of faulting, per the C header:
sequence lengths past the table (or negative), page indices outside the pool, and
DASH `used` counts outside [0, capacity].  Each case must give, bit for bit, what
the same call gives with the clamped value, and that must match the oracle."""

import pytest
import torch

from workloads import make_paged, make_segments

from _parity import TOL_BF16, compare, gpu_available, oracle_paged, run_paged

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"

# decode rows (key-split kernel) and a 64-row query block (LDS-ring kernel)
SHAPES = {"decode": dict(sq=1, Hq=8, Hkv=2), "block": dict(sq=16, Hq=8, Hkv=2)}


@pytest.fixture(scope="module")
def sap():
    import segmented_attention_paged_amd as m

    m.load()
    return m


def _bitwise(a, b, what):
    (oa, la), (ob, lb) = a, b
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), what
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), what


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("splits", [1, 3])
def test_lengths_are_clamped_to_the_table(sap, shape, splits):
    # 4-page table rows (64 keys); request 0 claims 100 keys, request 2 a negative count
    inp = make_paged(B=3, D=128, P=16, seq_lens=[64, 64, 30], seed=51, **SHAPES[shape]).to(DEV)
    assert inp.block_table.shape[1] == 4
    ref = run_paged(inp, num_splits=splits)
    O, L = oracle_paged(inp)
    compare(*ref, O, L, TOL_BF16, what="clamped lengths")
    inp.seq_lens.copy_(torch.tensor([100, 64, 30], dtype=torch.int32))
    _bitwise(run_paged(inp, num_splits=splits), ref, "length past the table")
    inp.seq_lens.copy_(torch.tensor([64, 64, -5], dtype=torch.int32))
    out, lse = run_paged(inp, num_splits=splits)
    assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))
    _bitwise((out[:2], lse[:2]), (ref[0][:2], ref[1][:2]), "negative length")


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("splits", [1, 2])
def test_page_indices_are_clamped_into_the_pool(sap, shape, splits):
    inp = make_paged(B=2, D=128, P=16, seq_lens=[70, 50], seed=52, **SHAPES[shape]).to(DEV)
    pages = inp.cache.shape[0]
    bad = inp.block_table.clone()
    bad[0, 1] = -7
    bad[1, 2] = 1_000_000
    fixed = inp.block_table.clone()
    fixed[0, 1] = 0
    fixed[1, 2] = pages - 1
    inp.block_table.copy_(fixed)
    ref = run_paged(inp, num_splits=splits)
    compare(*ref, *oracle_paged(inp), TOL_BF16, what="clamped table")
    inp.block_table.copy_(bad)
    _bitwise(run_paged(inp, num_splits=splits), ref, "page index outside the pool")


@pytest.mark.parametrize("fused", [True, False])
def test_segment_counts_are_clamped(sap, fused):
    s = make_segments(N=3, Hq=8, Hkv=2, D=128, topk=3, bs=16, local=32, seed=53, zero_frac=0.0,
                      name="clamp").to(DEV)
    good = s.used.clone()
    good[0, 0] = 16  # capacity of a remote segment
    good[1, 3] = 32  # capacity of the local segment
    good[2, 1] = 0
    bad = good.clone()
    bad[0, 0] = 16 + 50
    bad[1, 3] = 1 << 20
    bad[2, 1] = -3

    def run(used):
        return sap.segment_attn_run(s.q, s.k, s.v, used, s.bias, bs=s.bs, local=s.local, fused=fused)

    _bitwise(run(bad), run(good), f"used outside [0, cap], fused={fused}")
