"""GPU parity at the five workloads' full sizes, in the launch configuration the bench times.

Every output row is compared: the oracle evaluates one request at a time (all its kv
heads) from host copies of exactly the pages that request reads, so host memory holds
one request's pages at once; every DASH query is compared in both the fused and the
two-stage form.  The bars apply to the whole output: max-abs and the LSE error over
every row, mean-abs over every value.
"""

import time

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


class Tally:
    """Error statistics accumulated over slices of one output."""

    def __init__(self, what):
        self.what, self.max_abs, self.abs_sum, self.count, self.lse = what, 0.0, 0.0, 0, 0.0

    def add(self, out, lse, O_ref, L_ref):
        o = out.astype(np.float64)
        mask = ~np.isnan(L_ref)
        og, oref = o[mask], O_ref[mask]
        assert np.all(np.isfinite(og)), f"{self.what}: non-finite output"
        err = np.abs(og - oref)
        self.max_abs = max(self.max_abs, float(err.max(initial=0)))
        self.abs_sum += float(err.sum())
        self.count += err.size
        lg, lr = lse.astype(np.float64)[mask], L_ref[mask]
        dead = np.isneginf(lr)
        assert np.array_equal(np.isneginf(lg), dead), f"{self.what}: -inf LSE pattern differs"
        assert np.all(og[dead] == 0), f"{self.what}: rows without keys are not 0"
        if (~dead).any():
            self.lse = max(self.lse, float(np.abs(lg[~dead] - lr[~dead]).max()))
        return int(mask.sum())

    def check(self, tol):
        mean = self.abs_sum / max(self.count, 1)
        print(f"{self.what}: {self.count} values, max-abs {self.max_abs:.3e}, mean-abs {mean:.3e}, "
              f"lse {self.lse:.3e}", flush=True)
        assert self.max_abs <= tol["max_abs"], f"{self.what}: max-abs {self.max_abs:.3e}"
        assert mean <= tol["mean_abs"], f"{self.what}: mean-abs {mean:.3e}"
        assert self.lse <= tol["lse"], f"{self.what}: lse err {self.lse:.3e}"


@pytest.mark.parametrize("name,causal", [
    ("c1_tiny", False), ("c2_gqa_decode", False), ("c3_query_block", False),
    ("c3w_query_block_window", False), ("c4_split_kv", False), ("c4f_split_kv_fp8", False),
    # the blocks the bench also times with the causal mask, and with fp8 queries
    ("c3_query_block", True), ("c3w_query_block_window", True), ("c3f_query_block_fp8", False),
])
def test_full_size_every_row(sap, name, causal):
    t0 = time.perf_counter()
    inp = paged_config(name, poison=True, device=DEV)
    out, lse = run_paged(inp, causal=causal)  # the config's own num_splits (0 = library choice)
    torch.cuda.synchronize()
    out_h = out.float().cpu().numpy()
    lse_h = lse.cpu().numpy()
    tally = Tally(f"{name} causal={causal}")
    rows = 0
    for b in range(inp.B):
        O, L = oracle_paged(inp, requests=[b], causal=causal)
        rows += tally.add(out_h[b], lse_h[b], O[b], L[b])
    assert rows == inp.B * inp.sq * inp.Hq  # every (request, token, head) row compared
    tally.check(TOL_FP8 if inp.kv_dtype == "fp8_e4m3" else TOL_BF16)
    print(f"{name} causal={causal}: {time.perf_counter() - t0:.1f} s", flush=True)


@pytest.mark.parametrize("fused", [True, False])
def test_full_size_dash_segments_every_query(sap, fused):
    t0 = time.perf_counter()
    s = segment_config("c5_dash_segments", poison=True, device=DEV)
    out, lse = sap.segment_attn_run(s.q, s.k, s.v, s.used, s.bias, bs=s.bs, local=s.local,
                                    fused=fused)
    torch.cuda.synchronize()
    used = s.used.cpu().numpy()
    O, L = oracle.segment_attention(to_numpy_bits(s.q.cpu()), to_numpy_bits(s.k.cpu()),
                                    to_numpy_bits(s.v.cpu()), used, s.bias.cpu().numpy(),
                                    topk=s.topk, bs=s.bs, local=s.local, scale=s.scale)
    assert not np.isnan(L).any()  # every query evaluated
    compare(out, lse, O, L, TOL_BF16, what=f"c5 fused={fused}")
    print(f"c5 fused={fused}: {time.perf_counter() - t0:.1f} s", flush=True)
