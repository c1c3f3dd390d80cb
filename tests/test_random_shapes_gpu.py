"""Seeded random shapes through the whole paged path against the oracle.

Each case draws a geometry (requests, query length, head counts and ratio, head
dim, page size, lengths including empty and shorter-than-block requests, window,
splits, causal or dense, cache and query types) from a fixed seed, so failures
reproduce by case number.
"""

import numpy as np
import pytest
import torch

from workloads import make_paged

from _parity import TOL_BF16, TOL_FP8, compare, gpu_available, oracle_paged, run_paged

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"
N_CASES = 160


@pytest.fixture(scope="module")
def sap():
    import segmented_attention_paged_amd as m

    m.load()
    return m


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    sq = int(rng.choice([1, 1, 2, 3, 4, 5, 8, 16, 17]))
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([1, 8, 16, 16, 24, 64]))
    B = int(rng.integers(1, 9))
    hi = int(rng.choice([40, 300, 1500]))
    lens = [int(x) for x in rng.integers(0, hi + 1, size=B)]
    if rng.random() < 0.3:
        lens[0] = int(rng.integers(0, sq + 1))  # empty or shorter than the block
    kv_dtype = "fp8_e4m3" if rng.random() < 0.3 else "bf16"
    q_dtype = "fp8_e4m3" if (kv_dtype == "fp8_e4m3" and rng.random() < 0.5) else "bf16"
    window = int(rng.choice([0, 0, 1, 7, 33, 200]))
    causal = bool(rng.random() < 0.4)
    splits = int(rng.choice([0, 1, 2, 5, -1, -3]))
    return dict(B=B, sq=sq, Hq=Hkv * G, Hkv=Hkv, D=D, P=P, seq_lens=lens, kv_dtype=kv_dtype,
                q_dtype=q_dtype), dict(window=window, causal=causal, splits=splits)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(sap, i):
    geo, run = draw_case(i)
    inp = make_paged(seed=5000 + i, poison=True, name=f"rand{i}", **geo).to(DEV)
    out, lse = run_paged(inp, num_splits=run["splits"], window=run["window"], causal=run["causal"])
    O, L = oracle_paged(inp, window=run["window"], causal=run["causal"])
    tol = TOL_FP8 if geo["kv_dtype"] == "fp8_e4m3" else TOL_BF16
    compare(out, lse, O, L, tol, what=f"case {i}: {geo} {run}")
