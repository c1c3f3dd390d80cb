"""Seeded random DASH segment geometries (fused and two-stage) against the oracle,
including topk = 63 (64 segments per query, the limit) and fp16 inputs."""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_segments, to_numpy_bits

from _parity import TOL_BF16, compare, gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"
N_CASES = 40


@pytest.fixture(scope="module")
def sap():
    import segmented_attention_paged_amd as m

    m.load()
    return m


def draw_case(i):
    rng = np.random.default_rng(7000 + i)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    topk = int(rng.choice([0, 1, 3, 8, 20, 63]))
    bs = int(rng.choice([8, 16, 24, 64]))
    local = int(rng.choice([8, 32, 40, 128]))
    N = int(rng.integers(1, 7))
    return dict(N=N, Hq=Hkv * G, Hkv=Hkv, D=int(rng.choice([64, 128])), topk=topk, bs=bs,
                local=local), float(rng.choice([0.0, 0.2, 0.6])), bool(rng.random() < 0.3)


@pytest.mark.parametrize("i", range(N_CASES))
@pytest.mark.parametrize("fused", [True, False])
def test_random_segments(sap, i, fused):
    geo, zero_frac, fp16 = draw_case(i)
    s = make_segments(seed=8000 + i, poison=True, zero_frac=zero_frac, name=f"seg{i}", **geo)
    O, L = oracle.segment_attention(to_numpy_bits(s.q), to_numpy_bits(s.k), to_numpy_bits(s.v),
                                    s.used.numpy(), s.bias.numpy(), topk=s.topk, bs=s.bs,
                                    local=s.local, scale=s.scale)
    d = s.to(DEV)
    q, k, v = d.q, d.k, d.v
    if fp16:  # the same values are not representable: compare against the fp16 inputs' oracle
        q, k, v = q.to(torch.float16), k.to(torch.float16), v.to(torch.float16)
        O, L = oracle.segment_attention(
            to_numpy_bits(q.cpu()), to_numpy_bits(k.cpu()), to_numpy_bits(v.cpu()),
            s.used.numpy(), s.bias.numpy(), topk=s.topk, bs=s.bs, local=s.local, scale=s.scale,
            q_dtype="fp16", kv_dtype="fp16")
    out, lse = sap.segment_attn_run(q, k, v, d.used, d.bias, bs=s.bs, local=s.local, fused=fused)
    compare(out, lse, O, L, TOL_BF16, what=f"case {i} {geo} zero={zero_frac} fp16={fp16}")
