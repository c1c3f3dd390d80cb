"""The Python binding rejects malformed tensors before any device pointer is passed on.

The kernels index every buffer from the shapes alone, so a wrong shape, dtype,
layout or device must stop the call on the host.  Shape and dtype checks come
before the device check, so CPU tensors exercise them here without a GPU.
"""

import pytest
import torch

import segmented_attention_paged_amd as sap


def _paged(B=2, sq=3, Hq=4, Hkv=2, D=64, P=16, W=5, pages=8):
    q = torch.zeros((B, sq, Hq, D), dtype=torch.bfloat16)
    cache = torch.zeros((pages, Hkv, P, 2 * D), dtype=torch.bfloat16)
    k, v = sap.kv_halves(cache, D)
    bt = torch.zeros((B, W), dtype=torch.int32)
    lens = torch.full((B,), 20, dtype=torch.int32)
    return q, k, v, bt, lens


def test_paged_run_shape_dtype_and_device_errors():
    q, k, v, bt, lens = _paged()
    with pytest.raises(ValueError, match="out must have shape"):
        sap.paged_attn_run(q, k, v, bt, lens, scale=0.1, out=torch.empty((2, 3, 4, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse must have shape"):
        sap.paged_attn_run(q, k, v, bt, lens, scale=0.1, lse=torch.empty((2, 3), dtype=torch.float32))
    with pytest.raises(TypeError, match="lse must be"):
        sap.paged_attn_run(q, k, v, bt, lens, scale=0.1, lse=torch.empty((2, 3, 4), dtype=torch.float16))
    with pytest.raises(ValueError, match="seq_lens must have shape"):
        sap.paged_attn_run(q, k, v, bt, lens[:1], scale=0.1)
    with pytest.raises(TypeError, match="seq_lens must be"):
        sap.paged_attn_run(q, k, v, bt, lens.to(torch.int64), scale=0.1)
    with pytest.raises(ValueError, match="block_table must be"):
        sap.paged_attn_run(q, k, v, bt[:1], lens, scale=0.1)
    with pytest.raises(ValueError, match="block_table must be"):
        sap.paged_attn_run(q, k, v, bt.t().contiguous().t(), lens, scale=0.1)  # column-major
    with pytest.raises(ValueError, match="q must be contiguous"):
        sap.paged_attn_run(q.transpose(1, 2).contiguous().transpose(1, 2), k, v, bt, lens, scale=0.1)
    # well-formed, but on the host: refused before any pointer reaches the library
    with pytest.raises(ValueError, match="GPU"):
        sap.paged_attn_run(q, k, v, bt, lens, scale=0.1)


def test_kv_views_must_carry_the_query_head_dim():
    # a [pages, Hkv, P, 2*64] cache split into 64-wide halves, read with a D=128 query:
    # each V read would run into the next token's K and past the pool's last slot
    q = torch.zeros((2, 1, 4, 128), dtype=torch.bfloat16)
    _, k, v, bt, lens = _paged(sq=1, D=64)
    with pytest.raises(ValueError, match="head_dim"):
        sap.paged_attn_run(q, k, v, bt, lens, scale=0.1)
    with pytest.raises(ValueError, match="head_dim"):
        sap.paged_attn_partial(q, k, v, bt, lens, scale=0.1, num_splits=2)
    with pytest.raises(ValueError, match="head_dim"):
        sap.paged_attn_run(q[..., :64].contiguous(), k, v[..., :32], bt, lens, scale=0.1)


def test_partial_and_combine_buffer_errors():
    q, k, v, bt, lens = _paged()
    with pytest.raises(ValueError, match="part_o must have shape"):
        sap.paged_attn_partial(q, k, v, bt, lens, scale=0.1, num_splits=2,
                               part_o=torch.empty((1, 6, 4, 64)))
    po = torch.zeros((3, 5, 4, 64))
    with pytest.raises(ValueError, match="part_lse must have shape"):
        sap.split_kv_combine(po, torch.zeros((3, 5, 2)))
    with pytest.raises(ValueError, match="out must have shape"):
        sap.split_kv_combine(po, torch.zeros((3, 5, 4)), out=torch.empty((5, 4, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        sap.split_kv_combine(po, torch.zeros((3, 5, 4)))
    N, G, Hq, D = 2, 3, 4, 64
    pso, psl = torch.zeros((N, G, Hq, D)), torch.zeros((N, G, Hq))
    used, bias = torch.ones((N, G), dtype=torch.int32), torch.zeros((N, G - 1))
    with pytest.raises(TypeError, match="used must be"):
        sap.segment_attn_combine(pso, psl, used.to(torch.int64), bias)
    with pytest.raises(ValueError, match="bias must have shape"):
        sap.segment_attn_combine(pso, psl, used, torch.zeros((N, G)))
    with pytest.raises(ValueError, match="bias"):
        sap.segment_attn_combine(pso, psl, used, None)


def test_segment_run_layout_errors():
    N, Hq, Hkv, D, topk, bs, local = 2, 4, 2, 64, 2, 8, 16
    T = N * (topk * bs + local)
    q = torch.zeros((N, Hq, D), dtype=torch.bfloat16)
    k = torch.zeros((T, Hkv, D), dtype=torch.bfloat16)
    used = torch.ones((N, topk + 1), dtype=torch.int32)
    bias = torch.zeros((N, topk))
    with pytest.raises(ValueError, match="k must have shape"):
        sap.segment_attn_run(q, k[:-1], k, used, bias, bs=bs, local=local)
    with pytest.raises(ValueError, match="k must be contiguous"):
        strided = torch.zeros((T, Hkv, 2 * D), dtype=torch.bfloat16)[..., :D]
        sap.segment_attn_run(q, strided, k, used, bias, bs=bs, local=local)
    with pytest.raises(ValueError, match="used must have shape"):
        sap.segment_attn_run(q, k, k, used[:, :2], bias, bs=bs, local=local)
    with pytest.raises(ValueError, match="GPU"):
        sap.segment_attn_run(q, k, k, used, bias, bs=bs, local=local)


def test_describe_host_needs_host_tensors_of_the_right_type():
    _, _, _, bt, lens = _paged()
    with pytest.raises(TypeError, match="seq_lens must be"):
        sap.paged_attn_describe_host(bt, lens.to(torch.int64), query_len=3, Hq=4, Hkv=2, D=64,
                                     page_size=16)
    lens_out, table, ranges = sap.paged_attn_describe_host(bt, lens, query_len=3, Hq=4, Hkv=2, D=64,
                                                           page_size=16)
    assert lens_out.tolist() == [20, 20]


def test_kv_write_geometry_errors():
    cache = torch.zeros((4, 2, 16, 128), dtype=torch.bfloat16)
    k, v = sap.kv_halves(cache, 64)
    key = torch.zeros((3, 2, 32), dtype=torch.bfloat16)
    slots = torch.zeros(3, dtype=torch.int64)
    with pytest.raises(ValueError, match="head_dim"):
        sap.paged_kv_write(key, key, slots, k, v)
    key = torch.zeros((3, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        sap.paged_kv_write(key, key, slots, k, v)
