"""Pins for the oracle's paged attention, Split-KV and DASH segment combine (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import kv_halves
from workloads import make_paged, make_segments, to_numpy_bits

from _brute import bf16_bits_to_float, brute_attention_row, brute_paged


def _np(inp):
    q = to_numpy_bits(inp.q)
    cache = to_numpy_bits(inp.cache)
    k, v = kv_halves(cache, inp.D)
    return q, k, v, inp.block_table.numpy(), inp.seq_lens.numpy()


def _run(inp, **kw):
    q, k, v, bt, lens = _np(inp)
    args = dict(scale=inp.scale, window=inp.window, k_scale=inp.k_scale, v_scale=inp.v_scale)
    args.update(kw)
    return oracle.paged_attention(q, "bf16", k, v, inp.kv_dtype, bt, lens, **args)


def _tiny(**kw):
    base = dict(B=3, sq=2, Hq=4, Hkv=2, D=8, P=4, seq_lens=[1, 7, 13], seed=11, poison=True)
    base.update(kw)
    return make_paged(**base)


# P1 -------------------------------------------------------------------------
def test_single_key_returns_its_value():
    inp = _tiny(seq_lens=[1, 1, 1])
    O, LSE = _run(inp)
    q, k, v, bt, lens = _np(inp)
    for b in range(inp.B):
        page = bt[b, 0]
        for h in range(inp.Hq):
            kvh = h // (inp.Hq // inp.Hkv)
            V = oracle.bf16_to_f64(v[page, kvh, 0])
            K = oracle.bf16_to_f64(k[page, kvh, 0])
            for t in range(inp.sq):
                assert np.array_equal(O[b, t, h], V)  # weight exactly 1
                logit = inp.scale * float(np.dot(oracle.bf16_to_f64(q[b, t, h]), K))
                assert LSE[b, t, h] == pytest.approx(logit, abs=1e-13)


# P2 -------------------------------------------------------------------------
def test_identical_keys_give_mean_value():
    inp = _tiny(seq_lens=[5, 9, 16], poison=False)
    # make every K row of every page equal, leaving V random
    c = inp.cache
    c[..., : inp.D] = c[0, 0, 0, : inp.D]
    O, LSE = _run(inp)
    q, k, v, bt, lens = _np(inp)
    Krow = oracle.bf16_to_f64(k[0, 0, 0])
    for b in range(inp.B):
        L = int(lens[b])
        for h in range(inp.Hq):
            kvh = h // 2
            Vs = np.stack([oracle.bf16_to_f64(v[bt[b, j // 4], kvh, j % 4]) for j in range(L)])
            for t in range(inp.sq):
                np.testing.assert_allclose(O[b, t, h], Vs.mean(0), rtol=0, atol=1e-13)
                s = inp.scale * float(np.dot(oracle.bf16_to_f64(q[b, t, h]), Krow))
                assert LSE[b, t, h] == pytest.approx(s + math.log(L), abs=1e-12)


# P3 -------------------------------------------------------------------------
def test_weights_sum_to_one():
    rng = np.random.default_rng(0)
    for n in [1, 2, 17, 300]:
        w = oracle.attention_weights(rng.normal(size=(5, 16)) * 3, rng.normal(size=(n, 16)) * 3, 0.7)
        assert np.all(np.abs(w.sum(1) - 1) < 1e-12) and np.all(w >= 0)


# P4 -------------------------------------------------------------------------
def test_page_permutation_invariance():
    inp = _tiny(poison=False, seq_lens=[3, 11, 16])
    O1, L1 = _run(inp)
    perm = torch.randperm(inp.pool, generator=torch.Generator().manual_seed(9))
    cache2 = torch.empty_like(inp.cache)
    cache2[perm] = inp.cache  # page p moves to perm[p]
    bt2 = perm[inp.block_table.long()].to(torch.int32)
    q, _, _, _, lens = _np(inp)
    k2, v2 = kv_halves(to_numpy_bits(cache2), inp.D)
    O2, L2 = oracle.paged_attention(q, "bf16", k2, v2, "bf16", bt2.numpy(), lens, scale=inp.scale)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


# P7 -------------------------------------------------------------------------
def test_brute_force_loops_agree():
    inp = _tiny(seq_lens=[2, 6, 13], window=0)
    O, LSE = _run(inp)
    q, k, v, bt, lens = _np(inp)
    cache = to_numpy_bits(inp.cache)
    res = brute_paged(q.tolist(), cache, bt.tolist(), lens.tolist(), Hkv=inp.Hkv, P=inp.P,
                      D=inp.D, scale=inp.scale, dec=bf16_bits_to_float)
    for (b, t, h), (out, lse) in res.items():
        np.testing.assert_allclose(O[b, t, h], out, rtol=0, atol=1e-12)
        assert LSE[b, t, h] == pytest.approx(lse, abs=1e-12)


def test_matches_torch_sdpa_fp64():
    inp = make_paged(B=2, sq=3, Hq=8, Hkv=2, D=16, P=4, seq_lens=[16, 16], seed=21)
    # identity table: request b owns pages in table order; rebuild contiguous K/V
    O, LSE = _run(inp)
    cache = inp.cache.to(torch.float64)
    G = inp.Hq // inp.Hkv
    for b in range(inp.B):
        pages = inp.block_table[b].long()
        kv = cache[pages]  # [4 pages, Hkv, P, 2D]
        kv = kv.permute(1, 0, 2, 3).reshape(inp.Hkv, -1, 2 * inp.D)  # [Hkv, L, 2D]
        K = kv[..., : inp.D].repeat_interleave(G, 0)
        V = kv[..., inp.D:].repeat_interleave(G, 0)
        qq = inp.q[b].to(torch.float64).permute(1, 0, 2)  # [Hq, sq, D]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, K, V, scale=inp.scale)
        np.testing.assert_allclose(O[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        s = inp.scale * qq @ K.transpose(1, 2)
        lse = torch.logsumexp(s, -1).permute(1, 0).numpy()
        np.testing.assert_allclose(LSE[b], lse, rtol=0, atol=1e-12)


def test_fp8_query_scale_folding_equals_prescaled_query():
    inp = make_paged(B=2, sq=3, Hq=4, Hkv=2, D=16, P=4, seq_lens=[5, 11], seed=23,
                     kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3")
    q8 = to_numpy_bits(inp.q)
    k, v = kv_halves(to_numpy_bits(inp.cache), inp.D)
    bt, lens = inp.block_table.numpy(), inp.seq_lens.numpy()
    kw = dict(scale=inp.scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
    O, L = oracle.paged_attention(q8, "fp8_e4m3", k, v, "fp8_e4m3", bt, lens, q_scale=inp.q_scale, **kw)
    qf = oracle.e4m3fn_to_f64(q8) * inp.q_scale
    O2, L2 = oracle.paged_attention(qf, "f64", k, v, "fp8_e4m3", bt, lens, **kw)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, L2, rtol=0, atol=1e-12)
    assert inp.q.dtype == torch.uint8 and 0.5 <= inp.q_scale <= 2.0


# Causal mask with an exact per-token window --------------------------------
@pytest.mark.parametrize("window", [0, 1, 3, 9])
def test_causal_brute_force_loops_agree(window):
    inp = _tiny(seq_lens=[2, 6, 13], sq=3)
    O, LSE = _run(inp, causal=True, window=window)
    q, k, v, bt, lens = _np(inp)
    res = brute_paged(q.tolist(), to_numpy_bits(inp.cache), bt.tolist(), lens.tolist(),
                      Hkv=inp.Hkv, P=inp.P, D=inp.D, scale=inp.scale, dec=bf16_bits_to_float,
                      window=window, causal=True)
    for (b, t, h), (out, lse) in res.items():
        np.testing.assert_allclose(O[b, t, h], out, rtol=0, atol=1e-12)
        assert LSE[b, t, h] == pytest.approx(lse, abs=1e-12)


@pytest.mark.parametrize("window", [0, 5])
def test_causal_matches_torch_sdpa_with_mask_fp64(window):
    inp = make_paged(B=2, sq=4, Hq=8, Hkv=2, D=16, P=4, seq_lens=[16, 16], seed=22)
    O, LSE = _run(inp, causal=True, window=window)
    cache = inp.cache.to(torch.float64)
    G = inp.Hq // inp.Hkv
    L, sq = 16, inp.sq
    pos = torch.arange(sq)[:, None] + (L - sq)
    j = torch.arange(L)[None, :]
    allowed = j <= pos
    if window:
        allowed &= j >= pos - (window - 1)
    for b in range(inp.B):
        kv = cache[inp.block_table[b].long()].permute(1, 0, 2, 3).reshape(inp.Hkv, -1, 2 * inp.D)
        K = kv[..., : inp.D].repeat_interleave(G, 0)
        V = kv[..., inp.D:].repeat_interleave(G, 0)
        qq = inp.q[b].to(torch.float64).permute(1, 0, 2)  # [Hq, sq, D]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, K, V, attn_mask=allowed,
                                                               scale=inp.scale)
        np.testing.assert_allclose(O[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        s = (inp.scale * qq @ K.transpose(1, 2)).masked_fill(~allowed, float("-inf"))
        np.testing.assert_allclose(LSE[b], torch.logsumexp(s, -1).permute(1, 0).numpy(),
                                   rtol=0, atol=1e-12)


def test_causal_token_equals_decode_of_truncated_sequence():
    # token t of a causal block sees exactly what a lone query at its position
    # sees in a dense decode over the first L - sq + t + 1 keys
    inp = _tiny(seq_lens=[3, 9, 13], sq=3)
    O, LSE = _run(inp, causal=True)
    q, k, v, bt, lens = _np(inp)
    for t in range(inp.sq):
        lens_t = lens - (inp.sq - 1 - t)
        Ot, Lt = oracle.paged_attention(q[:, t:t + 1], "bf16", k, v, "bf16", bt, lens_t,
                                        scale=inp.scale)
        np.testing.assert_allclose(O[:, t], Ot[:, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE[:, t], Lt[:, 0], rtol=0, atol=1e-12)


def test_causal_single_token_is_dense_and_wide_window_is_none():
    inp = _tiny(seq_lens=[1, 7, 13], sq=1)
    np.testing.assert_array_equal(_run(inp, causal=True)[0], _run(inp)[0])
    inp3 = _tiny(seq_lens=[3, 7, 13], sq=3)
    a, la = _run(inp3, causal=True, window=20)
    b, lb = _run(inp3, causal=True)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_causal_token_before_the_sequence_sees_nothing():
    # L < sq: the first tokens sit at negative positions and see no key
    inp = _tiny(seq_lens=[1, 2, 13], sq=3)
    O, LSE = _run(inp, causal=True)
    assert np.all(LSE[0, :2] == -np.inf) and np.all(O[0, :2] == 0)
    assert np.all(np.isfinite(LSE[0, 2])) and np.all(LSE[1, 0] == -np.inf)


# P13 ------------------------------------------------------------------------
def test_lse_matches_logaddexp():
    rng = np.random.default_rng(1)
    for n in [1, 3, 50]:
        q = rng.normal(size=(4, 8))
        K = rng.normal(size=(n, 8)) * 4
        _, lse = oracle.softmax_attention(q, K, np.zeros((n, 8)), 0.9)
        for r in range(4):
            assert lse[r] == pytest.approx(np.logaddexp.reduce(0.9 * (K @ q[r])), abs=1e-12)


def test_empty_sequence_gives_zero_and_minus_inf():
    inp = _tiny(seq_lens=[0, 5, 0])
    O, LSE = _run(inp)
    assert np.all(O[0] == 0) and np.all(np.isneginf(LSE[0]))
    assert np.all(O[2] == 0) and np.all(np.isneginf(LSE[2]))
    assert np.all(np.isfinite(O[1]))


# P9 -------------------------------------------------------------------------
def test_window_equals_attention_on_page_aligned_suffix():
    inp = _tiny(seq_lens=[40, 23, 64], window=9, P=8, Hq=4, Hkv=1)
    Ow, Lw = _run(inp)
    q, k, v, bt, lens = _np(inp)
    for b in range(inp.B):
        L = int(lens[b])
        start = max(0, (L - (9 + inp.sq - 1)) // 8) * 8
        res = brute_paged(q[b:b + 1].tolist(), to_numpy_bits(inp.cache), bt[b:b + 1].tolist(),
                          [L], Hkv=1, P=8, D=inp.D, scale=inp.scale, window=9,
                          dec=bf16_bits_to_float)
        for (_, t, h), (out, lse) in res.items():
            np.testing.assert_allclose(Ow[b, t, h], out, rtol=0, atol=1e-12)
        assert start % 8 == 0


def test_window_at_least_length_equals_no_window():
    inp = _tiny(seq_lens=[7, 13, 2], window=0, poison=False)
    O0, L0 = _run(inp)
    for w in [13, 14, 1000]:
        Ow, Lw = _run(inp, window=w)
        assert np.array_equal(O0, Ow) and np.array_equal(L0, Lw)


def test_window_via_restricted_table_is_same_attention():
    inp = _tiny(seq_lens=[40, 23, 64], window=9, P=8, Hq=4, Hkv=1)
    Ow, Lw = _run(inp)
    q, k, v, bt, lens = _np(inp)
    l2, t2 = oracle.restrict_to_window(lens, bt, 9, inp.sq, 8)
    O2, L2 = oracle.paged_attention(q, "bf16", k, v, "bf16", t2, l2, scale=inp.scale)
    assert np.array_equal(Ow, O2) and np.array_equal(Lw, L2)


# P10 ------------------------------------------------------------------------
def test_gqa_equals_mha_with_repeated_kv():
    inp = _tiny(poison=False, Hq=6, Hkv=2)
    O, LSE = _run(inp)
    q, k, v, bt, lens = _np(inp)
    G = 3
    k3 = np.repeat(k, G, axis=1)
    v3 = np.repeat(v, G, axis=1)
    O3, L3 = oracle.paged_attention(q, "bf16", k3, v3, "bf16", bt, lens, scale=inp.scale)
    assert np.array_equal(O, O3) and np.array_equal(LSE, L3)


# P11 ------------------------------------------------------------------------
def test_fp8_scale_folding_equals_prescaled_values():
    inp = _tiny(kv_dtype="fp8_e4m3", poison=False)
    assert 0.5 <= inp.k_scale <= 2 and 0.5 <= inp.v_scale <= 2
    O, LSE = _run(inp)
    q, k, v, bt, lens = _np(inp)
    kf = oracle.e4m3fn_to_f64(k) * inp.k_scale
    vf = oracle.e4m3fn_to_f64(v) * inp.v_scale
    O2, L2 = oracle.paged_attention(q, "bf16", kf, vf, "f64", bt, lens, scale=inp.scale)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(LSE, L2, rtol=0, atol=1e-13)


# P12 ------------------------------------------------------------------------
def test_strided_halves_equal_compact_planes():
    inp = _tiny(poison=False)
    O, LSE = _run(inp)
    q, k, v, bt, lens = _np(inp)
    kc, vc = np.ascontiguousarray(k), np.ascontiguousarray(v)
    assert kc.strides != k.strides
    O2, L2 = oracle.paged_attention(q, "bf16", kc, vc, "bf16", bt, lens, scale=inp.scale)
    assert np.array_equal(O, O2) and np.array_equal(LSE, L2)


def test_poison_never_reaches_results():
    inp = _tiny(poison=True, seq_lens=[5, 1, 13])
    O, LSE = _run(inp)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(LSE))


# P5 -------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 3, 16, 64])
@pytest.mark.parametrize("window", [0, 9])
def test_split_then_combine_equals_unsplit(S, window):
    inp = _tiny(seq_lens=[1, 30, 61], P=4, window=window, poison=True)
    O, LSE = _run(inp)
    q, k, v, bt, lens = _np(inp)
    po, pl = oracle.split_partials(q, "bf16", k, v, "bf16", bt, lens, scale=inp.scale,
                                   num_splits=S, window=window)
    assert po.shape[0] == S
    Oc, Lc = oracle.combine_splits(po, pl)
    np.testing.assert_allclose(Oc, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lc, LSE, rtol=0, atol=1e-12)
    if S == 64:  # more splits than pages: some splits are empty
        assert np.any(np.isneginf(pl))


def test_combine_all_dead_is_zero():
    po = np.full((3, 2, 5, 4), np.nan)
    pl = np.full((3, 2, 5), -np.inf)
    O, L = oracle.combine_splits(po, pl)
    assert np.all(O == 0) and np.all(np.isneginf(L))


# DASH segments (P6, P8) ----------------------------------------------------
def _seg(**kw):
    base = dict(N=5, Hq=4, Hkv=2, D=8, topk=3, bs=8, local=16, seed=31, poison=True, zero_frac=0.3)
    base.update(kw)
    return make_segments(**base)


def _seg_np(s):
    return (to_numpy_bits(s.q), to_numpy_bits(s.k), to_numpy_bits(s.v), s.used.numpy(),
            s.bias.numpy())


def _seg_run(s, q, k, v, used, bias):
    return oracle.segment_attention(q, k, v, used, bias, topk=s.topk, bs=s.bs, local=s.local,
                                    scale=s.scale)


def test_segments_two_stage_equals_union_closed_form():
    s = _seg()
    q, k, v, used, bias = _seg_np(s)
    assert (used == 0).any() and (used > 0).any()
    O, L = _seg_run(s, q, k, v, used, bias)
    Ou, Lu = oracle.segment_attention_union(q, k, v, used, bias, topk=s.topk, bs=s.bs,
                                            local=s.local, scale=s.scale)
    np.testing.assert_allclose(O, Ou, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lu, rtol=0, atol=1e-12)
    assert np.all(np.isfinite(O))


def test_segments_brute_force_union():
    s = _seg(N=2)
    q, k, v, used, bias = _seg_np(s)
    O, L = _seg_run(s, q, k, v, used, bias)
    per = s.topk * s.bs + s.local
    for n in range(s.N):
        for h in range(s.Hq):
            kvh = h // 2
            keys, vals, kb = [], [], []
            for g in range(s.topk + 1):
                base = n * per + (g * s.bs if g < s.topk else s.topk * s.bs)
                for j in range(int(used[n, g])):
                    keys.append([bf16_bits_to_float(x) for x in k[base + j, kvh]])
                    vals.append([bf16_bits_to_float(x) for x in v[base + j, kvh]])
                    kb.append(float(bias[n, g]) if g < s.topk else 0.0)
            qrow = [bf16_bits_to_float(x) for x in q[n, h]]
            out, lse = brute_attention_row(qrow, keys, vals, s.scale, kb)
            np.testing.assert_allclose(O[n, h], out, rtol=0, atol=1e-12)
            assert L[n, h] == pytest.approx(lse, abs=1e-12) or (math.isinf(lse) and np.isneginf(L[n, h]))


def test_dead_segment_changes_nothing():
    s = _seg(poison=False, zero_frac=0.0)
    q, k, v, used, bias = _seg_np(s)
    used = used.copy()
    used[1, 2] = 0
    used[3, s.topk] = 0  # a dead local segment
    O, L = _seg_run(s, q, k, v, used, bias)
    per = s.topk * s.bs + s.local
    k2, v2, b2 = k.copy(), v.copy(), bias.copy()
    base = 1 * per + 2 * s.bs
    k2[base:base + s.bs] = 0x7FC0  # NaN
    v2[base:base + s.bs] = 0x4000
    b2[1, 2] = 1e6
    base = 3 * per + s.topk * s.bs
    k2[base:base + s.local] = 0x7FC0
    v2[base:base + s.local] = 0x7FC0
    O2, L2 = _seg_run(s, q, k2, v2, used, b2)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_all_dead_query_is_zero():
    s = _seg(poison=False)
    q, k, v, used, bias = _seg_np(s)
    used = used.copy()
    used[2] = 0
    O, L = _seg_run(s, q, k, v, used, bias)
    assert np.all(O[2] == 0) and np.all(np.isneginf(L[2]))


def test_minus_inf_bias_weighs_nothing():
    # The page's combine takes a softmax over LSE + bias and then nan_to_num: a live
    # segment whose bias is -inf gets weight e^-inf = 0, exactly like a dead one, and a
    # query whose every live logit is -inf gets the NaN softmax zeroed, i.e. output 0.
    s = _seg(poison=False, zero_frac=0.0)
    q, k, v, used, bias = _seg_np(s)
    b2 = bias.copy()
    b2[1, 2] = -np.inf           # one remote segment of query 1
    b2[4, :] = -np.inf           # every remote segment of query 4 (the local one is live)
    b2[0, :] = -np.inf           # query 0: every remote segment, and its local one is dead
    u2 = used.copy()
    u2[0, s.topk] = 0
    O, L = _seg_run(s, q, k, v, u2, b2)
    ref_used = u2.copy()
    ref_used[1, 2] = 0
    ref_used[4, :s.topk] = 0
    ref_used[0, :] = 0
    Or, Lr = _seg_run(s, q, k, v, ref_used, bias)
    np.testing.assert_allclose(O, Or, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L[1:], Lr[1:], rtol=0, atol=1e-14)
    assert np.all(O[0] == 0) and np.all(np.isneginf(L[0]))
    Ou, Lu = oracle.segment_attention_union(q, k, v, u2, b2, topk=s.topk, bs=s.bs,
                                            local=s.local, scale=s.scale)
    np.testing.assert_allclose(Ou, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lu, L, rtol=0, atol=1e-12)
    # brute force over the union of live prefixes for the three queries touched
    per = s.topk * s.bs + s.local
    for n in (0, 1, 4):
        for h in range(s.Hq):
            kvh = h // 2
            keys, vals, kb = [], [], []
            for g in range(s.topk + 1):
                base = n * per + (g * s.bs if g < s.topk else s.topk * s.bs)
                for j in range(int(u2[n, g])):
                    keys.append([bf16_bits_to_float(x) for x in k[base + j, kvh]])
                    vals.append([bf16_bits_to_float(x) for x in v[base + j, kvh]])
                    kb.append(float(b2[n, g]) if g < s.topk else 0.0)
            qrow = [bf16_bits_to_float(x) for x in q[n, h]]
            out, lse = brute_attention_row(qrow, keys, vals, s.scale, kb)
            np.testing.assert_allclose(O[n, h], out, rtol=0, atol=1e-12)
            assert (math.isinf(lse) and np.isneginf(L[n, h])) or L[n, h] == pytest.approx(lse, abs=1e-12)


def test_full_segments_zero_bias_is_plain_attention():
    s = _seg(N=2, poison=False, zero_frac=0.0)
    q, k, v, used, bias = _seg_np(s)
    used = np.array([[s.bs] * s.topk + [s.local]] * s.N, np.int32)
    bias = np.zeros_like(bias)
    O, L = _seg_run(s, q, k, v, used, bias)
    per = s.topk * s.bs + s.local
    for n in range(s.N):
        for h in range(s.Hq):
            kvh = h // 2
            K = torch.tensor(oracle.bf16_to_f64(k[n * per:(n + 1) * per, kvh]))
            V = torch.tensor(oracle.bf16_to_f64(v[n * per:(n + 1) * per, kvh]))
            qq = torch.tensor(oracle.bf16_to_f64(q[n, h]))[None]
            ref = torch.nn.functional.scaled_dot_product_attention(qq[None], K[None], V[None],
                                                                   scale=s.scale)[0, 0]
            np.testing.assert_allclose(O[n, h], ref.numpy(), rtol=0, atol=1e-12)
            assert L[n, h] == pytest.approx(float(torch.logsumexp(s.scale * K @ qq[0], 0)), abs=1e-12)


def test_segment_combine_is_bias_weighted_softmax():
    # Direct check of the combine against hand arithmetic on two live segments.
    po = np.zeros((1, 3, 1, 2))
    po[0, 0, 0] = [1.0, 0.0]
    po[0, 1, 0] = [0.0, 1.0]
    po[0, 2, 0] = [5.0, 5.0]
    pl = np.array([[[0.0], [math.log(3.0)], [7.0]]])
    used = np.array([[4, 2, 0]])
    bias = np.array([[math.log(2.0), 0.0]])
    out, lse = oracle.combine_segments(po, pl, used, bias)
    # logits: ln2, ln3 ; weights 2/5, 3/5; local dead
    np.testing.assert_allclose(out[0, 0], [0.4, 0.6], atol=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(5.0), abs=1e-15)
