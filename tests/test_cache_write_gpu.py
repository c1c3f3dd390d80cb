"""GPU parity of the paged K/V cache write (through the C ABI) against the oracle.

Same-type writes and fp8 quantisation are integer/byte results: compared bit
for bit over the whole cache (written and untouched slots alike).
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import kv_halves as np_halves
from workloads import make_kv_write, make_paged, to_numpy_bits

from _parity import TOL_BF16, TOL_FP8, compare, gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


@pytest.fixture(scope="module")
def sap():
    import segmented_attention_paged_amd as m

    m.load()
    return m


def _gpu_write(sap, w, k=None, v=None):
    cache = w.cache.to(DEV)
    key, value, slots = w.key.to(DEV), w.value.to(DEV), w.slot_mapping.to(DEV)
    if k is None:
        k, v = sap.kv_halves(cache, w.D)
    sap.paged_kv_write(key, value, slots, k, v, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    return cache, k, v


def _oracle_write(w, slots=None):
    kc, vc = np_halves(to_numpy_bits(w.cache), w.D)
    s = w.slot_mapping.numpy() if slots is None else slots
    return oracle.write_kv_cache(to_numpy_bits(w.key), to_numpy_bits(w.value), w.in_dtype, kc, vc,
                                 s, w.P, w.cache_dtype, k_scale=w.k_scale, v_scale=w.v_scale)


CASES = {
    "bf16": dict(T=300, Hkv=4, D=128, P=16, pages=64, in_dtype="bf16", cache_dtype="bf16"),
    "fp16": dict(T=300, Hkv=4, D=128, P=16, pages=64, in_dtype="fp16", cache_dtype="fp16"),
    "bf16_fp8": dict(T=300, Hkv=4, D=128, P=16, pages=64, in_dtype="bf16", cache_dtype="fp8_e4m3"),
    "fp16_fp8": dict(T=200, Hkv=2, D=64, P=16, pages=32, in_dtype="fp16", cache_dtype="fp8_e4m3"),
    "fp8_saturating": dict(T=100, Hkv=2, D=128, P=16, pages=16, in_dtype="bf16",
                           cache_dtype="fp8_e4m3", value_scale=400.0),
    "fp8_subnormal": dict(T=100, Hkv=2, D=128, P=16, pages=16, in_dtype="bf16",
                          cache_dtype="fp8_e4m3", value_scale=2e-3),
    "page1_d64": dict(T=50, Hkv=3, D=64, P=1, pages=80, in_dtype="bf16", cache_dtype="bf16"),
    "page64_d256": dict(T=90, Hkv=1, D=256, P=64, pages=4, in_dtype="bf16", cache_dtype="bf16"),
    "all_slots": dict(T=256, Hkv=2, D=64, P=16, pages=16, in_dtype="bf16", cache_dtype="fp8_e4m3",
                      pad_frac=0.0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_write_matches_oracle_bitwise(sap, name):
    kw = dict(seed=31, pad_frac=0.15)
    kw.update(CASES[name])
    w = make_kv_write(**kw)
    cache, _, _ = _gpu_write(sap, w)
    kc, vc = _oracle_write(w)
    gk, gv = np_halves(to_numpy_bits(cache.cpu()), w.D)
    np.testing.assert_array_equal(gk, kc)
    np.testing.assert_array_equal(gv, vc)


def test_special_values_quantise_like_the_oracle(sap):
    w = make_kv_write(T=64, Hkv=1, D=128, P=16, pages=8, seed=5, cache_dtype="fp8_e4m3")
    w.k_scale, w.v_scale = 1.0, 0.75
    key = to_numpy_bits(w.key).copy()
    # every e4m3 midpoint, its bf16 neighbours, +-0, +-inf, NaN, huge and tiny values
    fin = oracle.E4M3FN_TABLE[:0x7F]
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    specials = np.concatenate([mids, -mids, np.float32([0.0, -0.0, np.inf, -np.inf, np.nan,
                                                        1e30, -1e30, 2.0 ** -12, -2.0 ** -12])])
    b = (specials.view(np.uint32) >> 16).astype(np.uint16)  # bf16 truncation keeps them exact
    key.reshape(-1)[: b.size] = b
    key.reshape(-1)[b.size: 2 * b.size] = b + 1
    w.key = torch.from_numpy(key.view(np.int16)).view(torch.bfloat16)
    cache, _, _ = _gpu_write(sap, w)
    kc, vc = _oracle_write(w)
    gk, gv = np_halves(to_numpy_bits(cache.cpu()), w.D)
    np.testing.assert_array_equal(gk, kc)
    np.testing.assert_array_equal(gv, vc)


def test_quotient_ties_after_fp32_rounding(sap):
    # values whose exact quotient x / s sits a hair above an e4m3fn midpoint but
    # rounds onto it in fp32: the tie must go to the even code, as in the oracle
    cases = []
    for s in np.arange(1.01, 2.0, 0.001, dtype=np.float64).astype(np.float32):
        for mid in (1.0625, 2.375, 0.15625, 13.0):
            x = np.float32(mid * float(s))
            if float(x) / float(s) != mid and np.float32(x) / np.float32(s) == np.float32(mid):
                cases.append((float(s), x))
    # the cache write takes bf16/fp16 rows: keep the cases whose x is an fp16 value
    cases = [(s, x) for s, x in cases if np.float32(np.float16(x)) == x][:8]
    assert cases
    for sc, x in cases:
        w = make_kv_write(T=4, Hkv=1, D=64, P=16, pages=1, seed=2, in_dtype="fp16",
                          cache_dtype="fp8_e4m3")
        w.k_scale = w.v_scale = sc
        w.key = torch.full((w.T, 1, w.D), float(x), dtype=torch.float16)
        w.value = torch.full((w.T, 1, w.D), -float(x), dtype=torch.float16)
        cache, _, _ = _gpu_write(sap, w)
        kc, vc = _oracle_write(w)
        gk, gv = np_halves(to_numpy_bits(cache.cpu()), w.D)
        np.testing.assert_array_equal(gk, kc)
        np.testing.assert_array_equal(gv, vc)


def test_separate_planes_and_token_strides(sap):
    # K and V in separate compact planes; key/value rows taken from a wider
    # fused buffer (token stride larger than Hkv*D)
    w = make_kv_write(T=70, Hkv=2, D=64, P=8, pages=20, seed=8, pad_frac=0.1)
    k = torch.full((w.pages, w.Hkv, w.P, w.D), 3.0, dtype=torch.bfloat16, device=DEV)
    v = torch.full_like(k, -5.0)
    wide = torch.zeros((w.T, 3, w.Hkv, w.D), dtype=torch.bfloat16)
    wide[:, 1], wide[:, 2] = w.key, w.value
    wide = wide.to(DEV)
    sap.paged_kv_write(wide[:, 1], wide[:, 2], w.slot_mapping.to(DEV), k, v)
    torch.cuda.synchronize()
    kc0 = to_numpy_bits(torch.full((w.pages, w.Hkv, w.P, w.D), 3.0, dtype=torch.bfloat16))
    vc0 = to_numpy_bits(torch.full((w.pages, w.Hkv, w.P, w.D), -5.0, dtype=torch.bfloat16))
    kc, vc = oracle.write_kv_cache(to_numpy_bits(w.key), to_numpy_bits(w.value), "bf16", kc0, vc0,
                                   w.slot_mapping.numpy(), w.P, "bf16")
    np.testing.assert_array_equal(to_numpy_bits(k.cpu()), kc)
    np.testing.assert_array_equal(to_numpy_bits(v.cpu()), vc)


def test_padding_out_of_pool_and_empty(sap):
    w = make_kv_write(T=40, Hkv=2, D=128, P=16, pages=4, seed=3)
    slots = w.slot_mapping.numpy().copy()
    slots[::2] = -1
    slots[1::4] = w.pages * w.P + 7
    w.slot_mapping = torch.from_numpy(slots)
    cache, k, v = _gpu_write(sap, w)
    kc, vc = _oracle_write(w)
    gk, gv = np_halves(to_numpy_bits(cache.cpu()), w.D)
    np.testing.assert_array_equal(gk, kc)
    np.testing.assert_array_equal(gv, vc)
    before = cache.clone()
    empty = torch.empty((0, w.Hkv, w.D), dtype=torch.bfloat16, device=DEV)
    sap.paged_kv_write(empty, empty, torch.empty(0, dtype=torch.int64, device=DEV), k, v)
    torch.cuda.synchronize()
    assert torch.equal(cache, before)


def test_rejects_bad_arguments(sap):
    w = make_kv_write(T=8, Hkv=2, D=64, P=16, pages=2, seed=1, cache_dtype="fp8_e4m3")
    cache = w.cache.to(DEV)
    k, v = sap.kv_halves(cache, w.D)
    key, value, slots = w.key.to(DEV), w.value.to(DEV), w.slot_mapping.to(DEV)
    with pytest.raises(sap.PagedAttnError, match="PA_EINVAL"):
        sap.paged_kv_write(key, value, slots, k, v, k_scale=0.0, v_scale=1.0)
    with pytest.raises(sap.PagedAttnError, match="PA_ENOTSUP"):
        sap.paged_kv_write(key.float(), value.float(), slots, k, v)
    c16 = torch.zeros((2, 2, 16, 2 * 64), dtype=torch.float16, device=DEV)
    k16, v16 = sap.kv_halves(c16, 64)
    with pytest.raises(sap.PagedAttnError, match="PA_ENOTSUP"):
        sap.paged_kv_write(key, value, slots, k16, v16)  # bf16 rows into an fp16 cache


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_write_then_attend(sap, kv_dtype):
    # a batch whose K/V rows are all written by paged_kv_write into an empty
    # (NaN-filled) pool, then read by paged_attn_run: matches the oracle's
    # attention over the oracle-written cache
    ref = make_paged(B=3, sq=2, Hq=8, Hkv=2, D=128, P=16, seq_lens=[5, 40, 130], seed=12)
    bt, lens = ref.block_table.numpy(), ref.seq_lens.numpy()
    rows_k, rows_v, slots = [], [], []
    kh, vh = np_halves(to_numpy_bits(ref.cache), ref.D)
    for b in range(ref.B):
        for j in range(int(lens[b])):
            page, off = int(bt[b, j // ref.P]), j % ref.P
            rows_k.append(kh[page, :, off])
            rows_v.append(vh[page, :, off])
            slots.append(page * ref.P + off)
    key = torch.from_numpy(np.stack(rows_k).view(np.int16)).view(torch.bfloat16)
    value = torch.from_numpy(np.stack(rows_v).view(np.int16)).view(torch.bfloat16)
    slot_t = torch.tensor(slots, dtype=torch.int64)
    pages = ref.cache.shape[0]
    k_scale, v_scale = (1.0, 1.0) if kv_dtype == "bf16" else (0.8, 1.3)
    if kv_dtype == "bf16":
        cache = torch.full((pages, ref.Hkv, ref.P, 2 * ref.D), float("nan"), dtype=torch.bfloat16)
    else:
        cache = torch.full((pages, ref.Hkv, ref.P, 2 * ref.D), 0x7F, dtype=torch.uint8)
    kc, vc = oracle.write_kv_cache(to_numpy_bits(key), to_numpy_bits(value), "bf16",
                                   *np_halves(to_numpy_bits(cache), ref.D), slot_t.numpy(), ref.P,
                                   kv_dtype, k_scale=k_scale, v_scale=v_scale)
    gcache = cache.to(DEV)
    gk, gv = sap.kv_halves(gcache, ref.D)
    sap.paged_kv_write(key.to(DEV), value.to(DEV), slot_t.to(DEV), gk, gv, k_scale=k_scale,
                       v_scale=v_scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_halves(to_numpy_bits(gcache.cpu()), ref.D)[0], kc)
    out, lse = sap.paged_attn_run(ref.q.to(DEV), gk, gv, ref.block_table.to(DEV),
                                  ref.seq_lens.to(DEV), scale=ref.scale, k_scale=k_scale,
                                  v_scale=v_scale)
    O, L = oracle.paged_attention(to_numpy_bits(ref.q), "bf16", kc, vc, kv_dtype, bt, lens,
                                  scale=ref.scale, k_scale=k_scale, v_scale=v_scale)
    compare(out, lse, O, L, TOL_BF16 if kv_dtype == "bf16" else TOL_FP8)


@pytest.mark.parametrize("cache_dtype", ["fp8_e4m3", "bf16"])
def test_full_size_sampled(sap, cache_dtype):
    # the measured shape: 65536 tokens x 8 kv heads x D=128 into a 16-slot-page
    # pool twice as large; 64 sampled tokens checked against the oracle, every
    # untouched slot checked unchanged
    w = make_kv_write(T=65536, Hkv=8, D=128, P=16, pages=8192, seed=40, cache_dtype=cache_dtype,
                      pad_frac=0.05, device=DEV)
    before = w.cache.clone()
    sap.paged_kv_write(w.key, w.value, w.slot_mapping, *sap.kv_halves(w.cache, w.D),
                       k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    slots = w.slot_mapping.cpu().numpy()
    written = torch.zeros(w.pages * w.P, dtype=torch.bool)
    written[torch.from_numpy(slots[slots >= 0])] = True
    per_slot = w.cache.view(w.pages, w.Hkv, w.P, -1).permute(0, 2, 1, 3).reshape(w.pages * w.P, -1)
    before_slot = before.view(w.pages, w.Hkv, w.P, -1).permute(0, 2, 1, 3).reshape(w.pages * w.P, -1)
    untouched = (~written).to(DEV)
    assert torch.equal(per_slot[untouched], before_slot[untouched])
    rng = np.random.default_rng(2)
    for t in rng.choice(np.flatnonzero(slots >= 0), size=64, replace=False):
        s = int(slots[t])
        kq = oracle.convert_row(to_numpy_bits(w.key[t].cpu()), "bf16", cache_dtype, w.k_scale)
        vq = oracle.convert_row(to_numpy_bits(w.value[t].cpu()), "bf16", cache_dtype, w.v_scale)
        row = to_numpy_bits(w.cache[s // w.P, :, s % w.P].cpu())
        np.testing.assert_array_equal(row[:, : w.D], kq)
        np.testing.assert_array_equal(row[:, w.D:], vq)
