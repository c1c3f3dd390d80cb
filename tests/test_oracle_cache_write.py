"""Pins for the oracle's paged K/V cache write and its e4m3fn encoder (CPU only)."""

import numpy as np
import torch

import oracle
from oracle.attention import kv_halves
from workloads import make_kv_write, to_numpy_bits


# e4m3fn encoder -------------------------------------------------------------
def _torch_codes(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encoder_matches_torch_on_every_bf16_in_range():
    # every bf16 value of magnitude <= 448 (torch's cast is RNE there; above it
    # torch gives NaN where the writer saturates)
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # the NaN patterns among them
        vals = oracle.bf16_to_f64(bits).astype(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    x = vals[keep]
    np.testing.assert_array_equal(oracle.e4m3fn_encode(x), _torch_codes(x))


def test_encoder_matches_torch_at_midpoints_and_neighbours():
    finite = oracle.E4M3FN_TABLE[:0x7F]  # 0 .. 448
    mids = ((finite[:-1] + finite[1:]) / 2).astype(np.float32)  # exact in fp32
    x = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(500))])
    x = np.concatenate([x, -x]).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3fn_encode(x), _torch_codes(x))


def test_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e4m3fn_encode(oracle.E4M3FN_TABLE[codes]), codes)


def test_encoder_saturates_and_keeps_nan():
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e30, np.inf, -464.0, -np.inf, np.nan, -np.nan],
                 dtype=np.float64)
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0xFF]
    assert oracle.e4m3fn_encode(x).tolist() == want


def test_encoder_ties_go_to_the_even_code():
    # 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3A; subnormal step 2^-9
    x = np.array([1.0625, 1.1875, 0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9, -1.0625])
    assert oracle.e4m3fn_encode(x).tolist() == [0x38, 0x3A, 0x00, 0x02, 0x02, 0xB8]


def test_quantize_rounds_the_quotient_to_fp32_first():
    # x / s lands a hair above the midpoint 1.0625 of 0x38 / 0x39 in exact
    # arithmetic but on it after rounding to fp32, where the tie goes to the
    # even code 0x38 (an fp64 quotient would give 0x39)
    found = 0
    for s in np.arange(1.01, 2.0, 0.001, dtype=np.float64).astype(np.float32):
        x = np.float32(1.0625 * float(s))
        if float(x) / float(s) > 1.0625 and np.float32(x) / np.float32(s) == np.float32(1.0625):
            assert oracle.quantize_e4m3fn(np.array([x]), float(s)).tolist() == [0x38]
            found += 1
    assert found > 10


def test_quantize_divides_in_fp32():
    # 1/3 is rounded to fp32 before encoding: (x / 3) for x = 3 * code value is exact
    vals = oracle.E4M3FN_TABLE[0x20:0x60].astype(np.float32) * np.float32(3.0)
    codes = oracle.quantize_e4m3fn(vals, 3.0)
    np.testing.assert_array_equal(codes, np.arange(0x20, 0x60, dtype=np.uint8))


# write_kv_cache -------------------------------------------------------------
def _case(**kw):
    base = dict(T=40, Hkv=2, D=8, P=4, pages=16, seed=21, pad_frac=0.2)
    base.update(kw)
    return make_kv_write(**base)


def _write(w, **kw):
    key, value = to_numpy_bits(w.key), to_numpy_bits(w.value)
    kc, vc = kv_halves(to_numpy_bits(w.cache), w.D)
    args = dict(k_scale=w.k_scale, v_scale=w.v_scale)
    args.update(kw)
    return oracle.write_kv_cache(key, value, w.in_dtype, kc, vc, w.slot_mapping.numpy(), w.P,
                                 w.cache_dtype, **args)


def test_padding_and_out_of_pool_slots_write_nothing():
    w = _case()
    slots = w.slot_mapping.numpy().copy()
    slots[::3] = -1
    slots[1::7] = w.pages * w.P + 5  # past the pool
    w.slot_mapping = torch.from_numpy(slots)
    kc, vc = _write(w)
    k0, v0 = kv_halves(to_numpy_bits(w.cache), w.D)
    written = np.zeros((w.pages, w.P), dtype=bool)
    for s in slots:
        if 0 <= s < w.pages * w.P:
            written[s // w.P, s % w.P] = True
    for page in range(w.pages):
        for off in range(w.P):
            if not written[page, off]:
                np.testing.assert_array_equal(kc[page, :, off], k0[page, :, off])
                np.testing.assert_array_equal(vc[page, :, off], v0[page, :, off])
    assert written.any()


def test_token_order_does_not_matter():
    w = _case()
    kc, vc = _write(w)
    perm = np.random.default_rng(5).permutation(w.T)
    w.key, w.value = w.key[perm], w.value[perm]
    w.slot_mapping = w.slot_mapping[perm]
    kc2, vc2 = _write(w)
    np.testing.assert_array_equal(kc, kc2)
    np.testing.assert_array_equal(vc, vc2)


def _attend_back(w, kc, vc, kv_dtype, k_scale, v_scale):
    """Paged attention of one query over the written tokens, in token order."""
    slots = w.slot_mapping.numpy()
    live = np.flatnonzero(slots >= 0)
    # one request whose pages are visited slot by slot: page table = the slots' pages
    # in token order, one token per page (page size 1 view of the written slots)
    def by_slot(c):  # [pages, Hkv, P, D] -> [slots, Hkv, 1, D]
        return c.transpose(0, 2, 1, 3).reshape(w.pages * w.P, w.Hkv, w.D)[slots[live]][:, :, None, :]

    k1, v1 = by_slot(kc), by_slot(vc)
    n = len(live)
    q = np.random.default_rng(9).standard_normal((1, 1, w.Hkv, w.D))
    bt = np.arange(n, dtype=np.int32)[None, :]
    O, L = oracle.paged_attention(q, "f64", k1, v1, kv_dtype, bt, np.array([n]), scale=0.3,
                                  k_scale=k_scale, v_scale=v_scale)
    return q, live, O, L


def test_write_then_attend_equals_attention_over_the_rows():
    w = _case(T=24, pad_frac=0.25)
    kc, vc = _write(w)
    q, live, O, L = _attend_back(w, kc, vc, w.cache_dtype, 1.0, 1.0)
    key = oracle.bf16_to_f64(to_numpy_bits(w.key))[live]
    value = oracle.bf16_to_f64(to_numpy_bits(w.value))[live]
    for h in range(w.Hkv):
        o, l = oracle.softmax_attention(q[0, 0, h][None, :], key[:, h], value[:, h], 0.3)
        np.testing.assert_allclose(O[0, 0, h], o[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[0, 0, h], l[0], rtol=0, atol=1e-12)


def test_fp8_write_then_attend_matches_scaled_codes():
    # the stored code times the scale is the value the read side uses: the
    # written cache read back with (k_scale, v_scale) equals attention over
    # scale * e4m3fn(x / scale), and stays within the e4m3 step of the input
    w = _case(T=24, pad_frac=0.25, cache_dtype="fp8_e4m3")
    kc, vc = _write(w)
    q, live, O, L = _attend_back(w, kc, vc, "fp8_e4m3", w.k_scale, w.v_scale)
    key = oracle.bf16_to_f64(to_numpy_bits(w.key))[live]
    value = oracle.bf16_to_f64(to_numpy_bits(w.value))[live]
    kq = oracle.E4M3FN_TABLE[oracle.quantize_e4m3fn(key, w.k_scale)] * w.k_scale
    vq = oracle.E4M3FN_TABLE[oracle.quantize_e4m3fn(value, w.v_scale)] * w.v_scale
    assert np.all(np.abs(kq - key) <= np.abs(key) / 16 + 2.0 ** -9 * w.k_scale)
    for h in range(w.Hkv):
        o, l = oracle.softmax_attention(q[0, 0, h][None, :], kq[:, h], vq[:, h], 0.3)
        np.testing.assert_allclose(O[0, 0, h], o[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[0, 0, h], l[0], rtol=0, atol=1e-12)


def test_same_dtype_write_copies_bits():
    w = _case(in_dtype="fp16", cache_dtype="fp16")
    kc, vc = _write(w)
    slots = w.slot_mapping.numpy()
    key, value = to_numpy_bits(w.key), to_numpy_bits(w.value)
    for t, s in enumerate(slots):
        if s >= 0:
            np.testing.assert_array_equal(kc[s // w.P, :, s % w.P], key[t])
            np.testing.assert_array_equal(vc[s // w.P, :, s % w.P], value[t])
