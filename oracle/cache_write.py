"""Paged K/V cache write (oracle; test infrastructure only).

Page vllm.v1.attention.backends.flashinfer_ts, ``do_kv_cache_update``: the new
key and value rows of every token go into the ``[pages, Hkv, P, 2*D]`` page
cache at that token's entry of ``slot_mapping``; the cache is viewed with its
token and head axes swapped and its last axis split into the K half (first D
values) and the V half (last D values), and the cache dtype string and the
layer's k_scale / v_scale go along with it.  The page shows that call, not the
body of the writer, so these readings fill the gaps:

* slot s is slot ``s % P`` of page ``s // P`` (page-major numbering, the same
  one the block table of the read side uses);
* a negative slot marks a padding token and writes nothing; so does a slot at
  or past ``pages * P`` (the writer never addresses outside the pool);
* a cache of the input's own 16-bit type receives the input bits unchanged;
* an e4m3fn cache stores ``e4m3fn(x / scale)`` with k_scale for K and v_scale
  for V, so that ``scale * stored`` is the real value exactly as the read side
  takes it: the quotient is the correctly rounded fp32 division, then rounded
  to the nearest finite e4m3fn value, ties to the even code, saturating at
  +-448 (a finite input never turns into NaN); NaN stays NaN;
* the slots of one call are distinct (with repeats, which token lands in a
  repeated slot is unspecified).
"""

from __future__ import annotations

import numpy as np

from .formats import E4M3FN_TABLE, decode

# non-negative finite e4m3fn values in code order 0x00 .. 0x7E (increasing)
_POS_VALUES = E4M3FN_TABLE[:0x7F].copy()
_E4M3FN_MAX = float(_POS_VALUES[-1])  # 448


def e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """Nearest finite e4m3fn code of each value (ties to the even code), saturating.

    Works on the exact value of each input (fp32 or fp64), by search in the
    table of finite values built from the format definition.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    flat, res = x.reshape(-1), out.reshape(-1)
    for i, v in enumerate(flat):
        if np.isnan(v):
            res[i] = 0x7F | (0x80 if np.signbit(v) else 0)
            continue
        sign = 0x80 if np.signbit(v) else 0
        a = min(abs(float(v)), _E4M3FN_MAX)
        hi = int(np.searchsorted(_POS_VALUES, a, side="left"))  # first value >= a
        if _POS_VALUES[hi] == a:
            code = hi
        else:
            lo = hi - 1
            dl, dh = a - _POS_VALUES[lo], _POS_VALUES[hi] - a
            if dl < dh:
                code = lo
            elif dh < dl:
                code = hi
            else:
                code = lo if lo % 2 == 0 else hi
        res[i] = code | sign
    return out


def quantize_e4m3fn(values: np.ndarray, scale: float) -> np.ndarray:
    """e4m3fn codes of ``values / scale``; the quotient is taken in fp32."""
    q = np.asarray(values, dtype=np.float32) / np.float32(scale)
    return e4m3fn_encode(q)


def convert_row(bits: np.ndarray, in_dtype: str, cache_dtype: str, scale: float) -> np.ndarray:
    """Stored form of input elements (bit patterns) in the cache's format."""
    if cache_dtype == in_dtype:
        return np.asarray(bits).copy()
    if cache_dtype == "fp8_e4m3":
        return quantize_e4m3fn(decode(bits, in_dtype), scale)
    raise ValueError(f"cannot store {in_dtype} into a {cache_dtype} cache")


def write_kv_cache(key_bits: np.ndarray, value_bits: np.ndarray, in_dtype: str,
                   k_cache: np.ndarray, v_cache: np.ndarray, slot_mapping: np.ndarray,
                   page_size: int, cache_dtype: str, k_scale: float = 1.0,
                   v_scale: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """Caches after writing the tokens.

    key_bits, value_bits: [T, Hkv, D] bit patterns of in_dtype.
    k_cache, v_cache: [pages, Hkv, P, D] bit patterns of cache_dtype (the two
    halves of the page); returned as new arrays, the inputs are not changed.
    """
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    capacity = kc.shape[0] * page_size
    for t, s in enumerate(np.asarray(slot_mapping, dtype=np.int64).tolist()):
        if s < 0 or s >= capacity:
            continue
        page, off = divmod(s, page_size)
        kc[page, :, off, :] = convert_row(key_bits[t], in_dtype, cache_dtype, k_scale)
        vc[page, :, off, :] = convert_row(value_bits[t], in_dtype, cache_dtype, v_scale)
    return kc, vc
