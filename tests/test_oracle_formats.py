"""Pins for the oracle's number-format decoding (CPU only)."""

import json
import math
import os

import numpy as np
import torch

from oracle import E4M3FN_TABLE, bf16_to_f64, e4m3fn_to_f64, fp16_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3fn_hand_worked_points():
    spec = json.load(open(os.path.join(GOLDEN, "e4m3fn_points.json")))
    for byte_s, val_s, _why in spec["points"]:
        byte = int(byte_s, 16)
        got = float(e4m3fn_to_f64(np.array([byte], np.uint8))[0])
        want = float(val_s)
        if math.isnan(want):
            assert math.isnan(got), byte_s
        else:
            assert got == want, (byte_s, got, want)
            assert math.copysign(1.0, got) == math.copysign(1.0, want), byte_s


def test_e4m3fn_table_matches_torch_for_all_bytes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = E4M3FN_TABLE
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(ours))
    assert np.array_equal(ref[~nan_ref], ours[~nan_ref])
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(ours[~nan_ref]))


def test_e4m3fn_bit_layout_by_integer_arithmetic():
    # independent restatement: value = (-1)^s * 2^(e-7) * (1 + m/8) for e > 0,
    # (-1)^s * 2^-6 * m/8 for e = 0
    for byte in range(256):
        s, e, m = byte >> 7, (byte >> 3) & 15, byte & 7
        if e == 15 and m == 7:
            assert math.isnan(E4M3FN_TABLE[byte])
            continue
        mag = math.ldexp(8 + m, e - 10) if e else math.ldexp(m, -9)
        assert E4M3FN_TABLE[byte] == (-mag if s else mag)


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(4096, generator=g) * 100).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_to_f64(bits), x.to(torch.float64).numpy())
    # specials
    specials = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F80, 0xFF80, 0x0001], np.uint16)
    vals = bf16_to_f64(specials)
    assert vals[2] == 1.0 and vals[3] == -1.0
    assert np.isinf(vals[4]) and np.isinf(vals[5])
    assert vals[6] == 2.0 ** -133  # smallest bf16 subnormal


def test_fp16_decode_matches_torch():
    g = torch.Generator().manual_seed(6)
    x = torch.randn(1024, generator=g).to(torch.float16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fp16_to_f64(bits), x.to(torch.float64).numpy())
