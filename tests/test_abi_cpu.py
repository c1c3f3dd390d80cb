"""C-ABI checks that need no GPU: exports, the host copy of the integer plan, argument errors."""

import ctypes
import os
import random
import re

import numpy as np
import pytest
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")

sap = pytest.importorskip("segmented_attention_paged_amd")
try:
    LIB = sap.load()
except RuntimeError as e:  # not built
    pytest.skip(str(e), allow_module_level=True)

from segmented_attention_paged_amd import _lib  # noqa: E402


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert "paged_attn_run" in names and "split_kv_combine" in names and "segment_attn_combine" in names
    for n in names:
        assert hasattr(LIB, n), n
        assert n in _lib.SIGNATURES, f"{n} has no ctypes binding"
    assert set(_lib.SIGNATURES) == set(names)


def test_binding_has_every_entry_point_by_name():
    # the Python binding mirrors the C ABI name for name
    for n in declared_functions():
        assert callable(getattr(sap, n, None)), f"segmented_attention_paged_amd.{n} is missing"
    assert sap.pa_version() == LIB.pa_version().decode()
    assert sap.paged_attn_plan(64, 1, 32, 8, 128, 16, 512)["splits"] == sap.resolve_splits(
        64, 1, 32, 8, 128, 16, 512)


def test_version_and_last_error():
    assert b"gfx950" in LIB.pa_version()
    assert isinstance(LIB.pa_last_error(), bytes)


def _host_plan(bt, lens, sq, P, window, S, Hq=8, Hkv=2, D=128):
    return sap.paged_attn_describe_host(torch.from_numpy(bt), torch.from_numpy(lens), query_len=sq,
                                        Hq=Hq, Hkv=Hkv, D=D, page_size=P, window=window,
                                        num_splits=S)


@pytest.mark.parametrize("seed", range(6))
def test_host_plan_matches_oracle_bit_exact(seed):
    rng = random.Random(seed)
    for _ in range(40):
        P = rng.choice([1, 8, 16, 64])
        sq = rng.randint(1, 16)
        window = rng.choice([0, 0, rng.randint(1, 300)])
        B = rng.randint(1, 6)
        lens = np.array([rng.randint(0, 700) for _ in range(B)], np.int32)
        W = max(1, int(max(-(-int(L) // P) for L in lens)) + rng.randint(0, 2))
        bt = np.array([[rng.randrange(10000) for _ in range(W)] for _ in range(B)], np.int32)
        S = rng.choice([1, 2, 3, 7, 16, 64])
        l2, t2, rngs = _host_plan(bt, lens, sq, P, window, S)
        el, et = oracle.restrict_to_window(lens, bt, window, sq, P)
        assert np.array_equal(l2.numpy(), el)
        assert np.array_equal(t2.numpy(), et)
        for b in range(B):
            n_pages = -(-int(el[b]) // P)
            for s, (first, count) in enumerate(oracle.split_page_ranges(n_pages, S)):
                tok0 = first * P
                ntok = max(0, min((first + count) * P, int(el[b])) - tok0)
                assert rngs[b, s].tolist() == [first, count, tok0, ntok]


def test_host_plan_fixed_chunks():
    bt = np.arange(40, dtype=np.int32).reshape(1, 40)
    lens = np.array([37 * 16 + 5], np.int32)
    l2, t2, r = _host_plan(bt, lens, 1, 16, 0, -8)  # chunks of 8 pages
    assert r.shape[1] == 5  # ceil(40 / 8)
    assert r[0, :, 1].tolist() == [8, 8, 8, 8, 6] and r[0, -1, 3].item() == 5 * 16 + 5


def test_auto_splits_are_valid():
    for shape in [(64, 1, 32, 8, 128, 16, 512, 0), (32, 16, 32, 8, 128, 16, 2048, 0),
                  (32, 16, 32, 8, 128, 16, 2048, 4096), (2, 1, 4, 1, 64, 16, 7, 0)]:
        S = sap.resolve_splits(*shape[:7], window=shape[7], num_splits=0)
        assert S >= 1
        ws = sap.workspace_size(*shape[:7], window=shape[7], num_splits=0)
        assert (ws == 0) == (S == 1)
    assert sap.resolve_splits(8, 1, 64, 8, 128, 16, 8192, 0, 16) == 16
    # automatic policy at the measured shapes: decode 4, query block 8 (4 with a 4096 window)
    assert sap.resolve_splits(64, 1, 32, 8, 128, 16, 512, 0, 0) == 4
    assert sap.resolve_splits(32, 16, 32, 8, 128, 16, 2048, 0, 0) == 8
    assert sap.resolve_splits(32, 16, 32, 8, 128, 16, 2048, 4096, 0) == 4
    assert sap.resolve_splits(2, 1, 4, 1, 64, 16, 7, 0, 0) == 1


def test_window_width_matches_oracle():
    for w, sq, P, W in [(0, 4, 16, 99), (4096, 16, 16, 2048), (20, 4, 16, 7), (1, 1, 16, 3),
                        (2**31 - 1, 1, 16, 5)]:
        assert sap.window_width(w, sq, P, W) == oracle.window_table_width(w, sq, P, W)
    # a width past int32 saturates instead of wrapping negative
    assert oracle.window_table_width(2**31 - 1, 8, 1, 5) > 2**31 - 1
    assert sap.window_width(2**31 - 1, 8, 1, 5) == 2**31 - 1


def _desc(dtype=_lib.PA_BF16, D=128, P=16, hkv=2):
    return _lib.PaKvDesc(16, 16 + 2 * D, hkv * P * 2 * D, P * 2 * D, 2 * D, P, hkv, 4, dtype, 1.0, 1.0)


def _run(**kw):
    a = dict(q=16, q_dtype=_lib.PA_BF16, desc=_desc(), bt=16, bt_stride=4, bt_width=4, lens=16,
             B=1, sq=1, Hq=4, D=128, scale=0.1, window=0, S=1, out=16, out_dtype=_lib.PA_BF16,
             lse=None, ws=None, ws_bytes=0)
    a.update(kw)
    return LIB.paged_attn_run(a["q"], a["q_dtype"], ctypes.byref(a["desc"]), a["bt"], a["bt_stride"],
                              a["bt_width"], a["lens"], a["B"], a["sq"], a["Hq"], a["D"], a["scale"],
                              a["window"], a["S"], a["out"], a["out_dtype"], a["lse"], a["ws"],
                              a["ws_bytes"], None)


def test_argument_errors_are_status_codes():
    # each of these is rejected on the host before anything is enqueued
    assert _run(q_dtype=_lib.PA_F32) == _lib.PA_ENOTSUP
    assert "query dtype" in _lib.last_error()
    assert _run(desc=_desc(dtype=_lib.PA_FP16)) == _lib.PA_ENOTSUP  # bf16 q, fp16 cache
    assert _run(D=96) == _lib.PA_EINVAL
    assert _run(Hq=3) == _lib.PA_EINVAL  # not a multiple of Hkv = 2
    assert _run(out_dtype=_lib.PA_FP8_E4M3) == _lib.PA_ENOTSUP
    assert _run(q=None) == _lib.PA_EINVAL
    assert _run(q=8) == _lib.PA_EINVAL  # misaligned
    d = _desc(dtype=_lib.PA_FP8_E4M3)
    d.k_scale = 0.0
    assert _run(desc=d) == _lib.PA_EINVAL
    assert _run(bt_stride=2) == _lib.PA_EINVAL
    assert _run(S=4, lens=16) == _lib.PA_EWORKSPACE
    # row counts that would overflow 32-bit arithmetic
    assert _run(B=1 << 16, sq=1 << 15) == _lib.PA_EINVAL and "2^31" in _lib.last_error()
    assert _run(Hq=2 * 1024, sq=1 << 21) == _lib.PA_EINVAL  # (Hq/Hkv)*sq = 2^31
    # empty problems are no-ops
    assert _run(B=0, q=None, out=None) == _lib.PA_OK
    assert _run(sq=0, q=None, out=None) == _lib.PA_OK


def test_segment_argument_errors():
    def seg(**kw):
        a = dict(q=16, qd=_lib.PA_BF16, k=16, v=16, kd=_lib.PA_BF16, used=16, bias=16, N=2, topk=2,
                 bs=64, local=128, Hq=4, Hkv=2, D=128, scale=0.1, fused=1, out=16,
                 od=_lib.PA_BF16)
        a.update(kw)
        return LIB.segment_attn_run(a["q"], a["qd"], a["k"], a["v"], a["kd"], a["used"], a["bias"],
                                    a["N"], a["topk"], a["bs"], a["local"], a["Hq"], a["Hkv"], a["D"],
                                    a["scale"], a["fused"], a["out"], a["od"], None, None, 0, None)
    assert seg(bs=60) == _lib.PA_EINVAL and "multiples of 8" in _lib.last_error()
    assert seg(local=124) == _lib.PA_EINVAL
    assert seg(qd=_lib.PA_F32) == _lib.PA_ENOTSUP
    assert seg(fused=0) == _lib.PA_EWORKSPACE
    assert seg(N=0, q=None) == _lib.PA_OK
    assert seg(N=1 << 26, topk=63) == _lib.PA_EINVAL and "2^31" in _lib.last_error()


def test_missing_library_fails_loudly():
    # a fresh interpreter pointed at a library that does not exist: the binding raises,
    # it does not fall back to anything
    import subprocess
    import sys
    code = ("import segmented_attention_paged_amd._lib as L\n"
            "L.LIB_PATH = '/nonexistent/libsapaged.so'\n"
            "try:\n"
            "    L.load()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert "raised:" in r.stdout and "is missing" in r.stdout, r.stdout + r.stderr
