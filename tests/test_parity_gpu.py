"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same bytes."""

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import kv_halves as np_halves
from workloads import make_paged, make_segments, paged_config, to_numpy_bits

from _parity import TOL_BF16, TOL_FP8, compare, gpu_available, oracle_paged, run_paged

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


@pytest.fixture(scope="module")
def sap():
    import segmented_attention_paged_amd as m

    m.load()
    return m


def _as(inp, q_dtype=None, kv16=None):
    """Re-type a bf16 workload (q and/or a 16-bit cache) to fp16, NaN poison kept."""
    if q_dtype is not None:
        inp.q = inp.q.to(q_dtype)
    if kv16 is not None:
        inp.cache = inp.cache.to(kv16)
        inp.kv_dtype = "fp16"
    return inp


SMALL = {
    "decode_d128_g4": dict(B=6, sq=1, Hq=32, Hkv=8, D=128, P=16, seq_lens=[1, 15, 16, 17, 300, 700]),
    "decode_d64_g8": dict(B=5, sq=1, Hq=16, Hkv=2, D=64, P=16, seq_lens=[0, 33, 64, 129, 500]),
    "block_sq16_g4": dict(B=4, sq=16, Hq=32, Hkv=8, D=128, P=16, seq_lens=[16, 100, 257, 640]),
    "block_sq16_window": dict(B=4, sq=16, Hq=32, Hkv=8, D=128, P=16, seq_lens=[16, 100, 257, 640],
                              window=100),
    "block_sq3_rt2": dict(B=3, sq=3, Hq=8, Hkv=1, D=128, P=16, seq_lens=[3, 50, 333]),
    "rows128_rg2": dict(B=2, sq=16, Hq=16, Hkv=2, D=64, P=16, seq_lens=[40, 200]),
    "page64": dict(B=3, sq=2, Hq=8, Hkv=2, D=128, P=64, seq_lens=[1, 100, 400]),
    "page8": dict(B=3, sq=1, Hq=4, Hkv=1, D=64, P=8, seq_lens=[7, 8, 90]),
    "page24_window": dict(B=2, sq=4, Hq=8, Hkv=4, D=128, P=24, seq_lens=[25, 200], window=30),
    "fp8_bf16q": dict(B=4, sq=1, Hq=16, Hkv=2, D=128, P=16, seq_lens=[5, 64, 300, 999],
                      kv_dtype="fp8_e4m3"),
    "fp8_sq16_window": dict(B=2, sq=16, Hq=8, Hkv=2, D=64, P=16, seq_lens=[20, 400],
                            kv_dtype="fp8_e4m3", window=64),
    "decode_sq4_window": dict(B=3, sq=4, Hq=8, Hkv=2, D=128, P=16, seq_lens=[4, 60, 300],
                              window=40),
    "page1": dict(B=2, sq=1, Hq=4, Hkv=2, D=64, P=1, seq_lens=[5, 40]),
    "many_requests": dict(B=70, sq=1, Hq=8, Hkv=2, D=64, P=16, seq_lens=("uniform", 0, 200)),
    # larger shapes: 300 requests of plain multi-head attention (G = 1), a 16-token block
    # with G = 16 (256 rows: four row groups), and 1024-token pages (64 tiles per page)
    "mha_300_requests": dict(B=300, sq=2, Hq=4, Hkv=4, D=64, P=16, seq_lens=("uniform", 0, 300)),
    "block_sq16_g16": dict(B=2, sq=16, Hq=64, Hkv=4, D=128, P=16, seq_lens=[100, 1000],
                           window=200),
    "page1024": dict(B=2, sq=4, Hq=8, Hkv=2, D=64, P=1024, seq_lens=[1500, 3000]),
}
SPLITS = [1, 0, 3, -2, 64]


def _small(name, seed=7):
    return make_paged(seed=seed, poison=True, name=name, **SMALL[name]).to(DEV)


@pytest.mark.parametrize("splits", [1, 0, 2, 3, 7, -1])
def test_c1_tiny_full_compare(sap, splits):
    inp = paged_config("c1_tiny", poison=True).to(DEV)
    out, lse = run_paged(inp, num_splits=splits)
    O, L = oracle_paged(inp)
    compare(out, lse, O, L, TOL_BF16, what=f"c1 S={splits}")


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("splits", SPLITS)
def test_small_cases(sap, name, splits):
    inp = _small(name)
    out, lse = run_paged(inp, num_splits=splits)
    O, L = oracle_paged(inp)
    tol = TOL_FP8 if inp.kv_dtype == "fp8_e4m3" else TOL_BF16
    compare(out, lse, O, L, tol, what=f"{name} S={splits}")


@pytest.mark.parametrize("name", ["decode_d128_g4", "block_sq16_window", "page24_window"])
def test_fp16(sap, name):
    inp = _as(_small(name), q_dtype=torch.float16, kv16=torch.float16)
    out, lse = run_paged(inp, num_splits=0, out_dtype=torch.float16)
    O, L = oracle_paged(inp)
    compare(out, lse, O, L, TOL_BF16, what=name)


def test_fp8_cache_fp16_query(sap):
    inp = _as(_small("fp8_bf16q"), q_dtype=torch.float16)
    out, lse = run_paged(inp, num_splits=2, out_dtype=torch.float16)
    O, L = oracle_paged(inp)
    compare(out, lse, O, L, TOL_FP8, what="fp8/fp16q")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16])
def test_output_dtypes(sap, out_dtype):
    inp = _small("decode_d128_g4")
    for splits in (1, 3):
        out, lse = run_paged(inp, num_splits=splits, out_dtype=out_dtype)
        assert out.dtype == out_dtype
        O, L = oracle_paged(inp)
        compare(out, lse, O, L, TOL_BF16, what=f"out {out_dtype} S={splits}")


def test_all_empty_requests(sap):
    inp = make_paged(B=3, sq=2, Hq=8, Hkv=2, D=128, P=16, seq_lens=[0, 0, 0], seed=3, poison=True,
                     table_width=2).to(DEV)
    for splits in (1, 4):
        out, lse = run_paged(inp, num_splits=splits)
        assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_zero_batch_is_noop(sap):
    inp = _small("decode_d64_g8")
    k, v = sap.kv_halves(inp.cache, inp.D)
    out = torch.full((0, 1, inp.Hq, inp.D), 7.0, dtype=torch.bfloat16, device=DEV)
    sap.paged_attn_run(inp.q[:0], k, v, inp.block_table[:0], inp.seq_lens[:0], scale=0.1, out=out)


def test_repeated_calls_share_one_workspace(sap):
    """Repeated split runs sharing one (never cleared) workspace: every call produces the
    same, correct result (the partials need no initialisation)."""
    inp = _small("block_sq16_window")
    k, v = sap.kv_halves(inp.cache, inp.D)
    W = inp.block_table.shape[1]
    O, L = oracle_paged(inp)
    for splits in (3, 5):
        need = sap.workspace_size(inp.B, inp.sq, inp.Hq, inp.Hkv, inp.D, inp.P, W, inp.window, splits)
        ws = sap.new_workspace(need, DEV)
        first = None
        for rep in range(4):
            out, lse = sap.paged_attn_run(inp.q, k, v, inp.block_table, inp.seq_lens, scale=inp.scale,
                                          window=inp.window, num_splits=splits, workspace=ws)
            compare(out, lse, O, L, TOL_BF16, what=f"S={splits} rep={rep}")
            if first is None:
                first = (out.clone(), lse.clone())
            else:
                assert torch.equal(out.view(torch.int16), first[0].view(torch.int16))


@pytest.mark.parametrize("name,splits", [("decode_d128_g4", 3), ("block_sq16_window", 2),
                                         ("decode_d64_g8", 1)])
def test_graph_capture_replays(sap, name, splits):
    """paged_attn_run captured into a graph (attention + combine) and replayed with eager
    work in between: every replay equals the eager result."""
    inp = _small(name)
    k, v = sap.kv_halves(inp.cache, inp.D)
    W = inp.block_table.shape[1]
    ws = sap.new_workspace(sap.workspace_size(inp.B, inp.sq, inp.Hq, inp.Hkv, inp.D, inp.P, W,
                                              inp.window, splits), DEV)
    out = torch.empty((inp.B, inp.sq, inp.Hq, inp.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((inp.B, inp.sq, inp.Hq), dtype=torch.float32, device=DEV)

    def call():
        sap.paged_attn_run(inp.q, k, v, inp.block_table, inp.seq_lens, scale=inp.scale,
                           window=inp.window, num_splits=splits, out=out, lse=lse, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    O, L = oracle_paged(inp)
    compare(ref_o, ref_l, O, L, TOL_BF16, what=f"{name} eager")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}"
        assert torch.equal(lse, ref_l), f"replay {rep}"


def test_graph_capture_segments(sap):
    s = make_segments(seed=17, poison=True, zero_frac=0.25, name="graph", **SEG["seg_small"]).to(DEV)
    out = torch.empty((s.N, s.Hq, s.D), dtype=torch.bfloat16, device=DEV)
    ws = sap.new_workspace(sap.segment_attn_workspace_size(s.N, s.topk, s.Hq, s.D), DEV)
    for fused in (True, False):
        def call():
            sap.segment_attn_run(s.q, s.k, s.v, s.used, s.bias, bs=s.bs, local=s.local, fused=fused,
                                 out=out, workspace=ws, return_lse=False)
        call()
        torch.cuda.synchronize()
        ref = out.clone()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            call()
        torch.cuda.current_stream().wait_stream(st)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        for rep in range(3):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"fused={fused} {rep}"


# ---- Split-KV partials and the combine ------------------------------------------
@pytest.mark.parametrize("name,S", [("decode_d128_g4", 3), ("block_sq16_window", 5), ("page64", 2),
                                    ("fp8_bf16q", 16)])
def test_partials_match_oracle(sap, name, S):
    inp = _small(name)
    k, v = sap.kv_halves(inp.cache, inp.D)
    po, pl = sap.paged_attn_partial(inp.q, k, v, inp.block_table, inp.seq_lens, scale=inp.scale,
                                    num_splits=S, window=inp.window, k_scale=inp.k_scale,
                                    v_scale=inp.v_scale)
    cache = to_numpy_bits(inp.cache.cpu())
    kk, vv = np_halves(cache, inp.D)
    Po, Pl = oracle.split_partials(to_numpy_bits(inp.q.cpu()), "bf16", kk, vv, inp.kv_dtype,
                                   inp.block_table.cpu().numpy(), inp.seq_lens.cpu().numpy(),
                                   scale=inp.scale, num_splits=S, window=inp.window,
                                   k_scale=inp.k_scale, v_scale=inp.v_scale)
    Po = Po.reshape(S, inp.B * inp.sq, inp.Hq, inp.D)
    Pl = Pl.reshape(S, inp.B * inp.sq, inp.Hq)
    live = ~np.isneginf(Pl)
    gl = pl.cpu().numpy()
    assert np.array_equal(np.isneginf(gl), ~live), "dead-split pattern differs"
    tol = TOL_FP8 if inp.kv_dtype == "fp8_e4m3" else TOL_BF16
    compare(po, None, Po, Pl, dict(tol, mean_abs=tol["mean_abs"]), mask=live, what=f"{name} parts")
    assert np.abs(gl[live] - Pl[live]).max() <= tol["lse"]


def test_split_combine_standalone(sap):
    rng = np.random.default_rng(4)
    S, rows, Hq, D = 7, 5, 6, 128
    po = rng.normal(size=(S, rows, Hq, D))
    pl = rng.normal(size=(S, rows, Hq)) * 3
    dead = rng.random((S, rows, Hq)) < 0.3
    dead[:, 2, 1] = True  # a row with no live split
    pl[dead] = -np.inf
    po[dead] = np.nan  # never read
    O, L = oracle.combine_splits(po, pl)
    t_o = torch.tensor(po, dtype=torch.float32, device=DEV)
    t_l = torch.tensor(pl, dtype=torch.float32, device=DEV)
    for od in (torch.float32, torch.bfloat16):
        out, lse = sap.split_kv_combine(t_o, t_l, out_dtype=od)
        tol = dict(max_abs=2e-5, mean_abs=2e-6, lse=1e-5) if od == torch.float32 else TOL_BF16
        compare(out, lse, O, L, tol, what=f"split combine {od}")


@pytest.mark.parametrize("part_dtype", [torch.float32, torch.bfloat16])
def test_segment_combine_standalone(sap, part_dtype):
    rng = np.random.default_rng(5)
    N, G, Hq, D = 6, 9, 4, 128
    po = rng.normal(size=(N, G, Hq, D))
    po = torch.tensor(po).to(part_dtype).double().numpy()  # what the kernel will read
    pl = rng.normal(size=(N, G, Hq)) * 2
    used = rng.integers(1, 64, size=(N, G)).astype(np.int32)
    used[rng.random((N, G)) < 0.3] = 0
    used[3] = 0  # all segments of query 3 dead
    bias = rng.normal(size=(N, G - 1)).astype(np.float32)
    po_nan = po.copy()
    po_nan[used == 0] = np.nan  # dead partials are never read
    O, L = oracle.combine_segments(po, pl, used, bias.astype(np.float64))
    out, lse = sap.segment_attn_combine(
        torch.tensor(po_nan, device=DEV).to(part_dtype), torch.tensor(pl, dtype=torch.float32, device=DEV),
        torch.tensor(used, device=DEV), torch.tensor(bias, device=DEV), out_dtype=torch.float32)
    compare(out, lse, O, L, dict(max_abs=2e-5, mean_abs=2e-6, lse=1e-5), what="segment combine")
    assert torch.all(out[3] == 0) and torch.all(torch.isneginf(lse[3]))


# ---- DASH segments --------------------------------------------------------------
SEG = {
    "seg_small": dict(N=6, Hq=8, Hkv=2, D=128, topk=3, bs=16, local=32),
    "seg_unaligned": dict(N=4, Hq=16, Hkv=4, D=64, topk=2, bs=8, local=24),
    "seg_g8": dict(N=3, Hq=32, Hkv=4, D=128, topk=8, bs=64, local=128),
    "seg_g32": dict(N=3, Hq=32, Hkv=1, D=128, topk=4, bs=16, local=40),  # 32-row groups
}


@pytest.mark.parametrize("name", sorted(SEG))
@pytest.mark.parametrize("fused", [True, False])
def test_segment_attention(sap, name, fused):
    s = make_segments(seed=11, poison=True, zero_frac=0.25, name=name, **SEG[name])
    used = s.used.clone()
    used[1] = 0  # one query with every segment empty
    s.used = used
    O, L = oracle.segment_attention(to_numpy_bits(s.q), to_numpy_bits(s.k), to_numpy_bits(s.v),
                                    s.used.numpy(), s.bias.numpy(), topk=s.topk, bs=s.bs,
                                    local=s.local, scale=s.scale)
    d = s.to(DEV)
    out, lse = sap.segment_attn_run(d.q, d.k, d.v, d.used, d.bias, bs=s.bs, local=s.local,
                                    fused=fused)
    compare(out, lse, O, L, TOL_BF16, what=f"{name} fused={fused}")


@pytest.mark.parametrize("fused", [True, False])
def test_segment_minus_inf_bias(sap, fused):
    # a live segment with bias -inf weighs nothing; a query whose live logits are all
    # -inf ends as out = 0, lse = -inf (the page's nan_to_num of a NaN softmax)
    s = make_segments(seed=19, poison=True, zero_frac=0.0, name="ninf", **SEG["seg_small"])
    bias = s.bias.clone()
    used = s.used.clone()
    bias[0, :] = float("-inf")
    used[0, s.topk] = 0          # query 0: nothing finite left
    bias[1, 0] = float("-inf")   # query 1: its first segment (a wave's first tile)
    bias[4, :] = float("-inf")   # query 4: only the local segment counts
    s.bias, s.used = bias, used
    O, L = oracle.segment_attention(to_numpy_bits(s.q), to_numpy_bits(s.k), to_numpy_bits(s.v),
                                    used.numpy(), bias.numpy(), topk=s.topk, bs=s.bs,
                                    local=s.local, scale=s.scale)
    d = s.to(DEV)
    out, lse = sap.segment_attn_run(d.q, d.k, d.v, d.used, d.bias, bs=s.bs, local=s.local,
                                    fused=fused)
    compare(out, lse, O, L, TOL_BF16, what=f"-inf bias fused={fused}")
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))


# ---- integer plan on the device --------------------------------------------------
@pytest.mark.parametrize("name", ["decode_d128_g4", "block_sq16_window", "page24_window"])
@pytest.mark.parametrize("splits", [1, 3, 0, -2])
def test_describe_bit_exact(sap, name, splits):
    inp = _small(name)
    lens, table, ranges = sap.paged_attn_describe(inp.block_table, inp.seq_lens, query_len=inp.sq,
                                                  Hq=inp.Hq, Hkv=inp.Hkv, D=inp.D, page_size=inp.P,
                                                  window=inp.window, num_splits=splits)
    el, et = oracle.restrict_to_window(inp.seq_lens.cpu().numpy(), inp.block_table.cpu().numpy(),
                                       inp.window, inp.sq, inp.P)
    assert np.array_equal(lens.cpu().numpy(), el)
    assert np.array_equal(table.cpu().numpy(), et)
    hl, ht, hr = sap.paged_attn_describe_host(inp.block_table.cpu(), inp.seq_lens.cpu(),
                                              query_len=inp.sq, Hq=inp.Hq, Hkv=inp.Hkv, D=inp.D,
                                              page_size=inp.P, window=inp.window, num_splits=splits)
    assert torch.equal(hr, ranges.cpu())
    if splits > 0:
        for b in range(inp.B):
            n_pages = -(-int(el[b]) // inp.P)
            got = [tuple(r[:2]) for r in ranges[b].cpu().tolist()]
            assert got == oracle.split_page_ranges(n_pages, splits)


# ---- bitwise invariants on the GPU -----------------------------------------------
def test_page_permutation_is_bitwise_invariant(sap):
    inp = _small("decode_d128_g4")
    out1, lse1 = run_paged(inp, num_splits=3)
    perm = torch.randperm(inp.pool, generator=torch.Generator().manual_seed(1)).to(DEV)
    cache2 = torch.empty_like(inp.cache)
    cache2[perm] = inp.cache
    inp.block_table = perm[inp.block_table.long()].to(torch.int32)
    inp.cache = cache2
    out2, lse2 = run_paged(inp, num_splits=3)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)


def test_strided_halves_equal_compact_planes_bitwise(sap):
    inp = _small("block_sq16_window")
    k, v = sap.kv_halves(inp.cache, inp.D)
    kc, vc = k.contiguous(), v.contiguous()
    assert kc.stride() != k.stride()
    a = sap.paged_attn_run(inp.q, k, v, inp.block_table, inp.seq_lens, scale=inp.scale,
                           window=inp.window, num_splits=2)
    b = sap.paged_attn_run(inp.q, kc, vc, inp.block_table, inp.seq_lens, scale=inp.scale,
                           window=inp.window, num_splits=2)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("fused", [True, False])
def test_dead_segment_is_bitwise_inert(sap, fused):
    s = make_segments(seed=13, zero_frac=0.0, name="inert", **SEG["seg_small"]).to(DEV)
    used = s.used.clone()
    used[2, 1] = 0
    out1, lse1 = sap.segment_attn_run(s.q, s.k, s.v, used, s.bias, bs=s.bs, local=s.local, fused=fused)
    k2, v2, b2 = s.k.clone(), s.v.clone(), s.bias.clone()
    base = 2 * s.per_query + 1 * s.bs
    k2[base:base + s.bs] = float("nan")
    v2[base:base + s.bs] = 1e4
    b2[2, 1] = 50.0
    out2, lse2 = sap.segment_attn_run(s.q, k2, v2, used, b2, bs=s.bs, local=s.local, fused=fused)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse1, lse2)


# ---- logit scale sign --------------------------------------------------------------
# A negative scale flips which keys dominate and a zero scale weighs every visible key
# alike; both must follow the plain softmax of scale * q.k.
@pytest.mark.parametrize("scale", [-0.09, 0.0, -1e-3])
@pytest.mark.parametrize("name", ["decode_d128_g4", "block_sq16_window", "fp8_bf16q",
                                  "fp8_sq16_window", "block_sq3_rt2"])
def test_logit_scale_sign(sap, name, scale):
    inp = _small(name)
    inp.scale = scale
    tol = TOL_FP8 if inp.kv_dtype == "fp8_e4m3" else TOL_BF16
    for causal in (False, True):
        for splits in (1, 3):
            out, lse = run_paged(inp, num_splits=splits, causal=causal)
            O, L = oracle_paged(inp, causal=causal)
            compare(out, lse, O, L, tol, what=f"{name} scale={scale} causal={causal} S={splits}")


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_logit_scale_sign_fp8_query(sap, scale):
    inp = make_paged(seed=29, poison=True, kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3", B=3, sq=16,
                     Hq=32, Hkv=8, D=128, P=16, seq_lens=[16, 257, 640]).to(DEV)
    inp.scale = scale
    out, lse = run_paged(inp, num_splits=0)
    O, L = oracle_paged(inp)
    compare(out, lse, O, L, TOL_FP8, what=f"fp8 q scale={scale}")


@pytest.mark.parametrize("scale", [-0.09, 0.0])
@pytest.mark.parametrize("fused", [True, False])
def test_logit_scale_sign_segments(sap, scale, fused):
    s = make_segments(seed=23, poison=True, zero_frac=0.25, name="sign", **SEG["seg_small"])
    O, L = oracle.segment_attention(to_numpy_bits(s.q), to_numpy_bits(s.k), to_numpy_bits(s.v),
                                    s.used.numpy(), s.bias.numpy(), topk=s.topk, bs=s.bs,
                                    local=s.local, scale=scale)
    d = s.to(DEV)
    out, lse = sap.segment_attn_run(d.q, d.k, d.v, d.used, d.bias, bs=s.bs, local=s.local,
                                    scale=scale, fused=fused)
    compare(out, lse, O, L, TOL_BF16, what=f"segments scale={scale} fused={fused}")


# ---- repeatability ----------------------------------------------------------------
# Every kernel is a fixed order of operations: repeated calls on the same inputs must
# agree bit for bit (a value read before the instruction producing it has finished
# shows up here first).
@pytest.mark.parametrize("name,splits", [("decode_d128_g4", 1), ("decode_d128_g4", 3),
                                         ("decode_d64_g8", 0), ("block_sq16_window", 2),
                                         ("block_sq3_rt2", 1), ("fp8_bf16q", 3),
                                         ("fp8_sq16_window", 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_repeated_calls_are_bitwise_equal(sap, name, splits, causal):
    inp = _small(name)
    ref = None
    for rep in range(12):
        out, lse = run_paged(inp, num_splits=splits, causal=causal)
        if ref is None:
            ref = (out.clone(), lse.clone())
            continue
        assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), f"rep {rep}"
        assert torch.equal(lse.view(torch.int32), ref[1].view(torch.int32)), f"rep {rep}"


@pytest.mark.parametrize("fused", [True, False])
def test_repeated_segment_calls_are_bitwise_equal(sap, fused):
    s = make_segments(seed=11, poison=True, zero_frac=0.25, name="rep", **SEG["seg_g8"]).to(DEV)
    ref = None
    for rep in range(12):
        out, lse = sap.segment_attn_run(s.q, s.k, s.v, s.used, s.bias, bs=s.bs, local=s.local,
                                        fused=fused)
        if ref is None:
            ref = (out.clone(), lse.clone())
            continue
        assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), f"rep {rep}"
        assert torch.equal(lse.view(torch.int32), ref[1].view(torch.int32)), f"rep {rep}"
