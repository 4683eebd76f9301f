"""Head dims 64 and 256: the append, bounds, selection, attention, sparse-V,
4-bit scan and step calls of the f16, int8 and group-wise (q8_0, q4_0, q5_0)
caches against the oracle (cpu-attn kernel card, "Requirements and limits": the head dimension
is any multiple of 16 up to 1024; these two and 128 are built).

Sizes span several tiles per wavefront, several parts and a ragged tail (the
f16 tile is 16 tokens, the int8 tile 32; a tile's 16-byte loads cover 8, 4 or
2 rows per instruction at D = 64, 128, 256).  Bars as at D = 128: appended
rows, codes, scales and bounds exact; int8 logit dots exact; selected sets
exact on the kernel's own scores; sparse-V keep decisions exact outside the
oracle's near-threshold band; the scan's index bit-exact and its bounds and
candidates as at head dim 128; f16 and group-wise outputs within 1e-3 and int8
outputs within 1e-4 of the method (per head and per element); the step
bit-identical to the calls it composes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import (DEV, assert_close, build_cache, padded_rows, quantized_host, rel_err,
                         run_dense, run_select, run_sparse, sel_tensor_from_lists)
from test_gpu_multi_token import check_dense as chunk_check_dense
from test_gpu_multi_token import check_quest as chunk_check_quest
from test_gpu_multi_token import run_chunk
from test_gpu_per_head import check as per_head_check
from test_gpu_per_head import run_per_head
from test_gpu_grouped import check_cache as grouped_check_cache
from test_gpu_grouped import reference as grouped_reference
from test_gpu_sparse_v import check_seq as sv_check_seq
from test_gpu_sparse_v import keep_bits as sv_keep_bits
from test_gpu_sparse_v import run_sv
from test_gpu_scan4 import build as scan4_index
from test_gpu_scan4 import check_index as scan4_check_index
from test_gpu_scan4 import check_scan as scan4_check_scan
from test_gpu_scan4 import run_scan as scan4_run
from test_gpu_step import _oracle_check, _run_case

import sparse_kv_cache_append_amd as skv

pytestmark = pytest.mark.gpu

DIMS = [64, 256]
GROUPED = ["q8_0", "q4_0", "q5_0"]
F16_TOL = 1e-3
I8_TOL = 1e-4


def _print(*a):
    print("[head dims]", *a, flush=True)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_append_exact(gpu_lib, D, kv):
    """Chunked appends (a block that straddles each chunk edge) against the
    oracle's rows, codes, scales and block bounds."""
    _print("append", D, kv)
    L = 300
    w = workloads.clustered([801, 802], 8, 2, D, [L, L], kv, n_dirs=8)
    cache = skv.Cache(2, 2, 320, D, kv, 64, device=DEV)
    k, v = padded_rows(w, L)
    kt, vt = torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV)
    p0 = 0
    for n in [37, 27, 64, 1, 99, 72]:
        pos0 = torch.full((2,), p0, dtype=torch.int32, device=DEV)
        skv.kv_append(cache, pos0, kt[:, p0:p0 + n].contiguous(), vt[:, p0:p0 + n].contiguous())
        p0 += n
    torch.cuda.synchronize()
    for b in range(2):
        if kv == "f16":
            assert np.array_equal(cache.k.cpu().numpy()[b, :, :L].view(np.uint16),
                                  w.k[b].view(np.uint16))
            assert np.array_equal(cache.v.cpu().numpy()[b, :, :L].view(np.uint16),
                                  w.v[b].view(np.uint16))
        else:
            kc, ks, vc, vs = quantized_host(w, b)
            assert np.array_equal(cache.k.cpu().numpy()[b, :, :L], kc)
            assert np.array_equal(cache.v.cpu().numpy()[b, :, :L], vc)
            assert np.array_equal(cache.k_scale.cpu().numpy()[b, :, :L].view(np.uint32),
                                  ks.view(np.uint32))
            assert np.array_equal(cache.v_scale.cpu().numpy()[b, :, :L].view(np.uint32),
                                  vs.view(np.uint32))
        kmin, kmax = oracle.block_bounds(w.k[b], L, 64)
        assert np.array_equal(cache.kmin.cpu().numpy()[b, :, :5], kmin)
        assert np.array_equal(cache.kmax.cpu().numpy()[b, :, :5], kmax)


DENSE = [
    # (B, H, Hkv, lens, n_split)
    (2, 8, 2, [130, 777], None),
    (1, 32, 8, [2049], 7),
    (3, 16, 16, [1, 333, 64], None),
    (1, 8, 1, [1000], 3),
    (2, 16, 8, [17, 1500], 1),
]


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kv", ["f16", "i8"])
@pytest.mark.parametrize("B,H,Hkv,lens,S", DENSE)
def test_dense(gpu_lib, D, kv, B, H, Hkv, lens, S):
    _print("dense", D, kv, B, H, Hkv, lens, S)
    w = workloads.gaussian(811 + D + sum(lens), B, H, Hkv, D, lens, kv)
    cache = build_cache(w)
    out, dbg = run_dense(cache, w, S, dbg=kv == "i8")
    for b in range(B):
        if kv == "f16":
            ref = oracle.attend_f16(w.q[b], w.k[b], w.v[b], w.softmax_scale)
            assert_close(out[b], ref, F16_TOL, b)
        else:
            kc, ks, vc, vs = quantized_host(w, b)
            dots, _, _ = oracle.int8_logit_dots(w.q[b], kc)
            assert np.array_equal(dbg[b, :, :lens[b]].astype(np.int64), dots), b
            meth = oracle.attend_i8(w.q[b], kc, ks, vc, vs, w.softmax_scale)
            assert_close(out[b], meth, I8_TOL, b)


def test_zero_query_gives_mean_of_values(gpu_lib):
    _print("q = 0")
    for D in DIMS:
        for kv in ("f16", "i8"):
            w = workloads.gaussian(820 + D, 1, 8, 2, D, [700], kv)
            w.q[:] = 0
            cache = build_cache(w)
            out, _ = run_dense(cache, w)
            if kv == "f16":
                ref = w.v[0].astype(np.float64).mean(axis=1)
            else:
                _, _, vc, vs = quantized_host(w, 0)
                ref = (vc.astype(np.float64) * vs.astype(np.float64)[..., None]).mean(axis=1)
            for h in range(8):
                assert_close(out[0, h], ref[h // 4], 1e-6, D, kv, h)


QUEST = [
    # (seeds, H, Hkv, lens, kv, k_sel, n_sink, n_recent)
    ([831, 832], 32, 8, [3000, 4097], "f16", [10, 12], 1, 2),
    ([833], 32, 4, [5001], "i8", [20], 1, 4),
    ([834, 835], 16, 8, [65, 2000], "f16", [0, 7], 2, 1),
    ([836], 8, 8, [1500], "i8", [6], 1, 2),
]


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("seeds,H,Hkv,lens,kv,k_sel,ns,nr", QUEST)
def test_quest_bounds_selection_attention(gpu_lib, D, seeds, H, Hkv, lens, kv, k_sel, ns, nr):
    _print("quest", D, lens, kv, k_sel)
    w = workloads.clustered(seeds, H, Hkv, D, lens, kv, n_dirs=16, k_sel=k_sel, n_sink=ns,
                            n_recent=nr)
    cache = build_cache(w)
    score, sel, cnt, _ = run_select(cache, w)
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    G = H // Hkv
    out = run_sparse(cache, w, sel, cnt)
    for b in range(w.B):
        nb = w.n_blocks(b)
        kmin, kmax = oracle.block_bounds(w.k[b], w.lens[b], w.block)
        ref = oracle.group_scores(oracle.upper_bounds(w.q[b], kmin, kmax), Hkv)
        np.testing.assert_allclose(score[b, :, :nb], ref, rtol=2e-6, atol=1e-4)
        for g in range(Hkv):
            own = oracle.select_blocks(score[b, g], nb, k_sel[b], ns, nr)["sel"]
            got = sel_h[b, g, :cnt_h[b, g]]
            assert np.array_equal(got, own), (b, g)
            toks = oracle.selected_tokens(got, w.lens[b], w.block)
            hs = slice(g * G, (g + 1) * G)
            if kv == "f16":
                r = oracle.attend_f16(w.q[b][hs], w.k[b][g:g + 1], w.v[b][g:g + 1],
                                      w.softmax_scale, tokens=toks)
                assert_close(out[b, hs], r, F16_TOL, b, g)
            else:
                kc, ks, vc, vs = quantized_host(w, b)
                sl = slice(g, g + 1)
                r = oracle.attend_i8(w.q[b][hs], kc[sl], ks[sl], vc[sl], vs[sl],
                                     w.softmax_scale, tokens=toks)
                assert_close(out[b, hs], r, I8_TOL, b, g)


STEP = [
    # name, factory(D), quest, append, extra
    ("quest-f16", lambda D: workloads.clustered(
        [841, 842], 32, 8, D, [2049, 3000], "f16", n_dirs=16, k_sel=[8, 20], n_sink=1,
        n_recent=2), True, True, {}),
    ("quest-i8 G8", lambda D: workloads.clustered(
        [843], 32, 4, D, [5000], "i8", n_dirs=16, k_sel=[30], n_sink=1, n_recent=4),
        True, True, {}),
    ("quest-f16 selection as its own kernel", lambda D: workloads.clustered(
        [844], 16, 8, D, [9000], "f16", n_dirs=16, k_sel=[60], n_sink=1, n_recent=2),
        True, True, {"S": 1}),
    ("dense-f16 append poisoned rows", lambda D: workloads.gaussian(
        845, 2, 32, 8, D, [65, 2000], "f16"), False, True, {"poison": True}),
    ("dense-i8 append poisoned rows G2", lambda D: workloads.gaussian(
        846, 2, 16, 8, D, [1025, 300], "i8"), False, True, {"poison": True, "S": 5}),
    ("dense-i8 first token of an empty cache", lambda D: workloads.gaussian(
        847, 1, 32, 4, D, [1], "i8"), False, True, {"lag": 1, "tight": True}),
    ("quest-q8_0", lambda D: workloads.clustered(
        [848, 849], 32, 8, D, [3000, 4097], "q8_0", n_dirs=16, k_sel=[10, 12], n_sink=1,
        n_recent=2), True, True, {}),
    ("quest-q5_0 G8 poisoned rows", lambda D: workloads.clustered(
        [850], 32, 4, D, [5001], "q5_0", n_dirs=16, k_sel=[20], n_sink=1, n_recent=4),
        True, True, {"poison": True}),
    ("dense-q4_0 append poisoned rows", lambda D: workloads.gaussian(
        851, 2, 32, 8, D, [65, 2000], "q4_0"), False, True, {"poison": True}),
    ("dense-q5_0 first token of an empty cache", lambda D: workloads.gaussian(
        852, 1, 32, 4, D, [1], "q5_0"), False, True, {"lag": 1, "tight": True}),
]


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kind", GROUPED)
def test_grouped_append_exact(gpu_lib, D, kind):
    """Group-wise codes (both q5_0 planes), f16 group scales and block bounds
    exact, appended whole and in 37-row chunks (blocks straddle the chunk
    edges), with a zero group and groups whose scale underflows and overflows
    f16 (the first and last group of a row included)."""
    _print("grouped append", D, kind)
    w = workloads.gaussian(890 + D, 2, 16, 4, D, [300, 129], kind)
    w.k[0][0, 5, :32] = 0.0
    w.k[0][1, 6, D - 32:] = 1e-9
    w.v[0][2, 7, 32:64] = 3e9
    for chunk in (None, 37):
        cache = build_cache(w, chunk=chunk)
        for b in range(w.B):
            grouped_check_cache(cache, w, b)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kind", GROUPED)
@pytest.mark.parametrize("H,Hkv,lens", [(32, 8, [2049, 100]), (8, 8, [513]), (16, 8, [1]),
                                        (32, 4, [4097])])
def test_grouped_dense(gpu_lib, D, kind, H, Hkv, lens):
    _print("grouped dense", D, kind, H, Hkv, lens)
    w = workloads.gaussian(893 + D + H + len(lens), len(lens), H, Hkv, D, lens, kind)
    cache = build_cache(w)
    for S in (None, 3):
        out, _ = run_dense(cache, w, n_split=S)
        for b in range(w.B):
            assert_close(out[b], grouped_reference(w, b), F16_TOL, D, kind, b, S)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kind", GROUPED)
def test_grouped_quest(gpu_lib, D, kind):
    """Bounds from the float32 keys, the selection on the kernel's own scores,
    attention over the selected blocks of a group-wise cache."""
    _print("grouped quest", D, kind)
    w = workloads.clustered([896, 897], 32, 8, D, [6000, 2600], kind, n_dirs=16,
                            k_sel=[20, 9], n_sink=1, n_recent=2)
    cache = build_cache(w)
    score, sel, cnt, _ = run_select(cache, w)
    out = run_sparse(cache, w, sel, cnt)
    s_h, c_h = sel.cpu().numpy(), cnt.cpu().numpy()
    for b in range(w.B):
        nb = w.n_blocks(b)
        kmin, kmax = oracle.block_bounds(w.k[b], w.lens[b], w.block)
        ref = oracle.group_scores(oracle.upper_bounds(w.q[b], kmin, kmax), w.Hkv)
        np.testing.assert_allclose(score[b, :, :nb], ref, rtol=2e-6, atol=1e-4)
        for g in range(w.Hkv):
            got = s_h[b, g, :c_h[b, g]]
            own = oracle.select_blocks(score[b, g], nb, w.k_sel[b], w.n_sink, w.n_recent)
            assert np.array_equal(got, own["sel"]), (b, g)
            toks = oracle.selected_tokens(got, w.lens[b], w.block)
            hs = slice(g * w.G, (g + 1) * w.G)
            assert_close(out[b, hs], grouped_reference(w, b, toks, hs, g), F16_TOL, b, g)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("name,make,quest,append,extra", STEP, ids=[c[0] for c in STEP])
def test_decode_step_equals_composed_calls(gpu_lib, D, name, make, quest, append, extra):
    """At these head dims the step runs the append as its own kernel (the
    folded appends move head dim 128 rows); still bit-identical to the five
    calls."""
    _print("step", D, name)
    w = make(D)
    out, sel = _run_case(w, quest, append, **extra)
    if not extra.get("lag"):
        _oracle_check(w, out, sel)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_decode_attn_select_equals_select_then_decode(gpu_lib, D, kv):
    _print("decode_attn_select", D, kv)
    L = 9000
    w = workloads.clustered([850], 32, 8, D, [L], kv, n_dirs=32, k_sel=[(-(-L // 64)) // 4],
                            n_sink=1, n_recent=2)
    cache = build_cache(w)
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    ks = torch.tensor(w.k_sel, dtype=torch.int32, device=DEV)
    max_sel = w.k_sel[0] + 3
    S = 16
    ws_a = torch.zeros(skv.workspace_bytes(1, 32, D, S), dtype=torch.uint8, device=DEV)
    ws_b = torch.full_like(ws_a, 255)
    score = torch.full((1, 8, cache.max_blocks), float("nan"), device=DEV)
    sel_a = torch.full((1, 8, max_sel), -7, dtype=torch.int32, device=DEV)
    sel_b = sel_a.clone()
    cnt_a = torch.full((1, 8), -7, dtype=torch.int32, device=DEV)
    cnt_b = cnt_a.clone()
    skv.block_bounds(cache, q, seq_len, L, score)
    skv.select_topk(score, seq_len, w.block, ks, w.n_sink, w.n_recent, sel_a, cnt_a)
    skv.decode_attn(cache, q, seq_len, L, w.softmax_scale, S, ws_a, sel_a, cnt_a)
    skv.decode_attn_select(cache, q, seq_len, L, w.softmax_scale, S, ws_b, score, ks, w.n_sink,
                           w.n_recent, sel_b, cnt_b)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b) and torch.equal(cnt_a, cnt_b)
    assert torch.equal(ws_a, ws_b)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("seeds,H,Hkv,lens,kv,ksel", [([861, 862], 32, 8, [5000, 777], "f16", [20, 4]),
                                                      ([863], 16, 4, [4100], "i8", [12]),
                                                      ([864], 32, 8, [3000], "q4_0", [10])])
def test_per_head_selection(gpu_lib, D, seeds, H, Hkv, lens, kv, ksel):
    """Per-query-head bounds, selection, union and attention at these head
    dims (bit-equal group scores, exact selections and unions, outputs
    element-wise)."""
    _print("per-head", D, lens, kv)
    w = workloads.clustered(seeds, H, Hkv, D, lens, kv, n_dirs=16, k_sel=ksel, n_sink=1,
                            n_recent=2)
    cache = build_cache(w)
    r = run_per_head(cache, w)
    per_head_check(w, r)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("seeds,H,Hkv,lens,kv,T", [([871, 872], 32, 8, [700, 1537], "f16", 4),
                                                   ([873], 32, 4, [2049], "i8", 2),
                                                   ([874], 8, 8, [1000], "i8", 8),
                                                   ([875], 32, 8, [900], "q8_0", 4)])
def test_dense_chunk(gpu_lib, D, seeds, H, Hkv, lens, kv, T):
    """A chunk of T query tokens (T x G MFMA columns, up to 16), dense."""
    _print("dense chunk", D, lens, kv, T)
    w = workloads.clustered(seeds, H, Hkv, D, lens, kv, n_dirs=16)
    qc = workloads.chunk_queries(w, T, seeds[0] + 50)
    cache = build_cache(w)
    r = run_chunk(cache, w, qc, quest=False)
    chunk_check_dense(w, qc, r)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("seeds,H,Hkv,lens,kv,T,ksel", [([881, 882], 32, 8, [5000, 1800], "f16", 4, [12, 5]),
                                                        ([883], 32, 4, [6001], "i8", 2, [20]),
                                                        ([884], 16, 8, [2500], "q5_0", 4, [9])])
def test_quest_chunk(gpu_lib, D, seeds, H, Hkv, lens, kv, T, ksel):
    """A chunk of T query tokens, each with its own Quest set."""
    _print("quest chunk", D, lens, kv, T)
    w = workloads.clustered(seeds, H, Hkv, D, lens, kv, n_dirs=16, k_sel=ksel, n_sink=1,
                            n_recent=2)
    qc = workloads.chunk_queries(w, T, seeds[0] + 60)
    cache = build_cache(w)
    r = run_chunk(cache, w, qc, quest=True)
    chunk_check_quest(w, qc, r)


def test_other_head_dims_are_refused(gpu_lib):
    """Head dim 96 (a multiple of 16, not built) raises SKV_EUNSUPPORTED
    before any launch."""
    _print("refused")
    c96 = skv.Cache(1, 2, 128, 96, "f16", 64, device=DEV)
    q = torch.zeros((1, 8, 96), dtype=torch.float32, device=DEV)
    sl = torch.tensor([10], dtype=torch.int32, device=DEV)
    score = torch.empty((1, 2, c96.max_blocks), dtype=torch.float32, device=DEV)
    with pytest.raises(skv.SkvError) as e:
        skv.block_bounds(c96, q, sl, 10, score)
    assert e.value.status == skv.SKV_EUNSUPPORTED
    idx = skv.Scan4Index(c96, device=DEV)
    with pytest.raises(skv.SkvError) as e:
        skv.scan4_build(c96, idx, torch.zeros(1, dtype=torch.int32, device=DEV), sl, 10)
    assert e.value.status == skv.SKV_EUNSUPPORTED
    torch.cuda.synchronize()


SPARSE_V = [
    # seed, kv, H, Hkv, lens, tau, eps
    (881, "f16", 32, 8, [1000, 2500], 1e-3, 0.0),
    (882, "f16", 16, 8, [4097, 64], 0.0, 0.5),
    (883, "i8", 32, 4, [3000], 0.0, 1.0),
    (884, "i8", 16, 8, [2049, 95, 1], 5e-4, 0.0),
    (887, "q4_0", 32, 8, [1500, 300], 1e-3, 0.0),
    (888, "q5_0", 16, 4, [2000], 0.0, 0.5),
    (889, "q8_0", 8, 8, [1100], 2e-3, 0.0),
]


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("seed,kv,H,Hkv,lens,tau,eps", SPARSE_V)
def test_sparse_v_dense_walk(gpu_lib, D, seed, kv, H, Hkv, lens, tau, eps):
    _print("sparse-v", D, seed, kv, H, Hkv, lens, tau, eps)
    w = workloads.clustered([seed + 10 * b for b in range(len(lens))], H, Hkv, D, lens, kv,
                            n_dirs=8, amp=5.0)
    cache = build_cache(w)
    out, kb = run_sv(cache, w, tau, eps)
    for b in range(w.B):
        sv_check_seq(w, b, out, kb, tau, eps)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_sparse_v_given_lists_and_zero_threshold(gpu_lib, D, kv):
    """Quest lists differing per KV head (a clipped last block) with both
    rules; and a zero threshold, which keeps every token and equals the dense
    attention."""
    _print("sparse-v lists", D, kv)
    w = workloads.clustered([885, 886], 32, 8, D, [5000, 3333], kv, n_dirs=8, amp=5.0)
    cache = build_cache(w)
    rng = np.random.default_rng(7)
    lists = []
    for b in range(w.B):
        nb = w.n_blocks(b)
        lists.append([np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, 17, replace=False)]))
                      for _ in range(w.Hkv)])
    max_sel = max(len(x) for row in lists for x in row)
    si, sc = sel_tensor_from_lists(lists, w.B, w.Hkv, max_sel)
    for tau, eps in ((2e-3, 0.0), (0.0, 0.3)):
        out, kb = run_sv(cache, w, tau, eps, sel=(si, sc))
        for b in range(w.B):
            sv_check_seq(w, b, out, kb, tau, eps, lists=lists[b])
    out, kb = run_sv(cache, w, 0.0, 0.0)
    for b in range(w.B):
        if kv == "f16":
            ref = oracle.attend_f16(w.q[b], w.k[b], w.v[b], w.softmax_scale)
            assert_close(out[b], ref, F16_TOL, b)
        else:
            kc, ks, vc, vs = quantized_host(w, b)
            assert_close(out[b], oracle.attend_i8(w.q[b], kc, ks, vc, vs, w.softmax_scale),
                         I8_TOL, b)
        for h in range(w.H):
            assert sv_keep_bits(kb[b, h], np.arange(w.lens[b])).all()


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("H,Hkv,lens,block", [(32, 8, [3000, 777], 64), (8, 8, [1500], 16),
                                              (16, 8, [1200], 32), (8, 1, [2049, 5], 128)])
def test_scan4_index_and_candidates(gpu_lib, D, H, Hkv, lens, block):
    """Every GQA group size (at D = 64 and G = 1 each lane takes one channel
    of the block's operands), 64- and 32-token tiles, ragged tails."""
    _print("scan4", D, H, Hkv, lens, block)
    w = workloads.clustered([970 + D + b for b in range(len(lens))], H, Hkv, D, lens, "f16",
                            n_dirs=8, amp=4.0, block=block)
    cache = build_cache(w)
    idx = scan4_index(cache, w)
    for delta in (0.0, 8.0):
        ub, cand, cnt = scan4_run(cache, idx, w, delta)
        for b in range(w.B):
            index = scan4_check_index(idx, w, b)
            scan4_check_scan(w, b, index, ub, cand, cnt, delta)


@pytest.mark.parametrize("D", DIMS)
def test_scan4_rebuild_after_append(gpu_lib, D):
    w = workloads.gaussian(975 + D, 2, 16, 4, D, [1000, 2049], "f16")
    cache = build_cache(w)
    lens_m1 = torch.tensor([L - 1 for L in w.lens], dtype=torch.int32, device=DEV)
    idx = scan4_index(cache, w, seq=lens_m1)
    pos = torch.tensor([L - 1 for L in w.lens], dtype=torch.int32, device=DEV)
    skv.scan4_build(cache, idx, pos, torch.tensor(w.lens, dtype=torch.int32, device=DEV),
                    max(w.lens))
    torch.cuda.synchronize()
    for b in range(w.B):
        scan4_check_index(idx, w, b)
