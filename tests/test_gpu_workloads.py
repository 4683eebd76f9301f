"""The five named decode workloads at full size, in the launch configuration
bench.py times (skv.default_split parts), against the oracle: through the
five calls, and through skv_decode_step (append of the last token folded into
the bounds pass, selection into the attention prologue) as bench.py runs it.

Every sequence, every query head and every int32 dot is compared: outputs
element-wise (per head: Frobenius-relative and largest element, against the
float64 oracle: f16 1e-3, int8 1e-4 against the int8 method), selected sets
bit-exact on the GPU's own scores and up to reported near-ties against the
float64 scores.  The strict 8e-3 int8 contract of the cpu-attn kernel card
("Correctness": fp32 attention on the dequantized cache) is asserted per
sequence, Frobenius-relative over its [H][D] output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import (DEV, assert_close, build_cache, prefilled_cache, quantized_host, rel_err, run_dense,
                         run_select, run_sparse, run_step)

pytestmark = pytest.mark.gpu

F16_TOL = 1e-3


def _print(*a):
    print(*a, flush=True)


def check_selection(w, b, score_gpu, sel, cnt, keys=None):
    """GPU scores vs exact-sum bounds; GPU sets == oracle selection of the GPU
    scores (exact) and == float64 selection up to reported near-ties."""
    nb = w.n_blocks(b)
    keys = w.k[b] if keys is None else keys
    kmin, kmax = oracle.block_bounds(keys, w.lens[b], w.block)
    ref = oracle.group_scores(oracle.upper_bounds(w.q[b], kmin, kmax), w.Hkv)
    np.testing.assert_allclose(score_gpu[b, :, :nb], ref, rtol=2e-6, atol=1e-4)
    near_total = 0
    lists = []
    for g in range(w.Hkv):
        got = sel[b, g, :cnt[b, g]]
        own = oracle.select_blocks(score_gpu[b, g], nb, w.k_sel[b], w.n_sink, w.n_recent)
        assert np.array_equal(got, own["sel"]), (b, g)
        r = oracle.select_blocks(ref[g], nb, w.k_sel[b], w.n_sink, w.n_recent)
        diff = set(got.tolist()) ^ set(r["sel"].tolist())
        assert diff <= set(r["near"].tolist()), (b, g, diff)
        near_total += len(diff)
        lists.append(got)
    return lists, near_total


def test_workload1_dense_f16_512(gpu_lib):
    _print("workload 1")
    w = workloads.named(1)
    cache = build_cache(w)
    out, _ = run_dense(cache, w)
    assert_close(out[0], oracle.attend_f16(w.q[0], w.k[0], w.v[0], w.softmax_scale), F16_TOL)


def test_workload2_dense_int8_8192(gpu_lib):
    _print("workload 2")
    w = workloads.named(2)
    cache = build_cache(w)
    out, dbg = run_dense(cache, w, dbg=True)
    kc, ks, vc, vs = quantized_host(w, 0)
    assert np.array_equal(cache.k.cpu().numpy()[0], kc)
    assert np.array_equal(cache.k_scale.cpu().numpy()[0].view(np.uint32), ks.view(np.uint32))
    dots, _, _ = oracle.int8_logit_dots(w.q[0], kc)
    assert np.array_equal(dbg[0].astype(np.int64), dots)
    meth = oracle.attend_i8(w.q[0], kc, ks, vc, vs, w.softmax_scale)
    con = oracle.attend_i8_dequant(w.q[0], kc, ks, vc, vs, w.softmax_scale)
    assert_close(out[0], meth, 1e-4)
    assert rel_err(out[0], con) < 8e-3


@pytest.fixture(scope="module")
def w3():
    w = workloads.named(3)
    return w, build_cache(w)


def test_workload3_dense_f16_32k(gpu_lib, w3):
    _print("workload 3 dense")
    w, cache = w3
    out, _ = run_dense(cache, w)
    assert_close(out[0], oracle.attend_f16(w.q[0], w.k[0], w.v[0], w.softmax_scale), F16_TOL)


def test_workload3_quest_f16_32k(gpu_lib, w3):
    _print("workload 3 quest")
    w, cache = w3
    score, sel, cnt, _ = run_select(cache, w)
    s_h, c_h = sel.cpu().numpy(), cnt.cpu().numpy()
    assert np.all(c_h == 131)
    lists, near = check_selection(w, 0, score, s_h, c_h)
    _print("near-tie differences", near)
    out = run_sparse(cache, w, sel, cnt)
    for g in range(w.Hkv):
        toks = oracle.selected_tokens(lists[g], w.lens[0], w.block)
        hs = slice(g * w.G, (g + 1) * w.G)
        ref = oracle.attend_f16(w.q[0][hs], w.k[0][g:g + 1], w.v[0][g:g + 1], w.softmax_scale,
                                tokens=toks)
        assert_close(out[0, hs], ref, F16_TOL)


@pytest.fixture(scope="module")
def w4():
    w = workloads.named(4)
    return w, build_cache(w, max_seq=65536)


SEQS4 = tuple(range(16))


def test_workload4_varlen_dense(gpu_lib, w4):
    _print("workload 4 dense")
    w, cache = w4
    out, _ = run_dense(cache, w)
    for b in SEQS4:
        ref = oracle.attend_f16(w.q[b], w.k[b], w.v[b], w.softmax_scale)
        assert_close(out[b], ref, F16_TOL, b)


def test_workload4_varlen_quest(gpu_lib, w4):
    _print("workload 4 quest")
    w, cache = w4
    score, sel, cnt, _ = run_select(cache, w)
    s_h, c_h = sel.cpu().numpy(), cnt.cpu().numpy()
    for b in range(w.B):
        nb = w.n_blocks(b)
        for g in range(w.Hkv):
            own = oracle.select_blocks(score[b, g], nb, w.k_sel[b], w.n_sink, w.n_recent)
            assert np.array_equal(s_h[b, g, :c_h[b, g]], own["sel"]), (b, g)
    out = run_sparse(cache, w, sel, cnt)
    for b in SEQS4:
        lists, _ = check_selection(w, b, score, s_h, c_h)
        for g in range(w.Hkv):
            toks = oracle.selected_tokens(lists[g], w.lens[b], w.block)
            hs = slice(g * w.G, (g + 1) * w.G)
            ref = oracle.attend_f16(w.q[b][hs], w.k[b][g:g + 1], w.v[b][g:g + 1],
                                    w.softmax_scale, tokens=toks)
            assert_close(out[b, hs], ref, F16_TOL, (b, g))


def test_workload5_quest_int8_256k(gpu_lib):
    _print("workload 5")
    w = workloads.named(5)
    cache = build_cache(w)
    score, sel, cnt, _ = run_select(cache, w)
    s_h, c_h = sel.cpu().numpy(), cnt.cpu().numpy()
    assert np.all(c_h == 517)
    # bounds come from the float32 keys before quantization
    lists, near = check_selection(w, 0, score, s_h, c_h, keys=w.k[0])
    _print("near-tie differences", near)
    kc, ks, vc, vs = quantized_host(w, 0)
    assert np.array_equal(cache.k.cpu().numpy()[0], kc)
    assert np.array_equal(cache.v.cpu().numpy()[0], vc)
    assert np.array_equal(cache.k_scale.cpu().numpy()[0].view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(cache.v_scale.cpu().numpy()[0].view(np.uint32), vs.view(np.uint32))
    out = run_sparse(cache, w, sel, cnt)
    meth = np.zeros((w.H, w.D))
    con = np.zeros((w.H, w.D))
    for g in range(w.Hkv):
        toks = oracle.selected_tokens(lists[g], w.lens[0], w.block)
        hs = slice(g * w.G, (g + 1) * w.G)
        sl = slice(g, g + 1)
        meth[hs] = oracle.attend_i8(w.q[0][hs], kc[sl], ks[sl], vc[sl], vs[sl], w.softmax_scale,
                                    tokens=toks)
        con[hs] = oracle.attend_i8_dequant(w.q[0][hs], kc[sl], ks[sl], vc[sl], vs[sl],
                                           w.softmax_scale, tokens=toks)
        assert_close(out[0, hs], meth[hs], 1e-4, g)
    _print("int8 Quest: contract error", rel_err(out[0], con), "method gap", rel_err(meth, con))
    assert rel_err(out[0], con) < 8e-3
    # dense int8 over all 262,144 tokens: every head, every int32 dot
    dense, dbg = run_dense(cache, w, dbg=True)
    dots, _, _ = oracle.int8_logit_dots(w.q[0], kc)
    assert np.array_equal(dbg[0].astype(np.int64), dots)
    del dbg, dots
    meth = oracle.attend_i8(w.q[0], kc, ks, vc, vs, w.softmax_scale)
    assert_close(dense[0], meth, 1e-4)
    con = oracle.attend_i8_dequant(w.q[0], kc, ks, vc, vs, w.softmax_scale)
    _print("int8 dense: contract error", rel_err(dense[0], con), "method gap", rel_err(meth, con))
    assert rel_err(dense[0], con) < 8e-3


# ------------------------------------------------------------ decode_step
def _check_quest_step(w, out, score, sel, cnt, seqs, keys_of=None):
    for b in seqs:
        keys = None if keys_of is None else keys_of(b)
        lists, near = check_selection(w, b, score, sel, cnt, keys=keys)
        _print("seq", b, "near-tie differences", near)
        if w.kv_dtype != "f16":
            kc, ks, vc, vs = quantized_host(w, b)
        for g in range(w.Hkv):
            toks = oracle.selected_tokens(lists[g], w.lens[b], w.block)
            hs = slice(g * w.G, (g + 1) * w.G)
            if w.kv_dtype == "f16":
                ref = oracle.attend_f16(w.q[b][hs], w.k[b][g:g + 1], w.v[b][g:g + 1],
                                        w.softmax_scale, tokens=toks)
                assert_close(out[b, hs], ref, F16_TOL, (b, g))
            else:
                sl = slice(g, g + 1)
                meth = oracle.attend_i8(w.q[b][hs], kc[sl], ks[sl], vc[sl], vs[sl],
                                        w.softmax_scale, tokens=toks)
                assert_close(out[b, hs], meth, 1e-4, (b, g))


def test_workload3_decode_step(gpu_lib):
    """The 32K Quest and dense steps exactly as bench.py times them."""
    _print("workload 3 decode_step")
    w = workloads.named(3)
    base = prefilled_cache(w)
    c2 = base.clone()
    out, (score, sel, cnt) = run_step(base, w, quest=True)
    assert np.all(cnt == 131)
    _check_quest_step(w, out, score, sel, cnt, [0])
    dense, _ = run_step(c2, w, quest=False)
    assert_close(dense[0], oracle.attend_f16(w.q[0], w.k[0], w.v[0], w.softmax_scale), F16_TOL)


def test_workload4_decode_step(gpu_lib):
    _print("workload 4 decode_step")
    w = workloads.named(4)
    base = prefilled_cache(w, max_seq=65536)
    c2 = base.clone()
    out, (score, sel, cnt) = run_step(base, w, quest=True)
    _check_quest_step(w, out, score, sel, cnt, SEQS4)
    dense, _ = run_step(c2, w, quest=False)
    for b in SEQS4:
        ref = oracle.attend_f16(w.q[b], w.k[b], w.v[b], w.softmax_scale)
        assert_close(dense[b], ref, F16_TOL, b)


def test_workload5_decode_step(gpu_lib):
    """The 262K int8 Quest step (fused selection over 4,091 candidates) and the
    dense int8 step, every head."""
    _print("workload 5 decode_step")
    w = workloads.named(5)
    base = prefilled_cache(w)
    c2 = base.clone()
    out, (score, sel, cnt) = run_step(base, w, quest=True)
    assert np.all(cnt == 517)
    _check_quest_step(w, out, score, sel, cnt, [0], keys_of=lambda b: w.k[b])
    dense, _ = run_step(c2, w, quest=False)
    kc, ks, vc, vs = quantized_host(w, 0)
    meth = oracle.attend_i8(w.q[0], kc, ks, vc, vs, w.softmax_scale)
    assert_close(dense[0], meth, 1e-4)
    con = oracle.attend_i8_dequant(w.q[0], kc, ks, vc, vs, w.softmax_scale)
    assert rel_err(dense[0], con) < 8e-3
