"""Group-wise quantized caches (q8_0, q4_0, q5_0) on the GPU against the oracle
(oracle/quant.py: quantize_groups; oracle/attention.py: attend_grouped):
the append's codes, f16 scales and side-cache bounds bit-exact (including
zero groups, scales below and beyond f16's range, round-half-even ties, and
appends in chunks that straddle blocks), the decode element-wise within 1e-3
of attention over the dequantized cache, dense and over Quest lists, at
small shapes (several tiles, ragged tails, every GQA group size) and at the
32K workload's shape."""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_cache_append_amd as skv
import workloads
from gpu_harness import (DEV, assert_close, build_cache, run_dense, run_select, run_sparse)
from oracle import quant

pytestmark = pytest.mark.gpu

QMAX = {"q8_0": quant.QMAX_Q8, "q4_0": quant.QMAX_Q4, "q5_0": quant.QMAX_Q5}
KINDS = ["q8_0", "q4_0", "q5_0"]


def _print(*a):
    print("[grouped]", *a, flush=True)


def host_codes(x, kind):
    """Oracle codes and scales, and the cache's byte layout of the codes."""
    codes, s16 = quant.quantize_groups(x, QMAX[kind])
    if kind == "q8_0":
        return codes.view(np.uint8), s16, codes, s16
    u = (codes.astype(np.int16) + QMAX[kind] + 1).astype(np.uint8)
    packed = ((u[..., 0::2] & 15) | ((u[..., 1::2] & 15) << 4)).astype(np.uint8)
    if kind == "q5_0":
        # (nibble plane, fifth-bit plane: bit c % 8 of byte c / 8)
        hi = np.packbits((u >> 4) & 1, axis=-1, bitorder="little")
        return (packed, hi), s16, codes, s16
    return packed, s16, codes, s16


def check_cache(cache, w, b=0):
    L = w.lens[b]
    for name, src in (("k", w.k[b]), ("v", w.v[b])):
        packed, s16, _, _ = host_codes(src, w.kv_dtype)
        if w.kv_dtype == "q5_0":
            lo, hi = cache.q5_planes(getattr(cache, name))
            assert np.array_equal(lo.cpu().numpy()[b, :, :L], packed[0]), name
            assert np.array_equal(hi.cpu().numpy()[b, :, :L], packed[1]), name
        else:
            got = getattr(cache, name).cpu().numpy()[b, :, :L]
            assert np.array_equal(got, packed), name
        gs = getattr(cache, name + "_scale").cpu().numpy()[b, :, :L]
        assert np.array_equal(gs.view(np.uint16), s16.view(np.uint16)), name
    kmin, kmax = oracle.block_bounds(w.k[b], L, w.block)
    nb = w.n_blocks(b)
    assert np.array_equal(cache.kmin.cpu().numpy()[b, :, :nb].view(np.uint16), kmin.view(np.uint16))
    assert np.array_equal(cache.kmax.cpu().numpy()[b, :, :nb].view(np.uint16), kmax.view(np.uint16))


def reference(w, b, tokens=None, hs=None, g=None):
    _, _, kc, ks = host_codes(w.k[b], w.kv_dtype)
    _, _, vc, vs = host_codes(w.v[b], w.kv_dtype)
    if g is None:
        return oracle.attend_grouped(w.q[b], kc, ks, vc, vs, w.softmax_scale, tokens)
    sl = slice(g, g + 1)
    return oracle.attend_grouped(w.q[b][hs], kc[sl], ks[sl], vc[sl], vs[sl], w.softmax_scale,
                                 tokens)


@pytest.mark.parametrize("kind", KINDS)
def test_append_codes_scales_bounds_exact(gpu_lib, kind):
    w = workloads.gaussian(901, 2, 16, 4, 128, [300, 129], kind)
    # edge rows: a zero group, a group whose scale underflows f16, one whose
    # scale overflows it, and values on round-half-even ties of the scale
    w.k[0][0, 5, :32] = 0.0
    w.k[0][1, 6, 32:64] = 1e-9
    w.v[0][2, 7, 64:96] = 3e9
    s = np.float32(np.float16(np.float32(QMAX[kind] * 0.5) / np.float32(QMAX[kind])))
    w.k[0][3, 8, 96:128] = (np.arange(32) % (2 * QMAX[kind] + 1) - QMAX[kind] + 0.5).astype(
        np.float32) * s
    w.k[0][3, 8, 96] = QMAX[kind] * s             # the group's absmax: scale exactly s
    for chunk in (None, 37):
        cache = build_cache(w, chunk=chunk)
        for b in range(w.B):
            check_cache(cache, w, b)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("H,Hkv,lens", [(32, 8, [2049, 100]), (8, 8, [513]), (16, 8, [1]),
                                        (32, 4, [4097])])
def test_dense_decode(gpu_lib, kind, H, Hkv, lens):
    w = workloads.gaussian(902 + H + len(lens), len(lens), H, Hkv, 128, lens, kind)
    cache = build_cache(w)
    for S in (None, 3):
        out, _ = run_dense(cache, w, n_split=S)
        for b in range(w.B):
            assert_close(out[b], reference(w, b), 1e-3, kind, b, S)


@pytest.mark.parametrize("kind", KINDS)
def test_quest_decode(gpu_lib, kind):
    """Quest over a grouped cache: bounds from the float32 keys, the
    selection, attention over the selected blocks (the step's composition is
    tested with the other step cases)."""
    w = workloads.clustered([903, 904], 32, 8, 128, [6000, 2600], kind, n_dirs=16,
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
            assert np.array_equal(got, own["sel"])
            toks = oracle.selected_tokens(got, w.lens[b], w.block)
            hs = slice(g * w.G, (g + 1) * w.G)
            assert_close(out[b, hs], reference(w, b, toks, hs, g), 1e-3, b, g)


def test_32k_workload_q8_q4_q5(gpu_lib):
    for kind in KINDS:
        w = workloads.quest32k_quant(kind)
        cache = build_cache(w)
        check_cache(cache, w)
        out, _ = run_dense(cache, w)
        assert_close(out[0], reference(w, 0), 1e-3, kind, "dense")
        score, sel, cnt, _ = run_select(cache, w)
        outq = run_sparse(cache, w, sel, cnt)
        s_h, c_h = sel.cpu().numpy(), cnt.cpu().numpy()
        for g in range(w.Hkv):
            toks = oracle.selected_tokens(s_h[0, g, :c_h[0, g]], w.lens[0], w.block)
            hs = slice(g * w.G, (g + 1) * w.G)
            assert_close(outq[0, hs], reference(w, 0, toks, hs, g), 1e-3, kind, g)
        full = oracle.attend_f16(w.q[0], w.k[0], w.v[0], w.softmax_scale)
        _print(kind, "dense output vs float32 cache (quantization error of the format):",
               float(np.linalg.norm(out[0] - full) / np.linalg.norm(full)))
