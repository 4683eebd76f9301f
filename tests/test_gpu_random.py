"""Seeded random configurations of the whole step against the oracle.

Each seed draws a cache type, a GQA grouping (G in 1, 2, 4, 8 and 1 to 8 KV
heads), a batch of 1 to 3 sequences of 1 to 2,499 tokens, a block size, a
split count, a Quest budget and sink/recent windows, then runs the dense step
and the Quest step (skv_decode_step, one-token append included) and checks:

* dense: the output against the float64 definition (f16: 1e-3; int8: 1e-4
  against the method-exact int8 oracle);
* Quest: the GPU's scores against the exact-sum bounds, its selected list
  bit for bit against the oracle's selection of those scores, and the output
  against attention over that list.

The draws cover grid sizes that are not multiples of the XCD count, rows
fewer and more than the XCDs, partial last tiles and empty parts.  A second
set of seeds also draws the cache type among all five (f16, int8, q8_0, q4_0,
q5_0; group-wise outputs within 1e-3 of the oracle on the dequantized cache)
and the head dim among 64, 128 and 256.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_harness import (assert_close, grouped_host, prefilled_cache, quantized_host, rel_err,
                         run_step)

pytestmark = pytest.mark.gpu

F16_TOL = 1e-3
I8_TOL_METHOD = 1e-4
SEEDS = list(range(16)) + [34]   # 34: 24 rows, dealt to the XCDs interleaved


def _workload(seed, kv=None, D=128):
    rng = np.random.default_rng(9100 + seed)
    kv = kv or ("f16" if seed % 2 == 0 else "i8")
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 4))
    block = int(rng.choice([16, 32, 64, 128]))
    lens = [int(x) for x in rng.integers(1, 2500, size=B)]
    k_sel = [int(rng.integers(0, -(-L // block) + 2)) for L in lens]
    n_sink, n_recent = int(rng.integers(0, 3)), int(rng.integers(0, 5))
    if max(k_sel) + n_sink + n_recent == 0:
        n_recent = 1                               # the list needs room for one entry
    n_split = int(rng.integers(1, 48))
    w = workloads.clustered([9200 + 10 * seed + b for b in range(B)], G * Hkv, Hkv, D, lens,
                            kv, n_dirs=16, block=block, k_sel=k_sel, n_sink=n_sink,
                            n_recent=n_recent)
    return w, n_split


def _attend(w, b, hs, g, tokens=None):
    if w.kv_dtype == "f16":
        return oracle.attend_f16(w.q[b][hs], w.k[b][g:g + 1], w.v[b][g:g + 1], w.softmax_scale,
                                 tokens=tokens), F16_TOL
    sl = slice(g, g + 1)
    if w.kv_dtype != "i8":
        kc, ks, vc, vs = grouped_host(w, b)
        return oracle.attend_grouped(w.q[b][hs], kc[sl], ks[sl], vc[sl], vs[sl],
                                     w.softmax_scale, tokens=tokens), F16_TOL
    kc, ks, vc, vs = quantized_host(w, b)
    return oracle.attend_i8(w.q[b][hs], kc[sl], ks[sl], vc[sl], vs[sl], w.softmax_scale,
                            tokens=tokens), I8_TOL_METHOD


KINDS = ["f16", "i8", "q8_0", "q4_0", "q5_0"]
SEEDS_ALL = list(range(100, 118))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_step_configurations(gpu_lib, seed):
    _check(*_workload(seed), seed)


@pytest.mark.parametrize("seed", SEEDS_ALL)
def test_random_step_every_cache_type_and_head_dim(gpu_lib, seed):
    kv = KINDS[seed % len(KINDS)]
    D = [64, 128, 256][(seed // len(KINDS)) % 3]
    _check(*_workload(seed, kv, D), seed)


def _check(w, S, seed):
    print("random step", seed, w.kv_dtype, "D", w.D, "B", w.B, "H", w.H, "Hkv", w.Hkv,
          "lens", w.lens, "block", w.block, "k_sel", w.k_sel, "sink", w.n_sink,
          "recent", w.n_recent, "n_split", S, flush=True)
    dense, _ = run_step(prefilled_cache(w), w, quest=False, n_split=S)
    out, (score, sel, cnt) = run_step(prefilled_cache(w), w, quest=True, n_split=S)
    for b in range(w.B):
        L = w.lens[b]
        nb = -(-L // w.block)
        kmin, kmax = oracle.block_bounds(w.k[b], L, w.block)
        ref_scores = oracle.group_scores(oracle.upper_bounds(w.q[b], kmin, kmax), w.Hkv)
        np.testing.assert_allclose(score[b, :, :nb], ref_scores, rtol=2e-6, atol=1e-4)
        for g in range(w.Hkv):
            hs = slice(g * w.G, (g + 1) * w.G)
            ref, tol = _attend(w, b, hs, g)
            assert_close(dense[b, hs], ref, tol, ("dense", b, g))
            got = sel[b, g, :cnt[b, g]]
            own = oracle.select_blocks(score[b, g], nb, w.k_sel[b], w.n_sink, w.n_recent)
            assert np.array_equal(got, own["sel"]), ("selection", b, g)
            toks = oracle.selected_tokens(got, L, w.block)
            ref, tol = _attend(w, b, hs, g, tokens=toks)
            assert_close(out[b, hs], ref, tol, ("quest", b, g))
