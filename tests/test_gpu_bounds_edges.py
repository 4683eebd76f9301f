"""Bounds edge cases on the GPU against the oracle (oracle/quest.py:
block_bounds, upper_bounds; sparse_attn.md, "Method: Quest-style min/max
block bounds"): blocks whose f16 side cache holds an infinity (int8 keys past
the f16 range, directed rounding) next to finite blocks, with 8 and 16 query
rows per KV head (the scoring path of the matrix cores, which keeps the vector
path for a tile holding an infinity) and 4 (the vector path); a query channel
of exactly 0 against an infinite bound contributes 0.  Group, per-head and
chunk scores."""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_cache_append_amd as skv
from gpu_harness import DEV
from oracle import multi_token as mt

pytestmark = pytest.mark.gpu


def _cache_with_inf(seed, Hkv, L, blk):
    rng = np.random.default_rng(seed)
    D = 128
    k = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    k[:, 3 * blk + 5, 0] = 70000.0            # block 3: kmax = +inf in channel 0
    k[:, 20 * blk + 1, 1] = -90000.0          # block 20 (the second tile): kmin = -inf, channel 1
    cache = skv.Cache(1, Hkv, L, D, "i8", blk, device=DEV)
    kt = torch.from_numpy(np.ascontiguousarray(np.transpose(k, (1, 0, 2))[None])).to(DEV)
    vt = torch.from_numpy(np.ascontiguousarray(np.transpose(v, (1, 0, 2))[None])).to(DEV)
    skv.kv_append(cache, torch.zeros(1, dtype=torch.int32, device=DEV), kt, vt)
    return cache, k


def _check(got, ref):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isposinf(got), np.isposinf(ref))
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    assert not np.any(np.isnan(got))
    np.testing.assert_allclose(got[fin], ref[fin], rtol=2e-6, atol=1e-4)


@pytest.mark.parametrize("G", [4, 8])
def test_group_and_per_head_bounds_with_infinite_blocks(gpu_lib, G):
    Hkv, blk, L = 2, 16, 16 * 40
    cache, k = _cache_with_inf(31 + G, Hkv, L, blk)
    rng = np.random.default_rng(40 + G)
    q = rng.standard_normal((1, Hkv * G, 128)).astype(np.float32)
    q[0, 0, 0] = 0.0                          # head 0: q = 0 against kmax = +inf
    q[0, 1, 0] = 2.0                          # head 1: q > 0 against it: +inf
    qd = torch.from_numpy(q).to(DEV)
    sl = torch.tensor([L], dtype=torch.int32, device=DEV)
    nb = L // blk
    sg = torch.full((1, Hkv, cache.max_blocks), float("nan"), device=DEV)
    sh = torch.full((1, Hkv * G, cache.max_blocks), float("nan"), device=DEV)
    skv.block_bounds(cache, qd, sl, L, sg)
    skv.block_bounds_heads(cache, qd, sl, L, sh)
    torch.cuda.synchronize()
    kmin, kmax = oracle.block_bounds(k, L, blk)
    ub = oracle.upper_bounds(q[0], kmin, kmax)
    # the planted cases: q = 0 against +inf adds 0, q > 0 against it gives +inf
    assert np.isfinite(ub[0, 3]) and np.isposinf(ub[1, 3])
    got_h = sh.cpu().numpy()[0, :, :nb]
    _check(got_h, ub)
    gmax = got_h.reshape(Hkv, G, nb).max(axis=1)
    got_g = sg.cpu().numpy()[0, :, :nb]
    assert np.array_equal(gmax.view(np.uint32), got_g.view(np.uint32))
    _check(got_g, oracle.group_scores(ub, Hkv))


def test_chunk_bounds_with_infinite_blocks(gpu_lib):
    Hkv, blk, L, T, G = 2, 16, 16 * 40, 4, 4
    cache, k = _cache_with_inf(51, Hkv, L, blk)
    rng = np.random.default_rng(52)
    qc = rng.standard_normal((1, T, Hkv * G, 128)).astype(np.float32)
    qc[0, 2, 0, 0] = 0.0
    qd = torch.from_numpy(qc).to(DEV)
    sl = torch.tensor([L], dtype=torch.int32, device=DEV)
    sc = torch.full((1, Hkv, T, cache.max_blocks), float("nan"), device=DEV)
    skv.block_bounds_multi(cache, qd, sl, L, sc)
    torch.cuda.synchronize()
    kmin, kmax = oracle.block_bounds(k, L, blk)
    scores, _ = mt.select_multi(qc[0], kmin, kmax, L, blk, k_sel=4)
    got = sc.cpu().numpy()[0]
    for t, Lt in enumerate(mt.token_lengths(L, T)):
        nb_t = -(-int(Lt) // blk)
        _check(got[:, t, :nb_t], scores[t])
