"""Pins for oracle.quest: side cache, bound soundness, selection rules.

The selection brute force below decides membership by counting, for each
candidate, how many candidates beat it (larger score, or equal score and lower
index); that is an independent statement of "top-K, ties to the lower index"
that shares nothing with the oracle's sort.
"""
import math

import numpy as np
import pytest

import oracle
import workloads


def test_bounds_are_channel_min_max_over_clipped_blocks():
    rng = np.random.default_rng(0)
    L, B = 130, 64
    k = rng.standard_normal((2, L, 8)).astype(np.float16)
    kmin, kmax = oracle.block_bounds(k, L, B)
    assert kmin.shape == (2, 3, 8) and kmin.dtype == np.float16
    for g in range(2):
        for j in range(3):
            rows = k[g, j * B:min(L, (j + 1) * B)]
            assert rows.shape[0] == (64 if j < 2 else 2)
            for d in range(8):
                assert kmin[g, j, d] == min(rows[:, d].tolist())
                assert kmax[g, j, d] == max(rows[:, d].tolist())


def test_float32_keys_get_directed_f16_bounds():
    rng = np.random.default_rng(1)
    k = (rng.standard_normal((1, 200, 16)) * 3).astype(np.float32)
    kmin, kmax = oracle.block_bounds(k, 200, 64)
    for j in range(4):
        rows = k[0, j * 64:min(200, (j + 1) * 64)]
        lo = rows.min(axis=0)
        hi = rows.max(axis=0)
        assert np.all(kmin[0, j].astype(np.float32) <= lo)
        assert np.all(kmax[0, j].astype(np.float32) >= hi)
        assert np.all(np.nextafter(kmin[0, j], np.float16(np.inf)).astype(np.float32) > lo)
        assert np.all(np.nextafter(kmax[0, j], np.float16(-np.inf)).astype(np.float32) < hi)


def test_bounds_of_a_prefix_merge_into_bounds_of_the_whole():
    """Incremental fill == from-scratch: min/max over a block equals the
    min/max-merge of the bounds of any split of its rows (page section
    'All-KV-types composition')."""
    rng = np.random.default_rng(2)
    k = rng.standard_normal((2, 64, 16)).astype(np.float32)
    full = oracle.block_bounds(k, 64, 64)
    a = oracle.block_bounds(k[:, :23], 23, 64)
    b = oracle.block_bounds(k[:, 23:], 41, 64)
    assert np.array_equal(np.minimum(a[0], b[0]), full[0])
    assert np.array_equal(np.maximum(a[1], b[1]), full[1])


@pytest.mark.parametrize("kv", ["f16", "f32"])
def test_upper_bound_is_sound_with_zero_tolerance(kv):
    """UB[h][j] >= q.k_t for every token of block j (exact sums via fsum)."""
    w = workloads.clustered([11], 8, 2, 32, [300], "f16" if kv == "f16" else "i8",
                            n_dirs=4, block=64)
    keys = w.k[0]
    kmin, kmax = oracle.block_bounds(keys, 300, 64)
    ub = oracle.upper_bounds(w.q[0], kmin, kmax)
    q = w.q[0].astype(np.float64)
    for h in range(8):
        g = h // 4
        for j in range(ub.shape[1]):
            rows = keys[g, j * 64:min(300, (j + 1) * 64)].astype(np.float64)
            best = max(math.fsum(q[h] * r) for r in rows)
            assert ub[h, j] >= best
    # and equality when a block holds one token (kmin == kmax == k)
    one = keys[:, :1]
    kmin1, kmax1 = oracle.block_bounds(one, 1, 64)
    ub1 = oracle.upper_bounds(w.q[0], kmin1, kmax1)
    if kv == "f16":
        for h in range(8):
            assert ub1[h, 0] == math.fsum(q[h] * one[h // 4, 0].astype(np.float64))


def test_upper_bound_picks_kmax_for_positive_and_kmin_for_negative_q():
    kmin = np.array([[[-1.0, -2.0, 0.5]]], np.float16)
    kmax = np.array([[[3.0, 1.0, 4.0]]], np.float16)
    q = np.array([[2.0, -1.0, 0.0]], np.float32)
    # 2*3 + (-1)(-2) + 0 = 8
    assert oracle.upper_bounds(q, kmin, kmax)[0, 0] == 8.0


def test_group_score_is_max_over_the_group():
    ub = np.array([[1.0, 5.0], [2.0, 0.0], [7.0, 7.0], [-1.0, 8.0]])
    assert oracle.group_scores(ub, 2).tolist() == [[2.0, 5.0], [7.0, 8.0]]


def brute_select(score, nb, k, n_sink, n_recent):
    forced = {j for j in range(nb) if j < n_sink or j >= nb - n_recent}
    cands = [j for j in range(nb) if j not in forced]
    chosen = set()
    for j in cands:
        beaten = sum(1 for i in cands if score[i] > score[j] or (score[i] == score[j] and i < j))
        if beaten < k:
            chosen.add(j)
    return sorted(forced | chosen)


@pytest.mark.parametrize("nb,k,ns,nr", [(1, 3, 1, 2), (2, 1, 1, 2), (5, 1, 1, 2), (20, 4, 1, 2),
                                        (20, 0, 1, 2), (20, 17, 1, 2), (20, 30, 1, 2),
                                        (33, 7, 2, 4), (64, 10, 0, 0), (64, 10, 1, 0)])
def test_selection_matches_counting_brute_force(nb, k, ns, nr):
    rng = np.random.default_rng(nb * 100 + k)
    for trial in range(5):
        score = rng.integers(-3, 4, size=nb).astype(np.float32)   # many exact ties
        if trial % 2:
            score = rng.standard_normal(nb).astype(np.float32)
        r = oracle.select_blocks(score, nb, k, ns, nr)
        assert r["sel"].tolist() == brute_select(score.tolist(), nb, k, ns, nr)
        n_forced = len({j for j in range(nb) if j < ns or j >= nb - nr})
        assert len(r["sel"]) == min(nb, k + n_forced)


def test_zero_query_selects_the_lowest_index_candidates():
    """q = 0 makes every bound +-0; ties go to the lower index, and -0 == +0."""
    score = np.zeros(40, np.float32)
    score[::3] = -0.0
    r = oracle.select_blocks(score, 40, 5, 1, 2)
    assert r["sel"].tolist() == [0, 1, 2, 3, 4, 5, 38, 39]


def test_select_all_when_budget_covers_every_candidate():
    score = np.random.default_rng(3).standard_normal(50)
    assert oracle.select_blocks(score, 50, 47, 1, 2)["sel"].tolist() == list(range(50))
    assert oracle.select_blocks(score, 50, 1000, 1, 2)["sel"].tolist() == list(range(50))


def test_forced_blocks_are_kept_even_with_lowest_scores():
    score = np.arange(30, dtype=np.float64)          # block 0 lowest, last blocks highest
    score[-2:] = -100
    r = oracle.select_blocks(score, 30, 3, 1, 2)
    assert r["sel"].tolist() == [0, 25, 26, 27, 28, 29]
    r2 = oracle.select_blocks(score, 30, 3, 1, 2, forced_in_candidates=True)
    assert r2["sel"].tolist() == [0, 25, 26, 27, 28, 29]  # OR reading: top-3 of all = 25,26,27


def test_planted_aligned_block_survives_selection():
    """A block whose keys all point along q (norm 40, well above the bound of a
    noisy block) must be selected (the retrieval
    role of the page's needle gate)."""
    w = workloads.clustered([5], 4, 1, 64, [64 * 40], "f16", n_dirs=8, block=64)
    k = w.k[0].copy()
    q = w.q[0]
    u = q[0] / np.linalg.norm(q[0])
    k[0, 64 * 17:64 * 18] = (40 * u).astype(np.float16)
    kmin, kmax = oracle.block_bounds(k, 64 * 40, 64)
    sc = oracle.group_scores(oracle.upper_bounds(q, kmin, kmax), 1)
    r = oracle.select_blocks(sc[0], 40, 4, 1, 2)
    assert 17 in r["sel"].tolist()


def test_near_tie_report():
    score = np.array([5.0, 3.0, 3.00001, 2.99999, 1.0, 0.0, 0.0], np.float64)
    r = oracle.select_blocks(score, 7, 2, 0, 0)
    assert r["sel"].tolist() == [0, 2]
    assert r["cutoff"] == 3.00001
    assert r["near"].tolist() == [1, 2, 3]


def test_selected_tokens_clip_last_block():
    t = oracle.selected_tokens(np.array([0, 2]), 150, 64)
    assert t.tolist() == list(range(64)) + list(range(128, 150))


def test_sparse_with_every_block_selected_equals_dense_bit_for_bit():
    """Select-all anchor (page section 'Gate ladder': K_SEL = n_blocks makes
    sparse equal dense)."""
    w = workloads.clustered([6], 8, 2, 32, [333], "f16", n_dirs=4, block=64)
    nb = w.n_blocks(0)
    kmin, kmax = oracle.block_bounds(w.k[0], 333, 64)
    sc = oracle.group_scores(oracle.upper_bounds(w.q[0], kmin, kmax), 2)
    dense = oracle.attend_f16(w.q[0], w.k[0], w.v[0], w.softmax_scale)
    for g in range(2):
        sel = oracle.select_blocks(sc[g], nb, nb, 1, 2)["sel"]
        toks = oracle.selected_tokens(sel, 333, 64)
        sp = oracle.attend_f16(w.q[0], w.k[0], w.v[0], w.softmax_scale, tokens=toks)
        assert np.array_equal(sp[g * 4:(g + 1) * 4], dense[g * 4:(g + 1) * 4])


def test_zero_query_channel_contributes_zero_even_against_infinite_bounds():
    kmin = np.array([[[-np.inf, -1.0]]], np.float16)
    kmax = np.array([[[np.inf, 2.0]]], np.float16)
    q = np.array([[0.0, 3.0]], np.float32)
    assert oracle.upper_bounds(q, kmin, kmax)[0, 0] == 6.0


def test_nan_keys_are_left_out_of_the_envelope():
    """Reading taken for NaN keys: they do not enter a channel's min/max.  The
    pin is a plain Python min/max over the non-NaN values of each channel
    (+inf / -inf when none is left)."""
    rng = np.random.default_rng(7)
    for dt in (np.float16, np.float32):
        k = rng.standard_normal((2, 70, 16)).astype(dt)
        k[0, 3, 5] = np.nan                  # one NaN in a block
        k[1, 64:70, 2] = np.nan              # a whole (partial) block's channel
        kmin, kmax = oracle.block_bounds(k, 70, 64)
        for g in range(2):
            for j in range(2):
                for d in range(16):
                    vals = [float(x) for x in k[g, j * 64:min(70, (j + 1) * 64), d]
                            if not np.isnan(x)]
                    lo = min(vals) if vals else np.inf
                    hi = max(vals) if vals else -np.inf
                    if dt == np.float16:
                        assert float(kmin[g, j, d]) == lo and float(kmax[g, j, d]) == hi
                    else:
                        assert float(kmin[g, j, d]) <= lo and float(kmax[g, j, d]) >= hi
                        if vals:
                            assert float(kmin[g, j, d]) > lo - 2e-3 * (abs(lo) + 1)
        assert kmin[1, 1, 2] == np.inf and kmax[1, 1, 2] == -np.inf
