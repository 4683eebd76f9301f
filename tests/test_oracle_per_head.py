"""Pins of the per-query-head block selection (oracle/quest.py:
select_blocks_per_head, union_with_heads; sparse_attn.md, "S2/S3 engineering
design" item 2 and "Open questions")."""
import numpy as np

import oracle
from oracle import quest


def test_one_head_per_group_is_the_group_max_rule():
    rng = np.random.default_rng(1)
    ub = rng.standard_normal((1, 300))
    per = quest.select_blocks_per_head(ub, 300, 40, 1, 2)
    grp = oracle.select_blocks(oracle.group_scores(ub, 1)[0], 300, 40, 1, 2)
    assert np.array_equal(per[0]["sel"], grp["sel"])


def test_identical_heads_share_the_group_set():
    """G heads with the same query: every head's set is the group-max set."""
    rng = np.random.default_rng(2)
    k = rng.standard_normal((1, 64 * 50, 32)).astype(np.float16)
    kmin, kmax = oracle.block_bounds(k, 64 * 50, 64)
    q = np.repeat(rng.standard_normal((1, 32)).astype(np.float32), 4, axis=0)
    ub = oracle.upper_bounds(q, kmin, kmax)
    per = quest.select_blocks_per_head(ub, 50, 10, 1, 2)
    grp = oracle.select_blocks(oracle.group_scores(ub, 1)[0], 50, 10, 1, 2)
    for r in per:
        assert np.array_equal(r["sel"], grp["sel"])
    u, m = quest.union_with_heads([r["sel"] for r in per])
    assert np.array_equal(u, grp["sel"]) and np.all(m == 0b1111)


def test_each_head_takes_its_own_top_k_by_brute_force():
    rng = np.random.default_rng(3)
    for trial in range(30):
        nb = int(rng.integers(1, 80))
        G = int(rng.choice([1, 2, 4, 8]))
        k_sel = int(rng.integers(0, nb + 2))
        ub = np.round(rng.standard_normal((G, nb)), 1)        # ties happen
        per = quest.select_blocks_per_head(ub, nb, k_sel, 1, 2)
        for i in range(G):
            forced = {0} | set(range(max(0, nb - 2), nb))
            cands = [j for j in range(nb) if j not in forced]
            order = sorted(cands, key=lambda j: (-ub[i, j], j))
            want = sorted(forced | set(order[:k_sel]))
            assert per[i]["sel"].tolist() == want


def test_union_and_head_masks():
    sets = [np.array([0, 3, 9]), np.array([0, 4, 9, 11]), np.array([]), np.array([3])]
    u, m = quest.union_with_heads(sets)
    assert u.tolist() == [0, 3, 4, 9, 11]
    assert m.tolist() == [0b0011, 0b1001, 0b0010, 0b0011, 0b0010]
    # every head's set is recovered from the union and its bit
    for i, s in enumerate(sets):
        assert u[(m >> i) & 1 == 1].tolist() == sorted(np.asarray(s).tolist())


def test_attention_over_a_heads_own_set_from_the_union():
    """Attending with head i's tokens equals attending over the union with
    the blocks head i did not choose left out (the kernel's masked walk)."""
    rng = np.random.default_rng(4)
    L, D = 64 * 20 + 7, 16
    k = rng.standard_normal((1, L, D)).astype(np.float16)
    v = rng.standard_normal((1, L, D)).astype(np.float16)
    q = rng.standard_normal((2, D)).astype(np.float32)
    sets = [np.array([0, 5, 19, 20]), np.array([0, 2, 20])]
    u, m = quest.union_with_heads(sets)
    for i in range(2):
        own = oracle.attend_f16(q[i:i + 1], k, v, 0.25, oracle.selected_tokens(sets[i], L, 64))
        via = oracle.attend_f16(q[i:i + 1], k, v, 0.25,
                                oracle.selected_tokens(u[(m >> i) & 1 == 1], L, 64))
        assert np.array_equal(own, via)
