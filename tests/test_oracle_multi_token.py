"""Pins of the multi-token query oracle (oracle/multi_token.py; sparse_attn.md,
"S2/S3 engineering design" item 2 and "Open questions": the prefill selector
takes many query tokens per call).

Each pin checks the oracle against something other than itself: causal
attention written as one masked softmax per KV head, the dense path when every
block is selected, causality as an invariant, the forced windows of each
token's own prefix, and a brute-force union."""
import numpy as np

import oracle
from oracle import multi_token as mt


def _masked_causal(q, k, v, scale, L):
    """Causal attention of the chunk as one [T][L] score matrix per head with
    -inf above each token's prefix (the textbook masked form)."""
    T, H, D = q.shape
    Hkv = k.shape[0]
    G = H // Hkv
    lens = [L - T + 1 + t for t in range(T)]
    out = np.zeros((T, H, D))
    for h in range(H):
        kg = k[h // G, :L].astype(np.float64)
        vg = v[h // G, :L].astype(np.float64)
        s = (q[:, h].astype(np.float64) @ kg.T) * scale             # [T][L]
        mask = np.arange(L)[None, :] >= np.array(lens)[:, None]
        s = np.where(mask, -np.inf, s)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h] = (w / w.sum(axis=1, keepdims=True)) @ vg
    return out


def _case(seed, T, H, Hkv, L, D=32):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    k = rng.standard_normal((Hkv, L, D)).astype(np.float16)
    v = rng.standard_normal((Hkv, L, D)).astype(np.float16)
    return q, k, v


def test_token_lengths():
    assert mt.token_lengths(100, 4).tolist() == [97, 98, 99, 100]
    assert mt.token_lengths(2, 4).tolist() == [0, 0, 1, 2]
    assert mt.token_lengths(5, 1).tolist() == [5]


def test_dense_equals_the_masked_causal_softmax():
    for seed, T, H, Hkv, L in [(1, 4, 8, 2, 130), (2, 2, 4, 4, 65), (3, 8, 2, 1, 40),
                               (4, 3, 6, 3, 3)]:
        q, k, v = _case(seed, T, H, Hkv, L)
        got = mt.attend_f16_multi(q, k, v, 0.2, L)
        ref = _masked_causal(q, k, v, 0.2, L)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_one_token_is_the_decode_step():
    q, k, v = _case(5, 1, 8, 2, 97)
    got = mt.attend_f16_multi(q, k, v, 0.3, 97)[0]
    ref = _masked_causal(q, k, v, 0.3, 97)[0]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_tokens_before_the_chunk_start_attend_to_nothing():
    q, k, v = _case(6, 4, 4, 2, 2)
    out = mt.attend_f16_multi(q, k, v, 0.25, 2)
    assert np.all(out[0] == 0) and np.all(out[1] == 0)
    assert np.all(np.isfinite(out)) and np.any(out[3] != 0)


def test_causality_later_keys_do_not_reach_earlier_tokens():
    q, k, v = _case(7, 4, 8, 2, 200)
    base = mt.attend_f16_multi(q, k, v, 0.2, 200)
    k2, v2 = k.copy(), v.copy()
    k2[:, 199] = 50.0                       # only the last token sees position 199
    v2[:, 199] = -7.0
    other = mt.attend_f16_multi(q, k2, v2, 0.2, 200)
    assert np.array_equal(base[:3], other[:3])
    assert not np.allclose(base[3], other[3])


def test_int8_dense_equals_a_masked_method_form():
    """The int8 method per token: its own query codes and scale, logits from the
    integer dots, softmax over its prefix -- written out as one masked matrix."""
    rng = np.random.default_rng(8)
    T, H, Hkv, L, D = 3, 4, 2, 90, 32
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    kf = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    vf = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    kc, ks = oracle.quantize_rows(kf)
    vc, vs = oracle.quantize_rows(vf)
    got = mt.attend_i8_multi(q, kc, ks, vc, vs, 0.2, L)
    G = H // Hkv
    for t in range(T):
        qc, qs = oracle.quantize_rows(q[t])
        Lt = L - T + 1 + t
        for h in range(H):
            g = h // G
            dots = kc[g, :Lt].astype(np.int64) @ qc[h].astype(np.int64)
            s = dots * np.float64(qs[h]) * ks[g, :Lt].astype(np.float64) * 0.2
            w = np.exp(s - s.max())
            w /= w.sum()
            ref = w @ (vc[g, :Lt].astype(np.float64) * vs[g, :Lt, None].astype(np.float64))
            np.testing.assert_allclose(got[t, h], ref, rtol=1e-12, atol=1e-12)


def test_selecting_every_block_is_dense():
    q, k, v = _case(9, 4, 8, 2, 64 * 6 + 5)
    L = 64 * 6 + 5
    kmin, kmax = oracle.block_bounds(k, L, 64)
    _, sels = mt.select_multi(q, kmin, kmax, L, 64, k_sel=100, n_sink=1, n_recent=2)
    got = mt.attend_f16_quest_multi(q, k, v, 0.2, L, [[s["sel"] for s in r] for r in sels], 64)
    np.testing.assert_allclose(got, _masked_causal(q, k, v, 0.2, L), rtol=1e-12, atol=1e-12)


def test_each_token_keeps_the_forced_windows_of_its_own_prefix():
    """A chunk that crosses a block boundary: tokens before it have one block
    fewer; every set holds that token's sink and recent blocks and nothing at or
    past its own block count."""
    rng = np.random.default_rng(10)
    T, H, Hkv, D, blk = 4, 8, 2, 32, 16
    L = 16 * 9 + 2                          # tokens 0, 1 end in block 8; 2, 3 in block 9
    k = rng.standard_normal((Hkv, L, D)).astype(np.float16)
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    kmin, kmax = oracle.block_bounds(k, L, blk)
    scores, sels = mt.select_multi(q, kmin, kmax, L, blk, k_sel=3, n_sink=1, n_recent=2)
    lens = mt.token_lengths(L, T)
    for t in range(T):
        nb_t = -(-int(lens[t]) // blk)
        assert scores[t].shape == (Hkv, nb_t)
        for g in range(Hkv):
            s = set(sels[t][g]["sel"].tolist())
            assert {0, nb_t - 2, nb_t - 1} <= s and max(s) < nb_t and len(s) == 3 + 3


def test_bound_is_sound_for_every_key_a_token_sees():
    rng = np.random.default_rng(11)
    T, H, Hkv, D, blk, L = 3, 4, 2, 32, 8, 77
    k = rng.standard_normal((Hkv, L, D)).astype(np.float16)
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    kmin, kmax = oracle.block_bounds(k, L, blk)
    scores, _ = mt.select_multi(q, kmin, kmax, L, blk, k_sel=2)
    G = H // Hkv
    for t, Lt in enumerate(mt.token_lengths(L, T)):
        for g in range(Hkv):
            for pos in range(int(Lt)):
                for h in range(g * G, (g + 1) * G):
                    dot = float(np.dot(q[t, h].astype(np.float64), k[g, pos].astype(np.float64)))
                    assert scores[t][g, pos // blk] >= dot


def test_union_by_brute_force():
    rng = np.random.default_rng(12)
    for _ in range(40):
        T = int(rng.choice([1, 2, 4, 8]))
        sets = [np.array(sorted(set(rng.integers(0, 50, int(rng.integers(0, 20))).tolist())))
                for _ in range(T)]
        u, m = mt.union_tokens(sets)
        expect = sorted(set(j for s in sets for j in s.tolist()))
        assert u.tolist() == expect
        for i, j in enumerate(expect):
            assert m[i] == sum(1 << t for t in range(T) if j in sets[t].tolist())
