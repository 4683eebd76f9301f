"""Pins for oracle.attention: brute force on tiny inputs and closed forms.

The brute force here is an independent scalar statement of
softmax(q k^T * scale) V in plain Python (``math.exp``, ``math.fsum``); the
closed forms (one token, q = 0, equal keys, two tokens) follow from the
definition by hand.  A dropped scale, a wrong GQA index, a transposed operand
or a missing max-shift in the oracle fails one of them.
"""
import math

import numpy as np
import pytest

import oracle


def brute_attention(q, k, v, scale, G):
    """Scalar softmax attention: q [H][D], k/v [Hkv][L][D] nested lists."""
    H = len(q)
    out = []
    for h in range(H):
        g = h // G
        logits = [math.fsum(qd * kd for qd, kd in zip(q[h], krow)) * scale for krow in k[g]]
        mx = max(logits)
        w = [math.exp(s - mx) for s in logits]
        z = math.fsum(w)
        D = len(q[h])
        out.append([math.fsum(w[t] * v[g][t][d] for t in range(len(w))) / z for d in range(D)])
    return np.array(out)


CASES = [(L, D, H, Hkv) for L in (1, 2, 3, 63, 64, 65, 130)
         for D in (16,) for (H, Hkv) in ((1, 1), (4, 1), (8, 2))] + \
        [(257, 128, 32, 8), (64, 128, 4, 1)]


@pytest.mark.parametrize("L,D,H,Hkv", CASES)
def test_f16_matches_scalar_brute_force(L, D, H, Hkv):
    rng = np.random.default_rng(L * 1000 + D + H)
    k = rng.standard_normal((Hkv, L, D)).astype(np.float16)
    v = rng.standard_normal((Hkv, L, D)).astype(np.float16)
    q = (2.0 * rng.standard_normal((H, D))).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    got = oracle.attend_f16(q, k, v, scale)
    ref = brute_attention(q.astype(float).tolist(), k.astype(float).tolist(),
                          v.astype(float).tolist(), scale, H // Hkv)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("L,D,H,Hkv", [(1, 16, 4, 1), (65, 16, 8, 2), (130, 128, 4, 2)])
def test_i8_matches_scalar_brute_force(L, D, H, Hkv):
    """The int8 method written as scalar code from its formula: integer dot of
    codes, times the three scales; weights times v_scale times v code."""
    rng = np.random.default_rng(7 + L)
    kf = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    vf = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    q = rng.standard_normal((H, D)).astype(np.float32)
    kc, ks = oracle.quantize_rows(kf)
    vc, vs = oracle.quantize_rows(vf)
    qc, qs = oracle.quantize_rows(q)
    scale = 1.0 / math.sqrt(D)
    G = H // Hkv
    ref = []
    for h in range(H):
        g = h // G
        logits = []
        for t in range(L):
            dot = sum(int(a) * int(b) for a, b in zip(qc[h], kc[g, t]))
            logits.append(dot * float(qs[h]) * float(ks[g, t]) * scale)
        mx = max(logits)
        w = [math.exp(s - mx) for s in logits]
        z = math.fsum(w)
        ref.append([math.fsum(w[t] * float(vs[g, t]) * int(vc[g, t, d]) for t in range(L)) / z
                    for d in range(D)])
    got = oracle.attend_i8(q, kc, ks, vc, vs, scale)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-12, atol=1e-13)


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((2, 1, 128)).astype(np.float16)
    v = rng.standard_normal((2, 1, 128)).astype(np.float16)
    q = rng.standard_normal((8, 128)).astype(np.float32) * 10
    out = oracle.attend_f16(q, k, v, 0.0883883)
    for h in range(8):
        assert np.array_equal(out[h], v[h // 4, 0].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    """q = 0 makes every logit 0, exp(0) = 1, so the output is mean(V) (the
    cpu-attn card's 'uniform-logit' construction, section 'Method')."""
    rng = np.random.default_rng(2)
    L = 300
    k = rng.standard_normal((2, L, 64)).astype(np.float16)
    v = rng.standard_normal((2, L, 64)).astype(np.float16)
    q = np.zeros((4, 64), dtype=np.float32)
    out = oracle.attend_f16(q, k, v, 0.125)
    for h in range(4):
        np.testing.assert_allclose(out[h], v[h // 2].astype(np.float64).mean(axis=0), rtol=0, atol=1e-15)
    # int8: q = 0 quantizes to all-zero codes with scale 0, logits all 0
    kc, ks = oracle.quantize_rows(k.astype(np.float32))
    vc, vs = oracle.quantize_rows(v.astype(np.float32))
    o8 = oracle.attend_i8(q, kc, ks, vc, vs, 0.125)
    for h in range(4):
        mean = (vc[h // 2].astype(np.float64) * vs[h // 2].astype(np.float64)[:, None]).mean(axis=0)
        np.testing.assert_allclose(o8[h], mean, rtol=0, atol=1e-15)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    row = rng.standard_normal(32).astype(np.float16)
    k = np.broadcast_to(row, (1, 50, 32)).copy()
    v = rng.standard_normal((1, 50, 32)).astype(np.float16)
    q = rng.standard_normal((3, 32)).astype(np.float32)
    out = oracle.attend_f16(q, k, v, 0.3)
    for h in range(3):
        np.testing.assert_allclose(out[h], v[0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_two_tokens_closed_form():
    """out = sigma(s0 - s1) v0 + (1 - sigma(s0 - s1)) v1."""
    rng = np.random.default_rng(4)
    k = rng.standard_normal((1, 2, 16)).astype(np.float16)
    v = rng.standard_normal((1, 2, 16)).astype(np.float16)
    q = rng.standard_normal((1, 16)).astype(np.float32)
    scale = 0.7
    s = [float(np.dot(q[0].astype(float), k[0, t].astype(float))) * scale for t in range(2)]
    sig = 1.0 / (1.0 + math.exp(-(s[0] - s[1])))
    ref = sig * v[0, 0].astype(float) + (1 - sig) * v[0, 1].astype(float)
    np.testing.assert_allclose(oracle.attend_f16(q, k, v, scale)[0], ref, rtol=1e-13, atol=1e-15)


def test_scale_and_gqa_mapping_matter():
    """Guards against a dropped softmax scale and a wrong KV-head index."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((2, 40, 16)).astype(np.float16)
    v = rng.standard_normal((2, 40, 16)).astype(np.float16)
    q = rng.standard_normal((4, 16)).astype(np.float32) * 3
    a = oracle.attend_f16(q, k, v, 0.25)
    b = oracle.attend_f16(q, k, v, 1.0)
    assert np.max(np.abs(a - b)) > 1e-3
    # heads 0,1 read KV head 0; heads 2,3 read KV head 1
    a0 = oracle.attend_f16(q[:2], k[:1], v[:1], 0.25)
    a1 = oracle.attend_f16(q[2:], k[1:], v[1:], 0.25)
    np.testing.assert_array_equal(a, np.concatenate([a0, a1]))


def test_token_restriction_equals_attention_on_the_subset():
    rng = np.random.default_rng(6)
    k = rng.standard_normal((1, 100, 16)).astype(np.float16)
    v = rng.standard_normal((1, 100, 16)).astype(np.float16)
    q = rng.standard_normal((2, 16)).astype(np.float32)
    T = np.array([0, 5, 6, 50, 99])
    np.testing.assert_array_equal(oracle.attend_f16(q, k, v, 0.5, tokens=T),
                                  oracle.attend_f16(q, k[:, T], v[:, T], 0.5))
    assert np.all(oracle.attend_f16(q, k, v, 0.5, tokens=np.array([], dtype=int)) == 0)


def test_int8_dots_are_exact_integers():
    rng = np.random.default_rng(8)
    kf = rng.standard_normal((2, 70, 128)).astype(np.float32)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    kc, _ = oracle.quantize_rows(kf)
    dots, qc, _ = oracle.int8_logit_dots(q, kc)
    for h in range(4):
        for t in (0, 33, 69):
            assert dots[h, t] == sum(int(a) * int(b) for a, b in zip(qc[h], kc[h // 2, t]))
    assert np.max(np.abs(dots)) <= 127 * 127 * 128


def test_int8_method_gap_to_dequantized_reference_is_the_query_rounding():
    """C3 (quantized q) vs R8 (float q) differ only by the query quantization.
    For N(0,1) data at D = 128 the logit error std is about scale_q/sqrt(12)*|k|
    ~ 6e-3 relative; a gap far outside [1e-3, 2e-2] means a broken oracle."""
    rng = np.random.default_rng(9)
    kf = rng.standard_normal((2, 2048, 128)).astype(np.float32)
    vf = rng.standard_normal((2, 2048, 128)).astype(np.float32)
    q = rng.standard_normal((8, 128)).astype(np.float32)
    kc, ks = oracle.quantize_rows(kf)
    vc, vs = oracle.quantize_rows(vf)
    a = oracle.attend_i8(q, kc, ks, vc, vs, 1 / math.sqrt(128))
    r = oracle.attend_i8_dequant(q, kc, ks, vc, vs, 1 / math.sqrt(128))
    rel = np.linalg.norm(a - r) / np.linalg.norm(r)
    assert 1e-3 < rel < 2e-2, rel
    # with an exactly representable query (codes times a power of two) the two agree
    q2 = np.zeros((8, 128), np.float32)
    q2[:, :5] = np.array([127, -64, 3, 0, 100], np.float32) / 128
    a2 = oracle.attend_i8(q2, kc, ks, vc, vs, 0.1)
    r2 = oracle.attend_i8_dequant(q2, kc, ks, vc, vs, 0.1)
    np.testing.assert_allclose(a2, r2, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("base", [2.0, math.e])
def test_combine_of_any_partition_equals_unsplit(base):
    rng = np.random.default_rng(10)
    L, D = 500, 32
    k = rng.standard_normal((1, L, D)).astype(np.float16)
    v = rng.standard_normal((1, L, D)).astype(np.float16)
    q = (3 * rng.standard_normal((1, D))).astype(np.float32)
    ref = oracle.attend_f16(q, k, v, 0.2)[0]
    cuts = np.sort(rng.choice(np.arange(1, L), size=6, replace=False))
    sets = np.split(np.arange(L), cuts) + [np.array([], dtype=int)]
    m, l, a = oracle.softmax_partials(q[0], k[0], v[0], 0.2, sets, base=base)
    np.testing.assert_allclose(oracle.combine_partials(m, l, a, base=base), ref, rtol=1e-13, atol=1e-15)
    # a non-contiguous partition too
    perm = rng.permutation(L)
    sets2 = [perm[:17], perm[17:300], perm[300:]]
    m, l, a = oracle.softmax_partials(q[0], k[0], v[0], 0.2, sets2, base=base)
    np.testing.assert_allclose(oracle.combine_partials(m, l, a, base=base), ref, rtol=1e-13, atol=1e-15)
    assert np.all(oracle.combine_partials(np.array([-np.inf]), np.array([0.0]), np.zeros((1, D))) == 0)
