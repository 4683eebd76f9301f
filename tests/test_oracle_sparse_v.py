"""Pins of the sparse-V oracle (oracle/sparse_v.py) against closed forms,
invariants and a pure-Python brute force (sparse_attn.md, "Compose" item 3,
"Stacking with sparse-V", "Adaptive tau (the eps mode)")."""
import math

import numpy as np
import pytest

import oracle
from oracle import sparse_v


def brute(qh, kg, vg, scale, tau, eps):
    """Pure Python: softmax over all tokens (math.exp, math.fsum), keep the
    tokens whose weight reaches the threshold, sum their weighted values."""
    s = [math.fsum(float(a) * float(b) for a, b in zip(qh, krow)) * scale for krow in kg]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    den = math.fsum(e)
    p = [x / den for x in e]
    th = eps / len(p) if eps > 0 else tau
    keep = [pi >= th for pi in p]
    D = len(vg[0])
    return [math.fsum(p[t] * float(vg[t][d]) for t in range(len(p)) if keep[t]) for d in range(D)]


@pytest.mark.parametrize("L,H,Hkv,tau,eps", [(1, 1, 1, 0.3, 0.0), (5, 2, 1, 0.15, 0.0),
                                             (33, 4, 2, 0.02, 0.0), (64, 4, 1, 0.0, 0.5),
                                             (130, 8, 2, 0.0, 2.0), (17, 2, 2, 0.0, 0.0)])
def test_matches_brute_force(L, H, Hkv, tau, eps):
    rng = np.random.default_rng(L * 7 + H)
    D = 16
    q = (2.0 * rng.standard_normal((H, D))).astype(np.float32)
    k = rng.standard_normal((Hkv, L, D)).astype(np.float16)
    v = rng.standard_normal((Hkv, L, D)).astype(np.float16)
    out, keep, _ = oracle.attend_f16_sparse_v(q, k, v, 0.25, tau=tau, eps=eps)
    G = H // Hkv
    for h in range(H):
        ref = brute(q[h], k[h // G], v[h // G], 0.25, tau, eps)
        np.testing.assert_allclose(out[h], ref, rtol=1e-12, atol=1e-14)


def test_zero_threshold_is_the_dense_result_bit_for_bit():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((8, 128)).astype(np.float32)
    k = rng.standard_normal((2, 300, 128)).astype(np.float16)
    v = rng.standard_normal((2, 300, 128)).astype(np.float16)
    toks = np.array([0, 5, 6, 100, 299])
    for t in (None, toks):
        out, keep, _ = oracle.attend_f16_sparse_v(q, k, v, 0.1, tokens=t)
        assert keep.all()
        assert np.array_equal(out, oracle.attend_f16(q, k, v, 0.1, tokens=t))
    kc, ks = oracle.quantize_rows(rng.standard_normal((2, 300, 128)).astype(np.float32))
    vc, vs = oracle.quantize_rows(rng.standard_normal((2, 300, 128)).astype(np.float32))
    out, keep, _ = oracle.attend_i8_sparse_v(q, kc, ks, vc, vs, 0.1)
    assert keep.all()
    assert np.array_equal(out, oracle.attend_i8(q, kc, ks, vc, vs, 0.1))


@pytest.mark.parametrize("qmax", [oracle.QMAX_Q8, oracle.QMAX_Q4, oracle.QMAX_Q5])
def test_grouped_caches(qmax):
    """Group-wise caches: the brute force on the values scale * code, and a
    zero threshold equal to the dense group-wise oracle bit for bit."""
    rng = np.random.default_rng(qmax)
    H, Hkv, L, D = 4, 2, 40, 64
    q = (2.0 * rng.standard_normal((H, D))).astype(np.float32)
    kc, ks = oracle.quantize_groups(rng.standard_normal((Hkv, L, D)).astype(np.float32), qmax)
    vc, vs = oracle.quantize_groups(rng.standard_normal((Hkv, L, D)).astype(np.float32), qmax)
    G = H // Hkv
    for tau, eps in ((0.02, 0.0), (0.0, 0.5)):
        out, keep, _ = oracle.attend_grouped_sparse_v(q, kc, ks, vc, vs, 0.25, tau=tau, eps=eps)
        assert not keep.all()
        for h in range(H):
            g = h // G
            kd = [[float(ks[g, t, d // 32]) * int(kc[g, t, d]) for d in range(D)]
                  for t in range(L)]
            vd = [[float(vs[g, t, d // 32]) * int(vc[g, t, d]) for d in range(D)]
                  for t in range(L)]
            np.testing.assert_allclose(out[h], brute(q[h], kd, vd, 0.25, tau, eps),
                                       rtol=1e-12, atol=1e-14)
    toks = np.array([0, 3, 4, 39])
    for t in (None, toks):
        out, keep, _ = oracle.attend_grouped_sparse_v(q, kc, ks, vc, vs, 0.1, tokens=t)
        assert keep.all()
        assert np.array_equal(out, oracle.attend_grouped(q, kc, ks, vc, vs, 0.1, tokens=t))


def test_two_tokens_closed_form():
    """Logits ln 9 and 0: weights 0.9 and 0.1.  tau 0.2 keeps only the first
    token, and the normalizer still counts both: out = 0.9 v0 (not v0)."""
    D = 4
    q = np.zeros((1, D), np.float32)
    q[0, 0] = 1.0
    k = np.zeros((1, 2, D))
    k[0, 0, 0] = math.log(9.0)
    v = np.array([[[1.0, 2.0, 3.0, 4.0], [10.0, 20.0, 30.0, 40.0]]])
    out, keep, _ = oracle.attend_f16_sparse_v(q, k, v, 1.0, tau=0.2)
    assert keep.tolist() == [[True, False]]
    np.testing.assert_allclose(out[0], 0.9 * v[0, 0], rtol=1e-14)
    out, keep, _ = oracle.attend_f16_sparse_v(q, k, v, 1.0, tau=0.05)
    np.testing.assert_allclose(out[0], 0.9 * v[0, 0] + 0.1 * v[0, 1], rtol=1e-14)
    # adaptive: eps / n = eps / 2; eps 0.3 -> threshold 0.15 drops the second
    out, keep, _ = oracle.attend_f16_sparse_v(q, k, v, 1.0, eps=0.3)
    assert keep.tolist() == [[True, False]]
    # eps > 0 takes precedence over tau
    out, keep, _ = oracle.attend_f16_sparse_v(q, k, v, 1.0, tau=0.95, eps=0.1)
    assert keep.all()


def test_uniform_weights():
    """q = 0: every weight is 1/n.  A static tau above 1/n drops everything
    (out = 0); at or below 1/n keeps everything (out = mean V).  The adaptive
    rule keeps everything for eps <= 1 and nothing above."""
    rng = np.random.default_rng(5)
    n, D = 40, 8
    q = np.zeros((2, D), np.float32)
    k = rng.standard_normal((1, n, D)).astype(np.float16)
    v = rng.standard_normal((1, n, D)).astype(np.float16)
    mean = np.asarray(v[0], np.float64).mean(axis=0)
    out, keep, _ = oracle.attend_f16_sparse_v(q, k, v, 1.0, tau=1.0 / n * 1.001)
    assert not keep.any() and np.all(out == 0)
    out, keep, _ = oracle.attend_f16_sparse_v(q, k, v, 1.0, tau=1.0 / n * 0.999)
    np.testing.assert_allclose(out[0], mean, rtol=1e-12, atol=1e-15)
    out, keep, _ = oracle.attend_f16_sparse_v(q, k, v, 1.0, eps=0.999)
    assert keep.all()
    out, keep, _ = oracle.attend_f16_sparse_v(q, k, v, 1.0, eps=1.001)
    assert not keep.any()


def test_adaptive_rule_bounds_the_dropped_mass():
    """Every dropped token has p < eps / n, so the dropped mass is < eps."""
    rng = np.random.default_rng(9)
    for trial in range(20):
        n = int(rng.integers(2, 400))
        s = rng.standard_normal(n) * rng.uniform(0.5, 6.0)
        p = np.exp(s - s.max())
        p /= p.sum()
        for eps in (0.01, 0.1, 0.5):
            keep, _ = sparse_v.keep_mask(p, eps=eps)
            assert p[~keep].sum() < eps


def test_kept_sets_are_nested_in_tau():
    rng = np.random.default_rng(11)
    p = np.exp(rng.standard_normal(500) * 3)
    p /= p.sum()
    prev = np.ones(500, bool)
    for tau in (0.0, 1e-5, 1e-4, 1e-3, 1e-2, 0.1):
        keep, _ = sparse_v.keep_mask(p, tau=tau)
        assert np.all(prev | ~keep) and np.all(keep <= prev)
        prev = keep


def test_near_threshold_report():
    p = np.array([0.1, 0.1 * (1 + 5e-5), 0.1 * (1 - 5e-5), 0.2, 0.05])
    keep, near = sparse_v.keep_mask(p, tau=0.1)
    assert keep.tolist() == [True, True, False, True, False]
    assert near.tolist() == [True, True, True, False, False]


def test_a_renormalizing_variant_would_fail_the_closed_form():
    """Planted mistake: renormalizing over the kept tokens gives v0 instead
    of 0.9 v0 in the two-token case, which the closed form above rejects."""
    p = np.array([0.9, 0.1])
    keep = np.array([True, False])
    wrong = (p * keep) / (p * keep).sum()
    v = np.array([[1.0, 2.0], [10.0, 20.0]])
    assert not np.allclose(wrong @ v, 0.9 * v[0])
