"""Pins of the 4-bit scan (oracle/scan4.py; Certified Sparse Attention via
Perturbed Retrieval: abstract, appendix layout table)."""
import math

import numpy as np
import pytest

import oracle
from oracle import scan4


def keys(seed, Hkv=2, L=200, D=32, dt=np.float16):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((Hkv, L, D)) * rng.uniform(0.1, 5.0, (Hkv, 1, D))
    return k.astype(dt)


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_index_invariants(dt):
    k = keys(1, dt=dt)
    codes, lo, step, err = scan4.build_index(k, 200, 64)
    assert codes.max() <= 15 and lo.shape == (2, 4, 32)
    kf = np.asarray(k, np.float32)
    for j in range(4):
        blk = kf[:, 64 * j:64 * j + 64]
        assert np.array_equal(lo[:, j], blk.min(axis=1))
        rec = scan4.reconstruct(codes, lo, step, 64)[:, 64 * j:64 * j + 64]
        e = np.abs(blk.astype(np.float64) - rec)
        # the recorded error is the largest float32 error, and it bounds
        # the exact one up to that float32 rounding
        assert np.all(e.max(axis=1) <= err[:, j].astype(np.float64) * (1 + 2 ** -23) + 1e-30)
        # nearest level: within half a step (plus rounding)
        assert np.all(e <= step[:, j][:, None, :].astype(np.float64) * (0.5 + 1e-5) + 1e-30)
        # the extremes are codes 0 and 15 where step > 0
        c = codes[:, 64 * j:64 * j + 64]
        live = step[:, j] > 0
        assert np.all(c.min(axis=1)[live] == 0) and np.all(c.max(axis=1)[live] == 15)


def test_constant_channel_has_zero_step_and_error():
    k = keys(2, L=64)
    k[0, :, 3] = 1.5
    codes, lo, step, err = scan4.build_index(k, 64, 64)
    assert step[0, 0, 3] == 0 and err[0, 0, 3] == 0 and np.all(codes[0, :, 3] == 0)


def test_bounds_are_sound_with_zero_tolerance():
    """LB <= q.k <= UB, both sides correctly rounded sums (math.fsum), no
    tolerance."""
    k = keys(3, L=150)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 32)).astype(np.float32)
    codes, lo, step, err = scan4.build_index(k, 150, 64)
    lb, ub = scan4.scan_bounds(q, codes, lo, step, err, 64)
    for h in range(4):
        g = h // 2
        for t in range(150):
            s = math.fsum(float(a) * float(b) for a, b in zip(q[h], k[g, t]))
            assert lb[h, t] <= s <= ub[h, t]


def test_brute_force_bounds():
    k = keys(5, Hkv=1, L=70, D=16)
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 16)).astype(np.float32)
    codes, lo, step, err = scan4.build_index(k, 70, 32)
    lb, ub = scan4.scan_bounds(q, codes, lo, step, err, 32)
    for h in range(2):
        for t in range(70):
            j = t // 32
            rec = [float(np.float32(lo[0, j, d] + np.float32(step[0, j, d] * np.float32(codes[0, t, d]))))
                   for d in range(16)]
            s = math.fsum(float(q[h, d]) * rec[d] for d in range(16))
            r = math.fsum(abs(float(q[h, d])) * float(err[0, j, d]) for d in range(16))
            assert lb[h, t] == s - r and ub[h, t] == s + r


def test_candidates_contain_the_exact_set():
    k = keys(7, Hkv=1, L=300, D=32)
    rng = np.random.default_rng(8)
    q = (rng.standard_normal((2, 32)) * 2).astype(np.float32)
    codes, lo, step, err = scan4.build_index(k, 300, 64)
    lb, ub = scan4.scan_bounds(q, codes, lo, step, err, 64)
    for h in range(2):
        exact = np.array([math.fsum(float(a) * float(b) for a, b in zip(q[h], k[0, t]))
                          for t in range(300)])
        for delta in (0.0, 1.0, 5.0):
            cand, _, _ = scan4.candidates(lb[h], ub[h], delta)
            assert np.all(cand[exact >= exact.max() - delta])
        cand, _, _ = scan4.candidates(lb[h], ub[h], 1e30)
        assert cand.all()


def test_exact_index_gives_exact_candidates():
    """Keys on the index's own grid (every channel takes two values per
    block): the reconstruction is exact, err = 0, LB = UB = q.k, and the
    candidates are exactly the tokens within delta of the best."""
    rng = np.random.default_rng(9)
    k = np.where(rng.random((1, 128, 16)) < 0.5, 0.0, 1.5).astype(np.float32)
    k[0, 0], k[0, 64] = 0.0, 1.5                      # both levels in both blocks
    k[0, 1], k[0, 65] = 1.5, 0.0
    codes, lo, step, err = scan4.build_index(k, 128, 64)
    assert np.all(err == 0)
    q = rng.standard_normal((1, 16)).astype(np.float32)
    lb, ub = scan4.scan_bounds(q, codes, lo, step, err, 64)
    assert np.array_equal(lb, ub)
    exact = k[0].astype(np.float64) @ q[0].astype(np.float64)
    np.testing.assert_allclose(ub[0], exact, rtol=1e-12, atol=1e-12)


def test_float64_bounds_agree_with_the_exact_sums():
    k = keys(11, L=130)
    rng = np.random.default_rng(12)
    q = rng.standard_normal((4, 32)).astype(np.float32)
    idx = scan4.build_index(k, 130, 64)
    lb, ub = scan4.scan_bounds(q, *idx, 64)
    lb2, ub2 = scan4.scan_bounds_f64(q, *idx, 64)
    np.testing.assert_allclose(lb2, lb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ub2, ub, rtol=1e-12, atol=1e-12)


def test_cache_keys_are_the_dequantized_values():
    """int8: the float32 product of code and scale (correctly rounded);
    group-wise: scale * code exactly (the float64 dequantization)."""
    rng = np.random.default_rng(44)
    x = rng.standard_normal((2, 50, 64)).astype(np.float32)
    kc, ks = oracle.quantize_rows(x)
    got = scan4.cache_keys(kc, ks)
    assert got.dtype == np.float32
    ref = (kc.astype(np.float64) * ks.astype(np.float64)[..., None]).astype(np.float32)
    assert np.array_equal(got, ref)                 # one rounding of the exact product
    for qmax in (oracle.QMAX_Q8, oracle.QMAX_Q4, oracle.QMAX_Q5):
        gc, gs = oracle.quantize_groups(x, qmax)
        got = scan4.cache_keys(gc, gs)
        assert np.array_equal(got.astype(np.float64), oracle.dequantize_groups(gc, gs))
