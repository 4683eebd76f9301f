"""Pins of the group-wise quantization (oracle/quant.py: quantize_groups;
sparse_attn.md, "All-KV-types composition": q8_0 / q4_0 blocks of 32 values;
"Method: Quest-style min/max block bounds": q5_0)
and of attention over such a cache (oracle/attention.py: attend_grouped)."""
import math

import numpy as np
import pytest

import oracle
from oracle import quant


@pytest.mark.parametrize("qmax", [quant.QMAX_Q8, quant.QMAX_Q4, quant.QMAX_Q5])
def test_group_invariants(qmax):
    rng = np.random.default_rng(qmax)
    x = (rng.standard_normal((3, 50, 128)) * rng.uniform(0.01, 30, (3, 50, 1))).astype(np.float32)
    x[0, 0, :32] = 0                                  # a zero group
    codes, s16 = quant.quantize_groups(x, qmax)
    assert codes.dtype == np.int8 and s16.dtype == np.float16 and s16.shape == (3, 50, 4)
    c = codes.reshape(3, 50, 4, 32).astype(np.int64)
    s = s16.astype(np.float64)
    g = x.reshape(3, 50, 4, 32).astype(np.float64)
    assert np.all(np.abs(c) <= qmax)
    nz = s > 0
    # the absmax element of every nonzero group gets the extreme code
    assert np.all(np.abs(c).max(axis=-1)[nz] == qmax)
    # the stored scale is the f16 rounding of absmax / QMAX (float32 division)
    a = np.abs(g).max(axis=-1)
    assert np.array_equal(s16, (a.astype(np.float32) / np.float32(qmax)).astype(np.float16))
    # every value within (1/2 + 1/16) of a scale step of its representation
    err = np.abs(g - c * s[..., None])
    assert np.all(err <= s[..., None] * (0.5 + 1.0 / 16) + 1e-30)
    # zero group
    assert s16[0, 0, 0] == 0 and np.all(codes[0, 0, :32] == 0)
    # idempotent: re-quantizing the represented values gives the same codes
    codes2, s2 = quant.quantize_groups(quant.dequantize_groups(codes, s16).astype(np.float32), qmax)
    assert np.array_equal(codes2, codes) and np.array_equal(s2, s16)


def test_group_rounding_brute_force():
    """Pure Python per value: rint(x / s) against the stored f16 scale, half
    to even, clamped."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 64)).astype(np.float32) * 3
    for qmax in (127, 7, 15):
        codes, s16 = quant.quantize_groups(x, qmax)
        for r in range(4):
            for grp in range(2):
                vals = [float(v) for v in x[r, 32 * grp:32 * grp + 32]]
                a = max(abs(v) for v in vals)
                s = float(np.float16(np.float32(a) / np.float32(qmax)))
                for i, v in enumerate(vals):
                    qv = float(np.float32(np.float32(v) / np.float32(s)))
                    want = max(-qmax, min(qmax, int(round(qv))))      # round half to even
                    assert codes[r, 32 * grp + i] == want


def test_group_scale_range_edges():
    x = np.zeros((2, 32), np.float32)
    x[0, 3] = 1e-10            # a / 127 below f16's smallest subnormal: scale 0, codes 0
    x[1, 5] = 1e8              # a / 7 beyond f16's range: scale inf, codes 0
    codes, s16 = quant.quantize_groups(x, 7)
    assert s16[0, 0] == 0 and np.all(codes[0] == 0)
    assert np.isinf(s16[1, 0]) and np.all(codes[1] == 0)


def test_attention_over_the_grouped_cache_is_the_definition():
    rng = np.random.default_rng(9)
    k = rng.standard_normal((2, 70, 64)).astype(np.float32)
    v = rng.standard_normal((2, 70, 64)).astype(np.float32)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    kc, ks = quant.quantize_groups(k, 127)
    vc, vs = quant.quantize_groups(v, 127)
    out = oracle.attend_grouped(q, kc, ks, vc, vs, 0.125)
    kd, vd = quant.dequantize_groups(kc, ks), quant.dequantize_groups(vc, vs)
    for h in range(4):
        g = h // 2
        s = [math.fsum(float(a) * float(b) for a, b in zip(q[h], kd[g, t])) * 0.125
             for t in range(70)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = math.fsum(e)
        ref = [math.fsum(e[t] / den * vd[g, t, d] for t in range(70)) for d in range(64)]
        np.testing.assert_allclose(out[h], ref, rtol=1e-12, atol=1e-14)
    # q8_0 stays close to the float32 cache; q4_0 is coarser
    full = oracle.attend_f16(q, k, v, 0.125)
    rel = np.linalg.norm(out - full) / np.linalg.norm(full)
    assert rel < 2e-2
