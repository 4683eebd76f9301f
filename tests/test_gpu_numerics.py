"""Numerical edges of the decode kernels' softmax-weighted sums, against the
float64 oracle.

The kernels feed the softmax weights to the matrix cores as an f16 high part
plus an f16 low part (int8: the weight times the token's V scale in a running
power-of-two unit).  Two input shapes stress the dynamic range of that split:

* a peaked query over a long flat tail: a few keys get weight 1 and every
  other key the same tiny weight (about 2^-18 of the peak), so the tail's
  weights are far below the f16 normal range while their total mass is a
  sizeable part of the normalizer; V has a non-zero mean, so a systematic
  loss on the tail shows up in every channel.  Run at 262,144 tokens with one
  part per KV head (each wavefront sees a peak first, then a quarter of the
  tail) and in the default launch configuration;
* outlier V rows: rows whose largest value is 10^3 times the others', early
  in every part and wavefront walk, for flat weights (q = 0) and a random
  query.

Outputs are checked per head and per element (see gpu_harness.close_report),
and for the outlier case also channel by channel, since the outlier channel
dominates a head's largest element.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_kv_cache_append_amd as skv
from gpu_harness import DEV, assert_close, build_cache, quantized_host, run_dense
from workloads import Workload

pytestmark = pytest.mark.gpu


def _print(*a):
    print("[numerics]", *a, flush=True)


NEEDLES = (0, 16, 32, 48, 64, 96)    # the first tile of every wavefront's walk (f16, int8)


def peaked_workload(kv_dtype, L=262144, H=32, Hkv=4, D=128, seed=91, needles=NEEDLES,
                    tail_log2=-17.0):
    """Tail keys: one random vector orthogonal to the KV head's direction u
    (logit ~ 0); needle keys (at ``needles``): c * u; query heads a_h * u with
    a_h * c / sqrt(D) = ln(2) * (-tail_log2) * f_h, f_h in [0.95, 1.1], so the
    tail's weight is about 2^(tail_log2 f_h) of a needle's.  V ~ 3 + N(0, 1)."""
    rng = np.random.default_rng(seed)
    G = H // Hkv
    u = rng.standard_normal((Hkv, D)).astype(np.float32)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    z = rng.standard_normal((Hkv, D)).astype(np.float32)
    z -= (z * u).sum(1, keepdims=True) * u
    gap = math.log(2.0) * (-tail_log2) * math.sqrt(D)         # a * c
    c = math.sqrt(gap)
    k = np.repeat(z[:, None, :], L, axis=1)
    for g in range(Hkv):
        k[g, list(needles)] = c * u[g]
    v = (3.0 + rng.standard_normal((Hkv, L, D))).astype(np.float32)
    f = np.linspace(0.95, 1.1, G)
    q = np.stack([c * f[h % G] * u[h // G] for h in range(H)]).astype(np.float32)[None]
    cast = (lambda x: x.astype(np.float16)) if kv_dtype == "f16" else (lambda x: x)
    return Workload(f"peaked-{kv_dtype} L{L}", 1, H, Hkv, D, [L], kv_dtype, [cast(k)],
                    [cast(v)], q)


def outlier_workload(kv_dtype, zero_q, L=32768, H=32, Hkv=8, D=128, seed=92, part=1024):
    """V ~ 2 + N(0, 1); at the first tokens of every wavefront's first tile in
    every ``part``-token part (f16 tiles of 16, int8 tiles of 32 tokens),
    channel 5 of the V row is 10^3 times the row's largest value."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    v = (2.0 + rng.standard_normal((Hkv, L, D))).astype(np.float32)
    pos = [p + o for p in range(0, L, part) for o in (0, 16, 32, 48, 64, 96)]
    v[:, pos, 5] = 1e3 * np.abs(v[:, pos]).max(axis=-1)
    q = np.zeros((1, H, D), np.float32) if zero_q else rng.standard_normal((1, H, D)).astype(
        np.float32)
    cast = (lambda x: x.astype(np.float16)) if kv_dtype == "f16" else (lambda x: x)
    return Workload(f"outlier-{kv_dtype}", 1, H, Hkv, D, [L], kv_dtype, [cast(k)], [cast(v)], q)


def reference(w):
    if w.kv_dtype == "f16":
        return oracle.attend_f16(w.q[0], w.k[0], w.v[0], w.softmax_scale), 1e-3
    kc, ks, vc, vs = quantized_host(w, 0)
    return oracle.attend_i8(w.q[0], kc, ks, vc, vs, w.softmax_scale), 1e-4


def tail_share(w):
    """Fraction of each head's softmax mass on the tail keys (float64)."""
    kf = np.asarray(w.k[0], np.float64)
    out = []
    for h in range(w.H):
        s = kf[h // w.G] @ np.asarray(w.q[0, h], np.float64) * w.softmax_scale
        p = np.exp(s - s.max())
        out.append(1.0 - p[list(NEEDLES)].sum() / p.sum())
    return np.array(out)


@pytest.mark.parametrize("kv_dtype", ["f16", "i8"])
def test_peaked_query_flat_tail_262k(gpu_lib, kv_dtype):
    w = peaked_workload(kv_dtype)
    share = tail_share(w)
    _print(kv_dtype, "tail share of the mass", share.min(), share.max())
    assert share.min() > 0.05         # the tail matters to every head
    cache = build_cache(w)
    ref, tol = reference(w)
    for S in (1, None):
        out, _ = run_dense(cache, w, n_split=S)
        _print(kv_dtype, "parts", S)
        assert_close(out[0], ref, tol, kv_dtype, S)


def _channelwise(got, ref, tol):
    """Every element within tol of itself (plus tol * 1e-2 of its head's
    largest value for elements near zero)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    floor = 1e-2 * np.abs(ref).max(axis=-1, keepdims=True)
    bad = np.abs(got - ref) > tol * (np.abs(ref) + floor)
    return int(bad.sum())


@pytest.mark.parametrize("kv_dtype", ["f16", "i8"])
@pytest.mark.parametrize("zero_q", [True, False])
def test_outlier_v_rows_early_in_every_part(gpu_lib, kv_dtype, zero_q):
    w = outlier_workload(kv_dtype, zero_q)
    cache = build_cache(w)
    ref, tol = reference(w)
    out, _ = run_dense(cache, w)
    _print(kv_dtype, "q = 0" if zero_q else "random q")
    assert_close(out[0], ref, tol, kv_dtype, zero_q)
    assert _channelwise(out[0], ref, tol) == 0
    # the same with the parts' lists given explicitly (sparse walk, every block)
    nb = w.n_blocks(0)
    sel = torch.arange(nb, dtype=torch.int32, device=DEV).repeat(1, w.Hkv, 1).contiguous()
    cnt = torch.full((1, w.Hkv), nb, dtype=torch.int32, device=DEV)
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    S = skv.default_split(1, w.Hkv, nb, kv_dtype=w.kv_dtype, sparse=True)
    ws = torch.empty(skv.workspace_bytes(1, w.H, w.D, S), dtype=torch.uint8, device=DEV)
    o2 = torch.empty((1, w.H, w.D), dtype=torch.float32, device=DEV)
    skv.decode_attn(cache, q, seq_len, w.lens[0], w.softmax_scale, S, ws, sel, cnt)
    skv.combine(ws, 1, w.H, w.D, S, o2)
    torch.cuda.synchronize()
    o2 = o2.cpu().numpy()
    assert_close(o2[0], ref, tol, kv_dtype, zero_q, "list")
    assert _channelwise(o2[0], ref, tol) == 0
