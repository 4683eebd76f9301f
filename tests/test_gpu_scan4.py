"""The 4-bit key index and its GQA-shared scan on the GPU (skv_scan4_build,
skv_scan4_candidates) against the oracle (oracle/scan4.py): the index (codes,
lo, step, err) bit-exact, rebuilding from an append position equal to a full
build, the upper bounds within float32 rounding of the exact ones, the
candidate sets equal up to tokens within rounding of the threshold, and
every token within delta of the best exact score among the GPU's candidates
(up to the same band).  Over int8 and group-wise caches the keys are the
cache's (code x scale, one float32 product: oracle scan4.cache_keys)."""
import copy
import math

import numpy as np
import pytest
import torch

import sparse_kv_cache_append_amd as skv
import workloads
from gpu_harness import DEV, build_cache, device_inputs, grouped_host, quantized_host
from oracle import scan4

pytestmark = pytest.mark.gpu


def _print(*a):
    print("[scan4]", *a, flush=True)


def build(cache, w, pos0=None, seq=None, max_len=None):
    idx = skv.Scan4Index(cache, device=DEV)
    p = torch.zeros(w.B, dtype=torch.int32, device=DEV) if pos0 is None else pos0
    s = torch.tensor(w.lens, dtype=torch.int32, device=DEV) if seq is None else seq
    skv.scan4_build(cache, idx, p, s, max(w.lens) if max_len is None else max_len)
    torch.cuda.synchronize()
    return idx


def check_index(idx, w, b):
    L = w.lens[b]
    codes, lo, step, err = scan4.build_index(w.k[b], L, w.block)
    packed = idx.codes4.cpu().numpy()[b, :, :L]
    got = np.empty(codes.shape, np.uint8)
    got[..., 0::2] = packed & 15
    got[..., 1::2] = packed >> 4
    assert np.array_equal(got, codes)
    nb = w.n_blocks(b)
    for name, ref in (("lo", lo), ("step", step), ("err", err)):
        g = getattr(idx, name).cpu().numpy()[b, :, :nb]
        assert np.array_equal(g.view(np.uint32), ref.view(np.uint32)), name
    return codes, lo, step, err


def run_scan(cache, idx, w, delta, S=None):
    q, seq_len = device_inputs(w)
    max_len = max(w.lens)
    S = S or skv.scan4_default_split(w.B, w.Hkv, max(-(-max_len // w.block), 1))
    ws = torch.empty(skv.scan4_workspace_bytes(w.B, w.H, S, max_len), dtype=torch.uint8,
                     device=DEV)
    cand = torch.full((w.B, w.H, max(-(-max_len // 32), 1)), -1, dtype=torch.int32, device=DEV)
    cnt = torch.full((w.B, w.H), -7, dtype=torch.int32, device=DEV)
    skv.scan4_candidates(cache, idx, q, seq_len, max_len, delta, S, ws, cand, cnt)
    torch.cuda.synchronize()
    ub = ws[:w.B * w.H * max_len * 4].view(torch.float32).view(w.B, w.H, max_len).cpu().numpy()
    return ub, cand.cpu().numpy().view(np.uint32), cnt.cpu().numpy()


def check_scan(w, b, index, ub_gpu, cand, cnt, delta):
    codes, lo, step, err = index
    L = w.lens[b]
    lb, ub = scan4.scan_bounds_f64(w.q[b], codes, lo, step, err, w.block)
    rec = scan4.reconstruct(codes, lo, step, w.block).astype(np.float64)
    jb = np.arange(L) // w.block
    n_band = 0
    for h in range(w.H):
        g = h // w.G
        qh = w.q[b][h].astype(np.float64)
        # the float32 evaluation's natural scale per token
        scale = np.abs(rec[g]) @ np.abs(qh) + np.abs(qh) @ err[g].astype(np.float64).T[:, jb] \
            + np.abs(qh) @ np.abs(lo[g].astype(np.float64)).T[:, jb]
        tol = 2e-5 * scale + 1e-6
        bad = np.nonzero(np.abs(ub_gpu[b, h, :L] - ub[h]) > tol)[0]
        assert bad.size == 0, (b, h, bad.size, bad[:6].tolist(), ub_gpu[b, h, bad[:6]].tolist(),
                               ub[h][bad[:6]].tolist(), tol[bad[:6]].tolist())
        c_ref, _, th = scan4.candidates(lb[h], ub[h], delta)
        bits = ((cand[b, h][np.arange(L) // 32] >> (np.arange(L) % 32).astype(np.uint32)) & 1
                ).astype(bool)
        # words past the tokens are zero
        tail = np.arange(L, cand.shape[2] * 32)
        assert not np.any((cand[b, h][tail // 32] >> (tail % 32).astype(np.uint32)) & 1)
        band = np.abs(ub[h] - th) <= 2 * tol + 2e-5 * (abs(th) + 1)
        assert not np.any((bits != c_ref) & ~band), (b, h)
        n_band += int(np.sum(bits != c_ref))
        assert cnt[b, h] == int(bits.sum())
        exact = np.asarray(w.k[b][g], np.float64) @ qh
        need = exact >= exact.max() - delta
        assert not np.any(need & ~bits & ~band), (b, h)
    return n_band


@pytest.mark.parametrize("H,Hkv,lens,block", [(32, 8, [3000, 777], 64), (8, 8, [1500], 16),
                                              (16, 8, [4100], 128), (32, 4, [2049, 1], 64),
                                              (16, 4, [2500], 96), (8, 4, [5000, 300], 256)])
def test_index_and_candidates(gpu_lib, H, Hkv, lens, block):
    w = workloads.clustered([950 + b for b in range(len(lens))], H, Hkv, 128, lens, "f16",
                            n_dirs=8, amp=4.0, block=block)
    cache = build_cache(w)
    idx = build(cache, w)
    for delta in (0.0, 2.0, 8.0):
        ub, cand, cnt = run_scan(cache, idx, w, delta)
        for b in range(w.B):
            index = check_index(idx, w, b)
            nb = check_scan(w, b, index, ub, cand, cnt, delta)
            _print(H, Hkv, lens, block, "delta", delta, "seq", b, "candidates",
                   cnt[b].tolist()[:4], "band differences", nb)


def test_rebuild_after_append_equals_full_build(gpu_lib):
    w = workloads.gaussian(960, 2, 16, 4, 128, [1000, 2049], "f16")
    cache = build_cache(w)
    lens_m1 = torch.tensor([L - 1 for L in w.lens], dtype=torch.int32, device=DEV)
    idx = build(cache, w, seq=lens_m1)                       # index of L - 1 tokens
    pos = torch.tensor([L - 1 for L in w.lens], dtype=torch.int32, device=DEV)
    skv.scan4_build(cache, idx, pos, torch.tensor(w.lens, dtype=torch.int32, device=DEV),
                    max(w.lens))                              # the new token's block
    torch.cuda.synchronize()
    for b in range(w.B):
        check_index(idx, w, b)


def test_32k_workload_scan(gpu_lib):
    w = workloads.named(3)
    cache = build_cache(w)
    idx = build(cache, w)
    ub, cand, cnt = run_scan(cache, idx, w, 8.0)
    index = check_index(idx, w, 0)
    nb = check_scan(w, 0, index, ub, cand, cnt, 8.0)
    _print("32K delta 8: candidates per head", cnt[0].tolist(), "band differences", nb)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("kv", ["i8", "q8_0", "q4_0", "q5_0"])
def test_quantized_caches(gpu_lib, kv, D):
    """The index built from the keys the cache holds, bit-exact; bounds and
    candidates against those keys."""
    w = workloads.clustered([990 + D, 991 + D], 32, 8, D, [3000, 777], kv, n_dirs=8, amp=4.0,
                            block=64)
    cache = build_cache(w)
    idx = build(cache, w)
    wk = copy.copy(w)
    host = quantized_host if kv == "i8" else grouped_host
    wk.k = [scan4.cache_keys(*host(w, b)[:2]) for b in range(w.B)]
    for delta in (0.0, 8.0):
        ub, cand, cnt = run_scan(cache, idx, w, delta)
        for b in range(w.B):
            index = check_index(idx, wk, b)
            nb = check_scan(wk, b, index, ub, cand, cnt, delta)
            _print(kv, D, "delta", delta, "seq", b, "band differences", nb)
