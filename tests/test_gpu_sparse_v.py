"""Sparse-V decode attention (skv_decode_attn_sparse_v + skv_combine)
against the float64 oracle (oracle/sparse_v.py).

The keep decisions are compared bit by bit through the kernel's keep mask:
they must equal the oracle's except for tokens whose weight lies within the
oracle's near-threshold band (the kernel decides in float32).  The output is
compared element-wise with the oracle evaluated on the kernel's own
decisions (f16 and group-wise caches 1e-3, int8 cache 1e-4 against the int8
method), and with
the oracle's own decisions within the same bar plus the mass of the tokens
decided differently.  Sizes span several tiles, ragged tails, every GQA group
size, dense walks and given block lists, and both rules (static tau,
adaptive eps)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_cache_append_amd as skv
import workloads
from gpu_harness import (DEV, assert_close, build_cache, grouped_host, quantized_host,
                         sel_tensor_from_lists)

pytestmark = pytest.mark.gpu


def _print(*a):
    print("[sparse-v]", *a, flush=True)


def run_sv(cache, w, tau, eps, sel=None, n_split=None):
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    max_len = max(w.lens)
    if sel is not None:
        si, sc = sel
        units = int(si.shape[2])
    else:
        si = sc = None
        units = max(-(-max_len // w.block), 1)
    S = n_split or skv.default_split(w.B, w.Hkv, units, kv_dtype=w.kv_dtype,
                                     sparse=sel is not None)
    ws = torch.full((skv.sparse_v_workspace_bytes(w.B, w.H, w.Hkv, w.D, S, max_len),), 0x7F,
                    dtype=torch.uint8, device=DEV)
    keep = torch.zeros((w.B, w.H, max(-(-max_len // 32), 1)), dtype=torch.int32, device=DEV)
    out = torch.empty((w.B, w.H, w.D), dtype=torch.float32, device=DEV)
    skv.decode_attn_sparse_v(cache, q, seq_len, max_len, w.softmax_scale, S, ws, tau=tau,
                             eps=eps, sel_idx=si, sel_cnt=sc,
                             keep_mask=keep if max_len > 0 else None)
    skv.combine(ws, w.B, w.H, w.D, S, out)
    torch.cuda.synchronize()
    kb = keep.cpu().numpy().view(np.uint32)
    return out.cpu().numpy(), kb


def keep_bits(words, tokens):
    tokens = np.asarray(tokens, np.int64)
    return ((words[tokens // 32] >> (tokens % 32).astype(np.uint32)) & 1).astype(bool)


def check_seq(w, b, out, kb, tau, eps, tokens=None, lists=None):
    """Sequence b: decisions and output against the oracle (per KV head when
    lists give each KV head its own blocks)."""
    tol = 1e-4 if w.kv_dtype == "i8" else 1e-3
    if w.kv_dtype == "i8":
        kc, ks, vc, vs = quantized_host(w, b)
    elif w.kv_dtype != "f16":
        kc, ks, vc, vs = grouped_host(w, b)
    n_diff = n_near = 0
    for g in range(w.Hkv):
        hs = slice(g * w.G, (g + 1) * w.G)
        toks = np.arange(w.lens[b]) if lists is None else oracle.selected_tokens(
            lists[g], w.lens[b], w.block)
        sl = slice(g, g + 1)
        if w.kv_dtype == "f16":
            def ref(keep=None):
                return oracle.attend_f16_sparse_v(w.q[b][hs], w.k[b][g:g + 1], w.v[b][g:g + 1],
                                                  w.softmax_scale, tau, eps, toks, keep)
        elif w.kv_dtype == "i8":
            def ref(keep=None):
                return oracle.attend_i8_sparse_v(w.q[b][hs], kc[sl], ks[sl], vc[sl], vs[sl],
                                                 w.softmax_scale, tau, eps, toks, keep)
        else:
            def ref(keep=None):
                return oracle.attend_grouped_sparse_v(w.q[b][hs], kc[sl], ks[sl], vc[sl],
                                                      vs[sl], w.softmax_scale, tau, eps, toks,
                                                      keep)
        o_ref, k_ref, near = ref()
        k_gpu = np.stack([keep_bits(kb[b, h], toks) for h in range(g * w.G, (g + 1) * w.G)])
        diff = k_gpu != k_ref
        assert not np.any(diff & ~near), ("decisions differ outside the near band", b, g,
                                         int((diff & ~near).sum()))
        n_diff += int(diff.sum())
        n_near += int(near.sum())
        o_own, _, _ = ref(k_gpu)
        assert_close(out[b, hs], o_own, tol, b, g)
    return n_diff, n_near


CASES = [
    # seed, kv, H, Hkv, lens, tau, eps
    (701, "f16", 32, 8, [1000, 2500], 1e-3, 0.0),
    (702, "f16", 8, 8, [513], 2e-2, 0.0),
    (703, "f16", 16, 8, [4097, 64], 0.0, 0.5),
    (704, "f16", 64, 8, [3001], 0.0, 2.0),
    (705, "i8", 32, 8, [1000, 2500], 1e-3, 0.0),
    (706, "i8", 32, 4, [7000], 0.0, 1.0),
    (707, "i8", 16, 16, [333], 1e-2, 0.0),
    (708, "i8", 16, 8, [2049, 95, 1], 5e-4, 0.0),
    (741, "q8_0", 32, 8, [1000, 2500], 1e-3, 0.0),       # group-wise caches
    (742, "q4_0", 16, 8, [4097, 64], 0.0, 0.5),
    (743, "q5_0", 32, 4, [3001], 0.0, 1.0),
    (744, "q4_0", 16, 16, [333], 1e-2, 0.0),
    (745, "q5_0", 8, 8, [2049, 95, 1], 5e-4, 0.0),
]


@pytest.mark.parametrize("seed,kv,H,Hkv,lens,tau,eps", CASES)
def test_sparse_v_dense_walk(gpu_lib, seed, kv, H, Hkv, lens, tau, eps):
    _print("dense", seed, kv, H, Hkv, lens, tau, eps)
    w = workloads.clustered([seed + 10 * b for b in range(len(lens))], H, Hkv, 128, lens, kv,
                            n_dirs=8, amp=5.0)
    cache = build_cache(w)
    out, kb = run_sv(cache, w, tau, eps)
    for b in range(w.B):
        nd, nn = check_seq(w, b, out, kb, tau, eps)
        _print("seq", b, "decisions differing (all near the threshold):", nd, "near:", nn)


@pytest.mark.parametrize("kv", ["f16", "i8", "q8_0", "q4_0", "q5_0"])
def test_sparse_v_given_lists(gpu_lib, kv):
    """Quest lists (host-built, differing per KV head, with a clipped last
    block) and sparse-V inside them."""
    w = workloads.clustered([711, 712], 32, 8, 128, [5000, 3333], kv, n_dirs=8, amp=5.0)
    cache = build_cache(w)
    rng = np.random.default_rng(5)
    lists = []
    for b in range(w.B):
        nb = w.n_blocks(b)
        lists.append([np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, 17, replace=False)]))
                      for _ in range(w.Hkv)])
    max_sel = max(len(x) for row in lists for x in row)
    si, sc = sel_tensor_from_lists(lists, w.B, w.Hkv, max_sel)
    for tau, eps in ((2e-3, 0.0), (0.0, 0.3)):
        out, kb = run_sv(cache, w, tau, eps, sel=(si, sc))
        for b in range(w.B):
            check_seq(w, b, out, kb, tau, eps, lists=lists[b])


@pytest.mark.parametrize("kv", ["f16", "i8", "q8_0", "q4_0", "q5_0"])
def test_sparse_v_zero_threshold_is_dense(gpu_lib, kv):
    w = workloads.gaussian(721, 2, 32, 8, 128, [3000, 777], kv)
    cache = build_cache(w)
    out, kb = run_sv(cache, w, 0.0, 0.0)
    for b in range(w.B):
        if kv == "f16":
            ref = oracle.attend_f16(w.q[b], w.k[b], w.v[b], w.softmax_scale)
            assert_close(out[b], ref, 1e-3, b)
        elif kv != "i8":
            kc, ks, vc, vs = grouped_host(w, b)
            assert_close(out[b], oracle.attend_grouped(q=w.q[b], k_codes=kc, k_scales=ks,
                                                       v_codes=vc, v_scales=vs,
                                                       scale=w.softmax_scale), 1e-3, b)
        else:
            kc, ks, vc, vs = quantized_host(w, b)
            assert_close(out[b], oracle.attend_i8(w.q[b], kc, ks, vc, vs, w.softmax_scale),
                         1e-4, b)
        for h in range(w.H):
            assert keep_bits(kb[b, h], np.arange(w.lens[b])).all()


def test_sparse_v_edges(gpu_lib):
    """An empty sequence beside others (zeros), a threshold above every
    weight (nothing kept: zeros), one part per KV head and many parts."""
    w = workloads.gaussian(731, 3, 16, 4, 128, [0, 1, 200], "f16")
    cache = build_cache(w)
    for S in (1, 9):
        out, kb = run_sv(cache, w, 1e-3, 0.0, n_split=S)
        assert np.all(out[0] == 0)
        for b in (1, 2):
            check_seq(w, b, out, kb, 1e-3, 0.0)
    out, kb = run_sv(cache, w, 2.0, 0.0)
    assert np.all(out == 0) and not kb.any()


@pytest.mark.parametrize("tau", [1e-4, 1e-3])
def test_sparse_v_32k_quest_workload(gpu_lib, tau):
    """The 32K workload: Quest selection (skv_select_topk on the GPU's own
    scores) then sparse-V over the selected blocks, in the launch
    configuration bench.py times."""
    from gpu_harness import run_select
    w = workloads.named(3)
    cache = build_cache(w)
    _, sel, cnt, _ = run_select(cache, w)
    s_h, c_h = sel.cpu().numpy(), cnt.cpu().numpy()
    lists = [[s_h[0, g, :c_h[0, g]] for g in range(w.Hkv)]]
    out, kb = run_sv(cache, w, tau, 0.0, sel=(sel, cnt))
    nd, nn = check_seq(w, 0, out, kb, tau, 0.0, lists=lists[0])
    kept = sum(int(keep_bits(kb[0, h], oracle.selected_tokens(lists[0][h // w.G], w.lens[0],
                                                                w.block)).sum())
               for h in range(w.H))
    _print("32K Quest + sparse-V tau", tau, "kept (head, token) pairs", kept, "differing", nd)
