"""skv_decode_step_static (scratch in the library's fixed per-GPU array,
nothing allocated) against skv_decode_step (caller scratch buffers): the same
kernels, so every result is bit-identical -- the output, the appended rows,
scales and bounds, the selected lists.  Two calls in a row, the second on a
smaller input (the array keeps the first call's contents), for a Quest and a
dense step; a call whose scratch would not fit is rejected before anything
runs."""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_cache_append_amd as skv
import workloads
from gpu_harness import DEV, assert_close, new_token, prefilled_cache

pytestmark = pytest.mark.gpu


def _print(*a):
    print("[no-alloc]", *a, flush=True)


def _cache_bits(c):
    return [t.view(torch.uint8).clone() for t in (c.k, c.v, c.k_scale, c.v_scale, c.kmin, c.kmax)
            if t is not None]


def _pair(w, quest):
    """One step through each entry point on identical caches."""
    base = prefilled_cache(w)
    ca, cb = base.clone(), base.clone()
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    max_len = max(w.lens)
    pos, kn, vn = new_token(w)
    kw = {}
    if quest:
        max_sel = max(w.k_sel) + w.n_sink + w.n_recent
        S = skv.default_split(w.B, w.Hkv, max_sel, kv_dtype=w.kv_dtype, sparse=True)
        ks = torch.tensor(w.k_sel, dtype=torch.int32, device=DEV)
        kw = dict(k_sel=ks, n_sink=w.n_sink, n_recent=w.n_recent)
        sel = [torch.full((w.B, w.Hkv, max_sel), -7, dtype=torch.int32, device=DEV)
               for _ in range(2)]
        cnt = [torch.full((w.B, w.Hkv), -7, dtype=torch.int32, device=DEV) for _ in range(2)]
    else:
        S = skv.default_split(w.B, w.Hkv, -(-max_len // w.block), kv_dtype=w.kv_dtype)
    outs = [torch.full((w.B, w.H, w.D), float("nan"), device=DEV) for _ in range(2)]
    ws = torch.empty(skv.workspace_bytes(w.B, w.H, w.D, S), dtype=torch.uint8, device=DEV)
    extra_a = dict(kw)
    extra_b = dict(kw)
    if quest:
        extra_a.update(score=torch.empty((w.B, w.Hkv, ca.max_blocks), device=DEV),
                       sel_idx=sel[0], sel_cnt=cnt[0])
        extra_b.update(sel_idx=sel[1], sel_cnt=cnt[1])
    skv.decode_step(ca, q, seq_len, max_len, w.softmax_scale, S, ws, outs[0], pos0=pos,
                    k_new=kn, v_new=vn, **extra_a)
    skv.decode_step_static(cb, q, seq_len, max_len, w.softmax_scale, S, outs[1], pos0=pos,
                           k_new=kn, v_new=vn, **extra_b)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    for ta, tb in zip(_cache_bits(ca), _cache_bits(cb)):
        assert torch.equal(ta, tb)
    if quest:
        assert torch.equal(sel[0], sel[1]) and torch.equal(cnt[0], cnt[1])
    return outs[1].cpu().numpy()


@pytest.mark.parametrize("kv_dtype", ["f16", "i8"])
def test_static_step_matches_the_step_twice_second_smaller(gpu_lib, kv_dtype):
    big = workloads.clustered([601, 602], 32, 8, 128, [20000, 9000], kv_dtype, n_dirs=32,
                              k_sel=[78, 35], n_sink=1, n_recent=2)
    small = workloads.clustered([603], 16, 4, 128, [3001], kv_dtype, n_dirs=16, k_sel=[11],
                                n_sink=1, n_recent=2)
    for quest in (True, False):
        for w in (big, small):
            _print(kv_dtype, "quest" if quest else "dense", w.lens)
            out = _pair(w, quest)
            if kv_dtype == "f16" and not quest:
                for b in range(w.B):
                    assert_close(out[b], oracle.attend_f16(w.q[b], w.k[b], w.v[b],
                                                           w.softmax_scale), 1e-3, b)


@pytest.mark.parametrize("kv_dtype,D", [("q5_0", 128), ("f16", 256), ("i8", 64),
                                        ("q4_0", 256)])
def test_static_step_other_formats_and_head_dims(gpu_lib, kv_dtype, D):
    """The same pairing for group-wise caches and head dims 256 and 64 (where
    the step runs its append as its own kernel)."""
    w = workloads.clustered([605], 32, 8, D, [5000], kv_dtype, n_dirs=16, k_sel=[20], n_sink=1,
                            n_recent=2)
    for quest in (True, False):
        _print(kv_dtype, D, "quest" if quest else "dense")
        _pair(w, quest)


def test_static_step_rejects_what_does_not_fit(gpu_lib):
    w = workloads.gaussian(604, 1, 32, 8, 128, [256], "f16")
    cache = prefilled_cache(w, whole=True)
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    out = torch.zeros((1, 32, 128), device=DEV)
    S = 4096          # 4 * 32 * 4096 * 130 bytes of partial states: more than the array
    assert skv.workspace_bytes(1, 32, 128, S) > skv.static_scratch_bytes()
    with pytest.raises(skv.SkvError) as e:
        skv.decode_step_static(cache, q, seq_len, 256, w.softmax_scale, S, out)
    assert e.value.status == skv.SKV_ERANGE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
