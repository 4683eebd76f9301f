"""skv_decode_step against the five calls it composes.

The step folds the one-token append into the bounds pass and the block
selection into the attention kernel's prologue; neither changes any
arithmetic, so every result must be bit-identical to kv_append ->
block_bounds -> select_topk -> decode_attn -> combine on an identical cache:
the output, the appended rows, scales and side-cache bounds, the scores and
the selected lists, for each size class of the folded selection.  The dense
step folds the append into the attention kernel instead; its cases start
from poisoned rows at the append positions.  The
fallback paths (selection as its own kernel when a
part spans more than 64 list entries or a row has more than 4096 blocks; the
dense step) are held to the same bar.  One output per case is also checked
against the float64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_cache_append_amd as skv
import workloads
from gpu_harness import (DEV, assert_close, new_token as _new_token, prefilled_cache as _prefilled,
                         quantized_host, rel_err)

pytestmark = pytest.mark.gpu


def _print(*a):
    print("[step]", *a, flush=True)


def _buffers(w, cache, quest, max_sel, S):
    out = torch.full((w.B, w.H, w.D), float("nan"), device=DEV)
    ws = torch.empty(skv.workspace_bytes(w.B, w.H, w.D, S), dtype=torch.uint8, device=DEV)
    if not quest:
        return out, ws, None, None, None
    score = torch.full((w.B, w.Hkv, cache.max_blocks), float("nan"), device=DEV)
    sel = torch.full((w.B, w.Hkv, max_sel), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((w.B, w.Hkv), -7, dtype=torch.int32, device=DEV)
    return out, ws, score, sel, cnt


def _cache_tensors(c):
    return [t for t in (c.k, c.v, c.k_scale, c.v_scale, c.kmin, c.kmax) if t is not None]


def _poison_rows(cache, pos):
    """Fill the rows the step's append will write with values no correct
    result can depend on (NaN halves; int8 code -128 and NaN scales; q8_0 /
    q4_0 / q5_0 bytes 0x80 (both q5_0 planes) and NaN group scales)."""
    for b, p in enumerate(pos.tolist()):
        if cache.kv_dtype == "f16":
            cache.k[b, :, p] = float("nan")
            cache.v[b, :, p] = float("nan")
        elif cache.kv_dtype == "q5_0":
            for t in (cache.k, cache.v):
                for plane in cache.q5_planes(t):
                    plane[b, :, p] = 0x80
            cache.k_scale[b, :, p] = float("nan")
            cache.v_scale[b, :, p] = float("nan")
        elif cache.kv_dtype in ("q8_0", "q4_0"):
            cache.k[b, :, p] = 0x80
            cache.v[b, :, p] = 0x80
            cache.k_scale[b, :, p] = float("nan")
            cache.v_scale[b, :, p] = float("nan")
        else:
            cache.k[b, :, p] = -128
            cache.v[b, :, p] = -128
            cache.k_scale[b, :, p] = float("nan")
            cache.v_scale[b, :, p] = float("nan")


def _run_case(w, quest, append, S=None, max_seq=None, max_sel=None, poison=False, lag=0,
              tight=False, no_oracle=False):
    """``poison``: the append positions hold NaN / out-of-range data before the
    step; ``lag``: seq_len excludes the last ``lag`` tokens (with lag 1 the new
    token lies past every walk); ``tight``: max_len is the largest seq_len
    (0 for an empty cache) instead of the largest L_b."""
    base = _prefilled(w, max_seq, whole=not append)
    if poison:
        _poison_rows(base, _new_token(w)[0])
    ca, cb = base.clone(), base.clone()
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor([L - lag for L in w.lens], dtype=torch.int32, device=DEV)
    max_len = max(w.lens) - (lag if tight else 0)
    ks = torch.tensor(w.k_sel, dtype=torch.int32, device=DEV) if quest else None
    if quest:
        max_sel = max_sel or (max(w.k_sel) + w.n_sink + w.n_recent)
        S = S or skv.default_split(w.B, w.Hkv, max_sel, kv_dtype=w.kv_dtype, sparse=True)
    else:
        S = S or skv.default_split(w.B, w.Hkv, -(-max_len // w.block), kv_dtype=w.kv_dtype)
    pos, kn, vn = _new_token(w)
    out_a, ws_a, sc_a, sel_a, cnt_a = _buffers(w, ca, quest, max_sel, S)
    out_b, ws_b, sc_b, sel_b, cnt_b = _buffers(w, cb, quest, max_sel, S)
    # composed calls
    if append:
        skv.kv_append(ca, pos, kn, vn)
    if quest:
        skv.block_bounds(ca, q, seq_len, max_len, sc_a)
        skv.select_topk(sc_a, seq_len, w.block, ks, w.n_sink, w.n_recent, sel_a, cnt_a)
        skv.decode_attn(ca, q, seq_len, max_len, w.softmax_scale, S, ws_a, sel_a, cnt_a)
    else:
        skv.decode_attn(ca, q, seq_len, max_len, w.softmax_scale, S, ws_a)
    skv.combine(ws_a, w.B, w.H, w.D, S, out_a)
    # one step
    skv.decode_step(cb, q, seq_len, max_len, w.softmax_scale, S, ws_b, out_b,
                    pos0=pos if append else None, k_new=kn if append else None,
                    v_new=vn if append else None, k_sel=ks, n_sink=w.n_sink,
                    n_recent=w.n_recent, score=sc_b, sel_idx=sel_b, sel_cnt=cnt_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(ws_a, ws_b)      # the same partial states, bit for bit
    for ta, tb in zip(_cache_tensors(ca), _cache_tensors(cb)):
        assert torch.equal(ta.view(torch.uint8), tb.view(torch.uint8))     # bits (NaN rows too)
    if quest:
        assert torch.equal(sel_a, sel_b)
        assert torch.equal(cnt_a, cnt_b)
        for b, L in enumerate(w.lens):
            nb = -(-L // w.block)
            a_, b_ = sc_a[b, :, :nb], sc_b[b, :, :nb]
            bad = (a_.view(torch.int32) != b_.view(torch.int32)).nonzero().tolist()
            assert not bad, ("scores differ", b, bad[:8],
                             [(float(a_[i, j]), float(b_[i, j])) for i, j in bad[:8]])
    return out_b.cpu().numpy(), (sel_b.cpu().numpy(), cnt_b.cpu().numpy()) if quest else None


def _with_nan_key(w):
    """Channels 3 and 77 of the last (appended) key are NaN in every KV head."""
    for b, L in enumerate(w.lens):
        w.k[b][:, L - 1, 3] = np.nan
        w.k[b][:, L - 1, 77] = np.nan
    return w


def _oracle_check(w, out, sel):
    """Sequence 0's output against the float64 definition over the step's
    own selected blocks (f16 within 1e-3; int8 within 1e-4 of the method)."""
    G = w.G
    for g in range(w.Hkv):
        hs = slice(g * G, (g + 1) * G)
        toks = None
        if sel is not None:
            s, c = sel
            toks = oracle.selected_tokens(s[0, g, :c[0, g]], w.lens[0], w.block)
        if w.kv_dtype == "f16":
            ref = oracle.attend_f16(w.q[0][hs], w.k[0][g:g + 1], w.v[0][g:g + 1],
                                    w.softmax_scale, tokens=toks)
            assert_close(out[0, hs], ref, 1e-3)
        elif w.kv_dtype in ("q8_0", "q4_0", "q5_0"):
            qmax = {"q8_0": oracle.QMAX_Q8, "q4_0": oracle.QMAX_Q4,
                    "q5_0": oracle.QMAX_Q5}[w.kv_dtype]
            kc, ksc = oracle.quantize_groups(w.k[0][g:g + 1], qmax)
            vc, vsc = oracle.quantize_groups(w.v[0][g:g + 1], qmax)
            ref = oracle.attend_grouped(w.q[0][hs], kc, ksc, vc, vsc, w.softmax_scale,
                                        tokens=toks)
            assert_close(out[0, hs], ref, 1e-3)
        else:
            kc, ksc, vc, vsc = quantized_host(w, 0)
            sl = slice(g, g + 1)
            ref = oracle.attend_i8(w.q[0][hs], kc[sl], ksc[sl], vc[sl], vsc[sl],
                                   w.softmax_scale, tokens=toks)
            assert_close(out[0, hs], ref, 1e-4)


STEP_CASES = [
    # name, workload factory, quest, append, extra
    ("quest-f16 fresh+mid block", lambda: workloads.clustered(
        [501, 502], 32, 8, 128, [2049, 3000], "f16", n_dirs=16, k_sel=[8, 20],
        n_sink=1, n_recent=2), True, True, {}),
    ("quest-i8 G8", lambda: workloads.clustered(
        [503], 32, 4, 128, [5000], "i8", n_dirs=32, k_sel=[30], n_sink=1, n_recent=4),
        True, True, {}),
    ("quest-f16 G1 block 16", lambda: workloads.clustered(
        [504], 8, 8, 128, [1500], "f16", n_dirs=8, block=16, k_sel=[20], n_sink=1,
        n_recent=2), True, True, {}),
    ("quest-f16 G2 L=1 in batch", lambda: workloads.clustered(
        [505, 506], 16, 8, 128, [1, 700], "f16", n_dirs=8, k_sel=[3, 3], n_sink=1,
        n_recent=2), True, True, {}),
    ("quest-f16 no append", lambda: workloads.clustered(
        [507], 32, 8, 128, [4096], "f16", n_dirs=16, k_sel=[16], n_sink=1, n_recent=2),
        True, False, {}),
    ("quest-f16 long parts (select kernel)", lambda: workloads.clustered(
        [508], 32, 8, 128, [32768], "f16", n_dirs=64, k_sel=[128], n_sink=1, n_recent=2),
        True, True, {"S": 2}),
    ("quest-f16 >4096 blocks (select kernel)", lambda: workloads.clustered(
        [509], 16, 4, 128, [3000], "f16", n_dirs=8, k_sel=[10], n_sink=1, n_recent=2),
        True, True, {"max_seq": 64 * 4100}),
    # the folded selection holds 2, 4 or 16 keys per thread by row size:
    # 513 candidates (the first row past 2 x 256), exactly 512 (no sink)
    ("quest-f16 513 candidates", lambda: workloads.clustered(
        [513], 16, 8, 128, [514 * 64 - 10], "f16", n_dirs=32, k_sel=[130], n_sink=1,
        n_recent=2), True, True, {}),
    ("quest-i8 512 candidates no sink", lambda: workloads.clustered(
        [514], 32, 4, 128, [512 * 64], "i8", n_dirs=32, k_sel=[100], n_sink=0,
        n_recent=4), True, True, {}),
    # 7 parts: the published slices do not divide the list evenly
    ("quest-f16 7 parts", lambda: workloads.clustered(
        [515, 516], 32, 8, 128, [6000, 9000], "f16", n_dirs=16, k_sel=[20, 33], n_sink=1,
        n_recent=2), True, True, {"S": 7}),
    ("dense-f16 varlen", lambda: workloads.gaussian(
        510, 3, 16, 4, 128, [100, 64, 2500], "f16"), False, True, {}),
    # the dense step writes the new token from the attention kernel: its rows
    # start out poisoned; positions at a block's first token (fresh bounds),
    # mid block, position 0, a part count that does not divide the blocks
    ("dense-f16 append poisoned rows", lambda: workloads.gaussian(
        518, 3, 32, 8, 128, [65, 1, 4097], "f16"), False, True, {"poison": True}),
    ("dense-i8 append poisoned rows G8", lambda: workloads.gaussian(
        519, 2, 32, 4, 128, [3000, 129], "i8"), False, True, {"poison": True}),
    ("dense-i8 append 7 parts", lambda: workloads.gaussian(
        520, 2, 16, 8, 128, [2050, 700], "i8"), False, True, {"poison": True, "S": 7}),
    ("dense-f16 append block 16", lambda: workloads.gaussian(
        527, 2, 32, 8, 128, [1601, 999], "f16", block=16), False, True, {"poison": True}),
    ("dense-i8 append block 128 G2", lambda: workloads.gaussian(
        528, 2, 16, 8, 128, [1025, 2000], "i8", block=128), False, True, {"poison": True}),
    ("dense-f16 append 40 parts G1", lambda: workloads.gaussian(
        521, 1, 8, 8, 128, [999], "f16"), False, True, {"poison": True, "S": 40}),
    # seq_len without the new token: the append still lands, no walk reads it
    ("dense-f16 append past the length", lambda: workloads.gaussian(
        522, 2, 32, 8, 128, [2, 300], "f16"), False, True, {"lag": 1}),
    ("dense-i8 append past the length", lambda: workloads.gaussian(
        523, 2, 32, 8, 128, [1, 129], "i8"), False, True, {"lag": 1}),
    ("dense-i8 no append", lambda: workloads.gaussian(
        511, 1, 32, 8, 128, [1000], "i8"), False, False, {}),
    # the first token of an empty cache: seq_len 0, max_len 0, position 0 (the
    # part that writes the row is found with at least one block per part)
    ("dense-f16 first token of an empty cache", lambda: workloads.gaussian(
        529, 2, 32, 8, 128, [1, 1], "f16"), False, True, {"lag": 1, "tight": True}),
    ("dense-i8 first token of an empty cache", lambda: workloads.gaussian(
        530, 1, 32, 4, 128, [1], "i8"), False, True, {"lag": 1, "tight": True}),
    # a NaN channel in the appended key: every path leaves that channel out of
    # the block's min/max (the new token itself is not attended: lag 1)
    ("quest-f16 NaN channel in the new key", lambda: _with_nan_key(workloads.clustered(
        [531, 532], 32, 8, 128, [3000, 4097], "f16", n_dirs=16, k_sel=[10, 12],
        n_sink=1, n_recent=2)), True, True, {"lag": 1}),
    ("quest-i8 NaN channel in the new key", lambda: _with_nan_key(workloads.clustered(
        [533], 32, 4, 128, [5001], "i8", n_dirs=16, k_sel=[20], n_sink=1, n_recent=4)),
        True, True, {"lag": 1}),
    # group-wise quantized caches: append, bounds, select and attention as
    # the step's own kernels
    ("quest-q8_0", lambda: workloads.clustered(
        [541, 542], 32, 8, 128, [3000, 4097], "q8_0", n_dirs=16, k_sel=[10, 12], n_sink=1,
        n_recent=2), True, True, {}),
    ("quest-q4_0 G8", lambda: workloads.clustered(
        [543], 32, 4, 128, [5001], "q4_0", n_dirs=16, k_sel=[20], n_sink=1, n_recent=4),
        True, True, {}),
    # the group-wise append folded into the Quest step's bounds pass: a NaN
    # channel, poisoned rows, and a token past the launched tiles (the row's
    # first workgroup then appends it whole)
    ("quest-q8_0 NaN channel in the new key", lambda: _with_nan_key(workloads.clustered(
        [552, 553], 32, 8, 128, [3001, 4100], "q8_0", n_dirs=16, k_sel=[10, 12], n_sink=1,
        n_recent=2)), True, True, {"lag": 1}),
    ("quest-q4_0 poisoned rows", lambda: workloads.clustered(
        [554], 16, 8, 128, [2049], "q4_0", n_dirs=16, k_sel=[9], n_sink=1, n_recent=2),
        True, True, {"poison": True}),
    ("quest-q4_0 token past the launched tiles", lambda: workloads.clustered(
        [555], 32, 4, 128, [64 * 16 + 1], "q4_0", n_dirs=16, k_sel=[5], n_sink=1, n_recent=2),
        True, True, {"lag": 1, "tight": True}),
    ("quest-q8_0 first token of an empty cache", lambda: workloads.clustered(
        [556], 32, 8, 128, [1], "q8_0", n_dirs=4, k_sel=[1], n_sink=1, n_recent=1),
        True, True, {"lag": 1, "tight": True}),
    ("dense-q8_0 append poisoned rows", lambda: workloads.gaussian(
        544, 2, 32, 8, 128, [65, 2000], "q8_0"), False, True, {"poison": True}),
    ("dense-q4_0 append 5 parts G2", lambda: workloads.gaussian(
        545, 2, 16, 8, 128, [1025, 300], "q4_0"), False, True, {"poison": True, "S": 5}),
    ("quest-q5_0", lambda: workloads.clustered(
        [557, 558], 32, 8, 128, [3000, 4097], "q5_0", n_dirs=16, k_sel=[10, 12], n_sink=1,
        n_recent=2), True, True, {}),
    ("quest-q5_0 poisoned rows G8", lambda: workloads.clustered(
        [559], 32, 4, 128, [5001], "q5_0", n_dirs=16, k_sel=[20], n_sink=1, n_recent=4),
        True, True, {"poison": True}),
    ("quest-q5_0 NaN channel in the new key", lambda: _with_nan_key(workloads.clustered(
        [560], 16, 8, 128, [2049], "q5_0", n_dirs=16, k_sel=[9], n_sink=1, n_recent=2)),
        True, True, {"lag": 1}),
    ("quest-q5_0 token past the launched tiles", lambda: workloads.clustered(
        [561], 32, 4, 128, [64 * 16 + 1], "q5_0", n_dirs=16, k_sel=[5], n_sink=1, n_recent=2),
        True, True, {"lag": 1, "tight": True}),
    ("dense-q5_0 append poisoned rows", lambda: workloads.gaussian(
        562, 2, 32, 8, 128, [65, 2000], "q5_0"), False, True, {"poison": True}),
    ("dense-q5_0 first token of an empty cache", lambda: workloads.gaussian(
        563, 1, 32, 8, 128, [1], "q5_0"), False, True, {"lag": 1, "tight": True}),
    # part counts whose merge takes 1, 2, 3 and 4 wavefronts per head
    ("quest-f16 8 parts", lambda: workloads.clustered(
        [546, 547], 32, 8, 128, [3000, 4097], "f16", n_dirs=16, k_sel=[10, 12], n_sink=1,
        n_recent=2), True, True, {"S": 8}),
    ("quest-i8 32 parts G8", lambda: workloads.clustered(
        [548], 32, 4, 128, [9001], "i8", n_dirs=16, k_sel=[60], n_sink=1, n_recent=4),
        True, True, {"S": 32}),
    ("quest-f16 64 parts", lambda: workloads.clustered(
        [549, 550], 32, 8, 128, [20000, 1500], "f16", n_dirs=16, k_sel=[100, 10], n_sink=1,
        n_recent=2), True, True, {"S": 64}),
    ("quest-i8 40 parts", lambda: workloads.clustered(
        [551], 16, 8, 128, [12000], "i8", n_dirs=16, k_sel=[80], n_sink=1, n_recent=2),
        True, True, {"S": 40}),
    ("dense-f16 NaN channel in the new key", lambda: _with_nan_key(workloads.gaussian(
        534, 2, 32, 8, 128, [700, 1025], "f16")), False, True, {"lag": 1}),
]


@pytest.mark.parametrize("name,make,quest,append,extra", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_decode_step_equals_composed_calls(gpu_lib, name, make, quest, append, extra):
    _print(name)
    w = make()
    out, sel = _run_case(w, quest, append, **extra)
    if not extra.get("lag"):
        _oracle_check(w, out, sel)


def test_decode_step_replays_in_a_hip_graph(gpu_lib):
    """The three launches of a Quest step captured once and replayed several
    times (with eager work between the replays) give the eager result each
    time; the step allocates nothing and leaves no memset in the graph."""
    _print("step graph")
    w = workloads.clustered([512], 32, 8, 128, [8192], "f16", n_dirs=16, k_sel=[32],
                            n_sink=1, n_recent=2)
    base = _prefilled(w)
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    ks = torch.tensor(w.k_sel, dtype=torch.int32, device=DEV)
    pos, kn, vn = _new_token(w)
    max_sel = 35
    S = skv.default_split(1, 8, max_sel)
    out, ws, sc, sel, cnt = _buffers(w, base, True, max_sel, S)

    def step():
        skv.decode_step(base, q, seq_len, 8192, w.softmax_scale, S, ws, out, pos0=pos,
                        k_new=kn, v_new=vn, k_sel=ks, score=sc, sel_idx=sel, sel_cnt=cnt)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    ref_sel = sel.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        out.fill_(float("nan"))
        sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(sel, ref_sel)


def test_decode_step_all_scores_equal(gpu_lib):
    """q = 0: every block bound is 0, so more than 64 candidates tie on the
    cut key and the folded selection takes its index-order branch; the lowest
    candidate indices win (the tie rule), as in skv_select_topk."""
    _print("step q=0")
    w = workloads.clustered([517], 32, 8, 128, [20000], "f16", n_dirs=16, k_sel=[70],
                            n_sink=1, n_recent=2)
    w.q[:] = 0
    out, (sel, cnt) = _run_case(w, True, True)
    nb = -(-20000 // 64)
    want = list(range(0, 1 + 70)) + [nb - 2, nb - 1]
    for g in range(w.Hkv):
        assert cnt[0, g] == len(want)
        assert list(sel[0, g, :cnt[0, g]]) == want
    _oracle_check(w, out, (sel, cnt))


def test_int8_decode_step_replays_in_a_hip_graph(gpu_lib):
    """The int8 Quest step (append folded into bounds, selection folded into
    the attention prologue with 4 keys per thread) captured once and replayed
    with eager work between the replays gives the eager result each time."""
    _print("int8 step graph")
    w = workloads.clustered([518], 32, 4, 128, [40000], "i8", n_dirs=32, k_sel=[80],
                            n_sink=1, n_recent=4)
    base = _prefilled(w)
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    ks = torch.tensor(w.k_sel, dtype=torch.int32, device=DEV)
    pos, kn, vn = _new_token(w)
    max_sel = 85
    S = skv.default_split(1, 4, max_sel, kv_dtype="i8", sparse=True)
    out, ws, sc, sel, cnt = _buffers(w, base, True, max_sel, S)

    def step():
        skv.decode_step(base, q, seq_len, 40000, w.softmax_scale, S, ws, out, pos0=pos,
                        k_new=kn, v_new=vn, k_sel=ks, n_sink=1, n_recent=4, score=sc,
                        sel_idx=sel, sel_cnt=cnt)

    step()
    torch.cuda.synchronize()
    ref, ref_sel = out.clone(), sel.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        out.fill_(float("nan"))
        sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(sel, ref_sel)
    _oracle_check(w, out.cpu().numpy(), (sel.cpu().numpy(), cnt.cpu().numpy()))


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_dense_decode_step_replays_in_a_hip_graph(gpu_lib, kv):
    """The dense step (append folded into the attention kernel, then combine)
    captured once and replayed; before each replay the append positions are
    poisoned again by eager work, so every replay must take the new token
    from k_new / v_new and write it back, as the eager step did."""
    _print("dense step graph", kv)
    w = workloads.gaussian(524, 2, 32, 8, 128, [5000, 4097], kv)
    base = _prefilled(w)
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    pos, kn, vn = _new_token(w)
    S = skv.default_split(2, 8, -(-5000 // 64), kv_dtype=kv)
    out, ws, _, _, _ = _buffers(w, base, False, 0, S)

    def step():
        skv.decode_step(base, q, seq_len, 5000, w.softmax_scale, S, ws, out, pos0=pos,
                        k_new=kn, v_new=vn)

    _poison_rows(base, pos)
    step()
    torch.cuda.synchronize()
    ref = out.clone()
    ref_cache = [t.clone() for t in _cache_tensors(base)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        out.fill_(float("nan"))
        _poison_rows(base, pos)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        for a, b in zip(ref_cache, _cache_tensors(base)):
            assert torch.equal(a, b)
    _oracle_check(w, out.cpu().numpy(), None)


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_dense_decode_step_without_side_cache(gpu_lib, kv):
    """A cache built without Quest bounds: the dense step's folded append
    writes the rows (and int8 scales) only, bit-identical to kv_append +
    decode_attn + combine."""
    _print("dense step, no side cache", kv)
    w = workloads.gaussian(525, 2, 16, 4, 128, [3001, 64], kv)
    pos, kn, vn = _new_token(w)
    dt = np.float16 if kv == "f16" else np.float32
    rows = max(w.lens) - 1
    k = np.zeros((w.B, rows, w.Hkv, w.D), dt)
    v = np.zeros((w.B, rows, w.Hkv, w.D), dt)
    for b, L in enumerate(w.lens):
        k[b, :L - 1] = np.transpose(w.k[b][:, :L - 1], (1, 0, 2))
        v[b, :L - 1] = np.transpose(w.v[b][:, :L - 1], (1, 0, 2))
    base = skv.Cache(w.B, w.Hkv, max(w.lens), w.D, kv, w.block, bounds=False, device=DEV)
    skv.kv_append(base, torch.zeros(w.B, dtype=torch.int32, device=DEV),
                  torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV))
    _poison_rows(base, pos)
    ca, cb = base.clone(), base.clone()
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    S = skv.default_split(w.B, w.Hkv, -(-max(w.lens) // w.block), kv_dtype=kv)
    out_a, ws_a, _, _, _ = _buffers(w, ca, False, 0, S)
    out_b, ws_b, _, _, _ = _buffers(w, cb, False, 0, S)
    skv.kv_append(ca, pos, kn, vn)
    skv.decode_attn(ca, q, seq_len, max(w.lens), w.softmax_scale, S, ws_a)
    skv.combine(ws_a, w.B, w.H, w.D, S, out_a)
    skv.decode_step(cb, q, seq_len, max(w.lens), w.softmax_scale, S, ws_b, out_b, pos0=pos,
                    k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    assert cb.kmin is None
    assert torch.equal(out_a, out_b)
    for ta, tb in zip(_cache_tensors(ca), _cache_tensors(cb)):
        assert torch.equal(ta, tb)
    _oracle_check(w, out_b.cpu().numpy(), None)


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_dense_decode_step_out_of_range_positions(gpu_lib, kv):
    """Append positions the append kernel skips (negative, or at or past the
    cache capacity) are skipped by the dense step's folded append too: the
    cache is untouched for those sequences and everything stays
    bit-identical to kv_append + decode_attn + combine."""
    _print("dense step, out-of-range positions", kv)
    w = workloads.gaussian(526, 3, 32, 8, 128, [700, 1000, 1500], kv)
    base = _prefilled(w, max_seq=1500)
    _, kn, vn = _new_token(w)
    pos = torch.tensor([-1, 1500, 1499], dtype=torch.int32, device=DEV)
    ca, cb = base.clone(), base.clone()
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    S = skv.default_split(w.B, w.Hkv, -(-1500 // w.block), kv_dtype=kv)
    out_a, ws_a, _, _, _ = _buffers(w, ca, False, 0, S)
    out_b, ws_b, _, _, _ = _buffers(w, cb, False, 0, S)
    skv.kv_append(ca, pos, kn, vn)
    skv.decode_attn(ca, q, seq_len, 1500, w.softmax_scale, S, ws_a)
    skv.combine(ws_a, w.B, w.H, w.D, S, out_a)
    skv.decode_step(cb, q, seq_len, 1500, w.softmax_scale, S, ws_b, out_b, pos0=pos,
                    k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    for ta, tb, t0 in zip(_cache_tensors(ca), _cache_tensors(cb), _cache_tensors(base)):
        assert torch.equal(ta, tb)
        assert torch.equal(tb[:2], t0[:2])      # sequences 0 and 1 were not written


@pytest.mark.parametrize("k_sel", [100, 300])
def test_decode_step_tie_classes(gpu_lib, k_sel):
    """Blocks that repeat 8 contents have 8 distinct bounds per KV head, each
    shared by about 64 candidates, so the cut falls inside a tie class: the
    folded selection must give the oracle's rule on the step's own scores
    (the K best, exact ties to the lower index)."""
    _print("step tie classes", k_sel)
    w = workloads.clustered([519], 32, 8, 128, [512 * 64], "f16", n_dirs=8, k_sel=[k_sel],
                            n_sink=1, n_recent=2)
    for j in range(8, 512):
        src = j % 8
        w.k[0][:, j * 64:(j + 1) * 64] = w.k[0][:, src * 64:(src + 1) * 64]
    base = _prefilled(w)
    cb = base.clone()
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    ks = torch.tensor(w.k_sel, dtype=torch.int32, device=DEV)
    max_sel = k_sel + 3
    S = skv.default_split(1, 8, max_sel, sparse=True)
    pos, kn, vn = _new_token(w)
    out, ws, sc, sel, cnt = _buffers(w, cb, True, max_sel, S)
    skv.decode_step(cb, q, seq_len, 512 * 64, w.softmax_scale, S, ws, out, pos0=pos, k_new=kn,
                    v_new=vn, k_sel=ks, n_sink=1, n_recent=2, score=sc, sel_idx=sel, sel_cnt=cnt)
    torch.cuda.synchronize()
    score, s_h, c_h = sc.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy()
    for g in range(8):
        assert len(np.unique(score[0, g, 1:510])) <= 8
        own = oracle.select_blocks(score[0, g], 512, k_sel, 1, 2)["sel"]
        assert np.array_equal(s_h[0, g, :c_h[0, g]], own), g
    _oracle_check(w, out.cpu().numpy(), (s_h, c_h))


@pytest.mark.parametrize("kv_dtype,L,S", [("f16", 32768, 32), ("i8", 20000, 24), ("f16", 3000, 1),
                                          ("q8_0", 9000, 16), ("q4_0", 32768, 32),
                                          ("q5_0", 32768, 32)])
def test_decode_attn_select_equals_select_then_decode(gpu_lib, kv_dtype, L, S):
    """skv_decode_attn_select (selection folded into the attention prologue;
    with S = 1 a part spans more than 64 entries and the selection runs as
    its own kernel) writes the same list and partial states as select_topk +
    decode_attn, bit for bit."""
    _print("decode_attn_select", kv_dtype, L, S)
    w = workloads.clustered([540], 32, 8, 128, [L], kv_dtype, n_dirs=32,
                            k_sel=[(-(-L // 64)) // 4], n_sink=1, n_recent=2)
    cache = _prefilled(w, whole=True)
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=DEV)
    ks = torch.tensor(w.k_sel, dtype=torch.int32, device=DEV)
    max_sel = w.k_sel[0] + 3
    _, ws_a, score, sel_a, cnt_a = _buffers(w, cache, True, max_sel, S)
    _, ws_b, _, sel_b, cnt_b = _buffers(w, cache, True, max_sel, S)
    ws_a.zero_()
    ws_b.fill_(255)
    skv.block_bounds(cache, q, seq_len, L, score)
    skv.select_topk(score, seq_len, w.block, ks, w.n_sink, w.n_recent, sel_a, cnt_a)
    skv.decode_attn(cache, q, seq_len, L, w.softmax_scale, S, ws_a, sel_a, cnt_a)
    skv.decode_attn_select(cache, q, seq_len, L, w.softmax_scale, S, ws_b, score, ks, w.n_sink,
                           w.n_recent, sel_b, cnt_b)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b) and torch.equal(cnt_a, cnt_b)
    assert torch.equal(ws_a, ws_b)
