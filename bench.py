"""Decode-step attention benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: append the new
token (kv_append), Quest upper bounds (block_bounds), top-K selection
(select_topk), attention over the selected blocks (decode_attn) and the
split-K merge (combine), issued as one skv_decode_step (three launches:
append folded into the bounds pass, selection into the attention
prologue); the same five calls issued one by one are timed too.  The headline workload is the 32K-context GQA
decode (B=1, H=32, Hkv=8, D=128, f16 KV, block 64, K_SEL=128 + sink + 2
recent); the same cache is also timed with the dense step (two launches:
the append folded into decode_attn, then combine) for the sparse/dense
ratio.  The other named
workloads (512-token dense f16, 8K int8, the 16-sequence 16K-64K batch,
262K int8 Quest) are timed the same way and reported under "workloads".

Timing protocol:
* Inputs are resident in HBM before the timed region.
* Cold cache: step i reads copy i % R of the cache, R chosen so that R
  consecutive steps touch more than twice the 256 MB last-level cache.
* W warmup steps, then exactly K steps captured in one HIP graph
  (torch.cuda.CUDAGraph over the library's launches), replayed once
  untimed, then 5 times, each replay bracketed by HIP events on the replay
  stream; the median replay / K is the time per step.  The stream-launch
  time of K eager steps is reported too.
* Warm cache (secondary, headline steps only): the same K-step graph on one
  copy of the cache, so a step's bytes may stay in the last-level cache.
* The dominant kernel is timed alone the same way (K launches in one
  graph, median of 5 event-timed replays): for the Quest step its own
  attention kernel, decode_attn_select (selection in the prologue), and
  decode_attn over the given list beside it; achieved GB/s = algorithmic
  bytes per launch / average launch time.
* The CPU baseline: the float64 oracle's step of every timed workload on
  a bounded sample of its (sequence, KV head) units, on one core and on a
  pool of up to 16 cores, scaled to one step, run before the GPU is used.

Prints ONE JSON line (one GPU).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step + achieved KV GB/s (% HBM peak) at 32K, H=32/Hkv=8, D=128"
HBM_PEAK_GBPS = 8000.0
LLC_BYTES = 256 * 2 ** 20


# ------------------------------------------------------------- accounting
def kv_bytes_per_token(kv_dtype: str, D: int) -> int:
    """Algorithmic bytes of one attended (token, KV head): K and V rows, plus
    the two float32 scales for int8, or the f16 scale of every 32-channel
    group of both rows for q8_0 (int8 codes), q4_0 (4-bit codes) and q5_0
    (5-bit codes: a nibble plane plus a plane of fifth bits)."""
    if kv_dtype == "f16":
        return 4 * D
    if kv_dtype == "i8":
        return 2 * D + 8
    codes = {"q8_0": D, "q4_0": D // 2, "q5_0": D // 2 + D // 8}[kv_dtype]
    return 2 * (codes + 2 * (D // 32))


def side_cache_bytes_per_block(D: int) -> int:
    """kmin and kmax rows of one (block, KV head), f16."""
    return 2 * 2 * D


def scan4_index_bytes(lens, Hkv: int, D: int, block: int, reads_per_token: int = 1) -> int:
    """Bytes one scan of the 4-bit index reads: D / 2 bytes of codes per
    (token, KV head) (read reads_per_token times: 1 for the GQA-shared scan, G
    when every query head scans on its own) and lo, step, err (3 x D float32)
    per (block, KV head)."""
    toks = sum(lens) * Hkv
    nblk = sum(-(-L // block) for L in lens) * Hkv
    return toks * (D // 2) * reads_per_token + nblk * 3 * D * 4

def step_bytes(lens, Hkv, H, D, kv_dtype, block, attended_blocks=None):
    """Algorithmic bytes of one decode step.

    attended_blocks: None for dense, else {(b, g): list of selected blocks}.
    Returns dict(kv=..., bounds=..., q_out=..., total=...)."""
    per_tok = kv_bytes_per_token(kv_dtype, D)
    kv = 0
    bounds = 0
    for b, L in enumerate(lens):
        nb = -(-L // block)
        if attended_blocks is None:
            kv += L * Hkv * per_tok
        else:
            bounds += nb * Hkv * side_cache_bytes_per_block(D)
            for g in range(Hkv):
                toks = sum(min(block, L - j * block) for j in attended_blocks[(b, g)])
                kv += toks * per_tok
    q_out = 2 * len(lens) * H * D * 4
    return {"kv": kv, "bounds": bounds, "q_out": q_out, "total": kv + bounds + q_out}


# ------------------------------------------------------------- HBM traffic
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_quest32k.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_kv_cache_append_amd", "csrc", f)
                  for f in ("decode_kernels.h", "decode_mfma.hip", "decode_core.h",
                            "device_common.h", "launch.h", "select_core.h", "fused_walk.h")]


def kernel_source_digest() -> str:
    """sha256 over the code of the sources the decode kernel is compiled from
    (comments and whitespace removed, so an edit to a comment keeps it)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        text = open(f, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", "", text).encode())
    return h.hexdigest()


def recorded_traffic(kernel: str):
    """HBM bytes per launch of the timed kernel from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    factors recorded there), or None when the summary is missing, is for
    another kernel, or the kernel source changed since it was taken."""
    try:
        fields = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        if fields.get("kernel_source_sha256") != kernel_source_digest() or fields.get("kernel") != kernel:
            return None
        return int(float(fields["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


# ------------------------------------------------------------- cpu baseline
CPU_POOL_MAX = 16          # the GPU machine's CPU share for one GPU


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _one_thread():
    """Limit the BLAS pools of this process to one thread."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl is in the image
        return None


class OracleStep:
    """The oracle's decode step of one workload, split into its independent
    (sequence, KV head) units: dense attention of the unit's G query heads,
    or the Quest pipeline of the unit (the appended token's block bounds,
    the upper bounds of every block for the G heads, their max, the top-K
    selection, attention over the selected blocks).  The cache state (the
    side cache before the step, the int8 codes and scales) is prepared
    outside the timed region: it is the cache the step finds in memory."""

    def __init__(self, w, quest: bool):
        import oracle
        self.w, self.quest, self.oracle = w, quest, oracle
        self.units = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
        self.kmin, self.kmax, self.codes = {}, {}, {}
        for b in range(w.B):
            L = w.lens[b]
            if quest:
                # the side cache as it stands before the step (tokens < L - 1)
                mn, mx = oracle.block_bounds(w.k[b][:, :L - 1], L - 1, w.block) if L > 1 else (
                    None, None)
                self.kmin[b], self.kmax[b] = mn, mx
            if w.kv_dtype == "i8":
                kc, ks = oracle.quantize_rows(w.k[b])
                vc, vs = oracle.quantize_rows(w.v[b])
                self.codes[b] = (kc, ks, vc, vs)
            elif w.kv_dtype in ("q8_0", "q4_0", "q5_0"):
                qmax = {"q8_0": oracle.QMAX_Q8, "q4_0": oracle.QMAX_Q4,
                        "q5_0": oracle.QMAX_Q5}[w.kv_dtype]
                kc, ks = oracle.quantize_groups(w.k[b], qmax)
                vc, vs = oracle.quantize_groups(w.v[b], qmax)
                self.codes[b] = (kc, ks, vc, vs)

    def unit(self, bg):
        o, w = self.oracle, self.w
        b, g = bg
        L = w.lens[b]
        hs = slice(g * w.G, (g + 1) * w.G)
        q = w.q[b][hs]
        toks = None
        if self.quest:
            # append: the new token's block, min/max-merged (from scratch over
            # the block is the same bytes, min and max being exact)
            j = (L - 1) // w.block
            bmn, bmx = o.block_bounds(w.k[b][g:g + 1, j * w.block:L], L - j * w.block, w.block)
            if self.kmin[b] is None:
                mn, mx = bmn, bmx
            else:
                # the token's block replaces the old one, or starts a new one
                mn = np.concatenate([self.kmin[b][g:g + 1, :j], bmn], axis=1)
                mx = np.concatenate([self.kmax[b][g:g + 1, :j], bmx], axis=1)
            sc = o.group_scores(o.upper_bounds(q, mn, mx), 1)[0]
            r = o.select_blocks(sc, w.n_blocks(b), w.k_sel[b], w.n_sink, w.n_recent)
            toks = o.selected_tokens(r["sel"], L, w.block)
        if w.kv_dtype == "f16":
            return o.attend_f16(q, w.k[b][g:g + 1], w.v[b][g:g + 1], w.softmax_scale, tokens=toks)
        kc, ks, vc, vs = self.codes[b]
        sl = slice(g, g + 1)
        if w.kv_dtype == "i8":
            return o.attend_i8(q, kc[sl], ks[sl], vc[sl], vs[sl], w.softmax_scale, tokens=toks)
        return o.attend_grouped(q, kc[sl], ks[sl], vc[sl], vs[sl], w.softmax_scale, tokens=toks)


_POOL_STEP = None


_POOL_LIMIT = None


def _pool_init():
    global _POOL_LIMIT
    _POOL_LIMIT = _one_thread()


def _pool_noop(i):
    return i


def _pool_unit(i):
    t0 = time.perf_counter()
    _POOL_STEP.unit(_POOL_STEP.units[i])
    return time.perf_counter() - t0


def cpu_baseline(w, quest: bool, budget_s: float = 4.0):
    """The oracle's step of workload w on the host cores, on a bounded sample
    of its (sequence, KV head) units, scaled to one whole step:
    * one core: units run one after another on one thread, until budget_s
      has passed (at least one unit); us/step = mean unit time x units;
    * all cores: a pool of min(cores, units) forked workers (one thread
      each) runs one unit per worker at once (best of up to 3 rounds);
      us/step = wall time x ceil(units / workers).
    Runs before the GPU is touched (the pool forks this process)."""
    import multiprocessing as mp
    global _POOL_STEP
    st = OracleStep(w, quest)
    n = len(st.units)
    lim = _one_thread()
    times = []
    t_all = time.perf_counter()
    for i in range(n):
        t0 = time.perf_counter()
        st.unit(st.units[i])
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > budget_s:
            break
    if lim is not None and hasattr(lim, "unregister"):
        lim.unregister()
    one = sum(times) / len(times) * n
    cores = max(1, min(len(os.sched_getaffinity(0)), CPU_POOL_MAX))
    workers = min(cores, n)
    _POOL_STEP = st
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_pool_init) as pool:
        pool.map(_pool_noop, range(4 * workers), chunksize=1)     # workers up
        wall = float("inf")
        t_end = time.perf_counter() + budget_s
        for rep in range(3):                                      # best of up to 3
            t0 = time.perf_counter()
            pool.map(_pool_unit, range(workers), chunksize=1)
            wall = min(wall, time.perf_counter() - t0)
            if time.perf_counter() > t_end:
                break
    _POOL_STEP = None
    allc = wall * math.ceil(n / workers)
    what = ("Quest step (append's block bounds, upper bounds, group max, top-K, attention "
            "over the selected blocks)" if quest else "dense attention")
    return {"workload": w.name, "step": "quest" if quest else "dense", "units": n,
            "one_core": {"value": round(one * 1e6, 1), "unit": "us/step", "cores": 1,
                         "sample": f"{len(times)} of {n} (sequence, KV head) units, scaled"},
            "all_cores": {"value": round(allc * 1e6, 1), "unit": "us/step", "cores": workers,
                          "sample": f"{workers} units at once on {workers} workers, scaled "
                                    f"x{math.ceil(n / workers)}"},
            "what": f"float64 NumPy oracle, {what}"}


# ------------------------------------------------------------- GPU bench
class Timer:
    """Graph- and stream-timed replays of a step function f(i) over a ring of
    R cache copies (step i reads copy i % R)."""

    REPS = 5

    def __init__(self, torch, R, steps, warmup, use_graph):
        self.torch, self.R, self.K, self.W, self.use_graph = torch, R, steps, warmup, use_graph

    def stream(self, fn):
        """Host wall time per step of K eager steps (launch-bound when a step's
        GPU time is below the host's launch time)."""
        torch = self.torch
        for i in range(self.W):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(self.K):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / self.K

    def _replays(self, g, st):
        """Median over REPS timed replays of graph g on stream st, HIP events
        recorded on st around each replay; seconds per replay."""
        torch = self.torch
        ts = []
        with torch.cuda.stream(st):
            g.replay()                                   # untimed
            for _ in range(self.REPS):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                g.replay()
                e1.record(st)
                st.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    def graph(self, fn):
        """Device time per step of exactly K steps captured in one HIP graph
        (step i reads copy i % R): median of REPS replays, each bracketed by
        HIP events on the replay stream.  Returns (None, K) when graphs are
        off."""
        if not self.use_graph:
            return None, self.K
        torch, R, K = self.torch, self.R, self.K
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            for i in range(max(self.W, R)):
                fn(i)
        st.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for i in range(K):
                fn(i)
        dt = self._replays(g, st) / K
        del g
        return dt, K

    def kernel(self, fn):
        """Average duration of one launch of fn (K launches in one graph,
        median of REPS replays, HIP events on the launch stream)."""
        torch, R, K = self.torch, self.R, self.K
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            for i in range(R):
                fn(i)
        st.synchronize()
        if not self.use_graph:
            ts = []
            for _ in range(self.REPS):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(st):
                    e0.record(st)
                    for i in range(K):
                        fn(i)
                    e1.record(st)
                st.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / K)
            return float(np.median(ts))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for i in range(K):
                fn(i)
        dt = self._replays(g, st) * 1e6 / K
        del g
        return dt


def padded_prefill(w, rows):
    """[B][rows][Hkv][D] rows 0..L_b-2 of every sequence, padded past L_b - 2
    with copies of that row (the pad never changes a block's min/max and is
    never attended: positions >= L_b - 1 are rewritten or unread)."""
    dt = np.float16 if w.kv_dtype == "f16" else np.float32
    k = np.empty((w.B, rows, w.Hkv, w.D), dt)
    v = np.empty((w.B, rows, w.Hkv, w.D), dt)
    for b, L in enumerate(w.lens):
        n = L - 1
        k[b, :n] = np.transpose(w.k[b][:, :n], (1, 0, 2))
        v[b, :n] = np.transpose(w.v[b][:, :n], (1, 0, 2))
        k[b, n:] = k[b, n - 1]
        v[b, n:] = v[b, n - 1]
    return k, v


def _warm_us(torch, args, step):
    """The same step on one cache copy every time (warm: the step's bytes may
    stay in the last-level cache between steps), µs per step; a secondary
    figure beside the cold-ring one."""
    T1 = Timer(torch, 1, args.steps, args.warmup, not args.no_graph)
    gr, _ = T1.graph(lambda i: step(0))
    return (gr if gr is not None else T1.stream(lambda i: step(0))) * 1e6


def measure(w, args, quest: bool, dense: bool, detail: bool = False):
    """Time the dense and/or Quest decode step of workload w on a cold ring of
    cache copies.  Returns a dict of per-step figures (and, with detail, the
    device state used for the roofline kernel timing)."""
    import torch
    import sparse_kv_cache_append_amd as skv
    dev = torch.device("cuda:0")
    B, H, Hkv, D, blk = w.B, w.H, w.Hkv, w.D, w.block
    Lmax = max(w.lens)
    src_dt = torch.float16 if w.kv_dtype == "f16" else torch.float32
    base = skv.Cache(B, Hkv, Lmax, D, w.kv_dtype, blk, bounds=True, device=dev)
    k0, v0 = padded_prefill(w, Lmax - 1)
    skv.kv_append(base, torch.zeros(B, dtype=torch.int32, device=dev),
                  torch.from_numpy(k0).to(dev), torch.from_numpy(v0).to(dev))
    del k0, v0
    new_k = torch.from_numpy(np.stack([w.k[b][:, L - 1] for b, L in enumerate(w.lens)])[:, None]
                             .copy()).to(dev).to(src_dt).contiguous()
    new_v = torch.from_numpy(np.stack([w.v[b][:, L - 1] for b, L in enumerate(w.lens)])[:, None]
                             .copy()).to(dev).to(src_dt).contiguous()
    pos_last = torch.tensor([L - 1 for L in w.lens], dtype=torch.int32, device=dev)
    seq_len = torch.tensor(w.lens, dtype=torch.int32, device=dev)
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(dev)
    nb_max = -(-Lmax // blk)
    per_tok = kv_bytes_per_token(w.kv_dtype, D)

    k_sel = list(w.k_sel) if (quest and w.k_sel) else None
    max_sel = (max(k_sel) + w.n_sink + w.n_recent) if k_sel else 0
    # bytes one step touches; the ring is sized for the smaller step so that
    # R consecutive steps of either kind exceed twice the last-level cache
    touches = []
    if dense:
        touches.append(sum(w.lens) * Hkv * per_tok)
    if k_sel:
        touches.append(B * Hkv * max_sel * blk * per_tok + B * Hkv * nb_max * 512)
    per_copy = sum(t.numel() * t.element_size() for t in
                   (base.k, base.v, base.k_scale, base.v_scale, base.kmin, base.kmax)
                   if t is not None)
    R = args.ring or min(256, max(2, math.ceil(2 * LLC_BYTES / max(min(touches), 1)) + 1))
    R = max(1, min(R, int(args.ring_budget_gb * 2 ** 30 // max(per_copy, 1))))
    caches = [base] + [base.clone() for _ in range(R - 1)]
    torch.cuda.synchronize()
    T = Timer(torch, R, args.steps, args.warmup, not args.no_graph)
    res = {"workload": w.name, "cache_copies": R}

    if dense:
        S_d = args.n_split or skv.default_split(B, Hkv, nb_max, kv_dtype=w.kv_dtype)
        ws_d = torch.empty(skv.workspace_bytes(B, H, D, S_d), dtype=torch.uint8, device=dev)
        out_d = torch.empty((B, H, D), dtype=torch.float32, device=dev)

        def dense_step(i):
            skv.decode_step(caches[i % R], q, seq_len, Lmax, w.softmax_scale, S_d, ws_d, out_d,
                            pos0=pos_last, k_new=new_k, v_new=new_v)

        st = T.stream(dense_step)
        gr, n = T.graph(dense_step)
        us = (gr if gr is not None else st) * 1e6
        warm = _warm_us(torch, args, dense_step) if detail else None
        dec_us = T.kernel(lambda i: skv.decode_attn(caches[i % R], q, seq_len, Lmax,
                                                    w.softmax_scale, S_d, ws_d))
        db = step_bytes(w.lens, Hkv, H, D, w.kv_dtype, blk, None)
        dec_bytes = db["kv"] + B * H * D * 4
        res["dense"] = {"us_per_step": round(us, 3), "stream_us_per_step": round(st * 1e6, 3),
                        "steps": n, "n_split": S_d, "bytes_per_step": db["total"],
                        "GBps": round(db["total"] / us / 1e3, 1),
                        "pct_hbm_peak": round(100 * db["total"] / us / 1e3 / HBM_PEAK_GBPS, 2),
                        "decode_attn_us": round(dec_us, 3),
                        "decode_attn_GBps": round(dec_bytes / dec_us / 1e3, 1),
                        "decode_attn_pct_peak": round(100 * dec_bytes / dec_us / 1e3
                                                      / HBM_PEAK_GBPS, 2)}
        if warm is not None:
            res["dense"]["warm_us_per_step"] = round(warm, 3)

    if k_sel:
        ks = torch.tensor(k_sel, dtype=torch.int32, device=dev)
        score = torch.empty((B, Hkv, base.max_blocks), dtype=torch.float32, device=dev)
        sel = torch.empty((B, Hkv, max_sel), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        S_q = args.n_split or skv.default_split(B, Hkv, max_sel, kv_dtype=w.kv_dtype, sparse=True)
        ws_q = torch.empty(skv.workspace_bytes(B, H, D, S_q), dtype=torch.uint8, device=dev)
        out_q = torch.empty((B, H, D), dtype=torch.float32, device=dev)

        def quest_step(i):
            skv.decode_step(caches[i % R], q, seq_len, Lmax, w.softmax_scale, S_q, ws_q, out_q,
                            pos0=pos_last, k_new=new_k, v_new=new_v, k_sel=ks,
                            n_sink=w.n_sink, n_recent=w.n_recent, score=score, sel_idx=sel,
                            sel_cnt=cnt)

        def quest_calls(i):
            c = caches[i % R]
            skv.kv_append(c, pos_last, new_k, new_v)
            skv.block_bounds(c, q, seq_len, Lmax, score)
            skv.select_topk(score, seq_len, blk, ks, w.n_sink, w.n_recent, sel, cnt)
            skv.decode_attn(c, q, seq_len, Lmax, w.softmax_scale, S_q, ws_q, sel, cnt)
            skv.combine(ws_q, B, H, D, S_q, out_q)

        st = T.stream(quest_step)
        gr, n = T.graph(quest_step)
        us = (gr if gr is not None else st) * 1e6
        warm = _warm_us(torch, args, quest_step) if detail else None
        gr_c, _ = T.graph(quest_calls)
        calls_us = (gr_c if gr_c is not None else T.stream(quest_calls)) * 1e6
        quest_step(0)
        torch.cuda.synchronize()
        sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
        attended = {(b, g): sel_h[b, g, :cnt_h[b, g]].tolist() for b in range(B) for g in range(Hkv)}
        qb = step_bytes(w.lens, Hkv, H, D, w.kv_dtype, blk, attended)
        dec_bytes = qb["kv"] + B * H * D * 4
        dec_us = T.kernel(lambda i: skv.decode_attn(caches[i % R], q, seq_len, Lmax,
                                                    w.softmax_scale, S_q, ws_q, sel, cnt))
        # the step's own attention kernel: the selection folded into its
        # prologue (the scores are the step's, identical for every copy)
        sel_us = T.kernel(lambda i: skv.decode_attn_select(
            caches[i % R], q, seq_len, Lmax, w.softmax_scale, S_q, ws_q, score, ks, w.n_sink,
            w.n_recent, sel, cnt))
        n_att = sum(len(x) for x in attended.values())
        n_all = sum(-(-L // blk) for L in w.lens) * Hkv
        res["quest"] = {"us_per_step": round(us, 3), "stream_us_per_step": round(st * 1e6, 3),
                        "five_calls_us_per_step": round(calls_us, 3),
                        "steps": n, "n_split": S_q, "bytes_per_step": qb["total"],
                        "kv_bytes": qb["kv"], "bounds_bytes": qb["bounds"],
                        "blocks_attended_frac": round(n_att / n_all, 4),
                        "GBps": round(qb["total"] / us / 1e3, 1),
                        "pct_hbm_peak": round(100 * qb["total"] / us / 1e3 / HBM_PEAK_GBPS, 2),
                        "decode_attn_us": round(dec_us, 3),
                        "decode_attn_GBps": round(dec_bytes / dec_us / 1e3, 1),
                        "decode_attn_pct_peak": round(100 * dec_bytes / dec_us / 1e3
                                                      / HBM_PEAK_GBPS, 2),
                        "decode_attn_select_us": round(sel_us, 3),
                        "decode_attn_select_pct_peak": round(100 * dec_bytes / sel_us / 1e3
                                                             / HBM_PEAK_GBPS, 2)}
        if warm is not None:
            res["quest"]["warm_us_per_step"] = round(warm, 3)
        if detail:
            res["_roofline"] = (dec_bytes, sel_us, dec_us)
        if not args.no_per_head:
            res["quest_per_head"] = measure_per_head(T, skv, torch, w, caches, R, q, seq_len, Lmax,
                                                     new_k, new_v, pos_last, ks, res["quest"])
        if not args.no_scan4:
            res["scan4"] = measure_scan4(T, skv, torch, w, caches, R, q, seq_len, Lmax,
                                         args.scan4_delta)
        n_chunk = min(args.chunk_tokens, 16 // w.G)
        if n_chunk > 1:
            res["chunk"] = measure_chunk(T, skv, torch, w, caches, R, seq_len, Lmax, n_chunk,
                                         res.get("dense"), res["quest"])
        if args.sparse_v_tau > 0:
            res["quest_sparse_v"] = measure_sparse_v(
                T, skv, torch, w, caches, R, q, seq_len, Lmax, new_k, new_v, pos_last, ks, score,
                sel, cnt, attended, args.sparse_v_tau, calls_us)
        if "dense" in res:
            res["quest_over_dense"] = round(res["quest"]["us_per_step"]
                                            / res["dense"]["us_per_step"], 4)
    del caches
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def measure_chunk(T, skv, torch, w, caches, R, seq_len, Lmax, n_tok, dense_res, quest_res):
    """A chunk of n_tok query tokens per sequence (the last n_tok positions;
    queries from workloads.chunk_queries): the chunk's append (kv_append of
    n_tok rows), then dense (decode_attn_multi + combine) or Quest
    (block_bounds_multi, select_topk_multi, select_union_tokens,
    decode_attn_multi over each token's own blocks, combine).  Compared with
    n_tok single-token steps of the same workload.  Bytes: the side cache
    (Quest), the KV rows of every block some token attends (read once for the
    chunk), n_tok queries and outputs."""
    import workloads
    B, H, Hkv, D, blk = w.B, w.H, w.Hkv, w.D, w.block
    dev = seq_len.device
    qc = torch.from_numpy(workloads.chunk_queries(w, n_tok, 7000 + n_tok)).to(dev)
    rng = np.random.default_rng(7100)
    dt = torch.float16 if w.kv_dtype == "f16" else torch.float32
    nk = torch.from_numpy(rng.standard_normal((B, n_tok, Hkv, D), dtype=np.float32)).to(dev, dt)
    nv = torch.from_numpy(rng.standard_normal((B, n_tok, Hkv, D), dtype=np.float32)).to(dev, dt)
    pos = (seq_len - n_tok).clamp(min=0).to(torch.int32)
    max_blocks = caches[0].max_blocks
    max_sel = max(w.k_sel) + w.n_sink + w.n_recent
    max_union = min(max_blocks, n_tok * max_sel)
    sc = torch.empty((B, Hkv, n_tok, max_blocks), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Hkv, n_tok, max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hkv, n_tok), dtype=torch.int32, device=dev)
    uni = torch.empty((B, Hkv, max_union), dtype=torch.int32, device=dev)
    ucnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    um = torch.empty((B, Hkv, max_union), dtype=torch.int32, device=dev)
    ks = torch.tensor(w.k_sel, dtype=torch.int32, device=dev)
    nb = -(-Lmax // blk)
    S_d = skv.default_split(B, Hkv, nb, kv_dtype=w.kv_dtype)
    S_q = skv.default_split(B, Hkv, max_union, kv_dtype=w.kv_dtype, sparse=True)
    ws_d = torch.empty(skv.workspace_bytes(B, n_tok * H, D, S_d), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(skv.workspace_bytes(B, n_tok * H, D, S_q), dtype=torch.uint8, device=dev)
    out = torch.empty((B, n_tok * H, D), dtype=torch.float32, device=dev)

    def dense_step(i):
        c = caches[i % R]
        skv.kv_append(c, pos, nk, nv)
        skv.decode_attn_multi(c, qc, seq_len, Lmax, w.softmax_scale, S_d, ws_d)
        skv.combine(ws_d, B, n_tok * H, D, S_d, out)

    def quest_step(i):
        c = caches[i % R]
        skv.kv_append(c, pos, nk, nv)
        skv.block_bounds_multi(c, qc, seq_len, Lmax, sc)
        skv.select_topk_multi(sc, seq_len, blk, ks, w.n_sink, w.n_recent, sel, cnt)
        skv.select_union_tokens(sel, cnt, w.G, max_blocks, uni, ucnt, um)
        skv.decode_attn_multi(c, qc, seq_len, Lmax, w.softmax_scale, S_q, ws_q, uni, ucnt, um)
        skv.combine(ws_q, B, n_tok * H, D, S_q, out)

    quest_step(0)
    torch.cuda.synchronize()
    u_h, c_h = uni.cpu().numpy(), ucnt.cpu().numpy()
    attended = {(b, g): u_h[b, g, :c_h[b, g]].tolist() for b in range(B) for g in range(Hkv)}
    qio = (n_tok - 1) * B * H * D * 4 * 2                     # the extra queries and outputs
    qb = step_bytes(w.lens, Hkv, H, D, w.kv_dtype, blk, attended)
    db = step_bytes(w.lens, Hkv, H, D, w.kv_dtype, blk, None)
    res = {"n_tokens": n_tok, "columns_per_kv_head": n_tok * w.G}
    gr, _ = T.graph(quest_step)
    us = (gr if gr is not None else T.stream(quest_step)) * 1e6
    n_all = sum(-(-L // blk) for L in w.lens) * Hkv
    res["quest"] = {"us_per_step": round(us, 3),
                    "vs_single_token_steps": round(us / (n_tok * quest_res["us_per_step"]), 4),
                    "bytes_per_step": qb["total"] + qio,
                    "union_blocks_frac": round(sum(len(x) for x in attended.values()) / n_all, 4),
                    "pct_hbm_peak": round(100 * (qb["total"] + qio) / us / 1e3 / HBM_PEAK_GBPS, 2),
                    "n_split": S_q}
    if dense_res is not None:
        gr, _ = T.graph(dense_step)
        us = (gr if gr is not None else T.stream(dense_step)) * 1e6
        res["dense"] = {"us_per_step": round(us, 3),
                        "vs_single_token_steps": round(us / (n_tok * dense_res["us_per_step"]), 4),
                        "bytes_per_step": db["total"] + qio,
                        "pct_hbm_peak": round(100 * (db["total"] + qio) / us / 1e3
                                              / HBM_PEAK_GBPS, 2),
                        "n_split": S_d}
    return res


def measure_per_head(T, skv, torch, w, caches, R, q, seq_len, Lmax, new_k, new_v, pos_last, ks,
                     group_res):
    """The Quest step with one block set per query head: kv_append,
    block_bounds_heads, select_topk over the H per-head rows, select_union,
    decode_attn_heads (each head over its own blocks, the union read once
    for the group), combine.  Bytes: the side cache, the KV rows of the
    union's blocks, q and the output."""
    B, H, Hkv, D, blk = w.B, w.H, w.Hkv, w.D, w.block
    dev = q.device
    max_sel = max(w.k_sel) + w.n_sink + w.n_recent
    max_blocks = caches[0].max_blocks
    max_union = min(max_blocks, w.G * max_sel)
    sc = torch.empty((B, H, max_blocks), dtype=torch.float32, device=dev)
    sel = torch.empty((B, H, max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H), dtype=torch.int32, device=dev)
    uni = torch.empty((B, Hkv, max_union), dtype=torch.int32, device=dev)
    ucnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    um = torch.empty((B, Hkv, max_union), dtype=torch.int32, device=dev)
    S = skv.default_split(B, Hkv, max_union, kv_dtype=w.kv_dtype, sparse=True)
    ws = torch.empty(skv.workspace_bytes(B, H, D, S), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, D), dtype=torch.float32, device=dev)

    def step(i):
        c = caches[i % R]
        skv.kv_append(c, pos_last, new_k, new_v)
        skv.block_bounds_heads(c, q, seq_len, Lmax, sc)
        skv.select_topk(sc, seq_len, blk, ks, w.n_sink, w.n_recent, sel, cnt)
        skv.select_union(sel, cnt, Hkv, max_blocks, uni, ucnt, um)
        skv.decode_attn_heads(c, q, seq_len, Lmax, w.softmax_scale, S, ws, uni, ucnt, um)
        skv.combine(ws, B, H, D, S, out)

    step(0)
    torch.cuda.synchronize()
    u_h, c_h = uni.cpu().numpy(), ucnt.cpu().numpy()
    attended = {(b, g): u_h[b, g, :c_h[b, g]].tolist() for b in range(B) for g in range(Hkv)}
    qb = step_bytes(w.lens, Hkv, H, D, w.kv_dtype, blk, attended)
    gr, _ = T.graph(step)
    us = (gr if gr is not None else T.stream(step)) * 1e6
    dec_bytes = qb["kv"] + B * H * D * 4
    dec_us = T.kernel(lambda i: skv.decode_attn_heads(caches[i % R], q, seq_len, Lmax,
                                                      w.softmax_scale, S, ws, uni, ucnt, um))
    n_all = sum(-(-L // blk) for L in w.lens) * Hkv
    return {"us_per_step": round(us, 3),
            "vs_group_five_calls": round(us / group_res["five_calls_us_per_step"], 4),
            "bytes_per_step": qb["total"], "kv_bytes": qb["kv"],
            "union_blocks_frac": round(sum(len(x) for x in attended.values()) / n_all, 4),
            "GBps": round(qb["total"] / us / 1e3, 1),
            "pct_hbm_peak": round(100 * qb["total"] / us / 1e3 / HBM_PEAK_GBPS, 2),
            "decode_attn_heads_us": round(dec_us, 3),
            "decode_attn_heads_pct_peak": round(100 * dec_bytes / dec_us / 1e3 / HBM_PEAK_GBPS, 2),
            "n_split": S}


def measure_scan4(T, skv, torch, w, caches, R, q, seq_len, Lmax, delta):
    """The GQA-shared 4-bit scan: skv_scan4_candidates over every token
    (index built beforehand, as an append would keep it).  Bytes: the 4-bit
    codes (D / 2 per (token, KV head), read once for the G heads) and the
    per-block lo / step / err (3 x D x 4 B per (block, KV head)); the UB
    values the two passes exchange are implementation traffic."""
    B, H, Hkv, D, blk = w.B, w.H, w.Hkv, w.D, w.block
    dev = q.device
    idx = [skv.Scan4Index(c, device=dev) for c in caches]
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    for c, ix in zip(caches, idx):
        skv.scan4_build(c, ix, zero, seq_len, Lmax)
    S = skv.scan4_default_split(B, Hkv, -(-Lmax // blk))
    ws = torch.empty(skv.scan4_workspace_bytes(B, H, S, Lmax), dtype=torch.uint8, device=dev)
    cand = torch.empty((B, H, -(-Lmax // 32)), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    us = T.kernel(lambda i: skv.scan4_candidates(caches[i % R], idx[i % R], q, seq_len, Lmax,
                                                 delta, S, ws, cand, cnt))
    build_us = T.kernel(lambda i: skv.scan4_build(caches[i % R], idx[i % R], zero, seq_len,
                                                  Lmax))
    byts = scan4_index_bytes(w.lens, Hkv, D, blk) + B * H * D * 4
    per_head = scan4_index_bytes(w.lens, Hkv, D, blk, reads_per_token=w.G) + B * H * D * 4
    n_c = int(cnt.sum().item())
    del idx
    return {"delta": delta, "us": round(us, 3), "bytes": byts,
            "pct_hbm_peak": round(100 * byts / us / 1e3 / HBM_PEAK_GBPS, 2),
            "per_head_scan_bytes": per_head,
            "candidates_frac": round(n_c / (sum(w.lens) * H), 5),
            "build_all_us": round(build_us, 3), "n_split": S}


def measure_sparse_v(T, skv, torch, w, caches, R, q, seq_len, Lmax, new_k, new_v, pos_last, ks,
                     score, sel, cnt, attended, tau, calls_us):
    """The Quest step with sparse-V inside the selected blocks (static tau):
    kv_append, block_bounds, select_topk, decode_attn_sparse_v (its q.K pass
    and its value pass over the kept rows), combine.  Bytes: the side cache,
    the K rows of the selected blocks, the V rows some head of the group
    keeps (read once for the group), q and the output; the logits the two
    passes exchange are implementation traffic, reported beside them."""
    B, H, Hkv, D, blk = w.B, w.H, w.Hkv, w.D, w.block
    S = skv.default_split(B, Hkv, int(sel.shape[2]), kv_dtype=w.kv_dtype, sparse=True)
    dev = q.device
    ws = torch.empty(skv.sparse_v_workspace_bytes(B, H, Hkv, D, S, Lmax), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    keep = torch.zeros((B, H, -(-Lmax // 32)), dtype=torch.int32, device=dev)
    skv.decode_attn_sparse_v(caches[0], q, seq_len, Lmax, w.softmax_scale, S, ws, tau=tau,
                             sel_idx=sel, sel_cnt=cnt, keep_mask=keep)
    torch.cuda.synchronize()
    kw = keep.cpu().numpy().view(np.uint32)
    row_k = 2 * D if w.kv_dtype == "f16" else D + 4          # a K (or V) row and its scale
    k_bytes = v_bytes = 0
    kept_pairs = att_pairs = 0
    for b, L in enumerate(w.lens):
        for g in range(Hkv):
            toks = np.concatenate([np.arange(j * blk, min((j + 1) * blk, L))
                                   for j in attended[(b, g)]])
            bits = np.zeros(toks.size, bool)
            for h in range(g * w.G, (g + 1) * w.G):
                hb = (kw[b, h][toks // 32] >> (toks % 32).astype(np.uint32)) & 1
                kept_pairs += int(hb.sum())
                bits |= hb.astype(bool)
            att_pairs += w.G * toks.size
            k_bytes += toks.size * row_k
            v_bytes += int(bits.sum()) * row_k
    bounds = sum(-(-L // blk) for L in w.lens) * Hkv * side_cache_bytes_per_block(D)
    total = bounds + k_bytes + v_bytes + 2 * B * H * D * 4
    logit_bytes = 2 * 4 * sum(len(v) for v in attended.values()) * blk * w.G

    def sv_calls(i):
        c = caches[i % R]
        skv.kv_append(c, pos_last, new_k, new_v)
        skv.block_bounds(c, q, seq_len, Lmax, score)
        skv.select_topk(score, seq_len, blk, ks, w.n_sink, w.n_recent, sel, cnt)
        skv.decode_attn_sparse_v(c, q, seq_len, Lmax, w.softmax_scale, S, ws, tau=tau,
                                 sel_idx=sel, sel_cnt=cnt)
        skv.combine(ws, B, H, D, S, out)

    gr, _ = T.graph(sv_calls)
    us = (gr if gr is not None else T.stream(sv_calls)) * 1e6
    pair_us = T.kernel(lambda i: skv.decode_attn_sparse_v(
        caches[i % R], q, seq_len, Lmax, w.softmax_scale, S, ws, tau=tau, sel_idx=sel,
        sel_cnt=cnt))
    att_bytes = k_bytes + v_bytes + B * H * D * 4
    return {"tau": tau, "us_per_step": round(us, 3),
            "vs_five_calls_without": round(us / calls_us, 4),
            "bytes_per_step": total, "k_bytes": k_bytes, "v_bytes_kept": v_bytes,
            "kept_head_token_frac": round(kept_pairs / max(att_pairs, 1), 5),
            "v_rows_read_frac": round(v_bytes / max(k_bytes, 1), 5),
            "logit_bytes_exchanged": logit_bytes,
            "sparse_v_pair_us": round(pair_us, 3),
            "sparse_v_pair_pct_peak": round(100 * att_bytes / pair_us / 1e3 / HBM_PEAK_GBPS, 2),
            "n_split": S}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--ring", type=int, default=0, help="cache copies (0 = auto, cold cache)")
    ap.add_argument("--ring-budget-gb", type=float, default=24.0,
                    help="upper bound on the memory of the cache copies of one workload")
    ap.add_argument("--n-split", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--mode", choices=("both", "quest", "dense"), default="both",
                    help="which step of the 32K workload to time (profiling runs use one)")
    ap.add_argument("--workloads", default="1,2,4,5,3@16384,3q8,3q4,3q5,3d64,3d256",
                    help="other workloads to time besides the 32K headline ('' = none; "
                         "3@L = the 32K Quest generator at context L; 3q8 / 3q4 / 3q5 = over a "
                         "q8_0 / q4_0 / q5_0 cache; 3d64 / 3d256 = at head dim 64 / 256; both, "
                         "e.g. 3q4d256)")
    ap.add_argument("--chunk-tokens", type=int, default=4,
                    help="query tokens per chunk for the multi-token measurement (0 = off)")
    ap.add_argument("--no-per-head", action="store_true",
                    help="skip the Quest steps with one block set per query head")
    ap.add_argument("--no-scan4", action="store_true",
                    help="skip the GQA-shared 4-bit scan timing")
    ap.add_argument("--scan4-delta", type=float, default=8.0,
                    help="candidate margin of the 4-bit scan, in q.k units")
    ap.add_argument("--sparse-v-tau", type=float, default=1e-3,
                    help="also time the Quest steps with sparse-V at this static threshold "
                         "(0 = off)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB three times "
                         "(a plain copy of known size that scales HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path has no "
              "multi-GPU mode in this build", file=sys.stderr)
        sys.exit(2)

    import workloads

    # the workloads, drawn once (host arrays) for the CPU baseline and the GPU
    jobs = [(workloads.named(3), args.mode in ("both", "quest"),
             args.mode in ("both", "dense"), True)]
    for tok in [t.strip() for t in args.workloads.split(",") if t.strip()]:
        if tok.startswith("3@"):
            # the 32K generator at another length (Quest vs dense from 16K up)
            jobs.append((workloads.quest32k_at(int(tok[2:])), True, True, False))
        elif tok != "3" and re.fullmatch(r"3(q[458])?(d\d+)?", tok):
            # the 32K generator over a group-wise quantized cache (3q8, 3q4,
            # 3q5) and / or at another head dim (3d64, 3d256, 3q4d256)
            m = re.fullmatch(r"3(q[458])?(d\d+)?", tok)
            kv = {None: "f16", "q8": "q8_0", "q4": "q4_0", "q5": "q5_0"}[m.group(1)]
            D = int(m.group(2)[1:]) if m.group(2) else 128
            jobs.append((workloads.quest32k_dim(D, kv), True, True, False))
        elif int(tok) != 3:
            w = workloads.named(int(tok))
            jobs.append((w, bool(w.k_sel), True, False))

    # the oracle on the host cores, before anything touches the GPU (its
    # all-cores leg forks this process)
    cpu_rows = []
    if not args.no_cpu:
        for w, quest, dense, _ in jobs:
            if quest:
                cpu_rows.append(cpu_baseline(w, quest=True))
            if dense:
                cpu_rows.append(cpu_baseline(w, quest=False))

    import torch
    import sparse_kv_cache_append_amd as skv

    skv.load()
    torch.cuda.set_device(0)
    w3 = jobs[0][0]
    head = None
    others = []
    for w, quest, dense, detail in jobs:
        r = measure(w, args, quest=quest, dense=dense, detail=detail)
        if detail:
            head = r
        else:
            others.append(r)

    hq, hd = head.get("quest"), head.get("dense")
    top = hq if hq is not None else hd
    if hq is not None:
        rk = ("decode_f16_mfma, selection in the prologue (decode_attn_select over the "
              "selected blocks: the Quest step's attention kernel)")
        rb, rus, _ = head["_roofline"]
    else:
        rk = "decode_f16_mfma (decode_attn, dense)"
        rus = hd["decode_attn_us"]
        rb = step_bytes(w3.lens, w3.Hkv, w3.H, w3.D, "f16", w3.block, None)["kv"] + w3.H * w3.D * 4
    ach = rb / (rus * 1e-6) / 1e9
    us = top["us_per_step"]
    res = {
        "metric": METRIC,
        "value": us,
        "unit": "us/step",
        "n_gpus": 1,
        "steps": top["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w3.name,
                   "step": ("decode_step: kv_append + block_bounds + select_topk + "
                            "decode_attn(selected blocks) + combine in 3 launches")
                           if hq is not None else
                           "decode_step: kv_append + decode_attn(dense) + combine in 2 launches",
                   "cache_copies": head["cache_copies"],
                   "launch": "hipgraph" if not args.no_graph else "stream",
                   "n_split": top["n_split"]},
        "achieved_GBps": top["GBps"],
        "pct_hbm_peak": top["pct_hbm_peak"],
        "quest": hq,
        "dense": hd,
        "quest_over_dense_time": head.get("quest_over_dense"),
        "quest_sparse_v": head.get("quest_sparse_v"),
        "quest_per_head": head.get("quest_per_head"),
        "scan4": head.get("scan4"),
        "chunk": head.get("chunk"),
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": recorded_traffic(rk), "kernel": rk,
                     "avg_launch_us": round(rus, 3), "bytes_per_launch": rb},
        "workloads": others,
    }
    if args.copy_probe_mib > 0:
        a = torch.ones(args.copy_probe_mib * 2 ** 18, dtype=torch.float32, device="cuda:0")
        b2 = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b2.copy_(a)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = {"read": a.numel() * 4, "written": a.numel() * 4}
    if cpu_rows:
        top_cpu = cpu_rows[0]
        res["cpu_baseline"] = {
            "value": top_cpu["all_cores"]["value"], "unit": "us/step",
            "cores": top_cpu["all_cores"]["cores"], "kind": "oracle",
            "sample": f"{top_cpu['workload']} {top_cpu['step']} step: "
                      f"{top_cpu['all_cores']['sample']}; {top_cpu['what']}",
            "cpu_model": _cpu_model(),
            "single_core": top_cpu["one_core"],
            "per_config": cpu_rows}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
