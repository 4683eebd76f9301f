"""Decode-step attention benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: append the new
token (kv_append), Quest upper bounds (block_bounds), top-K selection
(select_topk), attention over the selected blocks (decode_attn) and the
split-K merge (combine).  The workload is the 32K-context GQA decode
(B=1, H=32, Hkv=8, D=128, f16 KV, block 64, K_SEL=128 + sink + 2 recent);
the same cache is also timed with dense decode (append + decode_attn +
combine) for the sparse/dense ratio.

Timing protocol:
* Inputs are resident in HBM before the timed region.
* Cold cache: every step reads one of R cache copies, R chosen so the copies
  a ring touches exceed 2x the 256 MB last-level cache, so steps read HBM.
* W warmup steps, then exactly K timed steps between synchronizations;
  the steps are captured once in a HIP graph (torch.cuda.CUDAGraph over the
  library's launches on the capture stream) and replayed; the stream-launch
  time is reported too.
* The dominant kernel (decode_attn) is timed alone: R launches (one per cache
  copy) captured in a HIP graph, replayed, HIP events on the replay stream;
  achieved GB/s = algorithmic bytes per launch / average launch time.

Prints ONE JSON line (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
import json
import math
import os
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
    the two float32 scales for int8."""
    return 4 * D if kv_dtype == "f16" else 2 * D + 8


def side_cache_bytes_per_block(D: int) -> int:
    """kmin and kmax rows of one (block, KV head), f16."""
    return 2 * 2 * D


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
                  for f in ("decode_mfma.hip", "device_common.h", "launch.h")]


def kernel_source_digest() -> str:
    """sha256 over the sources the decode kernel is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
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
def cpu_baseline(w, budget_s: float = 12.0):
    """The oracle's Quest step (append the token, bounds, selection, sparse
    attention) on the host cores, single-threaded, repeated for ~budget_s."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl is in the image
        limiter = None
    L = w.lens[0]
    keys, vals, q = w.k[0], w.v[0], w.q[0]

    def step():
        # append: the new token's row joins its block's bounds (from scratch is
        # the same bytes, by exactness of min/max)
        kmin, kmax = oracle.block_bounds(keys, L, w.block)
        sc = oracle.group_scores(oracle.upper_bounds(q, kmin, kmax), w.Hkv)
        out = np.zeros((w.H, w.D))
        for g in range(w.Hkv):
            r = oracle.select_blocks(sc[g], w.n_blocks(0), w.k_sel[0], w.n_sink, w.n_recent)
            toks = oracle.selected_tokens(r["sel"], L, w.block)
            hs = slice(g * w.G, (g + 1) * w.G)
            out[hs] = oracle.attend_f16(q[hs], keys[g:g + 1], vals[g:g + 1], w.softmax_scale,
                                        tokens=toks)
        return out

    n = 0
    t0 = time.perf_counter()
    while True:
        step()
        n += 1
        if time.perf_counter() - t0 > budget_s or n >= 50:
            break
    dt = (time.perf_counter() - t0) / n
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": dt * 1e6, "unit": "us/step", "cores": 1, "kind": "oracle",
            "sample": f"{n} full Quest steps of the same workload (float64 NumPy oracle: "
                      f"bounds with exact sums, selection, attention over the selected "
                      f"blocks), one thread, on {cpu}"}


# ------------------------------------------------------------- GPU bench
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--ring", type=int, default=0, help="cache copies (0 = auto, cold cache)")
    ap.add_argument("--n-split", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--mode", choices=("both", "quest", "dense"), default="both",
                    help="which step to time (profiling runs use one)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB three times "
                         "(a plain copy of known size that scales HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path has no "
              "multi-GPU mode in this build", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_kv_cache_append_amd as skv
    import workloads

    skv.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.named(3)
    B, H, Hkv, D, blk = w.B, w.H, w.Hkv, w.D, w.block
    L = w.lens[0]
    k_sel = w.k_sel[0]
    max_sel = k_sel + w.n_sink + w.n_recent
    nb = -(-L // blk)

    # ring of cache copies, each holding L-1 tokens; every step appends token L-1
    src_k = torch.from_numpy(np.ascontiguousarray(np.transpose(w.k[0], (1, 0, 2))[None])).to(dev)
    src_v = torch.from_numpy(np.ascontiguousarray(np.transpose(w.v[0], (1, 0, 2))[None])).to(dev)
    quest_touch = max_sel * blk * Hkv * kv_bytes_per_token("f16", D) + nb * Hkv * 512
    R = args.ring or max(2, math.ceil(2 * LLC_BYTES / quest_touch) + 1)
    caches = []
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(R):
        c = skv.Cache(B, Hkv, L, D, "f16", blk, bounds=True, device=dev)
        skv.kv_append(c, zero, src_k[:, :L - 1].contiguous(), src_v[:, :L - 1].contiguous())
        caches.append(c)
    new_k = src_k[:, L - 1:L].contiguous()
    new_v = src_v[:, L - 1:L].contiguous()
    pos_last = torch.full((B,), L - 1, dtype=torch.int32, device=dev)
    q = torch.from_numpy(w.q).to(dev)
    seq_len = torch.full((B,), L, dtype=torch.int32, device=dev)
    ks = torch.full((B,), k_sel, dtype=torch.int32, device=dev)
    score = torch.empty((B, Hkv, caches[0].max_blocks), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Hkv, max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    S_q = args.n_split or skv.default_split(B, Hkv, max_sel)
    S_d = args.n_split or skv.default_split(B, Hkv, nb)
    ws_q = torch.empty(skv.workspace_bytes(B, H, D, S_q), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(skv.workspace_bytes(B, H, D, S_d), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def quest_step(i):
        c = caches[i % R]
        skv.kv_append(c, pos_last, new_k, new_v)
        skv.block_bounds(c, q, seq_len, L, score)
        skv.select_topk(score, seq_len, blk, ks, w.n_sink, w.n_recent, sel, cnt)
        skv.decode_attn(c, q, seq_len, L, w.softmax_scale, S_q, ws_q, sel, cnt)
        skv.combine(ws_q, B, H, D, S_q, out)

    def dense_step(i):
        c = caches[i % R]
        skv.kv_append(c, pos_last, new_k, new_v)
        skv.decode_attn(c, q, seq_len, L, w.softmax_scale, S_d, ws_d)
        skv.combine(ws_d, B, H, D, S_d, out)

    def time_stream(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def time_graph(fn, steps, warmup):
        for i in range(max(warmup, R)):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                fn(i)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // R)
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (reps * R), reps * R

    K, W = args.steps, args.warmup
    do_q, do_d = args.mode in ("both", "quest"), args.mode in ("both", "dense")
    quest_stream = time_stream(quest_step, K, W) if do_q else None
    dense_stream = time_stream(dense_step, K, W) if do_d else None
    quest_graph = dense_graph = None
    steps_done = K
    if not args.no_graph:
        if do_q:
            quest_graph, steps_done = time_graph(quest_step, K, W)
        if do_d:
            dense_graph, steps_done = time_graph(dense_step, K, W)

    # selected sets of this workload (for the byte accounting)
    quest_step(0)
    torch.cuda.synchronize()
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    attended = {(0, g): sel_h[0, g, :cnt_h[0, g]].tolist() for g in range(Hkv)}
    qb = step_bytes([L], Hkv, H, D, "f16", blk, attended)
    db = step_bytes([L], Hkv, H, D, "f16", blk, None)

    # dominant kernel alone: the fused decode over the selected blocks, R
    # launches (one per cache copy) captured in a HIP graph and replayed;
    # HIP events on the replay stream bracket K launches
    def time_kernel(fn):
        st = torch.cuda.Stream()
        if args.no_graph:
            with torch.cuda.stream(st):
                for i in range(R):
                    fn(i)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                for i in range(K):
                    fn(i)
                e1.record(st)
            st.synchronize()
            return e0.elapsed_time(e1) * 1e3 / K
        with torch.cuda.stream(st):
            for i in range(R):
                fn(i)
        st.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for i in range(R):
                fn(i)
        reps = max(1, K // R)
        with torch.cuda.stream(st):
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                g.replay()
            e1.record(st)
        st.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * R)

    dec_bytes = qb["kv"] + H * D * 4
    dense_dec_bytes = db["kv"] + H * D * 4
    dec_us = time_kernel(lambda i: skv.decode_attn(caches[i % R], q, seq_len, L, w.softmax_scale,
                                                   S_q, ws_q, sel, cnt)) if do_q else None
    dense_dec_us = time_kernel(lambda i: skv.decode_attn(caches[i % R], q, seq_len, L,
                                                         w.softmax_scale, S_d, ws_d)) if do_d else None

    def us(graph_t, stream_t):
        t = graph_t if graph_t is not None else stream_t
        return None if t is None else t * 1e6

    def rnd(x, n=3):
        return None if x is None else round(x, n)

    quest_us = us(quest_graph, quest_stream)
    dense_us = us(dense_graph, dense_stream)
    head_us = quest_us if quest_us is not None else dense_us
    head_bytes = qb["total"] if quest_us is not None else db["total"]
    gbps = head_bytes / (head_us * 1e-6) / 1e9
    if dec_us is not None:
        rk, rb, rus = "decode_f16_mfma (decode_attn over the selected blocks)", dec_bytes, dec_us
    else:
        rk, rb, rus = "decode_f16_mfma (decode_attn, dense)", dense_dec_bytes, dense_dec_us
    ach = rb / (rus * 1e-6) / 1e9
    traffic = recorded_traffic(rk)
    res = {
        "metric": METRIC,
        "value": round(head_us, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": steps_done,
        "warmup": W,
        "ms_per_step": round(head_us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name,
                   "step": ("kv_append + block_bounds + select_topk + decode_attn(selected blocks)"
                            " + combine") if quest_us is not None else
                           "kv_append + decode_attn(dense) + combine",
                   "cache_copies": R,
                   "launch": "hipgraph" if not args.no_graph else "stream",
                   "n_split": S_q if quest_us is not None else S_d},
        "achieved_GBps": round(gbps, 1),
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "bytes_per_step": qb if quest_us is not None else db,
        "dense": None if dense_us is None else {
            "us_per_step": rnd(dense_us), "bytes_per_step": db,
            "achieved_GBps": round(db["total"] / (dense_us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * db["total"] / (dense_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
            "n_split": S_d, "decode_attn_us": rnd(dense_dec_us),
            "decode_attn_GBps": round(dense_dec_bytes / (dense_dec_us * 1e-6) / 1e9, 1)},
        "quest_over_dense_time": (round(quest_us / dense_us, 4)
                                  if quest_us is not None and dense_us is not None else None),
        "stream_launch_us": {"quest": rnd(None if quest_stream is None else quest_stream * 1e6),
                             "dense": rnd(None if dense_stream is None else dense_stream * 1e6)},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": rk, "avg_launch_us": round(rus, 3), "bytes_per_launch": rb},
    }
    if args.copy_probe_mib > 0:
        a = torch.ones(args.copy_probe_mib * 2 ** 18, dtype=torch.float32, device=dev)
        b2 = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b2.copy_(a)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = {"read": a.numel() * 4, "written": a.numel() * 4}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
