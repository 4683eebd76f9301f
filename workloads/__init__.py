"""Seeded synthetic inputs for decode-step attention over a long KV cache.

This module only draws tensors. It holds none of the attention method's
arithmetic (no quantization, no bounds, no softmax), so that the HIP path and
the CPU oracle can both be fed from it without sharing any of the computation
they are compared on.

Two families of inputs are drawn, both with ``numpy.random.default_rng(seed)``
in float32:

* ``gaussian``: K, V, q i.i.d. N(0, 1).
* ``clustered``: per KV head ``n_dirs`` random unit directions; every
  ``block``-token block of keys picks one direction ``c`` uniformly and each
  key is ``amp * dir[c] + N(0, 1)``; V is N(0, 1); each query head picks a
  random direction of its KV head and is ``amp * dir + N(0, 1)``.  This plants
  the retrievable block structure the block selector is meant to find (the
  "needle block" role of the retrieval gate in the opencoti-llamafile
  sparse_attn.md page, section "Correctness gate").

Draw order is fixed (documented per function) so a seed names the bytes.

The five named workloads mirror GQA decode shapes (D = 128):

==  ===========================================================================
1   dense f16, B=1, H=8, Hkv=8, L=512, gaussian, seed 1001
2   dense int8, B=1, H=32, Hkv=8, L=8192, gaussian fp32 (quantized at append),
    seed 1002
3   Quest f16, B=1, H=32, Hkv=8, L=32768, clustered (64 dirs, amp 4), block 64,
    K_SEL=128, sink block 0, 2 recent blocks, seed 1003
4   batched varlen f16, B=16, L_b ~ U{16384..65536} (seed 1004), H=32, Hkv=8,
    clustered per sequence (seed 4000+b), K_SEL_b = floor(NB_b/4), sink 0,
    2 recent blocks
5   Quest int8, B=1, L=262144, H=32, Hkv=4, clustered (256 dirs, amp 4),
    block 64, K_SEL=512, sink block 0, 4 recent blocks, seed 1005
==  ===========================================================================
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
from typing import List, Optional

import numpy as np

__all__ = ["Workload", "gaussian", "clustered", "named", "quest32k_at", "quest32k_quant",
           "lengths_config4", "chunk_queries", "NAMED"]


@dataclasses.dataclass
class Workload:
    """One batch of decode-step inputs.

    ``k[b]``/``v[b]`` are ``[Hkv][L_b][D]``: float16 for an f16 cache, float32
    (pre-quantization) for an int8, q8_0 or q4_0 cache.  ``q`` is ``[B][H][D]`` float32.
    ``k_sel`` is the per-sequence top-K budget (None = dense only).
    """
    name: str
    B: int
    H: int
    Hkv: int
    D: int
    lens: List[int]
    kv_dtype: str            # "f16", "i8", "q8_0" or "q4_0"
    k: List[np.ndarray]
    v: List[np.ndarray]
    q: np.ndarray
    block: int = 64
    k_sel: Optional[List[int]] = None
    n_sink: int = 1
    n_recent: int = 2
    softmax_scale: float = 0.0

    def __post_init__(self):
        if self.softmax_scale == 0.0:
            self.softmax_scale = 1.0 / math.sqrt(self.D)

    @property
    def G(self) -> int:
        return self.H // self.Hkv

    def n_blocks(self, b: int) -> int:
        return -(-self.lens[b] // self.block)


def _cast(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    # f16 cache: round the float32 draw to float16 (round-to-nearest-even);
    # int8 cache: keep the float32 draw, it is what gets appended.
    return x.astype(np.float16) if kv_dtype == "f16" else x


def gaussian(seed: int, B: int, H: int, Hkv: int, D: int, lens, kv_dtype: str,
             name: str = "gaussian", **kw) -> Workload:
    """i.i.d. N(0,1) K, V, q.  Draw order: for each sequence b: K_b, V_b; then q."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    ks, vs = [], []
    for b in range(B):
        ks.append(_cast(rng.standard_normal((Hkv, lens[b], D), dtype=np.float32), kv_dtype))
        vs.append(_cast(rng.standard_normal((Hkv, lens[b], D), dtype=np.float32), kv_dtype))
    q = rng.standard_normal((B, H, D), dtype=np.float32)
    return Workload(name, B, H, Hkv, D, lens, kv_dtype, ks, vs, q, **kw)


def _clustered_sequence(rng, H, Hkv, D, L, n_dirs, amp, block, kv_dtype):
    """Draw order: dirs, per-block cluster ids, key noise, V, query cluster ids,
    query noise."""
    G = H // Hkv
    dirs = rng.standard_normal((Hkv, n_dirs, D), dtype=np.float32)
    dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
    nb = -(-L // block)
    cid = rng.integers(0, n_dirs, size=(Hkv, nb))
    k = rng.standard_normal((Hkv, L, D), dtype=np.float32)
    tok_cid = np.repeat(cid, block, axis=1)[:, :L]                  # [Hkv][L]
    for g in range(Hkv):
        k[g] += np.float32(amp) * dirs[g][tok_cid[g]]
    v = rng.standard_normal((Hkv, L, D), dtype=np.float32)
    qc = rng.integers(0, n_dirs, size=H)
    qn = rng.standard_normal((H, D), dtype=np.float32)
    q = np.stack([np.float32(amp) * dirs[h // G, qc[h]] for h in range(H)]) + qn
    return _cast(k, kv_dtype), _cast(v, kv_dtype), q.astype(np.float32)


def clustered(seeds, H: int, Hkv: int, D: int, lens, kv_dtype: str,
              n_dirs: int = 64, amp: float = 4.0, block: int = 64,
              name: str = "clustered", **kw) -> Workload:
    """Clustered keys, one generator per sequence (``seeds[b]``)."""
    lens = [int(x) for x in lens]
    B = len(lens)

    def one(b):
        rng = np.random.default_rng(seeds[b])
        return _clustered_sequence(rng, H, Hkv, D, lens[b], n_dirs, amp, block, kv_dtype)

    # Sequences draw from independent generators, so threads change no byte.
    workers = max(1, min(B, 8, os.cpu_count() or 1))
    if workers > 1:
        with cf.ThreadPoolExecutor(workers) as ex:
            seqs = list(ex.map(one, range(B)))
    else:
        seqs = [one(0)]
    ks = [s[0] for s in seqs]
    vs = [s[1] for s in seqs]
    qs = [s[2] for s in seqs]
    return Workload(name, B, H, Hkv, D, lens, kv_dtype, ks, vs, np.stack(qs),
                    block=block, **kw)


def lengths_config4() -> List[int]:
    rng = np.random.default_rng(1004)
    return [int(x) for x in rng.integers(16384, 65536, endpoint=True, size=16)]


NAMED = {
    1: "dense-f16 B1 H8/Hkv8 D128 L512",
    2: "dense-int8 B1 H32/Hkv8 D128 L8192",
    3: "quest-f16 B1 H32/Hkv8 D128 L32768 K_SEL128 sink1 recent2",
    4: "varlen-f16 B16 H32/Hkv8 D128 L16K-64K K_SEL=NB/4 sink1 recent2",
    5: "quest-int8 B1 H32/Hkv4 D128 L262144 K_SEL512 sink1 recent4",
}


def named(cfg: int) -> Workload:
    """The five named workloads at full size."""
    if cfg == 1:
        return gaussian(1001, 1, 8, 8, 128, [512], "f16", name=NAMED[1])
    if cfg == 2:
        return gaussian(1002, 1, 32, 8, 128, [8192], "i8", name=NAMED[2])
    if cfg == 3:
        return clustered([1003], 32, 8, 128, [32768], "f16", n_dirs=64,
                         name=NAMED[3], k_sel=[128], n_sink=1, n_recent=2)
    if cfg == 4:
        lens = lengths_config4()
        return clustered([4000 + b for b in range(16)], 32, 8, 128, lens, "f16",
                         n_dirs=64, name=NAMED[4],
                         k_sel=[(-(-L // 64)) // 4 for L in lens], n_sink=1, n_recent=2)
    if cfg == 5:
        return clustered([1005], 32, 4, 128, [262144], "i8", n_dirs=256,
                         name=NAMED[5], k_sel=[512], n_sink=1, n_recent=4)
    raise ValueError(f"unknown workload {cfg}")


def quest32k_quant(kv_dtype: str) -> Workload:
    """The 32K Quest workload's generator (H=32, Hkv=8, 64 directions, block
    64, K_SEL=128, sink 1, recent 2, seed 1003) drawn for a group-wise
    quantized cache ("q8_0", "q4_0" or "q5_0"): the float32 rows that get
    appended."""
    return quest32k_dim(128, kv_dtype)


def quest32k_at(L: int) -> Workload:
    """The 32K Quest workload's generator (H=32, Hkv=8, 64 directions, block
    64, sink 1, recent 2, seed 1003) at another context length, with the same
    25% coverage: K_SEL = floor(NB / 4)."""
    nb = -(-L // 64)
    return clustered([1003], 32, 8, 128, [L], "f16", n_dirs=64,
                     name=f"quest-f16 B1 H32/Hkv8 D128 L{L} K_SEL{nb // 4} sink1 recent2",
                     k_sel=[nb // 4], n_sink=1, n_recent=2)


def quest32k_dim(D: int, kv_dtype: str = "f16") -> Workload:
    """The 32K Quest workload's generator (H=32, Hkv=8, 64 directions, block
    64, K_SEL=128, sink 1, recent 2, seed 1003) at head dim D over a kv_dtype
    cache (f16 rows, or the float32 rows a quantized cache is filled from)."""
    return clustered([1003], 32, 8, D, [32768], kv_dtype, n_dirs=64,
                     name=f"quest-{kv_dtype} B1 H32/Hkv8 D{D} L32768 K_SEL128 sink1 recent2",
                     k_sel=[128], n_sink=1, n_recent=2)


def chunk_queries(w: Workload, T: int, seed: int, noise: float = 1.5) -> np.ndarray:
    """Queries of a chunk of T tokens per sequence, [B][T][H][D] float32:
    token 0 is the workload's own query, token t > 0 that query plus
    ``noise`` * N(0, 1) (drawn in token order), so the chunk's tokens lean on
    the same key directions but rank the blocks differently."""
    rng = np.random.default_rng(seed)
    out = np.empty((w.B, T, w.H, w.D), dtype=np.float32)
    out[:, 0] = w.q
    for t in range(1, T):
        out[:, t] = w.q + np.float32(noise) * rng.standard_normal((w.B, w.H, w.D),
                                                                 dtype=np.float32)
    return out
