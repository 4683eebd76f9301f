"""Quest-style block selection: side cache, upper bound, top-K + sink + recent.

Source: opencoti-llamafile docs/features/sparse_attn.md, "Sparse Attention --
Quest-style block-selector for long-context decode".
* Section "Method: Quest-style min/max block bounds": per (KV head, block)
  kmin[D], kmax[D] stored as f16, taken from the keys before quantization;
  per query the bound sum_d max(q_d*kmin_d, q_d*kmax_d); keep the top-K_SEL
  blocks by bound plus the recent window and the attention-sink block;
  unselected blocks are skipped entirely.
* Section "All-KV-types composition": the fill reads the new, pre-quantization
  keys and min/max-merges into the block that straddles the append point or
  overwrites a fully new block; min/max being exact, this equals recomputing
  the bounds from scratch.
* Section "S2/S3 engineering design", item 2 and "Open questions": the GQA
  group is reduced to one block set per KV head by taking the max of the
  per-head bounds over the group.
* Section "Budget policy": fixed top-K plus recent/sink.

Readings taken where the page leaves a step open:
* The top-K is chosen among the blocks that are not already forced (sink and
  recent), so every KV head attends exactly min(NB, K_SEL + |forced|) blocks
  (the page's "OR" of top-K with the forced set is kept as
  ``forced_in_candidates=True``).  Parity unpinned: no page number decides it.
* Sink = the first ``n_sink`` blocks (the page names one sink block); the
  recent window counts whole blocks, the partial last block included.
* Exact ties at the cut-off go to the lower block index; candidates within
  1e-5 relative of the cut-off are reported as near-ties (parity unpinned:
  the width is ours).
"""
from __future__ import annotations

import math

import numpy as np

from .quant import f16_round_down, f16_round_up

NEAR_TIE_REL = 1e-5


def block_bounds(keys: np.ndarray, L: int, block: int):
    """Per-block channel min/max of the pre-quantization keys of one sequence.

    keys [Hkv][L][D], float16 (f16 cache: exact) or float32 (int8 cache:
    kmin rounded toward -inf, kmax toward +inf into float16).
    Returns (kmin, kmax) float16 [Hkv][NB][D], NB = ceil(L / block).

    A NaN key value is left out of its channel's min and max (reading taken;
    the page does not say): a channel whose keys in the block are all NaN
    gets kmin = +inf, kmax = -inf, so it can only lower the block's bound.
    """
    Hkv, _, D = keys.shape
    nb = -(-L // block)
    kmin = np.empty((Hkv, nb, D), dtype=keys.dtype)
    kmax = np.empty((Hkv, nb, D), dtype=keys.dtype)
    for j in range(nb):
        blk = keys[:, j * block:min((j + 1) * block, L), :]
        nan = np.isnan(blk)
        kmin[:, j] = np.where(nan, np.inf, blk).min(axis=1)
        kmax[:, j] = np.where(nan, -np.inf, blk).max(axis=1)
    if keys.dtype == np.float16:
        return kmin, kmax
    return f16_round_down(kmin), f16_round_up(kmax)


def upper_bounds(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """UB[h][j] = sum_d max(q[h,d]*kmin[g,j,d], q[h,d]*kmax[g,j,d]), g = h//G.

    A channel with q_d == 0 contributes 0 (reading taken: the page's max of
    two products would be 0 * inf = NaN for an infinite bound, which only an
    int8 cache with |key| > 65504 can produce).

    Every product of a float32 q and a float16 bound is exact in float64, and
    the sum is ``math.fsum`` (correctly rounded), so UB is the exact bound
    rounded once; correctly rounded sums are monotone, which makes
    UB >= fl(max_t q.k_t) hold with no tolerance.  Returns float64 [H][NB].
    """
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    Hkv, nb, _ = kmin.shape
    G = H // Hkv
    ub = np.empty((H, nb), dtype=np.float64)
    for h in range(H):
        g = h // G
        with np.errstate(invalid="ignore"):
            lo = kmin[g].astype(np.float64) * q[h]
            hi = kmax[g].astype(np.float64) * q[h]
            terms = np.where(q[h] == 0, 0.0, np.maximum(lo, hi))     # [NB][D]
        ub[h] = [math.fsum(row) for row in terms]
    return ub


def group_scores(ub: np.ndarray, Hkv: int) -> np.ndarray:
    """score[g][j] = max over the G query heads of group g of UB[h][j]."""
    H, nb = ub.shape
    G = H // Hkv
    return ub.reshape(Hkv, G, nb).max(axis=1)


def select_blocks(score: np.ndarray, n_blocks: int, k_sel: int, n_sink: int = 1,
                  n_recent: int = 2, forced_in_candidates: bool = False):
    """Fixed top-K block selection for one (sequence, KV head).

    score [>= n_blocks] (any float dtype; compared by value, so -0 == +0).
    Forced F = the first n_sink blocks and the last n_recent blocks.
    Candidates C = all blocks not in F (all blocks if forced_in_candidates).
    Chosen = the k_sel largest candidates, ties to the lower index (all of C
    if k_sel >= |C|).  Returns a dict with
      ``sel``      ascending int64 array of F u chosen,
      ``cutoff``   the k_sel-th largest candidate score (None if no cut),
      ``near``     candidates within NEAR_TIE_REL * |cutoff| of the cutoff.
    """
    nb = int(n_blocks)
    k_sel = max(0, int(k_sel))
    forced = set(range(min(max(n_sink, 0), nb))) | set(range(max(0, nb - max(n_recent, 0)), nb))
    if forced_in_candidates:
        cands = list(range(nb))
    else:
        cands = [j for j in range(nb) if j not in forced]
    s = [float(score[j]) for j in cands]
    cutoff = None
    near = []
    if k_sel >= len(cands):
        chosen = cands
    else:
        order = sorted(range(len(cands)), key=lambda i: (-s[i], cands[i]))
        chosen = [cands[i] for i in order[:k_sel]]
        if k_sel > 0:
            cutoff = s[order[k_sel - 1]]
            tol = NEAR_TIE_REL * abs(cutoff)
            near = [cands[i] for i in range(len(cands)) if abs(s[i] - cutoff) <= tol]
    sel = np.array(sorted(forced | set(chosen)), dtype=np.int64)
    return {"sel": sel, "cutoff": cutoff, "near": np.array(sorted(near), dtype=np.int64)}


def selected_tokens(sel: np.ndarray, L: int, block: int) -> np.ndarray:
    """Token positions of the selected blocks, the last block clipped at L."""
    if len(sel) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(j * block, min((j + 1) * block, L)) for j in sel])


# ------------------------------------------------------- per-query-head sets
# sparse_attn.md, "S2/S3 engineering design" item 2 and "Open questions":
# the GQA group can be reduced to one block set per KV head (the max rule
# above) or each query head can keep its own set ("per-Q-head mask
# divergence", which the group max avoids).  The per-head variant: head h
# ranks blocks by its own bound UB[h] and takes its own top-K plus the same
# forced blocks; it attends to exactly its own blocks.  Its KV head's blocks
# are read once for the group: the union of the G sets, each block tagged
# with the heads that chose it.

def select_blocks_per_head(ub: np.ndarray, n_blocks: int, k_sel: int, n_sink: int = 1,
                           n_recent: int = 2):
    """ub [G][>= n_blocks]: the bounds of one KV head's G query heads.
    Returns one select_blocks result per head (same rule, own scores)."""
    return [select_blocks(ub[i], n_blocks, k_sel, n_sink, n_recent) for i in range(ub.shape[0])]


def union_with_heads(sets):
    """sets: G ascending block arrays (one per query head of a KV head).
    Returns (union ascending int64 [U], mask int64 [U]) with bit i of
    mask[u] set iff head i's set holds union[u]."""
    allb = sorted(set().union(*[set(np.asarray(s).tolist()) for s in sets])) if sets else []
    union = np.array(allb, dtype=np.int64)
    mask = np.zeros(union.size, dtype=np.int64)
    pos = {b: u for u, b in enumerate(allb)}
    for i, s in enumerate(sets):
        for b in np.asarray(s).tolist():
            mask[pos[b]] |= 1 << i
    return union, mask
