"""Multi-token queries: a chunk of T consecutive query tokens per sequence (a
chunked prefill, or a run of draft tokens to verify), each attending causally
to the cache, densely or through its own Quest block set.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: opencoti-llamafile sparse_attn.md, "S2/S3 engineering design" item 2
and "Open questions (resolve during impl)": the block selector is built for
the decode path first; a selector for the prefill path, where one call carries
many query tokens, is named there as a later stage without its rule.

Readings taken where the page leaves the rule open:
* The chunk's T tokens are the last T positions of the sequence: with L the
  sequence length (the chunk included), token t sits at position L - T + t and
  attends to the positions [0, L_t), L_t = L - T + 1 + t (causal); a token
  with L_t <= 0 attends to nothing (zeros).
* Each token is a decode query in its own right.  Dense: attention over its
  prefix.  Quest: its own upper bounds and group max over its G heads, its
  own top-K with the sink and the recent window counted over its own
  NB_t = ceil(L_t / block) blocks, attention over its own selected blocks
  with the last one clipped at L_t.
* The bounds are those of the side cache after the whole chunk is appended:
  a block may hold positions past L_t, so a token's bound covers a superset of
  the keys it sees and stays sound for them.
* A KV head's blocks are read once for the chunk: the ascending union of the
  T tokens' sets, each block tagged with the tokens that chose it.
"""
from __future__ import annotations

import numpy as np

from .attention import attend_f16, attend_i8
from .quest import group_scores, select_blocks, selected_tokens, upper_bounds


def token_lengths(L: int, T: int) -> np.ndarray:
    """L_t = L - T + 1 + t for t < T, floored at 0."""
    return np.array([max(int(L) - int(T) + 1 + t, 0) for t in range(int(T))], dtype=np.int64)


def attend_f16_multi(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, L: int):
    """q [T][H][D]; k, v [Hkv][>= L][D].  Token t attends densely to [0, L_t).
    Returns [T][H][D] float64."""
    T = q.shape[0]
    lens = token_lengths(L, T)
    return np.stack([attend_f16(q[t], k[:, :lens[t]], v[:, :lens[t]], scale)
                     for t in range(T)])


def attend_i8_multi(q, k_codes, k_scale, v_codes, v_scale, scale: float, L: int):
    """The int8 method for each token over its prefix (its own query codes and
    scale per head).  Returns [T][H][D] float64."""
    T = q.shape[0]
    lens = token_lengths(L, T)
    return np.stack([attend_i8(q[t], k_codes[:, :lens[t]], k_scale[:, :lens[t]],
                               v_codes[:, :lens[t]], v_scale[:, :lens[t]], scale)
                     for t in range(T)])


def select_multi(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray, L: int, block: int,
                 k_sel: int, n_sink: int = 1, n_recent: int = 2):
    """Each token's Quest selection.  q [T][H][D]; kmin, kmax [Hkv][NB][D] (the
    side cache of all L tokens).  Returns (scores, sels): scores[t] float64
    [Hkv][NB_t] (the group max of the token's bounds over its own blocks) and
    sels[t][g] the select_blocks result of token t and KV head g."""
    T = q.shape[0]
    Hkv = kmin.shape[0]
    lens = token_lengths(L, T)
    scores, sels = [], []
    for t in range(T):
        nb_t = -(-int(lens[t]) // block)
        ub = upper_bounds(q[t], kmin[:, :nb_t], kmax[:, :nb_t])
        sc = group_scores(ub, Hkv)
        scores.append(sc)
        sels.append([select_blocks(sc[g], nb_t, k_sel, n_sink, n_recent) for g in range(Hkv)])
    return scores, sels


def union_tokens(sets):
    """sets: the T tokens' ascending block arrays of one KV head.  Returns
    (union ascending int64 [U], mask int64 [U]): bit t of mask[u] set iff
    token t's set holds union[u]."""
    allb = sorted(set().union(*[set(np.asarray(s).tolist()) for s in sets])) if sets else []
    union = np.array(allb, dtype=np.int64)
    mask = np.zeros(union.size, dtype=np.int64)
    pos = {b: u for u, b in enumerate(allb)}
    for t, s in enumerate(sets):
        for b in np.asarray(s).tolist():
            mask[pos[b]] |= 1 << t
    return union, mask


def attend_f16_quest_multi(q, k, v, scale: float, L: int, sels, block: int):
    """Token t, KV head g: attention of the G heads of g over the tokens of
    sels[t][g] (ascending block indices) clipped at L_t.  Returns [T][H][D]."""
    T, H, D = q.shape
    Hkv = k.shape[0]
    G = H // Hkv
    lens = token_lengths(L, T)
    out = np.zeros((T, H, D), dtype=np.float64)
    for t in range(T):
        for g in range(Hkv):
            toks = selected_tokens(np.asarray(sels[t][g]), int(lens[t]), block)
            out[t, g * G:(g + 1) * G] = attend_f16(q[t, g * G:(g + 1) * G], k[g:g + 1],
                                                   v[g:g + 1], scale, toks)
    return out


def attend_i8_quest_multi(q, k_codes, k_scale, v_codes, v_scale, scale: float, L: int,
                          sels, block: int):
    """The int8 method per token and KV head over its selected blocks."""
    T, H, D = q.shape
    Hkv = k_codes.shape[0]
    G = H // Hkv
    lens = token_lengths(L, T)
    out = np.zeros((T, H, D), dtype=np.float64)
    for t in range(T):
        for g in range(Hkv):
            toks = selected_tokens(np.asarray(sels[t][g]), int(lens[t]), block)
            out[t, g * G:(g + 1) * G] = attend_i8(
                q[t, g * G:(g + 1) * G], k_codes[g:g + 1], k_scale[g:g + 1],
                v_codes[g:g + 1], v_scale[g:g + 1], scale, toks)
    return out
