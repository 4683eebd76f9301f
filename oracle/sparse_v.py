"""Sparse-V: within the attended tokens, leave out the value rows whose
softmax weight is negligible.  Computed from its definition in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: opencoti-llamafile sparse_attn.md -- "Compose (three sparsity
levers, three pipeline stages)", item 3 (inside the selected blocks, skip the
value work of positions whose post-softmax weight is negligible); "Stacking
with sparse-V" (a static threshold tau, to be retuned per configuration);
"Adaptive tau (the eps mode)" (a per-query threshold eps times the running
softmax denominator divided by the number of positions processed, so that the
dropped normalized mass stays below eps; eps = 0 falls back to the static
tau).

Readings taken where the page leaves a step open:
* The weight compared with the threshold is the normalized post-softmax
  weight p_t = exp(s_t - M) / sum_u exp(s_u - M) over every attended token of
  the query head (the page's kernel compares as it streams, against a running
  maximum and denominator; the whole-set values make the rule independent of
  the order and the split of the tokens).
* Static rule: keep t iff p_t >= tau.  Adaptive rule (eps > 0): keep t iff
  p_t >= eps / n, n the number of attended tokens -- the page's threshold
  eps * denominator / count, written for normalized weights.  Every dropped
  token then has p_t < eps / n, so the dropped mass is below eps.
* Only the value side is skipped: the normalizer keeps every token's weight,
  so out = sum over kept t of p_t v_t (the page skips the V dequantization
  and accumulation; the softmax sum is taken over all positions).
* tau = eps = 0 keeps every token (the dense result, bit for bit).
"""
from __future__ import annotations

import numpy as np

from .attention import _softmax_weights, int8_logit_dots
from .quant import dequantize_groups

NEAR_REL = 1e-4


def threshold(n: int, tau: float = 0.0, eps: float = 0.0) -> float:
    """The weight below which a token's value row is skipped."""
    if eps > 0.0:
        return float(eps) / max(int(n), 1)
    return float(tau)


def keep_mask(p: np.ndarray, tau: float = 0.0, eps: float = 0.0):
    """p: normalized weights of one head over its n attended tokens.  Returns
    (keep bool [n], near bool [n]); near marks weights within NEAR_REL of the
    threshold (a decision a float32 evaluation may take either way)."""
    th = threshold(p.size, tau, eps)
    keep = p >= th
    near = np.abs(p - th) <= NEAR_REL * th if th > 0 else np.zeros(p.size, bool)
    return keep, near


def _sparse_v_rows(logits: np.ndarray, vd: np.ndarray, tau: float, eps: float, keep=None):
    """One head: logits [n] float64, dequantized value rows [n][D] float64.
    Returns (out [D], keep [n], near [n], p [n])."""
    p = _softmax_weights(logits)
    k, near = keep_mask(p, tau, eps)
    if keep is not None:
        k = np.asarray(keep, bool)
    return (p * k) @ vd, k, near, p


def attend_f16_sparse_v(q, k, v, scale, tau=0.0, eps=0.0, tokens=None, keep=None):
    """Dense (or token-restricted) attention with sparse-V over an f16 cache.

    q [H][D] float32; k, v [Hkv][L][D]; tokens: optional attended positions.
    keep: optional [H][n] boolean decisions to use instead of the rule (to
    evaluate the output on another evaluation's decisions).  Returns
    (out [H][D] float64, keep [H][n], near [H][n]) over the attended tokens
    in ascending position order."""
    q = np.asarray(q, np.float64)
    H, D = q.shape
    Hkv = k.shape[0]
    G = H // Hkv
    idx = np.arange(k.shape[1]) if tokens is None else np.asarray(tokens)
    out = np.zeros((H, D))
    keeps = np.zeros((H, idx.size), bool)
    nears = np.zeros((H, idx.size), bool)
    if idx.size == 0:
        return out, keeps, nears
    for g in range(Hkv):
        kg = np.asarray(k[g][idx], np.float64)
        vg = np.asarray(v[g][idx], np.float64)
        hs = slice(g * G, (g + 1) * G)
        p = _softmax_weights((q[hs] @ kg.T) * np.float64(scale))        # [G][n]
        for i, h in enumerate(range(g * G, (g + 1) * G)):
            keeps[h], nears[h] = keep_mask(p[i], tau, eps)
        if keep is not None:
            keeps[hs] = np.asarray(keep, bool)[hs]
        out[hs] = (p * keeps[hs]) @ vg
    return out, keeps, nears


def attend_i8_sparse_v(q, k_codes, k_scale, v_codes, v_scale, scale, tau=0.0, eps=0.0,
                       tokens=None, keep=None):
    """The int8 method (exact integer q.k dots, see attention.attend_i8) with
    sparse-V.  Same returns as attend_f16_sparse_v."""
    H, D = q.shape
    Hkv = k_codes.shape[0]
    G = H // Hkv
    idx = np.arange(k_codes.shape[1]) if tokens is None else np.asarray(tokens)
    out = np.zeros((H, D))
    keeps = np.zeros((H, idx.size), bool)
    nears = np.zeros((H, idx.size), bool)
    if idx.size == 0:
        return out, keeps, nears
    dots, _, q_scale = int8_logit_dots(q, k_codes[:, idx])
    for g in range(Hkv):
        vd = v_codes[g, idx].astype(np.float64) * v_scale[g, idx].astype(np.float64)[:, None]
        ksg = k_scale[g, idx].astype(np.float64)
        for h in range(g * G, (g + 1) * G):
            s = dots[h].astype(np.float64) * np.float64(q_scale[h]) * ksg * np.float64(scale)
            out[h], keeps[h], nears[h], _ = _sparse_v_rows(
                s, vd, tau, eps, None if keep is None else keep[h])
    return out, keeps, nears


def attend_grouped_sparse_v(q, k_codes, k_scales, v_codes, v_scales, scale, tau=0.0, eps=0.0,
                            tokens=None, keep=None):
    """Sparse-V over a group-wise quantized cache (q8_0 / q4_0 / q5_0): the
    rule above on the dequantized keys and values scale * code (exact in
    float64), the query unquantized -- the group-wise attention's definition
    (attention.attend_grouped) with the value rows of negligible weight left
    out.  codes [Hkv][L][D] int8, scales [Hkv][L][D / 32] float16.  Same
    returns as attend_f16_sparse_v."""
    return attend_f16_sparse_v(q, dequantize_groups(k_codes, k_scales),
                               dequantize_groups(v_codes, v_scales), scale, tau, eps, tokens,
                               keep)
