"""Decode-step attention, computed from its definition in float64.

Sources:
* Definition: out_h = softmax(s) V with s_t = (q_h . k_t) * scale, one query
  token against every cached key of KV head g = h // (H // Hkv) (cpu-attn
  kernel card, section "Usage": GQA follows from shapes, query head h reads kv
  head h // (H // Hkv)).
* int8 method (cpu-attn kernel card, section "Method"): the logit of cached
  token s is the exact integer dot of the int8 query and key codes, times the
  query scale, the key scale of s and the softmax scale; the softmax is taken
  over those logits and the output sums softmax weight x value scale x value
  code over tokens.
* int8 contract reference (same card, sections "Correctness" and the
  introduction): float attention on the dequantized cache, which the kernel
  output must match within 8e-3 relative.
* Split-K combine: partial softmax states (max m, mass l, unnormalised
  numerator a) over disjoint token sets merge exactly after a common shift by
  the largest max, output = (sum of shifted numerators)/(sum of shifted
  masses).  The numerator/mass form is the one the SCSA guide states for its
  output (section "Mechanism", per-query step 4).
"""
from __future__ import annotations

import numpy as np

from .quant import dequantize_groups, quantize_rows


def _softmax_weights(s: np.ndarray) -> np.ndarray:
    """softmax along the last axis, float64, with max subtraction."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attend_f16(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
               tokens=None) -> np.ndarray:
    """Dense (or token-restricted) attention of one sequence.

    q [H][D] float32; k, v [Hkv][L][D] float16 (or any float); ``tokens`` an
    optional index array restricting the attended positions (Quest).  Returns
    [H][D] float64.  An empty token set gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    Hkv = k.shape[0]
    G = H // Hkv
    out = np.zeros((H, D), dtype=np.float64)
    for g in range(Hkv):
        kg = np.asarray(k[g], dtype=np.float64)
        vg = np.asarray(v[g], dtype=np.float64)
        if tokens is not None:
            kg = kg[tokens]
            vg = vg[tokens]
        if kg.shape[0] == 0:
            continue
        qg = q[g * G:(g + 1) * G]                       # [G][D]
        s = (qg @ kg.T) * np.float64(scale)             # [G][L]
        out[g * G:(g + 1) * G] = _softmax_weights(s) @ vg
    return out


def int8_logit_dots(q: np.ndarray, k_codes: np.ndarray):
    """Exact integer q.k dots of the int8 method.

    q [H][D] float32 is quantized per head (absmax rule); k_codes
    [Hkv][L][D] int8.  Returns (dots int64 [H][L], q_codes [H][D] int8,
    q_scale [H] float32).  |dot| <= 127*127*D, so for D <= 1024 the dot fits
    int32 and (D <= 128) is also exact in float32.
    """
    q_codes, q_scale = quantize_rows(q)
    H = q.shape[0]
    Hkv = k_codes.shape[0]
    G = H // Hkv
    dots = np.empty((H, k_codes.shape[1]), dtype=np.int64)
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        dots[hs] = (k_codes[g].astype(np.int64) @ q_codes[hs].astype(np.int64).T).T
    return dots, q_codes, q_scale


def attend_i8(q, k_codes, k_scale, v_codes, v_scale, scale, tokens=None):
    """The int8 method, exact up to float64 rounding.

    logit_t = dot_t * q_scale * k_scale[t] * scale (float64),
    out_d = sum_t softmax(logit)_t * v_scale[t] * v_code[t, d].
    q [H][D] f32; codes [Hkv][L][D] int8; scales [Hkv][L] f32.  Returns [H][D]
    float64.
    """
    H, D = q.shape
    Hkv = k_codes.shape[0]
    G = H // Hkv
    idx = np.arange(k_codes.shape[1]) if tokens is None else np.asarray(tokens)
    out = np.zeros((H, D), dtype=np.float64)
    if idx.size == 0:
        return out
    dots, _, q_scale = int8_logit_dots(q, k_codes[:, idx])
    for g in range(Hkv):
        vd = v_codes[g, idx].astype(np.float64) * v_scale[g, idx].astype(np.float64)[:, None]
        ksg = k_scale[g, idx].astype(np.float64)
        for h in range(g * G, (g + 1) * G):
            logit = (dots[h].astype(np.float64) * np.float64(q_scale[h]) * ksg
                     * np.float64(scale))
            out[h] = _softmax_weights(logit) @ vd
    return out


def attend_i8_dequant(q, k_codes, k_scale, v_codes, v_scale, scale, tokens=None):
    """Float attention on the dequantized int8 cache with the unquantized query:
    the reference the int8 output must match within 8e-3 relative.  Dequantized
    values code * scale are exact in float64."""
    kd = k_codes.astype(np.float64) * k_scale.astype(np.float64)[..., None]
    vd = v_codes.astype(np.float64) * v_scale.astype(np.float64)[..., None]
    return attend_f16(q, kd, vd, scale, tokens)


def softmax_partials(q_h: np.ndarray, k_g: np.ndarray, v_g: np.ndarray, scale: float,
                     token_sets, base: float = 2.0):
    """Partial softmax states of one head over disjoint token sets.

    For each set T: m = max_{t in T} s_t, l = sum_t base^(s_t - m),
    a = sum_t base^(s_t - m) v_t, with s_t = (q.k_t) * scale * log_base(e)
    (so that base^s equals e^(q.k*scale)).  An empty set gives m = -inf,
    l = 0, a = 0.  Used to test the combine step on its own.
    """
    q_h = np.asarray(q_h, dtype=np.float64)
    conv = 1.0 / np.log(base)
    ms, ls, as_ = [], [], []
    for T in token_sets:
        T = np.asarray(T, dtype=np.int64)
        if T.size == 0:
            ms.append(-np.inf); ls.append(0.0); as_.append(np.zeros(k_g.shape[-1]))
            continue
        s = (np.asarray(k_g[T], np.float64) @ q_h) * np.float64(scale) * conv
        m = np.max(s)
        w = np.power(base, s - m)
        ms.append(m); ls.append(np.sum(w)); as_.append(w @ np.asarray(v_g[T], np.float64))
    return np.array(ms), np.array(ls), np.stack(as_)


def combine_partials(m: np.ndarray, l: np.ndarray, a: np.ndarray, base: float = 2.0):
    """Merge partial softmax states: M = max_i m_i, out = sum_i base^(m_i-M) a_i
    / sum_i base^(m_i-M) l_i, skipping empty partials (m = -inf).  All partials
    empty gives zeros.  m, l [n]; a [n][D]."""
    m = np.asarray(m, dtype=np.float64)
    live = np.isfinite(m) & (np.asarray(l) > 0)
    if not np.any(live):
        return np.zeros(a.shape[-1], dtype=np.float64)
    M = np.max(m[live])
    w = np.power(base, m[live] - M)
    return (w @ np.asarray(a, np.float64)[live]) / np.sum(w * np.asarray(l, np.float64)[live])


def attend_grouped(q, k_codes, k_scales, v_codes, v_scales, scale, tokens=None):
    """Attention over a group-wise quantized cache (q8_0 / q4_0 / q5_0): the
    definition applied to the dequantized values scale * code (exact in
    float64), the query unquantized.  codes [Hkv][L][D] int8, scales
    [Hkv][L][D / 32] float16.  Returns [H][D] float64."""
    kd = dequantize_groups(k_codes, k_scales)
    vd = dequantize_groups(v_codes, v_scales)
    return attend_f16(q, kd, vd, scale, tokens)
