"""A 4-bit key index scanned once per GQA group, with deterministic score
bounds: a token-level candidate generator.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Certified Sparse Attention via Perturbed Retrieval" -- the abstract
(a 4-bit scan with deterministic bounds, shared across a grouped-query-
attention group, generates the candidates exactly but reads every key), the
appendix layout table (4-bit codes, 64 B per token at D = 128, read for every
token; per-block, per-channel fp32 scales lo and step) and the ablation table
(scanning per query head instead of per group reads 2.7-4.0x the bytes).  The
certificate, the perturbations and the sampling built on top of the scan are
another method and are not part of this.

Readings taken where the page leaves a step open:
* Per block of ``block`` consecutive tokens and per channel d: lo = min_t
  k_td, step = fl32(fl32(max_t k_td - lo) / 15), code = clamp(rint(fl32(
  fl32(k - lo) / step)), 0, 15) (0 when step == 0); the reconstruction is
  fl32(lo + fl32(step * code)) and err = max_t |fl32(k - recon)| is recorded per
  (block, channel), so |k_td - recon_td| <= err_d holds by construction (the
  page's bounds are "deterministic"; how it bounds is not printed).  All
  float32 steps are single IEEE operations (no fused multiply-add).
* For a query q and token t of block b: s~ = sum_d q_d recon_td, r = sum_d
  |q_d| err_bd, LB = s~ - r <= q.k_t <= UB = s~ + r.
* For an int8 or group-wise (q8_0 / q4_0 / q5_0) cache the index is built
  from the keys the cache holds, code x scale, each one float32 product
  (``cache_keys``): exact for the group-wise formats (a code of at most 8
  bits times an f16 scale fits in float32), correctly rounded for int8 (a
  float32 scale).
* Candidates of a query head for a margin delta >= 0 (in q.k units): every
  token whose exact q.k could be within delta of the largest,
  C = {t : UB_t >= max_u LB_u - delta}.  It contains {t : q.k_t >= max_u q.k_u
  - delta} (UB_t >= q.k_t >= max q.k - delta >= max LB - delta).
"""
from __future__ import annotations

import math

import numpy as np

LEVELS = 15
NEAR_REL = 1e-5


def cache_keys(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The keys a quantized cache holds, as float32: codes int8 [..., L, D];
    scales float32 [..., L] (int8, one per token) or float16 [..., L, D / 32]
    (group-wise, one per 32 channels).  Each value is one float32 product
    code * scale."""
    c = np.asarray(codes).astype(np.float32)
    sc = np.asarray(scales)
    if sc.ndim == c.ndim - 1:
        s = sc.astype(np.float32)[..., None]
    else:
        s = np.repeat(sc.astype(np.float32), 32, axis=-1)
    return (c * s).astype(np.float32)


def build_index(keys: np.ndarray, L: int, block: int):
    """keys [Hkv][L][D] (float16 or float32).  Returns (codes uint8
    [Hkv][L][D] in 0..15, lo, step, err float32 [Hkv][NB][D])."""
    k = np.asarray(keys[:, :L], dtype=np.float32)
    Hkv, _, D = k.shape
    nb = -(-L // block)
    codes = np.zeros((Hkv, L, D), np.uint8)
    lo = np.zeros((Hkv, nb, D), np.float32)
    step = np.zeros((Hkv, nb, D), np.float32)
    err = np.zeros((Hkv, nb, D), np.float32)
    for j in range(nb):
        blk = k[:, j * block:min((j + 1) * block, L)]
        mn = blk.min(axis=1)
        mx = blk.max(axis=1)
        st = ((mx - mn) / np.float32(LEVELS)).astype(np.float32)
        safe = np.where(st > 0, st, np.float32(1)).astype(np.float32)
        c = np.rint(((blk - mn[:, None]) / safe[:, None]).astype(np.float32))
        c = np.clip(c, 0, LEVELS)
        c = np.where((st > 0)[:, None], c, 0).astype(np.float32)
        rec = (mn[:, None] + (st[:, None] * c).astype(np.float32)).astype(np.float32)
        e = np.abs((blk - rec).astype(np.float32)).max(axis=1)
        codes[:, j * block:min((j + 1) * block, L)] = c.astype(np.uint8)
        lo[:, j], step[:, j], err[:, j] = mn, st, e
    return codes, lo, step, err


def reconstruct(codes, lo, step, block):
    """Float32 reconstruction lo + step * code of every indexed token."""
    Hkv, L, D = codes.shape
    j = np.arange(L) // block
    return (lo[:, j] + (step[:, j] * codes.astype(np.float32)).astype(np.float32)).astype(
        np.float32)


def scan_bounds(q: np.ndarray, codes, lo, step, err, block):
    """q [H][D] float32 (H = G x Hkv).  Returns (LB, UB) float64 [H][L]:
    sum_d q_d recon_td -/+ sum_d |q_d| err_bd, each sum correctly rounded
    (math.fsum of exact float64 products)."""
    q = np.asarray(q, np.float64)
    H, D = q.shape
    Hkv, L, _ = codes.shape
    G = H // Hkv
    rec = reconstruct(codes, lo, step, block).astype(np.float64)
    jb = np.arange(L) // block
    lb = np.empty((H, L))
    ub = np.empty((H, L))
    for h in range(H):
        g = h // G
        prod = rec[g] * q[h]                                          # exact in float64
        rad = err[g].astype(np.float64) * np.abs(q[h])                # [NB][D]
        r_blk = np.array([math.fsum(row) for row in rad])
        for t in range(L):
            s = math.fsum(prod[t])
            lb[h, t] = s - r_blk[jb[t]]
            ub[h, t] = s + r_blk[jb[t]]
    return lb, ub


def candidates(lb: np.ndarray, ub: np.ndarray, delta: float):
    """One head: C = {t : UB_t >= max LB - delta} as a bool mask, and the
    tokens within NEAR_REL of that threshold (a float32 evaluation may decide
    them either way)."""
    th = float(np.max(lb)) - float(delta)
    cand = ub >= th
    near = np.abs(ub - th) <= NEAR_REL * max(abs(th), 1.0)
    return cand, near, th


def scan_bounds_f64(q: np.ndarray, codes, lo, step, err, block):
    """scan_bounds with the sums taken as float64 products (BLAS order)
    instead of correctly rounded: within about 1e-13 relative of them, for
    inputs where the per-token Python sums would take minutes."""
    q = np.asarray(q, np.float64)
    H, D = q.shape
    Hkv, L, _ = codes.shape
    G = H // Hkv
    rec = reconstruct(codes, lo, step, block).astype(np.float64)
    jb = np.arange(L) // block
    lb = np.empty((H, L))
    ub = np.empty((H, L))
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        s = q[hs] @ rec[g].T                                          # [G][L]
        r = (np.abs(q[hs]) @ err[g].astype(np.float64).T)[:, jb]      # [G][L]
        lb[hs] = s - r
        ub[hs] = s + r
    return lb, ub
