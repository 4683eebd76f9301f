"""Quantization and rounding steps of the method, emulated exactly in float32.

Sources:
* cpu-attn kernel card (phanerozoic/cpu-attn), section "Method": K and V are
  quantized per token and per head with an absmax int8 rule at append time;
  section "Requirements and limits": per-token per-head absmax only.
* The same card's logit formula uses a quantized query (``q_i8``, ``q_scale``);
  it does not say how q is quantized.  Reading taken: the same per-row absmax
  rule, one scale per query head.
* opencoti-llamafile sparse_attn.md, section "Method: Quest-style min/max block
  bounds": the side cache stores kmin/kmax as f16.  When the pre-quantization
  keys are float32 (int8 cache), the reading taken is: round kmin toward -inf
  and kmax toward +inf so the stored envelope still contains every key.
"""
from __future__ import annotations

import numpy as np

QMAX = 127  # symmetric int8 range [-127, 127]


def quantize_rows(x: np.ndarray):
    """Absmax int8 quantization of each row (last axis) of a float32 array.

    For a row x: a = max_d |x_d| (exact); if a == 0 the scale is 0 and all
    codes are 0; otherwise scale = fl32(a / 127) and
    code_d = clamp(rint(fl32(x_d / scale)), -127, 127), rint rounding half to
    even.  Returns (codes int8 [..., D], scales float32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)                       # float32, exact
    scale = (a / np.float32(QMAX)).astype(np.float32)    # correctly rounded fl32 division
    safe = np.where(scale == 0, np.float32(1), scale).astype(np.float32)
    r = np.rint((x / safe[..., None]).astype(np.float32))
    r = np.clip(r, -QMAX, QMAX)
    r = np.where((scale == 0)[..., None], 0, r)
    return r.astype(np.int8), scale.astype(np.float32)


def f16_round_down(x: np.ndarray) -> np.ndarray:
    """Largest float16 value <= x (x float32).  Values below -65504 become -inf."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        r = x.astype(np.float16)                          # round to nearest even
        too_big = r.astype(np.float32) > x
        r = np.where(too_big, np.nextafter(r, np.float16(-np.inf)), r)
    return r.astype(np.float16)


def f16_round_up(x: np.ndarray) -> np.ndarray:
    """Smallest float16 value >= x (x float32).  Values above 65504 become +inf."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        r = x.astype(np.float16)
        too_small = r.astype(np.float32) < x
        r = np.where(too_small, np.nextafter(r, np.float16(np.inf)), r)
    return r.astype(np.float16)


# --------------------------------------------------- group-wise quantization
# opencoti-llamafile sparse_attn.md, "All-KV-types composition" and "Open
# questions": quantized caches (q8_0, q4_0) hold blocks of 32 values with a
# scale each (the quant block size, blck = 32), and the side cache is filled
# from the keys before quantization.  The cpu-attn card ("Requirements and
# limits") contrasts its per-token absmax with such group-wise scaling within
# a row.  Readings taken (the pages name the formats, not their arithmetic):
# * a group is 32 consecutive channels of one (token, KV head) row;
# * symmetric absmax per group, the int8 card's rule with QMAX levels each
#   side: q8_0 QMAX = 127, q4_0 QMAX = 7 (codes -7..7, stored as a nibble),
#   q5_0 QMAX = 15 (codes -15..15, five bits stored; sparse_attn.md names
#   q5_0 with q4_0 as the quantized caches the bounds compose with, "Method:
#   Quest-style min/max block bounds", and gives their block size 32, "Open
#   questions");
# * the scale is stored as f16: s = fl16(fl32(a / QMAX)); the codes are taken
#   against that stored scale, code = clamp(rint(fl32(x / s)), -QMAX, QMAX),
#   so a value is represented exactly as s * code; s == 0 (a zero group, or
#   a scale below f16's range) gives codes 0; a scale beyond f16's range
#   (|x| above 65504 * QMAX) rounds to inf and gives codes 0 as well.

GROUP = 32
QMAX_Q8 = 127
QMAX_Q4 = 7
QMAX_Q5 = 15


def quantize_groups(x: np.ndarray, qmax: int):
    """Group-wise absmax quantization of the last axis (a multiple of 32).

    x float32 [..., D].  Returns (codes int8 [..., D], scales float16
    [..., D / 32])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    assert D % GROUP == 0
    g = x.reshape(x.shape[:-1] + (D // GROUP, GROUP))
    a = np.max(np.abs(g), axis=-1)                                   # float32, exact
    with np.errstate(over="ignore"):
        s16 = (a / np.float32(qmax)).astype(np.float32).astype(np.float16)   # RNE to f16
    s = s16.astype(np.float32)
    ok = (s != 0) & np.isfinite(s)
    safe = np.where(ok, s, np.float32(1)).astype(np.float32)
    r = np.rint((g / safe[..., None]).astype(np.float32))
    r = np.clip(r, -qmax, qmax)
    r = np.where(ok[..., None], r, 0)
    return r.astype(np.int8).reshape(x.shape), s16


def dequantize_groups(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes int8 [..., D], scales float16 [..., D / 32] -> float64 values
    scale * code (exact in float64)."""
    D = codes.shape[-1]
    c = codes.astype(np.float64).reshape(codes.shape[:-1] + (D // GROUP, GROUP))
    return (c * scales.astype(np.float64)[..., None]).reshape(codes.shape)
