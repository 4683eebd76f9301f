// Device-side helpers shared by the gfx950 kernels: cross-lane reductions on
// 64-wide wavefronts, f16 bit handling, directed f32 -> f16 rounding, the
// absmax int8 row quantizer and order-preserving radix keys.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace skv {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------- XCD-aware placement
// The dispatcher hands the workgroups of a launch to the 8 XCDs in turn by
// linear id, and each XCD has its own L2.  xcd_slot renumbers a 1-D grid so
// that every XCD runs one contiguous range of work items ("slots"): a kernel
// that lays out its work row by row then keeps each row on one XCD (or on
// consecutive XCDs for rows larger than a range), the same XCD for every
// kernel of a step that uses this layout, so a consumer kernel finds its
// producer's lines (scores, partial states) in its own L2.  A bijection of
// [0, n) for any n; on a part with another XCD count it is just a
// permutation.
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t xcd_slot(uint32_t id, uint32_t n) {
  const uint32_t x = id % kXcds, k = id / kXcds, q = n / kXcds, rem = n % kXcds;
  return x * q + min(x, rem) + k;
}
// Row of the r-th row-sized range of slots.  With more rows than XCDs (a
// multiple of their count), XCD x takes rows x, x + 8, x + 16, ... rather than
// a run of consecutive rows, so every XCD gets the same KV head of every
// sequence and sequences of different lengths spread evenly over the XCDs.
__device__ __forceinline__ uint32_t xcd_row(uint32_t r, uint32_t rows) {
  if (rows <= kXcds || rows % kXcds != 0) return r;
  const uint32_t per = rows / kXcds;
  return (r % per) * kXcds + r / per;
}

// ---------------------------------------------------------------- DPP lanes
// DPP control codes (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over an aligned group of 8 lanes; every lane of the group gets the same
// bits (each step combines a lane with its mirror, a commutative op).
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp_f<kDppQuadXor1>(x);
  x += dpp_f<kDppQuadXor2>(x);
  x += dpp_f<kDppRowHalfMirror>(x);
  return x;
}
// Sum over aligned groups of 16 lanes (one DPP row).
__device__ __forceinline__ float group16_sum(float x) {
  x = group8_sum(x);
  x += dpp_f<kDppRowMirror>(x);
  return x;
}
// Max over aligned groups of 16 lanes (one DPP row); same bits in every lane.
__device__ __forceinline__ float group16_max(float x) {
  x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppRowMirror>(x));
  return x;
}


// ------------------------------------------------------- across the 4 rows
// gfx950 lane swaps (verified lane maps): permlane16_swap(x, x) returns, in
// every lane, the values of its row pair {row 2i, row 2i+1} as (row 2i,
// row 2i+1); permlane32_swap(x, x) returns (lower half, upper half).  So
// op(first, second) is the same bits in all lanes of the pair, and two steps
// reduce lanes l, l ^ 16, l ^ 32, l ^ 48 with VALU instructions only.
__device__ __forceinline__ uint32_t rows_pair_lo(uint32_t x, uint32_t& hi) {
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  hi = p[1];
  return p[0];
}
__device__ __forceinline__ uint32_t halves_lo(uint32_t x, uint32_t& hi) {
  const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  hi = p[1];
  return p[0];
}
__device__ __forceinline__ float rows_max(float x) {
  uint32_t h;
  float l = __uint_as_float(rows_pair_lo(__float_as_uint(x), h));
  x = fmaxf(l, __uint_as_float(h));
  l = __uint_as_float(halves_lo(__float_as_uint(x), h));
  return fmaxf(l, __uint_as_float(h));
}
__device__ __forceinline__ float rows_sum(float x) {
  uint32_t h;
  float l = __uint_as_float(rows_pair_lo(__float_as_uint(x), h));
  x = l + __uint_as_float(h);
  l = __uint_as_float(halves_lo(__float_as_uint(x), h));
  return l + __uint_as_float(h);
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppRowMirror>(x));
  return rows_max(x);
}

// ------------------------------------------------------ wavefront integers
// Inclusive prefix sum over the 64 lanes: DPP row shifts by 1, 2, 4, 8 scan
// each row of 16, then the row-15 and row-31 broadcasts carry the row totals
// into the rows above (verified on gfx950).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}
// AND / OR over the 64 lanes (every lane gets the result).
__device__ __forceinline__ uint32_t wave_and(uint32_t x) {
  x &= uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kDppQuadXor1, 0xF, 0xF, false));
  x &= uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kDppQuadXor2, 0xF, 0xF, false));
  x &= uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kDppRowHalfMirror, 0xF, 0xF, false));
  x &= uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kDppRowMirror, 0xF, 0xF, false));
  uint32_t h;
  x = rows_pair_lo(x, h) & h;
  x = halves_lo(x, h) & h;
  return x;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
  x |= uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kDppQuadXor1, 0xF, 0xF, false));
  x |= uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kDppQuadXor2, 0xF, 0xF, false));
  x |= uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kDppRowHalfMirror, 0xF, 0xF, false));
  x |= uint32_t(__builtin_amdgcn_update_dpp(0, int(x), kDppRowMirror, 0xF, 0xF, false));
  uint32_t h;
  x = rows_pair_lo(x, h) | h;
  x = halves_lo(x, h) | h;
  return x;
}

// ---------------------------------------------------------------- f16 bits
__device__ __forceinline__ float h2f(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}
__device__ __forceinline__ float h2f_lo(uint32_t w) { return h2f(uint16_t(w & 0xFFFFu)); }
__device__ __forceinline__ float h2f_hi(uint32_t w) { return h2f(uint16_t(w >> 16)); }

// Next f16 toward -inf / +inf of a non-NaN bit pattern.
__device__ __forceinline__ uint16_t f16_next_down(uint16_t u) {
  if ((u & 0x7FFFu) == 0) return 0x8001u;          // +-0 -> smallest negative subnormal
  return (u & 0x8000u) ? uint16_t(u + 1) : uint16_t(u - 1);
}
__device__ __forceinline__ uint16_t f16_next_up(uint16_t u) {
  if ((u & 0x7FFFu) == 0) return 0x0001u;
  return (u & 0x8000u) ? uint16_t(u - 1) : uint16_t(u + 1);
}
// Largest f16 <= x and smallest f16 >= x (x finite float32 or +-inf).
__device__ __forceinline__ uint16_t f32_to_f16_down(float x) {
  uint16_t r = __half_as_ushort(__float2half_rn(x));
  return (h2f(r) > x) ? f16_next_down(r) : r;
}
__device__ __forceinline__ uint16_t f32_to_f16_up(float x) {
  uint16_t r = __half_as_ushort(__float2half_rn(x));
  return (h2f(r) < x) ? f16_next_up(r) : r;
}
__device__ __forceinline__ uint16_t f16_min_bits(uint16_t a, uint16_t b) {
  return h2f(a) <= h2f(b) ? a : b;
}
__device__ __forceinline__ uint16_t f16_max_bits(uint16_t a, uint16_t b) {
  return h2f(a) >= h2f(b) ? a : b;
}

// ------------------------------------------------------- absmax int8 quant
// scale = a / 127 and x / scale are IEEE correctly rounded float32 divisions
// (this code is built without fast-math), rintf rounds half to even.
__device__ __forceinline__ float absmax_scale(float a) { return a / 127.0f; }
__device__ __forceinline__ int quant_code(float x, float scale) {
  if (scale == 0.0f) return 0;
  float r = rintf(x / scale);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return int(r);
}
// quant_code(x, scale) through inv = 1 / scale (correctly rounded).  For
// |x / scale| <= 128, y = x * inv carries two relative roundings of 2^-24, so
// it lies within 2^-16 of x / scale, and the correctly rounded quotient within
// 2^-17: the two are less than 2^-15 apart and round to the same integer
// unless |y| is within 2^-14 of a half-integer.  Such a value (and any
// non-finite y, e.g. a zero or subnormal scale) sets `exact`: the caller then
// takes quant_code for it.
__device__ __forceinline__ int quant_code_recip(float x, float inv, bool& exact) {
  const float y = x * inv;
  const float ay = fabsf(y);
  exact = !(fabsf(ay - floorf(ay) - 0.5f) > 0x1p-14f);
  const float r = fminf(fmaxf(rintf(y), -127.0f), 127.0f);
  return int(r);
}

// ------------------------------------------------------ radix select keys
// Order-preserving map float32 -> uint32 (larger float -> larger key), with
// -0 canonicalized to +0 so that the two compare equal.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace skv
