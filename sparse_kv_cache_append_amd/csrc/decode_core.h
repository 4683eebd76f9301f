// Shared pieces of the attention kernels (decode_kernels.h, sparse_v.hip,
// decode_grouped.hip):
// vector types, the 16-byte tile loads through per-tile buffer resources, the
// MFMA wrappers, the wave-uniform tile walk over a part's blocks (or its
// share of a selected list) and the exact int8 -> f16 widening of V codes.
// Included by the .hip sources only; everything here has internal linkage.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"

namespace skv {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));
#define SKV_LDS __attribute__((address_space(3)))

constexpr int kMWaves = 4;
constexpr int kMThreads = kMWaves * kWave;
constexpr int kD = 128;                // the head dimension every feature supports
constexpr int kRowBytesF16 = kD * 2;   // 256
constexpr int kRowBytesI8 = kD;        // 128

__device__ __forceinline__ int swz(int row) { return row & 15; }

// A full tile (4 KiB of K or V rows) as a raw buffer: the resource is built
// in scalar registers from the tile's first byte, the lane's 16-byte offset
// is loop-invariant and the row step is the instruction's immediate offset,
// so a tile's loads need no vector address arithmetic.  Records = the tile's
// bytes (the range check keeps every access inside it); word 3 is the plain
// untyped-buffer configuration of the CDNA resource descriptor.  aux = 2 is
// the nontemporal hint (each K/V byte is read once per step).
constexpr int kTileRsrcBytes = 4096;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kAuxNontemporal = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* t,
                                                           int bytes = kTileRsrcBytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(t), (short)0, bytes,
                                           kRsrcWord3);
}
__device__ __forceinline__ int4_t tile_load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0,
                                                                         kAuxNontemporal));
}

// Every refill of a tile fragment issues the same number of loads, also
// when the walk is over: then through a resource of zero records, which
// returns zeros and touches no memory.  The hardware load counter completes
// in order, and a path that issued fewer loads (a conditional refill) makes
// the compiler's wait at the next join conservative: the wave would then
// wait for every tile in flight, the one two steps ahead included, at each
// turn of the loop.

__device__ __forceinline__ float4_t mfma_f16_32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma_f16_16(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Tile walk of one wavefront: tiles w, w + kMWaves, ... of the part's
// sequence of T-row tiles (each block holds block / T tiles).
struct TileWalk {
  const int32_t* sel;
  int32_t jl, u0, n_units, tpb, block, L, nb;
  int32_t unit, sub;
  // per-query-head lists: the row's head mask per list entry (bit i: query
  // head i of the group chose the entry's block), lane i holding entry u0 + i
  const uint32_t* hsel = nullptr;
  uint32_t hl = ~0u;

  __device__ __forceinline__ void init(int w) {
    unit = w / tpb;
    sub = w - unit * tpb;
  }
  __device__ __forceinline__ bool more() const { return unit < n_units; }
  // tiles left in this wavefront's walk (it takes every kMWaves-th tile)
  __device__ __forceinline__ int32_t count() const {
    const int32_t left = (n_units - unit) * tpb - sub;
    return left > 0 ? (left + kMWaves - 1) / kMWaves : 0;
  }
  // first row and valid-row count of the current tile, then advance by kMWaves tiles
  // (the walk state is wave-uniform: it lives in scalar registers)
  // (HM: also the head mask of the tile's list entry)
  template <int T, bool HM = false>
  __device__ __forceinline__ void next(int32_t& r0, int32_t& nvalid, uint32_t* hm = nullptr) {
    int32_t j = u0 + unit;
    if constexpr (HM)
      *hm = unit < kWave ? uint32_t(__builtin_amdgcn_readlane(int32_t(hl), unit))
                         : uint32_t(__builtin_amdgcn_readfirstlane(int32_t(hsel[j])));
    if (sel != nullptr)
      j = unit < kWave ? __builtin_amdgcn_readlane(jl, unit)
                       : __builtin_amdgcn_readfirstlane(sel[j]);
    if (j < 0 || j >= nb) {
      r0 = 0;
      nvalid = 0;
    } else {
      r0 = j * block + sub * T;
      nvalid = __builtin_amdgcn_readfirstlane(min(min(T, block - sub * T), L - r0));
    }
    sub += kMWaves;
    while (sub >= tpb) { sub -= tpb; ++unit; }
  }
};

// A given list's count and this part's entries (lane i: entry u0 + i), requested
// at kernel entry together with the row length and the query, so the first
// tile loads wait for one round trip only.  Entries past the count are
// ignored through n_units.
struct ListSeed {
  int32_t cnt, jl;
  uint32_t hl;
};
__device__ __forceinline__ ListSeed list_seed(const int32_t* sel_idx, const int32_t* sel_cnt,
                                              int32_t max_sel, int64_t bg, int32_t split,
                                              int32_t units_per_split,
                                              const uint32_t* sel_hmask = nullptr) {
  ListSeed ls{0, -1, ~0u};
  if (sel_idx != nullptr) {
    const int lane = threadIdx.x % kWave;
    const int32_t e = split * units_per_split + lane;
    ls.cnt = sel_cnt[bg];
    if (lane < units_per_split && e < max_sel) {
      ls.jl = sel_idx[bg * max_sel + e];
      if (sel_hmask != nullptr) ls.hl = sel_hmask[bg * max_sel + e];
    }
  }
  return ls;
}

template <int T>
__device__ __forceinline__ TileWalk make_walk(const ListSeed& ls, const int32_t* sel_idx,
                                              int32_t max_sel, int64_t bg, int32_t L,
                                              int32_t block, int32_t split,
                                              int32_t units_per_split) {
  TileWalk tw;
  tw.block = block;
  tw.L = L;
  tw.nb = (L + block - 1) / block;
  tw.tpb = (block + T - 1) / T;
  int32_t total = tw.nb;
  tw.sel = nullptr;
  tw.jl = -1;
  tw.u0 = split * units_per_split;
  tw.hl = ls.hl;
  if (sel_idx != nullptr) {
    tw.sel = sel_idx + bg * max_sel;
    tw.jl = ls.jl;
    total = min(max(__builtin_amdgcn_readfirstlane(ls.cnt), 0), max_sel);
  }
  tw.n_units = max(0, min(units_per_split, total - tw.u0));
  return tw;
}

// The query rows behind the G MFMA columns of KV head g of sequence b: a
// chunk of ntok query tokens times gh = G / ntok heads, column i = token
// i / gh, head i % gh of the group.  q and the partial states are laid out
// [batch][ntok][Hkv * gh] rows; ntok = 1 gives the decode layout, row
// b * H + g * G + i.
struct QRows {
  int32_t ntok, gsh, H;    // tokens, log2 of the heads per token, heads per token
  __device__ __forceinline__ int64_t row(int32_t b, int32_t g, int i) const {
    return (int64_t(b) * ntok + (i >> gsh)) * H + (int64_t(g) << gsh) + (i & ((1 << gsh) - 1));
  }
};
template <int G>
__device__ __forceinline__ QRows make_qrows(int32_t ntok, int32_t Hkv) {
  const int32_t gh = G / ntok;
  return QRows{ntok, __builtin_ctz(uint32_t(gh)), Hkv * gh};
}

// Softmax bookkeeping of one tile for the 16 MFMA columns (heads): lane l
// owns head l%16 and rows 4*(l/16) + r of the tile; O holds N 16-channel
// blocks of the accumulators (N = D / 16).  s[r] are base-2 logits
// (-inf for masked rows); returns the weights p[r] and rescales O when the
// reference moves (by the change of reference times o_extra, a caller's exact
// power of two).
//
// With LAZY, the reference m_run is a lazy maximum: it moves to a tile's
// maximum only when that exceeds it by more than kLazySlack (base 2), so the
// weights stay below 2^kLazySlack (finite in fp32, and the f16 high + low
// split of P keeps its relative precision at any magnitude) while the
// accumulators are rescaled only on the few tiles that move it; O and l stay
// relative to the same m_run, which is all the merge and the combine need.
// (The int8 kernel, whose tiles carry more vector work, gains from skipping
// the rescale: 262K dense 53.6 -> 51.9 us; the f16 kernel does not, and keeps
// the exact running maximum.)
constexpr float kLazySlack = 8.0f;
template <int G, int NT, bool LAZY, int N>
__device__ __forceinline__ void tile_softmax(float (&s)[4 * NT], float& m_run, float& l_run,
                                             float4_t (&O)[N], float o_extra = 1.0f) {
  const int lane = threadIdx.x % kWave;
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 4 * NT; ++i) mx = fmaxf(mx, s[i]);
  mx = rows_max(mx);
  // -inf + slack = -inf: the first live tile of a head moves its reference
  const bool bump = LAZY ? mx > m_run + kLazySlack : mx > m_run;
  const float m_ref = bump ? mx : m_run;
  // exp2(-inf) = 0 covers masked logits; a head with nothing live yet keeps
  // factor 1 and weights exp2(-inf - 0) = 0
  const bool live = m_ref != -INFINITY;
  const float m_use = live ? m_ref : 0.0f;
  float ps = 0.0f;
#pragma unroll
  for (int i = 0; i < 4 * NT; ++i) {
    s[i] = __builtin_amdgcn_exp2f(s[i] - m_use);
    ps += s[i];
  }
  ps = rows_sum(ps);
  // heads past G are padding
  const bool moved = !LAZY || __ballot(bump && (lane % 16) < G) != 0;
  if (moved || o_extra != 1.0f) {
    const float cr = live ? __builtin_amdgcn_exp2f(m_run - m_ref) : 1.0f;
    l_run = l_run * cr + ps;
    // O rows are heads 4*(lane/16) + r; head h's factor is in lane h (column
    // h of every row holds it).  Only heads < G matter: rows past them hold
    // padding and may take any finite factor.  (G <= 16.)
    const int quad = lane / 16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cr), r));
      if (G > 4) {
        const float c4 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cr), 4 + r));
        if (G > 8) {
          const float c8 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cr), 8 + r));
          const float c12 =
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cr), 12 + r));
          c = quad == 0 ? c : (quad == 1 ? c4 : (quad == 2 ? c8 : c12));
        } else {
          c = quad > 0 ? c4 : c;
        }
      }
      c *= o_extra;
#pragma unroll
      for (int n = 0; n < N; ++n) O[n][r] *= c;
    }
  } else {
    l_run += ps;
  }
  m_run = m_ref;
}

// Merge the 4 wavefronts' states (heads < G) through LDS and write the
// part's partial softmax state.
template <int G, int N>
__device__ __forceinline__ void finish_mfma(float m_run, float l_run, const float4_t (&O)[N],
                                            float* lds, float* __restrict__ ws_m,
                                            float* __restrict__ ws_l, float* __restrict__ ws_o,
                                            const QRows& qr, int32_t b, int32_t g,
                                            int32_t n_split, int32_t split) {
  constexpr int D = 16 * N;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  float* lo = lds;                          // [waves][G][D]
  float* lm = lds + kMWaves * G * D;        // [waves][G]
  float* ll = lm + kMWaves * G;
  __syncthreads();                          // tile buffers are reused
  const int g4 = 4 * (lane / 16);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = g4 + r;
    if (h < G) {
#pragma unroll
      for (int n = 0; n < N; ++n) lo[(wave * G + h) * D + 16 * n + lane % 16] = O[n][r];
    }
  }
  if (lane < G) { lm[wave * G + lane] = m_run; ll[wave * G + lane] = l_run; }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kMThreads) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) M = fmaxf(M, lm[w * G + h]);
    float so = 0.0f, sl = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kMWaves; ++w) {
        const float mw = lm[w * G + h];
        const float a = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        so += a * lo[(w * G + h) * D + d];
        sl += a * ll[w * G + h];
      }
    }
    const int64_t ps = qr.row(b, g, h) * n_split + split;
    ws_o[ps * D + d] = so;
    if (d == 0) { ws_m[ps] = M; ws_l[ps] = sl; }
  }
}

// The int8 kernels' query as the B operand of the integer q.K product
// (column = head lc, k-chunk lg): x holds this lane's channels
// 64 kk + 16 lg + 0..15 of its head, kk < KK = D / 64 (zeros past the group);
// the head's absmax scale over all D channels (the 4 lanes of a column hold
// D / 4 channels each)
// and the codes, which equal the correctly rounded rint(x / scale) of the
// append quantizer bit for bit: taken through the reciprocal, with the rare
// value near a rounding boundary (flagged per lane) redone with the exact
// quotient.  coef = scale * softmax scale * log2 e (0 past the group).
template <int KK>
__device__ __forceinline__ void i8_query_operand(const float (&x)[KK][16], bool hv, float scale2,
                                                 int4_t (&qb)[KK], float& coef) {
  // one bit of the redo mask per value
  typedef typename std::conditional<(KK > 2), uint64_t, uint32_t>::type Mask;
  float a = 0.0f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(x[kk][i]));
  }
  a = rows_max(a);
  const float qs = absmax_scale(a);
  // codes through the reciprocal; the rare value near a rounding boundary
  // (flagged per lane) is redone with the exact quotient
  const float inv = 1.0f / qs;
  int c[KK][16];
  Mask redo = 0u;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      bool ex;
      c[kk][i] = quant_code_recip(x[kk][i], inv, ex);
      redo |= Mask(ex) << (16 * kk + i);
    }
  }
  if (__builtin_amdgcn_ballot_w64(redo != 0u) != 0u) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((redo >> (16 * kk + i)) & 1u) c[kk][i] = quant_code(x[kk][i], qs);
    }
  }
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t packed = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) packed |= (uint32_t(c[kk][4 * w + e]) & 0xFFu) << (8 * e);
      qb[kk][w] = hv ? int32_t(packed) : 0;
    }
  }
  coef = hv ? qs * scale2 : 0.0f;
}

// int8 V codes widened to f16 exactly: 1152 + c is exact in f16, minus 1152.
__device__ __forceinline__ half8_t widen_codes(int2_t w) {
  typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
  // v_perm_b32 picks bytes of {0x64646464, x}: selector 0..3 = bytes of x,
  // 4 = 0x64.  Each 16-bit half becomes 0x64 : (c + 128) = f16 1024 + c + 128.
  constexpr uint32_t kLoSel = 0x04010400u;   // (0x64, x1, 0x64, x0)
  constexpr uint32_t kHiSel = 0x04030402u;   // (0x64, x3, 0x64, x2)
  const half2_t off = half2_t{(_Float16)1152.0f, (_Float16)1152.0f};
  half8_t r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t x = uint32_t(w[k]) ^ 0x80808080u;         // c + 128 per byte
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, x, kLoSel);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, x, kHiSel);
    const half2_t a = __builtin_bit_cast(half2_t, lo) - off;
    const half2_t b = __builtin_bit_cast(half2_t, hi) - off;
    r[4 * k + 0] = a[0];
    r[4 * k + 1] = a[1];
    r[4 * k + 2] = b[0];
    r[4 * k + 3] = b[1];
  }
  return r;
}

}  // namespace
}  // namespace skv
