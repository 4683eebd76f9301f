// block_bounds: Quest upper bound of every block, reduced over the GQA group.
//
// UB_h(j) = sum_d max(q_hd * kmin_jd, q_hd * kmax_jd)  (sparse_attn.md,
// "Method: Quest-style min/max block bounds"), written here as
// q_hd * (q_hd > 0 ? kmax_jd : kmin_jd), which is the same value (rounding is
// monotone) and skips the second product; a channel with q_hd == 0 adds 0.
// score(j) = max over the G query heads of KV head g ("S2/S3 engineering
// design", item 2: one block set per KV head).
//
// The pass reads the whole side cache (512 B per block and KV head at
// D = 128), so it is spread over as many workgroups as there are 16-block
// tiles: 16 lanes per block, each lane holding D / 16 channels (at D = 128
// one 16-byte load of kmin and one of kmax), a 16-lane DPP sum per head, then
// the group max.  Head dims 64 and 256 score on the vector units and take no
// folded append.
//
// A decode step may fold its one-token append into this pass
// (launch_append_bounds), which saves a launch and a dependent round trip.
#include "decode_core.h"
#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int kBoundsThreads = 256;
constexpr int kLanesPerBlock = 16;
constexpr int kBlocksPerWG = kBoundsThreads / kLanesPerBlock;  // 16

enum AppendMode {
  kNoAppend = 0, kAppendF16 = 1, kAppendI8 = 2, kAppendQ8 = 3, kAppendQ4 = 4, kAppendQ5 = 5
};
constexpr bool is_grp_mode(int mode) {
  return mode == kAppendQ8 || mode == kAppendQ4 || mode == kAppendQ5;
}

// Group-wise caches (q8_0 / q4_0 / q5_0): 32-channel groups with an f16 scale
// each, the append kernel's arithmetic (decode_grouped.hip):
// s = f16(absmax / QMAX), code = clamp(rint(x / s), -QMAX, QMAX) against the
// stored scale (0 when s is 0 or not finite); q4_0 stores code + 8, channels
// 2i / 2i + 1 in the low / high nibble of byte i; q5_0 stores code + 16, its
// low four bits as q4_0 in a nibble plane and bit 4 in a plane of its own
// (bit c % 8 of byte c / 8), the planes one after the other per (sequence,
// KV head).
constexpr int kGrpChannels = 32;
template <int MODE>
struct GrpMode {
  static constexpr bool kNib = MODE != kAppendQ8;
  static constexpr bool kQ5 = MODE == kAppendQ5;
  static constexpr int kQmax = MODE == kAppendQ8 ? 127 : MODE == kAppendQ4 ? 7 : 15;
  static constexpr int kBias = kNib ? kQmax + 1 : 0;
  static constexpr int kRowBytes = kNib ? 64 : 128;
  static constexpr int kHiBytes = kQ5 ? 16 : 0;
  static constexpr int kTokBytes = kRowBytes + kHiBytes;
};
// byte offsets of token t of row bg: its code / nibble row, its fifth-bit row
template <int MODE>
__device__ __forceinline__ int64_t grp_row_b(int64_t bg, int32_t max_seq, int64_t t) {
  return bg * max_seq * GrpMode<MODE>::kTokBytes + t * GrpMode<MODE>::kRowBytes;
}
template <int MODE>
__device__ __forceinline__ int64_t grp_hi_b(int64_t bg, int32_t max_seq, int64_t t) {
  return bg * max_seq * GrpMode<MODE>::kTokBytes + int64_t(max_seq) * GrpMode<MODE>::kRowBytes +
         t * GrpMode<MODE>::kHiBytes;
}
__device__ __forceinline__ uint16_t grp_scale_bits_b(float a, int qmax) {
  return __half_as_ushort(__float2half_rn(a / float(qmax)));
}
__device__ __forceinline__ int grp_code_b(float x, float s, int qmax) {
  if (!(s > 0.0f && s < INFINITY)) return 0;
  float r = rintf(x / s);
  r = fminf(fmaxf(r, -float(qmax)), float(qmax));
  return int(r);
}

// Write the new token of (sequence b, KV head g) at position p0 -- the
// one-token case of skv_kv_append, same arithmetic -- and its block's bounds.
template <int D, int MODE>
__device__ __forceinline__ void append_one(const AppendOne& ap, uint16_t* __restrict__ kmin,
                                           uint16_t* __restrict__ kmax, int32_t b, int32_t g,
                                           int32_t Hkv, int32_t p0, int32_t jn, bool fresh,
                                           int32_t max_blocks) {
  const int tid = threadIdx.x;
  const int64_t bg = int64_t(b) * Hkv + g;
  const int64_t row = bg * ap.max_seq + p0;
  const int64_t bo = (bg * max_blocks + jn) * D;
  if constexpr (MODE == kAppendF16) {
    constexpr int kVec = D * 2 / 16;
    const uint4* ks = reinterpret_cast<const uint4*>(ap.k_new) + bg * kVec;
    const uint4* vs = reinterpret_cast<const uint4*>(ap.v_new) + bg * kVec;
    if (tid < kVec) reinterpret_cast<uint4*>(ap.k)[row * kVec + tid] = ks[tid];
    else if (tid < 2 * kVec) reinterpret_cast<uint4*>(ap.v)[row * kVec + tid - kVec] = vs[tid - kVec];
    const uint16_t* kn = static_cast<const uint16_t*>(ap.k_new) + bg * D;
    for (int d = tid; d < D; d += kBoundsThreads) {
      const uint16_t x = kn[d];
      const bool nan = (x & 0x7FFFu) > 0x7C00u;      // skipped, as by the append kernel
      uint16_t bmn = nan ? uint16_t(0x7C00u) : x, bmx = nan ? uint16_t(0xFC00u) : x;
      if (!fresh) {
        bmn = f16_min_bits(kmin[bo + d], bmn);
        bmx = f16_max_bits(kmax[bo + d], bmx);
      }
      kmin[bo + d] = bmn;
      kmax[bo + d] = bmx;
    }
  } else if constexpr (is_grp_mode(MODE)) {
    // one wavefront per row (K, V): lane l holds channels 2l, 2l + 1, a
    // group is one 16-lane row (the append kernel's layout and order)
    using F = GrpMode<MODE>;
    const int lane = tid % kWave, wave = tid / kWave;
    if (wave < 2) {
      const float2 x =
          reinterpret_cast<const float2*>(static_cast<const float*>(wave == 0 ? ap.k_new : ap.v_new) +
                                          bg * D)[lane];
      const float a = group16_max(fmaxf(fmaxf(0.0f, fabsf(x.x)), fabsf(x.y)));
      const uint16_t sb = grp_scale_bits_b(a, F::kQmax);
      const float sc = h2f(sb);
      const int c0 = grp_code_b(x.x, sc, F::kQmax), c1 = grp_code_b(x.y, sc, F::kQmax);
      uint8_t* base = static_cast<uint8_t*>(wave == 0 ? ap.k : ap.v);
      uint8_t* dst = base + grp_row_b<MODE>(bg, ap.max_seq, p0);
      if constexpr (F::kNib) {
        const int u0 = c0 + F::kBias, u1 = c1 + F::kBias;
        dst[lane] = uint8_t((u0 & 15) | ((u1 & 15) << 4));
        if constexpr (F::kQ5) {
          // fifth bits: channel 2l from h0 bit l, 2l + 1 from h1 bit l
          const uint64_t h0 = __ballot(u0 >> 4), h1 = __ballot(u1 >> 4);
          if (lane < 4) {
            const uint32_t e = uint32_t(h0 >> (16 * lane)) & 0xFFFFu;
            const uint32_t o = uint32_t(h1 >> (16 * lane)) & 0xFFFFu;
            uint32_t w = 0u;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              w |= (((e >> i) & 1u) << (2 * i)) | (((o >> i) & 1u) << (2 * i + 1));
            reinterpret_cast<uint32_t*>(base + grp_hi_b<MODE>(bg, ap.max_seq, p0))[lane] = w;
          }
        }
      } else {
        reinterpret_cast<uint16_t*>(dst)[lane] = uint16_t((c0 & 0xFF) | ((c1 & 0xFF) << 8));
      }
      if (lane % 16 == 0)
        reinterpret_cast<uint16_t*>(wave == 0 ? ap.ks : ap.vs)[row * (D / kGrpChannels) + lane / 16] = sb;
    }
    const float* kn = static_cast<const float*>(ap.k_new) + bg * D;
    for (int d = tid; d < D; d += kBoundsThreads) {
      const float x = kn[d];
      uint16_t bmn = f32_to_f16_down(fminf(INFINITY, x)), bmx = f32_to_f16_up(fmaxf(-INFINITY, x));
      if (!fresh) {
        bmn = f16_min_bits(kmin[bo + d], bmn);
        bmx = f16_max_bits(kmax[bo + d], bmx);
      }
      kmin[bo + d] = bmn;
      kmax[bo + d] = bmx;
    }
  } else {
    static_assert(D % kWave == 0, "D must be a multiple of 64");
    constexpr int E = D / kWave;
    const int lane = tid % kWave, wave = tid / kWave;
    if (wave < 2) {
      const float* x = static_cast<const float*>(wave == 0 ? ap.k_new : ap.v_new) + bg * D;
      float xv[E];
      float am = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        xv[e] = x[lane * E + e];
        am = fmaxf(am, fabsf(xv[e]));
      }
      am = wave_max(am);
      const float scale = absmax_scale(am);
      int8_t* dst = static_cast<int8_t*>(wave == 0 ? ap.k : ap.v) + row * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = int8_t(quant_code(xv[e], scale));
      if (lane == 0) (wave == 0 ? ap.ks : ap.vs)[row] = scale;
    }
    const float* kn = static_cast<const float*>(ap.k_new) + bg * D;
    for (int d = tid; d < D; d += kBoundsThreads) {
      const float x = kn[d];
      uint16_t bmn = f32_to_f16_down(fminf(INFINITY, x)), bmx = f32_to_f16_up(fmaxf(-INFINITY, x));
      if (!fresh) {
        bmn = f16_min_bits(kmin[bo + d], bmn);
        bmx = f16_max_bits(kmax[bo + d], bmx);
      }
      kmin[bo + d] = bmn;
      kmax[bo + d] = bmx;
    }
  }
}

// The append without extra round trips: every lane requested its 8 channels
// (8c .. 8c + 7) of the new token's K and V rows at entry.  The 16 lanes that
// hold the token's block (in the workgroup of its tile) merge the new key into
// that block's bounds, which they read at entry (the side cache as it was),
// and for f16 write the new rows; for int8, every thread of the row's first
// workgroup quantizes one value (each 16-lane slot holds the whole row: slots
// 0..7 take channel 8c + slot of K, slots 8..15 channel 8c + slot - 8 of V,
// with the row's absmax over the slot, one DPP row).  All of this is register work; the stores come at the end of the
// kernel, after the scoring, so no wait for the position or for a write
// stands in front of the bounds.
template <int MODE>
__device__ __forceinline__ void merge_new_key(bool fresh, const uint4& kx, const float (&kf)[8],
                                              uint16_t (&lb)[8], uint16_t (&hb)[8]) {
  uint16_t nmn[8], nmx[8];
  // a NaN channel leaves the bounds as they were (+inf / -inf in a fresh
  // block), the rule of the append kernel's min/max scan
  if constexpr (MODE == kAppendF16) {
    const uint32_t w[4] = {kx.x, kx.y, kx.z, kx.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const uint16_t x = uint16_t(hlf ? (w[i] >> 16) : (w[i] & 0xFFFFu));
        const bool nan = (x & 0x7FFFu) > 0x7C00u;
        nmn[2 * i + hlf] = nan ? uint16_t(0x7C00u) : x;
        nmx[2 * i + hlf] = nan ? uint16_t(0xFC00u) : x;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      nmn[e] = f32_to_f16_down(fminf(INFINITY, kf[e]));
      nmx[e] = f32_to_f16_up(fmaxf(-INFINITY, kf[e]));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lb[e] = fresh ? nmn[e] : f16_min_bits(lb[e], nmn[e]);
    hb[e] = fresh ? nmx[e] : f16_max_bits(hb[e], nmx[e]);
  }
}

__device__ __forceinline__ int8_t quant_slot_i8(const float (&kf)[8], const float (&vf)[8],
                                                float& ks, float& vs) {
  static_assert(kBlocksPerWG == 16 && kLanesPerBlock * 8 == 128, "16 slots of a 128-value row");
  float ka = 0.0f, va = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ka = fmaxf(ka, fabsf(kf[e]));
    va = fmaxf(va, fabsf(vf[e]));
  }
  ks = absmax_scale(group16_max(ka));
  vs = absmax_scale(group16_max(va));
  const int slot = int(threadIdx.x) / kLanesPerBlock, e = slot % 8;
  const bool is_v = slot >= 8;
  float x = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) x = e == i ? (is_v ? vf[i] : kf[i]) : x;
  return int8_t(quant_code(x, is_v ? vs : ks));
}

// Group-wise codes of the new row in the row's first workgroup: slot 0 (the
// first 16 lanes) quantizes K, slot 1 V, lane c its channels 8c .. 8c + 7; a
// group is 4 lanes (xor-shuffles 1, 2 give its absmax).  Returns the lane's
// codes packed as stored (q8_0: 8 bytes; q4_0: 4 bytes of nibbles; q5_0: 4
// bytes of nibbles and, in .y, the byte of fifth bits) and its group's scale
// bits.
template <int MODE>
__device__ __forceinline__ uint2 quant_slot_grp(const float (&kf)[8], const float (&vf)[8],
                                                uint16_t& sbits) {
  using F = GrpMode<MODE>;
  const bool is_v = int(threadIdx.x) / kLanesPerBlock == 1;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = is_v ? vf[e] : kf[e];
  // the append kernel's absmax: fmaxf over 0 and |x|, so a NaN value is left out
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) a = fmaxf(fmaxf(a, fabsf(x[e])), fabsf(x[e + 1]));
  a = fmaxf(a, __shfl_xor(a, 1));
  a = fmaxf(a, __shfl_xor(a, 2));
  sbits = grp_scale_bits_b(a, F::kQmax);
  const float sc = h2f(sbits);
  int c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) c[e] = grp_code_b(x[e], sc, F::kQmax);
  uint2 out = make_uint2(0u, 0u);
  if constexpr (F::kNib) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u0 = c[2 * i] + F::kBias, u1 = c[2 * i + 1] + F::kBias;
      out.x |= uint32_t((u0 & 15) | ((u1 & 15) << 4)) << (8 * i);
      out.y |= uint32_t(((u0 >> 4) & 1) | (((u1 >> 4) & 1) << 1)) << (2 * i);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out.x |= uint32_t(c[i] & 0xFF) << (8 * i);
      out.y |= uint32_t(c[4 + i] & 0xFF) << (8 * i);
    }
  }
  return out;
}

__device__ __forceinline__ uint4 pack_bits(const uint16_t (&h)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = uint32_t(h[2 * i]) | (uint32_t(h[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The bounds of one 16-block tile for R = NT * G query rows on the matrix
// cores, by one wavefront.  UB = q+ . kmax + q- . kmin with q+ = max(q, 0),
// q- = min(q, 0), channel by channel the vector path's product (the bound of
// a channel with q == 0 is 0 either way, the bounds here being finite): A =
// the blocks' kmin / kmax rows (f16, exact), B = q+ and q- of the query rows
// as f16 high + low parts, each row first scaled by a power of two that puts
// its largest |q| in [2^13, 2^14) (exact; undone on the result), so the low
// parts keep their precision.  Lane (lg, lc): A = block lc, B = query row
// lc, channels 32 kk + 8 lg .. + 7; result = blocks 4 lg + r, query row lc,
// then the max over each token's G rows (lanes of one 16-lane row).
template <int D, int G, int NT, bool PH>
__device__ __forceinline__ void score_mfma(const float* qs, const uint16_t (*sb)[kBlocksPerWG][D],
                                           float* __restrict__ score, int32_t b, int32_t g,
                                           int32_t Hkv, int32_t tile, int32_t nb,
                                           int32_t max_blocks) {
  static_assert(D == 128, "four 32-channel MFMA steps");
  constexpr int R = NT * G;
  const int lane = threadIdx.x % kWave, lg = lane / 16, lc = lane % 16;
  const bool cv = lc < R;
  const float* qrow = qs + (cv ? lc : 0) * D;
  float qv[4][8];
  float mq = 0.0f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const float4 a = *reinterpret_cast<const float4*>(qrow + 32 * kk + 8 * lg);
    const float4 c4 = *reinterpret_cast<const float4*>(qrow + 32 * kk + 8 * lg + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qv[kk][s] = cv ? x[s] : 0.0f;
      mq = fmaxf(mq, fabsf(qv[kk][s]));
    }
  }
  mq = rows_max(mq);                        // the row's 128 channels (4 lane groups)
  const int qe = mq > 0.0f ? 14 - __builtin_amdgcn_frexp_expf(mq) : 0;
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    half8_t ph, pl, nh, nl;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float x = ldexpf(qv[kk][s], qe);
      const float xp = fmaxf(x, 0.0f), xn = fminf(x, 0.0f);
      const _Float16 hp = (_Float16)xp, hn = (_Float16)xn;
      ph[s] = hp;
      pl[s] = (_Float16)(xp - (float)hp);
      nh[s] = hn;
      nl[s] = (_Float16)(xn - (float)hn);
    }
    const int chunk = 4 * kk + lg;
    const half8_t amin = *reinterpret_cast<const half8_t*>(&sb[0][lc][8 * (chunk ^ lc)]);
    const half8_t amax = *reinterpret_cast<const half8_t*>(&sb[1][lc][8 * (chunk ^ lc)]);
    acc = mfma_f16_32(amax, ph, acc);
    acc = mfma_f16_32(amax, pl, acc);
    acc = mfma_f16_32(amin, nh, acc);
    acc = mfma_f16_32(amin, nl, acc);
  }
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = ldexpf(acc[r], -qe);
  if constexpr (PH) {
    // per query head (NT == 1): every row's own bound
    if (cv) {
      const int64_t srow = (int64_t(b) * Hkv + g) * G + lc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int32_t j = tile * kBlocksPerWG + 4 * lg + r;
        if (j < nb) score[srow * max_blocks + j] = v[r];
      }
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int o = 1; o < G; o <<= 1) v[r] = fmaxf(v[r], __shfl_xor(v[r], o));
  }
  if (cv && lc % G == 0) {
    const int t = lc / G;
    const int64_t srow = NT == 1 ? int64_t(b) * Hkv + g : (int64_t(b) * Hkv + g) * NT + t;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t j = tile * kBlocksPerWG + 4 * lg + r;
      if (j < nb) score[srow * max_blocks + j] = v[r];
    }
  }
}

// MODE != kNoAppend: first append one token per sequence at pos0[b] (the// MODE != kNoAppend: first append one token per sequence at pos0[b] (the
// first workgroup of each (sequence, KV head) writes it) and score its block
// with the merged bounds.  The merge is computed from the new key in
// registers, so it does not matter whether this workgroup reads the side
// cache before or after the append writes it: min/max with the same key is
// idempotent, and a fresh block ignores the old values.
// PH: per-query-head bounds (score [batch][n_heads][max_blocks], no group
// max): each query head ranks the blocks by its own bound.
// NT > 1: a chunk of NT query tokens per sequence (q [batch][NT][H][D]); the
// side cache is read once for the NT x G query rows, and each token gets its
// own group max (score [batch][Hkv][NT][max_blocks]).
template <int D, int G, int MODE, bool PH = false, int NT = 1>
__global__ void __launch_bounds__(kBoundsThreads)
bounds_kernel(uint16_t* __restrict__ kmin, uint16_t* __restrict__ kmax,
              const float* __restrict__ q, const int32_t* __restrict__ seq_len,
              float* __restrict__ score, int32_t Hkv, int32_t max_len, int32_t block,
              int32_t max_blocks, int32_t tiles, int32_t n_rows, AppendOne ap) {
  static_assert(D == 64 || D == 128 || D == 256, "head dims 64, 128, 256");
  static_assert(D == 128 || MODE == kNoAppend, "head dims other than 128: no folded append");
  static_assert(NT == 1 || (MODE == kNoAppend && !PH), "token chunks: plain bounds only");
  constexpr int CPL = D / kLanesPerBlock;                      // channels per lane
  constexpr int kQ4 = NT * G * D / 4;                          // 16-byte query loads
  constexpr int kQPer = (kQ4 + kBoundsThreads - 1) / kBoundsThreads;
  static_assert(kQPer <= 4, "at most 16 query rows of at most 256 channels");
  // 1-D grid of tiles x Hkv x batch, row by row (XCD-aware slots: a row's
  // scores are written on the XCD whose L2 its decode parts read them from)
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t tile = int32_t(slot % uint32_t(tiles));
  const uint32_t row = xcd_row(slot / uint32_t(tiles), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int32_t j = tile * kBlocksPerWG + int32_t(threadIdx.x) / kLanesPerBlock;
  const int32_t c = threadIdx.x % kLanesPerBlock;  // channels CPL c .. CPL c + CPL - 1
  // Requests issued before anything waits (one round trip): the row length
  // (and append position), the group's G query rows (G * 512 B, one 16-byte
  // load per thread, staged once per workgroup in LDS) and this thread's
  // bounds, read for every block of the launched tile that exists in the
  // side cache; only those below the row's length are scored.
  const int32_t L_raw = seq_len[b];
  int32_t p0 = -1;
  if constexpr (MODE != kNoAppend) p0 = ap.pos0[b];
  const int32_t H = Hkv * G;
  // query row rr = token rr / G, head rr % G: q row (b NT + t) H + g G + h
  float4 qreg[kQPer];
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int e = int(threadIdx.x) + kBoundsThreads * i;
    const int rr = e / (D / 4);
    qreg[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (e < kQ4)
      qreg[i] = reinterpret_cast<const float4*>(
          q + ((int64_t(b) * NT + rr / G) * H + g * G + rr % G) * D)[e % (D / 4)];
  }
  // this lane's CPL bounds of each kind as CPL / 2 words (read once per
  // step: streaming loads, 16 bytes each, 8 bytes at D = 64)
  constexpr int kW = CPL / 2;
  uint32_t lw[kW], hw[kW];
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  if constexpr (D == 128) {
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (j < max_blocks) {
      const int64_t off = ((int64_t(b) * Hkv + g) * max_blocks + j) * D + c * 8;
      const u32x4 l4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kmin + off));
      const u32x4 h4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kmax + off));
      lo = make_uint4(l4.x, l4.y, l4.z, l4.w);
      hi = make_uint4(h4.x, h4.y, h4.z, h4.w);
    }
    lw[0] = lo.x; lw[1] = lo.y; lw[2] = lo.z; lw[3] = lo.w;
    hw[0] = hi.x; hw[1] = hi.y; hw[2] = hi.z; hw[3] = hi.w;
  } else {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const int64_t off = ((int64_t(b) * Hkv + g) * max_blocks + j) * D + c * CPL;
    const bool in = j < max_blocks;
    if constexpr (kW >= 4) {
#pragma unroll
      for (int i = 0; i < kW / 4; ++i) {
        u32x4 l4 = {0u, 0u, 0u, 0u}, h4 = {0u, 0u, 0u, 0u};
        if (in) {
          l4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kmin + off) + i);
          h4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kmax + off) + i);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) { lw[4 * i + e] = l4[e]; hw[4 * i + e] = h4[e]; }
      }
    } else {
      u32x2 l2 = {0u, 0u}, h2 = {0u, 0u};
      if (in) {
        l2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(kmin + off));
        h2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(kmax + off));
      }
      lw[0] = l2[0]; lw[1] = l2[1]; hw[0] = h2[0]; hw[1] = h2[1];
    }
  }
  // With the append: this lane's 8 channels of the new token's K and V rows,
  // requested here too (they do not depend on the position).
  const int64_t src = (int64_t(b) * Hkv + g) * D + c * 8;
  uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
  float kf[8], vf[8];
  if constexpr (MODE == kAppendF16) {
    kx = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(ap.k_new) + src);
    vx = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(ap.v_new) + src);
  } else if constexpr (MODE != kNoAppend) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = static_cast<const float*>(ap.k_new)[src + e];
      vf[e] = static_cast<const float*>(ap.v_new)[src + e];
    }
  }
  // keep those requests here, with the others (only the 16 owner lanes use
  // them, and the compiler would otherwise move them into that branch,
  // behind the wait for the position)
  if constexpr (MODE != kNoAppend) asm volatile("" ::: "memory");
  uint16_t lb[CPL], hb[CPL];
  {
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      lb[2 * i] = uint16_t(lw[i] & 0xFFFFu); lb[2 * i + 1] = uint16_t(lw[i] >> 16);
      hb[2 * i] = uint16_t(hw[i] & 0xFFFFu); hb[2 * i + 1] = uint16_t(hw[i] >> 16);
    }
  }
  bool own = false, own_wg = false;
  int64_t arow = 0, bo = 0;
  int8_t code = 0;
  float ks_new = 0.0f, vs_new = 0.0f;
  uint2 gcodes = make_uint2(0u, 0u);
  uint16_t gscale = 0;
  if constexpr (MODE != kNoAppend) {
    if (p0 >= 0 && p0 < ap.max_seq) {
      const int32_t jn = p0 / block;
      const bool fresh = (p0 % block) == 0;
      arow = (int64_t(b) * Hkv + g) * ap.max_seq + p0;
      bo = ((int64_t(b) * Hkv + g) * max_blocks + jn) * D + c * 8;
      if (jn / kBlocksPerWG < tiles) {
        own = j == jn;
        if (own) merge_new_key<MODE>(fresh, kx, kf, lb, hb);
        // int8 rows: by the row's first workgroup (dispatched first, so its
        // extra arithmetic is hidden behind the later tiles)
        if constexpr (MODE == kAppendI8) {
          own_wg = tile == 0;
          if (own_wg) code = quant_slot_i8(kf, vf, ks_new, vs_new);
        } else if constexpr (is_grp_mode(MODE)) {
          own_wg = tile == 0 && int(threadIdx.x) < 2 * kLanesPerBlock;
          if (own_wg) gcodes = quant_slot_grp<MODE>(kf, vf, gscale);
        }
      } else if (tile == 0) {
        // the token's block lies past the launched tiles: append it here
        append_one<D, MODE>(ap, kmin, kmax, b, g, Hkv, p0, jn, fresh, max_blocks);
      }
    }
  }
  const int32_t L = min(max(L_raw, 0), max_len);
  const int32_t nb = (L + block - 1) / block;
  const bool live = j < nb;
  float best = -INFINITY;
  // With 8 or more query rows per block the scoring runs on the matrix
  // cores (score_mfma; the per-head bounds too, so the group score stays the
  // max of the per-head values bit for bit); a workgroup whose live bounds
  // hold an infinity (an int8 cache with keys past the f16 range, or an
  // all-NaN channel) keeps the vector path, whose q == 0 rule the MFMA form
  // would turn into NaN.
  constexpr bool kMfma = NT * G >= 8 && D == 128;
  if (tile * kBlocksPerWG < nb) {          // else the whole tile is past the end
    __shared__ __attribute__((aligned(16))) float qs[NT * G * D];
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
      const int e = int(threadIdx.x) + kBoundsThreads * i;
      if (e < kQ4) reinterpret_cast<float4*>(qs)[e] = qreg[i];
    }
    if constexpr (kMfma) {
      // the tile's bounds, 16-byte chunks XOR-swizzled by block (the MFMA
      // reads 16 blocks at one chunk)
      __shared__ __attribute__((aligned(16))) uint16_t sb[2][kBlocksPerWG][D];
      const int jj = int(threadIdx.x) / kLanesPerBlock;
      *reinterpret_cast<uint4*>(&sb[0][jj][8 * (c ^ jj)]) = pack_bits(lb);
      *reinterpret_cast<uint4*>(&sb[1][jj][8 * (c ^ jj)]) = pack_bits(hb);
      bool inf = false;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        inf |= (lb[e] & 0x7FFFu) == 0x7C00u || (hb[e] & 0x7FFFu) == 0x7C00u;
      if (!__syncthreads_or(live && inf)) {
        if (threadIdx.x < kWave)
          score_mfma<D, G, NT, PH>(qs, sb, score, b, g, Hkv, tile, nb, max_blocks);
        goto scored;
      }
    } else {
      __syncthreads();
    }
    float mn[CPL], mx[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) { mn[e] = h2f(lb[e]); mx[e] = h2f(hb[e]); }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float qv[G][CPL];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float* qr = qs + (t * G + h) * D + c * CPL;
#pragma unroll
        for (int i = 0; i < CPL / 4; ++i) {
          const float4 a = reinterpret_cast<const float4*>(qr)[i];
          qv[h][4 * i] = a.x; qv[h][4 * i + 1] = a.y; qv[h][4 * i + 2] = a.z; qv[h][4 * i + 3] = a.w;
        }
      }
      float tbest = -INFINITY;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const float x = qv[h][e];
          const float kb = x > 0.0f ? mx[e] : mn[e];
          acc += (x != 0.0f) ? x * kb : 0.0f;
        }
        acc = group16_sum(acc);
        tbest = fmaxf(tbest, acc);
        if constexpr (PH) {
          if (live && c == 0) score[(int64_t(b) * H + g * G + h) * max_blocks + j] = acc;
        }
      }
      if constexpr (NT > 1) {
        if (live && c == 0) score[((int64_t(b) * Hkv + g) * NT + t) * max_blocks + j] = tbest;
      }
      best = tbest;
    }
    if (NT == 1 && !PH && live && c == 0) score[(int64_t(b) * Hkv + g) * max_blocks + j] = best;
  }
scored:
  // the append's stores
  if constexpr (MODE != kNoAppend) {
    if (own) {
      *reinterpret_cast<uint4*>(kmin + bo) = pack_bits(lb);
      *reinterpret_cast<uint4*>(kmax + bo) = pack_bits(hb);
      if constexpr (MODE == kAppendF16) {
        reinterpret_cast<uint4*>(static_cast<uint16_t*>(ap.k) + arow * D)[c] = kx;
        reinterpret_cast<uint4*>(static_cast<uint16_t*>(ap.v) + arow * D)[c] = vx;
      }
    }
    if constexpr (MODE == kAppendI8) {
      if (own_wg) {
        const int slot = int(threadIdx.x) / kLanesPerBlock;
        (static_cast<int8_t*>(slot >= 8 ? ap.v : ap.k) + arow * D)[8 * c + slot % 8] = code;
        if (threadIdx.x == 0) ap.ks[arow] = ks_new;
        if (threadIdx.x == 8 * kLanesPerBlock) ap.vs[arow] = vs_new;
      }
    } else if constexpr (is_grp_mode(MODE)) {
      if (own_wg) {
        using F = GrpMode<MODE>;
        const bool is_v = int(threadIdx.x) / kLanesPerBlock == 1;
        uint8_t* base = static_cast<uint8_t*>(is_v ? ap.v : ap.k);
        const int64_t bgr = int64_t(b) * Hkv + g;
        uint8_t* dst = base + grp_row_b<MODE>(bgr, ap.max_seq, p0);
        if constexpr (F::kNib) reinterpret_cast<uint32_t*>(dst)[c] = gcodes.x;
        else reinterpret_cast<uint2*>(dst)[c] = gcodes;
        if constexpr (F::kQ5) base[grp_hi_b<MODE>(bgr, ap.max_seq, p0) + c] = uint8_t(gcodes.y);
        if (c % 4 == 0)
          reinterpret_cast<uint16_t*>(is_v ? ap.vs : ap.ks)[arow * (D / kGrpChannels) + c / 4] =
              gscale;
      }
    }
  }
}

template <int G, int MODE, bool PH = false, int NT = 1, int D = 128>
hipError_t launch_bounds_g(const skv_cache& c, const float* q, const int32_t* seq_len,
                           int32_t max_len, float* score, const AppendOne& ap,
                           hipStream_t stream) {
  const int32_t max_blocks = (c.max_seq + c.block - 1) / c.block;
  const int32_t nb_max = (max_len + c.block - 1) / c.block;
  int32_t tiles = (nb_max + kBlocksPerWG - 1) / kBlocksPerWG;
  if (MODE != kNoAppend && tiles == 0) tiles = 1;           // the append still runs
  if (tiles == 0) return hipSuccess;
  const int64_t n_wg = int64_t(tiles) * c.n_kv_heads * c.batch;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(n_wg));
  bounds_kernel<D, G, MODE, PH, NT><<<grid, kBoundsThreads, 0, stream>>>(
      c.kmin, c.kmax, q, seq_len, score, c.n_kv_heads, max_len, c.block, max_blocks, tiles,
      c.n_kv_heads * c.batch, ap);
  return hipGetLastError();
}

template <int MODE, int D = 128, bool PH = false>
hipError_t launch_bounds_m(const skv_cache& c, const float* q, int32_t n_heads,
                           const int32_t* seq_len, int32_t max_len, float* score,
                           const AppendOne& ap, hipStream_t stream) {
  switch (n_heads / c.n_kv_heads) {
    case 1: return launch_bounds_g<1, MODE, PH, 1, D>(c, q, seq_len, max_len, score, ap, stream);
    case 2: return launch_bounds_g<2, MODE, PH, 1, D>(c, q, seq_len, max_len, score, ap, stream);
    case 4: return launch_bounds_g<4, MODE, PH, 1, D>(c, q, seq_len, max_len, score, ap, stream);
    case 8: return launch_bounds_g<8, MODE, PH, 1, D>(c, q, seq_len, max_len, score, ap, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_bounds(const skv_cache& c, const float* q, int32_t n_heads,
                         const int32_t* seq_len, int32_t max_len, float* score,
                         hipStream_t stream) {
  const AppendOne ap{};
  switch (c.head_dim) {
    case 64: return launch_bounds_m<kNoAppend, 64>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    case 128: return launch_bounds_m<kNoAppend>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    case 256:
      return launch_bounds_m<kNoAppend, 256>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    default: return hipErrorInvalidValue;
  }
}

namespace {

template <int D>
hipError_t launch_bounds_multi_d(const skv_cache& c, const float* q, int32_t n_tok,
                                 int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                                 float* score, hipStream_t stream) {
  const AppendOne ap{};
  const int G = n_heads / c.n_kv_heads;
#define SKV_BMT(GG, NN)                                                                        \
  if (G == GG && n_tok == NN)                                                                  \
    return launch_bounds_g<GG, kNoAppend, false, NN, D>(c, q, seq_len, max_len, score, ap, stream)
  SKV_BMT(1, 1); SKV_BMT(2, 1); SKV_BMT(4, 1); SKV_BMT(8, 1);
  SKV_BMT(1, 2); SKV_BMT(1, 4); SKV_BMT(1, 8);
  SKV_BMT(2, 2); SKV_BMT(2, 4); SKV_BMT(2, 8);
  SKV_BMT(4, 2); SKV_BMT(4, 4);
  SKV_BMT(8, 2);
#undef SKV_BMT
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bounds_multi(const skv_cache& c, const float* q, int32_t n_tok,
                               int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                               float* score, hipStream_t stream) {
  switch (c.head_dim) {
    case 64: return launch_bounds_multi_d<64>(c, q, n_tok, n_heads, seq_len, max_len, score, stream);
    case 128: return launch_bounds_multi_d<128>(c, q, n_tok, n_heads, seq_len, max_len, score, stream);
    case 256: return launch_bounds_multi_d<256>(c, q, n_tok, n_heads, seq_len, max_len, score, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bounds_heads(const skv_cache& c, const float* q, int32_t n_heads,
                               const int32_t* seq_len, int32_t max_len, float* score,
                               hipStream_t stream) {
  const AppendOne ap{};
  switch (c.head_dim) {
    case 64: return launch_bounds_m<kNoAppend, 64, true>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    case 128: return launch_bounds_m<kNoAppend, 128, true>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    case 256: return launch_bounds_m<kNoAppend, 256, true>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append_bounds(const skv_cache& c, const int32_t* pos0, const void* k_new,
                                const void* v_new, const float* q, int32_t n_heads,
                                const int32_t* seq_len, int32_t max_len, float* score,
                                hipStream_t stream) {
  if (c.head_dim != 128) return hipErrorInvalidValue;
  AppendOne ap{c.k, c.v, c.k_scale, c.v_scale, k_new, v_new, pos0, c.max_seq};
  switch (c.kv_dtype) {
    case SKV_F16:
      return launch_bounds_m<kAppendF16>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    case SKV_I8:
      return launch_bounds_m<kAppendI8>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    case SKV_Q8_0:
      return launch_bounds_m<kAppendQ8>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    case SKV_Q4_0:
      return launch_bounds_m<kAppendQ4>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    case SKV_Q5_0:
      return launch_bounds_m<kAppendQ5>(c, q, n_heads, seq_len, max_len, score, ap, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace skv
