// Group-wise quantized cache formats (q8_0, q4_0, q5_0) at head dims 64, 128
// and 256: the row layout and the exact widening of the codes to f16 shared by
// the attention kernels over such caches.  (The format itself, the codes'
// ranges and the planes are described with the cache descriptor.)
#pragma once

#include "decode_core.h"

namespace skv {
namespace {

constexpr int kGroup = 32;

enum GrpKind { kQ8 = 0, kQ4 = 1, kQ5 = 2 };
// Format K at head dim D (64, 128 or 256: D / 32 groups per row).
template <int K, int D = kD>
struct GrpFmt {
  static_assert(D == 64 || D == 128 || D == 256, "head dims 64, 128, 256");
  static constexpr bool kNib = K != kQ8;                   // nibble plane (q4_0, q5_0)
  static constexpr int kQmax = K == kQ8 ? 127 : K == kQ4 ? 7 : 15;
  static constexpr int kBias = K == kQ8 ? 0 : kQmax + 1;   // stored = code + bias
  static constexpr int kGroups = D / kGroup;               // 32-channel groups per row
  static constexpr int kRowBytes = kNib ? D / 2 : D;       // code / nibble row bytes
  static constexpr int kHiBytes = K == kQ5 ? D / 8 : 0;    // fifth-bit row bytes
  static constexpr int kTokBytes = kRowBytes + kHiBytes;   // per (token, KV head)
  static constexpr int kOcc = D > 128 ? 1 : 2;             // workgroups per CU (decode)
};
// Byte offsets of token t of row bg (sequence x KV head): its code (or
// nibble) row and, for q5_0, its fifth-bit row.
template <int K, int D = kD>
__device__ __forceinline__ int64_t grp_row_off(int64_t bg, int32_t max_seq, int64_t t) {
  using F = GrpFmt<K, D>;
  return bg * max_seq * F::kTokBytes + t * F::kRowBytes;
}
template <int K, int D = kD>
__device__ __forceinline__ int64_t grp_hi_off(int64_t bg, int32_t max_seq, int64_t t) {
  using F = GrpFmt<K, D>;
  return bg * max_seq * F::kTokBytes + int64_t(max_seq) * F::kRowBytes + t * F::kHiBytes;
}

// 32 nibble codes (16 bytes: byte i = channels 2i, 2i + 1, each code + 8) to
// 32 bytes in channel order, still biased (code + 8, 0..15): the bias comes
// off in the widening to f16 (widen_q4), in the same packed subtraction.
__device__ __forceinline__ void unpack_q4(const int4_t& w, int4_t& c0, int4_t& c1) {
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = uint32_t(w[i]);
    const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
    // (lo0, hi0, lo1, hi1) and (lo2, hi2, lo3, hi3)
    o[2 * i] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    o[2 * i + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
  c0 = int4_t{int(o[0]), int(o[1]), int(o[2]), int(o[3])};
  c1 = int4_t{int(o[4]), int(o[5]), int(o[6]), int(o[7])};
}

// q5_0: the nibbles as for q4_0, plus each channel's fifth bit (hi: bit i =
// channel i of the 32) as bit 4 of its byte: code + 16, 0..31.  The fifth bits
// of 4 channels go to bit 0 of 4 bytes by one 24-bit multiply: bit m of n
// (m < 4) lands at bit 8 m of n * 0x204081 (shifts 0, 7, 14, 21; no two
// products share a bit, so nothing carries).
__device__ __forceinline__ uint32_t spread4(uint32_t n) {
  return (n * 0x204081u) & 0x01010101u;
}
__device__ __forceinline__ void unpack_q5(const int4_t& w, uint32_t hi, int4_t& c0, int4_t& c1) {
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = uint32_t(w[i]);
    const uint32_t lo = x & 0x0F0F0F0Fu, hn = (x >> 4) & 0x0F0F0F0Fu;
    const uint32_t hb = hi >> (8 * i);                    // channels 8 i .. 8 i + 7
    o[2 * i] = __builtin_amdgcn_perm(hn, lo, 0x05010400u) | (spread4(hb & 15u) << 4);
    o[2 * i + 1] = __builtin_amdgcn_perm(hn, lo, 0x07030602u) | (spread4((hb >> 4) & 15u) << 4);
  }
  c0 = int4_t{int(o[0]), int(o[1]), int(o[2]), int(o[3])};
  c1 = int4_t{int(o[4]), int(o[5]), int(o[6]), int(o[7])};
}

// 8 biased bytes n = code + BIAS (q4_0: 8, q5_0: 16) to the f16 codes,
// exactly: each byte goes under a 0x64 high byte (f16 1024 + n), minus
// 1024 + BIAS.
template <int BIAS>
__device__ __forceinline__ half8_t widen_biased(int2_t w) {
  typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
  constexpr uint32_t kLoSel = 0x04010400u;   // (0x64, x1, 0x64, x0)
  constexpr uint32_t kHiSel = 0x04030402u;   // (0x64, x3, 0x64, x2)
  const half2_t off = half2_t{(_Float16)(1024.0f + BIAS), (_Float16)(1024.0f + BIAS)};
  half8_t r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t x = uint32_t(w[k]);
    const half2_t a = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, x, kLoSel)) - off;
    const half2_t b = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, x, kHiSel)) - off;
    r[4 * k + 0] = a[0];
    r[4 * k + 1] = a[1];
    r[4 * k + 2] = b[0];
    r[4 * k + 3] = b[1];
  }
  return r;
}

// The LDS codes of a tile as f16: q4_0 / q5_0 biased bytes or q8_0 int8 codes.
template <int K>
__device__ __forceinline__ half8_t widen_grp(int2_t w) {
  if constexpr (GrpFmt<K>::kNib) return widen_biased<GrpFmt<K>::kBias>(w);
  else return widen_codes(w);
}

// A lane's share of a tile's f16 scales, KG / 2 of them (groups
// (lane % 2) KG / 2 .. of token lane / 2: 2, 4 or 8 bytes at byte offset
// `off`, normally KG lane; an offset past the resource's records reads zeros
// without touching memory), packed in a uint2.
template <int KG>
__device__ __forceinline__ uint2 grp_scale_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (KG == 2) {
    return make_uint2(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kAuxNontemporal), 0u);
  } else if constexpr (KG == 4) {
    return make_uint2(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kAuxNontemporal), 0u);
  } else {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 a =
        __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAuxNontemporal));
    return make_uint2(a.x, a.y);
  }
}

// Stage a code tile of T = 32 tokens in LDS as one byte per channel (q8_0
// int8 codes, q4_0 / q5_0 code + bias), rows of D bytes with the 16-byte
// chunk c of row r at c ^ (r % min(D / 16, 16)).  c[i]: the lane's 16 bytes
// of HBM load i (chunk lane % HCPR of row HRPL i + lane / HCPR of the tile,
// HCPR = row bytes / 16, HRPL = 1024 / row bytes); h[i]: for q5_0 the fifth
// bits of those 32 channels.
template <int K, int D, int NL>
__device__ __forceinline__ void grp_stage(uint8_t* t, const int4_t (&c)[NL],
                                          const uint32_t (&h)[NL]) {
  using F = GrpFmt<K, D>;
  constexpr int kHcpr = F::kRowBytes / 16;
  constexpr int kHrpl = 1024 / F::kRowBytes;
  constexpr int kCpr = D / 16;
  constexpr int kSwz = kCpr < 16 ? kCpr : 16;
  const int lane = threadIdx.x % kWave;
  auto sw = [](int rw, int chunk) { return rw * D + 16 * (chunk ^ (rw & (kSwz - 1))); };
  if constexpr (F::kNib) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int rw = kHrpl * i + lane / kHcpr, ch = 2 * (lane % kHcpr);
      int4_t a0, a1;
      if constexpr (K == kQ5) unpack_q5(c[i], h[i], a0, a1);
      else unpack_q4(c[i], a0, a1);
      *reinterpret_cast<int4_t*>(t + sw(rw, ch)) = a0;
      *reinterpret_cast<int4_t*>(t + sw(rw, ch + 1)) = a1;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int rw = kHrpl * i + lane / kHcpr;
      *reinterpret_cast<int4_t*>(t + sw(rw, lane % kHcpr)) = c[i];
    }
  }
}

}  // namespace
}  // namespace skv
