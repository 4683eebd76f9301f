// Group-wise quantized caches (q8_0, q4_0, q5_0): append and decode
// attention at head dims D = 64, 128, 256.
//
// opencoti-llamafile sparse_attn.md, "All-KV-types composition": the side
// cache of the block selector is filled from the keys before quantization, so
// the Quest bound composes with quantized caches; "The decode win lives on
// quantized KV": a dense pass must dequantize every block, the block skip
// skips that work too.  The formats hold groups of 32 channels (the page's
// quant block size, blck = 32) with one scale each; the cpu-attn card
// ("Requirements and limits") contrasts its per-token scale with such
// group-wise scaling within a row.
//
// Layout: codes [batch][n_kv_heads][max_seq][row] with row = D bytes
// (q8_0, int8 codes -127..127) or D / 2 bytes (q4_0: channel 2i in the low
// nibble of byte i, channel 2i + 1 in the high nibble, each code + 8 with
// codes -7..7); q5_0 (codes -15..15, stored as code + 16 in five bits): per
// (sequence, KV head) a plane of max_seq D / 2-byte nibble rows (bits 0..3,
// as q4_0) followed by a plane of max_seq D / 8-byte rows of the fifth bits
// (bit c % 8 of byte c / 8 for channel c); scales
// [batch][n_kv_heads][max_seq][D / 32] f16, one per group of 32 channels.  Per group: a = max |x|,
// s = f16(a / QMAX) (QMAX 127, 7 or 15),
// code = clamp(rint(x / s), -QMAX, QMAX) against the stored scale, so a value
// is exactly s * code (s == 0 or not finite: codes 0).
//
// Decode (decode_grp_mfma) follows the int8 kernel's structure -- 32-token
// tiles, two in flight per wavefront, LDS staging with XOR-swizzled 16-byte
// chunks, MFMA for both contractions -- with:
//   q.K: the codes widened to f16 exactly (the int8 kernel's byte trick) as
//     the A operand, the query as f16 high + low parts (~22-bit precision) as
//     B; one v_mfma_f32_16x16x32_f16 pair per 32-channel group, so each
//     group's partial dot leaves the matrix core on its own and is weighted
//     by that (token, group)'s scale in float32 (4 FMAs per token and head);
//   P.V: the transposed V codes widened to f16 as B, and as A the weight
//     times the (token, group) V scale in a running power-of-two unit, split
//     into f16 high + low parts per group (each 16-channel MFMA block lies in
//     one group);
//   q4_0 tiles arrive as nibbles (half the bytes) and are spread to one
//     byte each (code + 8) in registers before the LDS stage, so both formats
//     share the LDS layout and the transposing reads; the bias comes off in
//     the exact widening to f16.
#include <type_traits>

#include "decode_core.h"
#include "device_common.h"
#include "fused_walk.h"
#include "grouped_core.h"
#include "launch.h"

namespace skv {
namespace {

// The fifth bits of 32 channels as a 32-bit word (bit i = channel i) from the
// two ballots of a row (lane l: h0 bit l = channel 2l, h1 bit l = channel
// 2l + 1), for lanes l < 4 (channels 32 l .. 32 l + 31).
__device__ __forceinline__ uint32_t q5_hi_word(uint64_t h0, uint64_t h1, int l) {
  const uint32_t e = uint32_t(h0 >> (16 * l)) & 0xFFFFu, o = uint32_t(h1 >> (16 * l)) & 0xFFFFu;
  uint32_t w = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) w |= (((e >> i) & 1u) << (2 * i)) | (((o >> i) & 1u) << (2 * i + 1));
  return w;
}

// The group-wise quantizer for one value given its group's absmax (the
// append's arithmetic): stored f16 scale and code.
__device__ __forceinline__ uint16_t grp_scale_bits(float a, int qmax) {
  return __half_as_ushort(__float2half_rn(a / float(qmax)));
}
__device__ __forceinline__ int grp_code(float x, float s, int qmax) {
  if (!(s > 0.0f && s < INFINITY)) return 0;
  float r = rintf(x / s);
  r = fminf(fmaxf(r, -float(qmax)), float(qmax));
  return int(r);
}

// ------------------------------------------------------------------ append
// One workgroup per (sequence, KV head, block touched by the append); one
// wavefront per new row, a 128-channel slice at a time: lane l holds channels
// 2l, 2l + 1 of the slice, a group is 16 lanes (one DPP row, whose max gives
// the group's absmax); at D = 64 lanes 32..63 hold nothing.  Bounds as for
// the int8 cache: the float32 keys' min / max rounded outward to f16.
constexpr int kAppendThreads = 256;

template <int K, int D>
__global__ void __launch_bounds__(kAppendThreads)
append_grp_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                  uint16_t* __restrict__ ksc, uint16_t* __restrict__ vsc,
                  uint16_t* __restrict__ kmin, uint16_t* __restrict__ kmax,
                  const float* __restrict__ kn, const float* __restrict__ vn,
                  const int32_t* __restrict__ pos0, int32_t n_new, int32_t Hkv,
                  int32_t max_seq, int32_t block, int32_t max_blocks) {
  using F = GrpFmt<K, D>;
  constexpr int kSlices = (D + 127) / 128;
  const int32_t g = blockIdx.y, b = blockIdx.z;
  const int32_t p0 = pos0[b];
  if (p0 < 0) return;
  const int32_t j = p0 / block + int32_t(blockIdx.x);
  const int64_t lo64 = max(int64_t(p0), int64_t(j) * block);
  const int64_t hi64 = min(min(int64_t(p0) + n_new, int64_t(j + 1) * block), int64_t(max_seq));
  if (lo64 >= hi64) return;
  const int32_t t0 = int32_t(lo64), t1 = int32_t(hi64);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  for (int32_t t = t0 + wave; t < t1; t += kAppendThreads / kWave) {
    const int64_t src = ((int64_t(b) * n_new + (t - p0)) * Hkv + g) * D;
    const int64_t bg = int64_t(b) * Hkv + g;
    const int64_t row = bg * max_seq + t;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) {
        const bool on = D >= 128 || 2 * lane < D;          // D = 64: lanes 0..31
        const float2 x = on ? reinterpret_cast<const float2*>((which == 0 ? kn : vn) + src)[64 * sl + lane]
                            : make_float2(0.0f, 0.0f);
        const float a = group16_max(fmaxf(fmaxf(0.0f, fabsf(x.x)), fabsf(x.y)));
        const uint16_t sb = grp_scale_bits(a, F::kQmax);
        const float s = h2f(sb);
        const int c0 = grp_code(x.x, s, F::kQmax), c1 = grp_code(x.y, s, F::kQmax);
        uint8_t* base = which == 0 ? kc : vc;
        uint8_t* dst = base + grp_row_off<K, D>(bg, max_seq, t);
        if constexpr (F::kNib) {
          const int u0 = c0 + F::kBias, u1 = c1 + F::kBias;
          if (on) dst[64 * sl + lane] = uint8_t((u0 & 15) | ((u1 & 15) << 4));
          if constexpr (K == kQ5) {
            const uint64_t h0 = __ballot(u0 >> 4), h1 = __ballot(u1 >> 4);
            if (lane < 4 && 128 * sl + 32 * lane < D)
              reinterpret_cast<uint32_t*>(base + grp_hi_off<K, D>(bg, max_seq, t))[4 * sl + lane] =
                  q5_hi_word(h0, h1, lane);
          }
        } else {
          if (on)
            reinterpret_cast<uint16_t*>(dst)[64 * sl + lane] =
                uint16_t((c0 & 0xFF) | ((c1 & 0xFF) << 8));
        }
        if (on && lane % 16 == 0)
          (which == 0 ? ksc : vsc)[row * F::kGroups + 4 * sl + lane / 16] = sb;
      }
    }
  }
  if (kmin == nullptr) return;
  const bool fresh = int64_t(j) * block >= p0;
  for (int32_t d = threadIdx.x; d < D; d += kAppendThreads) {
    float mn = INFINITY, mx = -INFINITY;
    for (int32_t t = t0; t < t1; ++t) {
      const float x = kn[((int64_t(b) * n_new + (t - p0)) * Hkv + g) * D + d];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    uint16_t bmn = f32_to_f16_down(mn), bmx = f32_to_f16_up(mx);
    const int64_t o = ((int64_t(b) * Hkv + g) * max_blocks + j) * D + d;
    if (!fresh) {
      bmn = f16_min_bits(kmin[o], bmn);
      bmx = f16_max_bits(kmax[o], bmx);
    }
    kmin[o] = bmn;
    kmax[o] = bmx;
  }
}

// ------------------------------------------------------------------ decode
constexpr int kPwShiftGrp = 7;

// SELR > 0: the block selection runs in the prologue (fused_walk), as in the
// f16 and int8 attention kernels.  HM: per-query-head lists (a head mask per
// list entry; the heads that did not choose a block leave it out).  The G
// MFMA columns are ntok query tokens x G / ntok heads (QRows), each token
// seeing the positions below its causal limit.
template <int G, int K, int SELR, int D, bool HM = false>
__global__ void __launch_bounds__(kMThreads, (GrpFmt<K, D>::kOcc))
decode_grp_mfma(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                const uint16_t* __restrict__ ksc, const uint16_t* __restrict__ vsc,
                const float* __restrict__ q, const int32_t* __restrict__ seq_len,
                const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
                int32_t max_sel, int32_t Hkv, int32_t max_seq, int32_t block, int32_t max_len,
                int32_t n_split, int32_t n_rows, int32_t units_per_split, float qscale2,
                float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
                FusedSelect fs, const uint32_t* __restrict__ sel_hmask, int32_t ntok) {
  using F = GrpFmt<K, D>;
  constexpr bool Q5 = K == kQ5;
  constexpr int KG = F::kGroups;
  constexpr int T = 32;
  constexpr int kCpr = D / 16;                              // LDS chunks per code row
  constexpr int kCodeBytes = T * D;                         // int8 codes in LDS (4 KiB at 128)
  constexpr int kScaleOff = 2 * kCodeBytes;                 // K, V scales as float [T][KG]
  constexpr int kBufBytes = 2 * kCodeBytes + 2 * T * KG * 4;
  constexpr int kTileBytes = T * F::kRowBytes;              // HBM bytes of a code tile
  constexpr int kLoads = kTileBytes / 1024;                 // 16-byte code loads per lane
  constexpr int kHcpr = F::kRowBytes / 16;                  // HBM chunks per code row
  constexpr int kHrpl = 1024 / F::kRowBytes;                // HBM rows per load instruction
  constexpr int kSb = KG;                                   // scale bytes per lane and tile
  static_assert(kLoads >= 1, "a tile is at least one load per lane");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMWaves][2][kBufBytes];
  static_assert(SELR == 0 || sizeof(smem) >= sizeof(SelectShared),
                "the prologue's selection runs in the tile buffers");
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t split = int32_t(slot % uint32_t(n_split));
  const uint32_t row = xcd_row(slot / uint32_t(n_split), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const QRows qr = make_qrows<G>(ntok, Hkv);
  const int64_t bg = int64_t(b) * Hkv + g;
  const int32_t L_raw = seq_len[b];
  ListSeed ls{};
  if constexpr (SELR == 0)
    ls = list_seed(sel_idx, sel_cnt, max_sel, bg, split, units_per_split,
                   HM ? sel_hmask : nullptr);
  // query as the B operand of the per-group q.K: column = query row lc,
  // k-chunk lg of group kk = channels 32 kk + 8 lg .. + 7; f16 high + low parts
  half8_t qhi[KG], qlo[KG];
  {
    const bool hv = lc < G;
    const float* qp = q + qr.row(b, g, hv ? lc : 0) * D;
#pragma unroll
    for (int kk = 0; kk < KG; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(qp + 32 * kk + 8 * lg);
      const float4 c = *reinterpret_cast<const float4*>(qp + 32 * kk + 8 * lg + 4);
      const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float v = hv ? x[s] * qscale2 : 0.0f;
        const _Float16 h = (_Float16)v;
        qhi[kk][s] = h;
        qlo[kk][s] = (_Float16)(v - (float)h);
      }
    }
  }
  const int32_t L = __builtin_amdgcn_readfirstlane(min(max(L_raw, 0), max_len));
  TileWalk tw;
  if constexpr (SELR > 0)
    tw = fused_walk<T, SELR>(fs, max_sel, bg, b, L, L_raw, block, split, units_per_split,
                            smem);
  else
    tw = make_walk<T>(ls, sel_idx, max_sel, bg, L, block, split, units_per_split);
  if constexpr (HM) tw.hsel = sel_hmask + bg * max_sel;
  tw.init(wave);
  float m_run = -INFINITY, l_run = 0.0f;
  float4_t O[2 * KG];
#pragma unroll
  for (int n = 0; n < 2 * KG; ++n) O[n] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const uint8_t* kbase = kc + grp_row_off<K, D>(bg, max_seq, 0);
  const uint8_t* vbase = vc + grp_row_off<K, D>(bg, max_seq, 0);
  const uint8_t* khbase = kc + grp_hi_off<K, D>(bg, max_seq, 0);       // q5_0 fifth bits
  const uint8_t* vhbase = vc + grp_hi_off<K, D>(bg, max_seq, 0);
  const uint8_t* ksb = reinterpret_cast<const uint8_t*>(ksc + bg * int64_t(max_seq) * KG);
  const uint8_t* vsb = reinterpret_cast<const uint8_t*>(vsc + bg * int64_t(max_seq) * KG);
  // Lane loads, per code tile: 16-byte chunk lane % kHcpr of row
  // kHrpl i + lane / kHcpr (q8_0 at D = 128: row 8 i + lane / 8; q4_0 / q5_0
  // at D = 128: row 16 i + lane / 4 of 64-byte nibble rows, 32 channels per
  // chunk).  Scales: KG bytes per lane = the KG / 2 f16 scales of groups
  // (lane % 2) KG / 2 .. of token lane / 2.  Buffer resources with the tile's
  // valid bytes: rows past the length read as zeros.
  // q5_0 also: the fifth bits of the lane's 32 channels of each of its rows
  // (4 bytes at 256 i + 4 lane of the tile's fifth-bit rows, at every D)
  struct Frag {
    int4_t k[kLoads], v[kLoads];
    uint32_t kh[kLoads], vh[kLoads];
    uint2 ks, vs;
    int32_t r0, nvalid;
    uint32_t hm;
  };
  auto issue = [&](Frag& f) {
    int32_t r0 = 0, nv = 0;
    uint32_t hm = ~0u;
    if (tw.more()) tw.next<T, HM>(r0, nv, &hm);
    f.r0 = r0;
    f.nvalid = nv;
    f.hm = hm;
    const uint32_t lo = 16u * uint32_t(lane);
    const int bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * F::kRowBytes);
    const auto kr = tile_rsrc(kbase + int64_t(r0) * F::kRowBytes, bytes);
    const auto vr = tile_rsrc(vbase + int64_t(r0) * F::kRowBytes, bytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      f.k[i] = tile_load(kr, lo + 1024 * i);
      f.v[i] = tile_load(vr, lo + 1024 * i);
    }
    if constexpr (Q5) {
      const int hbytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * F::kHiBytes);
      const auto khr = tile_rsrc(khbase + int64_t(r0) * F::kHiBytes, hbytes);
      const auto vhr = tile_rsrc(vhbase + int64_t(r0) * F::kHiBytes, hbytes);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        f.kh[i] = __builtin_amdgcn_raw_buffer_load_b32(khr, 256u * i + 4u * uint32_t(lane), 0,
                                                        kAuxNontemporal);
        f.vh[i] = __builtin_amdgcn_raw_buffer_load_b32(vhr, 256u * i + 4u * uint32_t(lane), 0,
                                                        kAuxNontemporal);
      }
    }
    const int sbytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * KG * 2);
    const auto ksr = tile_rsrc(ksb + int64_t(r0) * KG * 2, sbytes);
    const auto vsr = tile_rsrc(vsb + int64_t(r0) * KG * 2, sbytes);
    if constexpr (kSb == 2) {
      f.ks = make_uint2(__builtin_amdgcn_raw_buffer_load_b16(ksr, 2u * uint32_t(lane), 0,
                                                             kAuxNontemporal), 0u);
      f.vs = make_uint2(__builtin_amdgcn_raw_buffer_load_b16(vsr, 2u * uint32_t(lane), 0,
                                                             kAuxNontemporal), 0u);
    } else if constexpr (kSb == 4) {
      f.ks = make_uint2(__builtin_amdgcn_raw_buffer_load_b32(ksr, 4u * uint32_t(lane), 0,
                                                             kAuxNontemporal), 0u);
      f.vs = make_uint2(__builtin_amdgcn_raw_buffer_load_b32(vsr, 4u * uint32_t(lane), 0,
                                                             kAuxNontemporal), 0u);
    } else {
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 a = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(ksr, 8u * uint32_t(lane), 0, kAuxNontemporal));
      const u32x2 c = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(vsr, 8u * uint32_t(lane), 0, kAuxNontemporal));
      f.ks = make_uint2(a.x, a.y);
      f.vs = make_uint2(c.x, c.y);
    }
  };
  static_assert(kLoads * 1024 == kTileBytes, "whole 16-byte loads per lane");
  constexpr int kSwz = kCpr < 16 ? kCpr : 16;
  auto sw = [](int rw, int chunk) { return rw * D + 16 * (chunk ^ (rw & (kSwz - 1))); };
  constexpr int kExpUnset = -100000;
  int e_run = kExpUnset;
  constexpr int SPL = KG / 2;          // scales per lane: groups (lane % 2) SPL .. of token lane / 2
  typedef float floatS __attribute__((ext_vector_type(SPL)));

  auto process = [&](auto bufc, Frag& fr) {
    constexpr int kBuf = decltype(bufc)::value;
    uint8_t* kt = smem[wave][kBuf];
    uint8_t* vt = kt + kCodeBytes;
    float* stk = reinterpret_cast<float*>(kt + kScaleOff);          // [T][KG]
    float* stv = stk + T * KG;
    if constexpr (F::kNib) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int rw = kHrpl * i + lane / kHcpr, ch = 2 * (lane % kHcpr);
        int4_t a0, a1;
        if constexpr (Q5) unpack_q5(fr.k[i], fr.kh[i], a0, a1);
        else unpack_q4(fr.k[i], a0, a1);
        *reinterpret_cast<int4_t*>(kt + sw(rw, ch)) = a0;
        *reinterpret_cast<int4_t*>(kt + sw(rw, ch + 1)) = a1;
        if constexpr (Q5) unpack_q5(fr.v[i], fr.vh[i], a0, a1);
        else unpack_q4(fr.v[i], a0, a1);
        *reinterpret_cast<int4_t*>(vt + sw(rw, ch)) = a0;
        *reinterpret_cast<int4_t*>(vt + sw(rw, ch + 1)) = a1;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int rw = kHrpl * i + lane / kHcpr;
        *reinterpret_cast<int4_t*>(kt + sw(rw, lane % kHcpr)) = fr.k[i];
        *reinterpret_cast<int4_t*>(vt + sw(rw, lane % kHcpr)) = fr.v[i];
      }
    }
    // scales: f16 to float; V scales in the running power-of-two unit
    // 2^e_run >= every V scale so far, times 2^kPwShiftGrp
    float kv[SPL], vv[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const uint32_t kw = j < 2 ? fr.ks.x : fr.ks.y, vw = j < 2 ? fr.vs.x : fr.vs.y;
      kv[j] = (j & 1) ? h2f_hi(kw) : h2f_lo(kw);
      vv[j] = (j & 1) ? h2f_hi(vw) : h2f_lo(vw);
    }
    float vmx = vv[0];
#pragma unroll
    for (int j = 1; j < SPL; ++j) vmx = fmaxf(vmx, vv[j]);
    const int32_t vbits = __builtin_amdgcn_readfirstlane(__float_as_int(wave_max(vmx)));
    float unit = 1.0f;
    if (vbits > 0 && vbits < 0x7F800000) {
      const int32_t ex =
          __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(__int_as_float(vbits)));
      if (e_run == kExpUnset) {
        e_run = ex;
      } else if (ex > e_run) {
        unit = ldexpf(1.0f, e_run - ex);
        e_run = ex;
      }
    }
    const int e_use = e_run == kExpUnset ? 0 : e_run;
    {
      floatS ks4, vs4;
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        ks4[j] = kv[j];
        vs4[j] = ldexpf(vv[j], kPwShiftGrp - e_use);
      }
      reinterpret_cast<floatS*>(stk)[lane] = ks4;
      reinterpret_cast<floatS*>(stv)[lane] = vs4;
    }
    const int32_t nvalid = fr.nvalid, r0 = fr.r0;
    const uint32_t hm = fr.hm;
    issue(fr);
    // q.K per group: two 16-token halves, one MFMA pair per 32-channel group
    float sc[8];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float4_t acc[KG];
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
        const int rw = 16 * s + lc;
        const int2_t raw = *reinterpret_cast<const int2_t*>(kt + sw(rw, 2 * kk + lg / 2) +
                                                            8 * (lg & 1));
        const half8_t a = widen_grp<K>(raw);
        acc[kk] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        acc[kk] = mfma_f16_32(a, qhi[kk], acc[kk]);
        acc[kk] = mfma_f16_32(a, qlo[kk], acc[kk]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float* kr = stk + (16 * s + 4 * lg + r) * KG;
        if constexpr (KG == 4) {
          const float4 kss = *reinterpret_cast<const float4*>(kr);
          sc[4 * s + r] = acc[0][r] * kss.x + acc[1][r] * kss.y + acc[2][r] * kss.z +
                          acc[3][r] * kss.w;
        } else {
          float kss[KG];
#pragma unroll
          for (int kk = 0; kk < KG; kk += 2) {
            const float2 v2 = *reinterpret_cast<const float2*>(kr + kk);
            kss[kk] = v2.x;
            kss[kk + 1] = v2.y;
          }
          float a = acc[0][r] * kss[0];
#pragma unroll
          for (int kk = 1; kk < KG; ++kk) a += acc[kk][r] * kss[kk];
          sc[4 * s + r] = a;
        }
      }
    }
    if (nvalid < T || (ntok > 1 && r0 + T > L - ntok + 1)) {   // wave-uniform
      // rows past the row's length; with a chunk of query tokens, column lc
      // is token lc >> gsh, which sees the positions below
      // L - (ntok - 1 - token) only
      const int32_t lim = min(nvalid, L - (ntok - 1 - (lc >> qr.gsh)) - r0);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sc[e] = 16 * (e / 4) + 4 * lg + e % 4 < lim ? sc[e] : -INFINITY;
    }
    if constexpr (HM) {
      // the heads that did not choose this block leave it out
      const bool off = ((hm >> lc) & 1u) == 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = off ? -INFINITY : sc[e];
    }
    tile_softmax<G, 2, true>(sc, m_run, l_run, O, unit);
    // P.V: per 16-channel block n (group n / 2), A = weight x V scale of
    // (token tok(lg, e), group), f16 high + low; B = V codes of channels
    // 16 n + lc for tokens tok(lg, 0..7) (the int8 kernel's transposing read)
    float vsr[8][KG];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float* vr = stv + (16 * (e / 4) + 4 * lg + e % 4) * KG;
#pragma unroll
      for (int kk = 0; kk < KG; kk += 2) {
        if (KG >= 4 && kk % 4 == 0) {
          const float4 v4 = *reinterpret_cast<const float4*>(vr + kk);
          vsr[e][kk] = v4.x; vsr[e][kk + 1] = v4.y; vsr[e][kk + 2] = v4.z; vsr[e][kk + 3] = v4.w;
        } else if (KG < 4) {
          const float2 v2 = *reinterpret_cast<const float2*>(vr + kk);
          vsr[e][kk] = v2.x; vsr[e][kk + 1] = v2.y;
        }
      }
    }
    const int tr_row = 16 * ((lc / 2) / 4) + 4 * lg + (lc / 2) % 4;
#pragma unroll
    for (int grp = 0; grp < KG; ++grp) {
      half8_t phi, plo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float vsg = vsr[e][grp];
        const float pw = sc[e] * vsg;
        const _Float16 h = (_Float16)pw;
        phi[e] = h;
        plo[e] = (_Float16)(pw - (float)h);
      }
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const int n = 2 * grp + nn;
        const int off = sw(tr_row, n) + 8 * (lc & 1);
        const int2_t raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SKV_LDS int2_t*)(vt + off));
        const half8_t bv = widen_grp<K>(raw);
        O[n] = mfma_f16_32(phi, bv, O[n]);
        O[n] = mfma_f16_32(plo, bv, O[n]);
      }
    }
  };

  Frag f0, f1;
  const int32_t n_mine = tw.count();
  issue(f0);
  issue(f1);
  for (int32_t t = 0; t + 1 < n_mine; t += 2) {
    process(std::integral_constant<int, 0>{}, f0);
    process(std::integral_constant<int, 1>{}, f1);
  }
  if (n_mine & 1) process(std::integral_constant<int, 0>{}, f0);
  if (e_run != kExpUnset) {
#pragma unroll
    for (int n = 0; n < 2 * KG; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) O[n][r] = ldexpf(O[n][r], e_run - kPwShiftGrp);
    }
  }
  finish_mfma<G>(m_run, l_run, O, reinterpret_cast<float*>(&smem[0][0][0]), ws_m, ws_l, ws_o,
                 qr, b, g, n_split, split);
}

}  // namespace

namespace {

template <int D>
hipError_t launch_append_grouped_d(const skv_cache& c, const int32_t* pos0, int32_t n_new,
                                   const void* k_new, const void* v_new, hipStream_t stream) {
  const int32_t max_blocks = (c.max_seq + c.block - 1) / c.block;
  const int32_t n_aff = (n_new + c.block - 2) / c.block + 1;
  const dim3 grid(n_aff, c.n_kv_heads, c.batch);
  uint16_t* ks = reinterpret_cast<uint16_t*>(c.k_scale);
  uint16_t* vs = reinterpret_cast<uint16_t*>(c.v_scale);
#define SKV_APP_GRP(KK)                                                                         \
  append_grp_kernel<KK, D><<<grid, kAppendThreads, 0, stream>>>(                                \
      static_cast<uint8_t*>(c.k), static_cast<uint8_t*>(c.v), ks, vs, c.kmin, c.kmax,          \
      static_cast<const float*>(k_new), static_cast<const float*>(v_new), pos0, n_new,         \
      c.n_kv_heads, c.max_seq, c.block, max_blocks)
  switch (c.kv_dtype) {
    case SKV_Q8_0: SKV_APP_GRP(kQ8); break;
    case SKV_Q4_0: SKV_APP_GRP(kQ4); break;
    case SKV_Q5_0: SKV_APP_GRP(kQ5); break;
    default: return hipErrorInvalidValue;
  }
#undef SKV_APP_GRP
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_grouped_d(const DecodeParams& p, int G, hipStream_t stream) {
  const skv_cache& c = *p.c;
  const int32_t B = c.batch, S = p.n_split, nt = p.n_tok;
  const int32_t Hq = p.n_heads * nt;          // query rows: tokens x heads
  float* ws_m = p.ws + ws_m_offset(B, Hq, S);
  float* ws_l = p.ws + ws_l_offset(B, Hq, S);
  float* ws_o = p.ws + ws_o_offset(B, Hq, S);
  int32_t ups;
  if (p.sel_idx != nullptr) {
    ups = (p.max_sel + S - 1) / S;
  } else {
    const int32_t nb_max = (p.max_len + c.block - 1) / c.block;
    ups = (nb_max + S - 1) / S;
  }
  ups = ups < 1 ? 1 : ups;
  const int64_t n_wg = int64_t(S) * c.n_kv_heads * B;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(n_wg));
  const int32_t n_rows = c.n_kv_heads * B;
  const float scale2 = p.softmax_scale * kLog2e;
  const uint8_t* kc = static_cast<const uint8_t*>(c.k);
  const uint8_t* vc = static_cast<const uint8_t*>(c.v);
  const uint16_t* ks = reinterpret_cast<const uint16_t*>(c.k_scale);
  const uint16_t* vs = reinterpret_cast<const uint16_t*>(c.v_scale);
  const int fr = p.fused_r;
  const bool hmk = p.sel_hmask != nullptr;
#define SKV_GRP(GG, Q, SR, HMK)                                                                 \
  decode_grp_mfma<GG, Q, SR, D, HMK><<<grid, kMThreads, 0, stream>>>(                          \
      kc, vc, ks, vs, p.q, p.seq_len, p.sel_idx, p.sel_cnt, p.max_sel, c.n_kv_heads,           \
      c.max_seq, c.block, p.max_len, S, n_rows, ups, scale2, ws_m, ws_l, ws_o, p.fsel,         \
      p.sel_hmask, nt)
#define SKV_GRP_Q(GG, Q)                           \
  if (hmk) SKV_GRP(GG, Q, 0, true);                \
  else if (fr == 2) SKV_GRP(GG, Q, 2, false);      \
  else if (fr == 4) SKV_GRP(GG, Q, 4, false);      \
  else if (fr > 0) SKV_GRP(GG, Q, kFusedSelR, false); \
  else SKV_GRP(GG, Q, 0, false)
#define SKV_GRP_G(GG)                                          \
  if (c.kv_dtype == SKV_Q4_0) { SKV_GRP_Q(GG, kQ4); }            \
  else if (c.kv_dtype == SKV_Q5_0) { SKV_GRP_Q(GG, kQ5); }       \
  else { SKV_GRP_Q(GG, kQ8); }
// 16 columns: query-token chunks only (no fused variants)
#define SKV_GRP_Q16(Q)                                 \
  if (hmk) SKV_GRP(16, Q, 0, true);                    \
  else SKV_GRP(16, Q, 0, false)
  switch (G) {
    case 1: SKV_GRP_G(1); break;
    case 2: SKV_GRP_G(2); break;
    case 4: SKV_GRP_G(4); break;
    case 8: SKV_GRP_G(8); break;
    default:
      if (c.kv_dtype == SKV_Q4_0) { SKV_GRP_Q16(kQ4); }
      else if (c.kv_dtype == SKV_Q5_0) { SKV_GRP_Q16(kQ5); }
      else { SKV_GRP_Q16(kQ8); }
      break;
  }
#undef SKV_GRP_Q16
#undef SKV_GRP_G
#undef SKV_GRP_Q
#undef SKV_GRP
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_grouped(const skv_cache& c, const int32_t* pos0, int32_t n_new,
                                 const void* k_new, const void* v_new, hipStream_t stream) {
  switch (c.head_dim) {
    case 64: return launch_append_grouped_d<64>(c, pos0, n_new, k_new, v_new, stream);
    case 128: return launch_append_grouped_d<128>(c, pos0, n_new, k_new, v_new, stream);
    case 256: return launch_append_grouped_d<256>(c, pos0, n_new, k_new, v_new, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_grouped(const DecodeParams& p, hipStream_t stream) {
  const skv_cache& c = *p.c;
  if (c.block % 16 != 0) return hipErrorInvalidValue;
  // MFMA columns per KV head: n_tok query tokens x the group's heads
  const int32_t nt = p.n_tok;
  if (nt != 1 && nt != 2 && nt != 4 && nt != 8) return hipErrorInvalidValue;
  const int G = (p.n_heads / c.n_kv_heads) * nt;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return hipErrorInvalidValue;
  if (p.app.k_new != nullptr || p.dbg_logits != nullptr) return hipErrorInvalidValue;
  if (nt > 1 && p.fused_r > 0) return hipErrorInvalidValue;
  if (p.sel_hmask != nullptr && (p.sel_idx == nullptr || p.fused_r > 0))
    return hipErrorInvalidValue;
  switch (c.head_dim) {
    case 64: return launch_decode_grouped_d<64>(p, G, stream);
    case 128: return launch_decode_grouped_d<128>(p, G, stream);
    case 256: return launch_decode_grouped_d<256>(p, G, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace skv
