// A 4-bit key index and its GQA-shared scan with deterministic score bounds:
// a token-level candidate generator ("Certified Sparse Attention via
// Perturbed Retrieval": the abstract -- a 4-bit scan with deterministic
// bounds, shared across a GQA group, generates the candidates exactly but
// reads every key; the appendix layout table -- 4-bit codes, 64 B per token
// at D = 128, per-block per-channel fp32 lo / step; the ablation table --
// scanning per query head instead reads 2.7-4.0x the bytes).
//
// Index (per block of `block` tokens, per channel d; f16 cache keys):
//   lo = min k, step = fl32(fl32(max k - lo) / 15), code = clamp(rint(
//   fl32(fl32(k - lo) / step)), 0, 15) (0 if step == 0), recon = fl32(lo +
//   fl32(step * code)), err = max |fl32(k - recon)|, each one IEEE float32
//   operation (no fused multiply-add), so |k - recon| <= err.
// Bounds of token t in block b for query head h:
//   s~ = sum_d q_d recon_td = a_h + sum_d (q_d step_d) code_td,
//   a_h = sum_d q_d lo_d, r_h = sum_d |q_d| err_d,
//   LB = s~ - r_h <= q.k_t <= UB = s~ + r_h.
// Candidates of head h for a margin delta: UB_t >= max_u LB_u - delta.
//
// Head dims D = 64, 128, 256 (the index rows are D / 2 bytes of nibbles and
// D floats of lo / step / err per block).
//
// Kernels: scan4_build (one workgroup per (block, KV head, sequence));
// scan4_bounds (pass 1: split-K parts as the decode kernels, the codes of a
// KV head read once for its G query heads: q.K~ on the matrix cores with the
// codes widened to f16 as A and (q * step) as f16 high + low parts as B, one
// MFMA pair per 32 channels; writes UB per (head, token) and each part's
// largest LB per head); scan4_select (pass 2: the threshold from the parts'
// LB maxima, a ballot per 64 tokens into the candidate bitmask, the count).
#include <type_traits>

#include "decode_core.h"
#include "device_common.h"
#include "grouped_core.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int kLevels = 15;
constexpr int kScanBlockMax = 256;

// ------------------------------------------------------------------- build
// The block's keys (up to 64 tokens at a time) are staged in LDS with
// 16-byte loads, all in flight at once, then thread d < D reduces channel d
// (head dim D = 64, 128 or 256; a token's row of nibbles is D / 2 bytes).
constexpr int kBuildChunk = 64;
template <int D>
__global__ void __launch_bounds__(256)
scan4_build(const uint16_t* __restrict__ kc, const int32_t* __restrict__ pos0,
            const int32_t* __restrict__ seq_len, int32_t Hkv, int32_t max_seq, int32_t max_len,
            int32_t block, int32_t max_blocks, uint8_t* __restrict__ codes4,
            float* __restrict__ lo_out, float* __restrict__ step_out,
            float* __restrict__ err_out) {
  constexpr int kRow4 = D / 2;
  __shared__ uint8_t cs[kScanBlockMax][D];
  __shared__ __attribute__((aligned(16))) uint16_t ks[kBuildChunk][D];
  const int32_t g = blockIdx.y, b = blockIdx.z;
  const int32_t L = min(max(seq_len[b], 0), max_len);
  const int32_t p0 = pos0[b];
  const int32_t j = int32_t(blockIdx.x);
  const int32_t nb = (L + block - 1) / block;
  if (p0 < 0 || j < p0 / block || j >= nb) return;
  const int32_t t0 = j * block, t1 = min(t0 + block, L);
  const int64_t bg = int64_t(b) * Hkv + g;
  const int d = threadIdx.x;
  const uint4* krow = reinterpret_cast<const uint4*>(kc + (bg * max_seq) * D);
  // one chunk of rows into LDS: 16 bytes per thread per instruction
  auto stage = [&](int32_t c0, int32_t n) {
    __syncthreads();
    for (int32_t e = threadIdx.x; e < n * (D / 8); e += 256)
      reinterpret_cast<uint4*>(&ks[0][0])[e] = krow[int64_t(c0) * (D / 8) + e];
    __syncthreads();
  };
  float mn = INFINITY, mx = -INFINITY;
  for (int32_t c0 = t0; c0 < t1; c0 += kBuildChunk) {
    const int32_t n = min(kBuildChunk, t1 - c0);
    stage(c0, n);
    if (d < D) {
      for (int32_t t = 0; t < n; ++t) {
        const float x = h2f(ks[t][d]);
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
    }
  }
  float lo = mn, st = 0.0f, err = 0.0f;
  if (d < D) st = __fdiv_rn(__fsub_rn(mx, mn), float(kLevels));
  for (int32_t c0 = t0; c0 < t1; c0 += kBuildChunk) {
    const int32_t n = min(kBuildChunk, t1 - c0);
    if (block > kBuildChunk) stage(c0, n);           // else the chunk is still staged
    if (d >= D) continue;
    for (int32_t t = c0; t < c0 + n; ++t) {
      const float x = h2f(ks[t - c0][d]);
      float c = 0.0f;
      if (st > 0.0f) c = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(x, lo), st)), 0.0f), float(kLevels));
      // the product rounds on its own (the empty asm keeps the compiler from
      // fusing it with the sum into one multiply-add)
      float prod = st * c;
      asm volatile("" : "+v"(prod));
      const float rec = lo + prod;
      err = fmaxf(err, fabsf(__fsub_rn(x, rec)));
      cs[t - t0][d] = uint8_t(c);
    }
  }
  if (d < D) {
    const int64_t o = (bg * max_blocks + j) * D + d;
    lo_out[o] = lo;
    step_out[o] = st;
    err_out[o] = err;
  }
  __syncthreads();
  // pack: byte i of a token's row = channel 2i (low nibble), 2i + 1 (high)
  const int32_t n = (t1 - t0) * kRow4;
  uint8_t* dst = codes4 + (bg * max_seq + t0) * kRow4;
  for (int32_t e = threadIdx.x; e < n; e += 256) {
    const int32_t t = e / kRow4, i = e % kRow4;
    dst[e] = uint8_t(cs[t][2 * i] | (cs[t][2 * i + 1] << 4));
  }
}

// The key an int8 or group-wise cache holds at token t, channel d of row bg
// (sequence x KV head): code x scale as one float32 product (no fused
// multiply-add with what follows).
template <int D, int KV>
__device__ __forceinline__ float cache_key(const uint8_t* __restrict__ kc,
                                           const void* __restrict__ ks, int64_t bg,
                                           int32_t max_seq, int32_t t, int d) {
  if constexpr (KV == SKV_I8) {
    const int code = int(reinterpret_cast<const int8_t*>(kc)[(bg * max_seq + t) * D + d]);
    const float s = static_cast<const float*>(ks)[bg * max_seq + t];
    return __fmul_rn(float(code), s);
  } else {
    constexpr int K = KV == SKV_Q8_0 ? kQ8 : KV == SKV_Q4_0 ? kQ4 : kQ5;
    using F = GrpFmt<K, D>;
    const uint8_t* row = kc + grp_row_off<K, D>(bg, max_seq, t);
    int code;
    if constexpr (K == kQ8) {
      code = int(int8_t(row[d]));
    } else {
      const uint32_t by = row[d / 2];
      uint32_t n = (d & 1) ? (by >> 4) : (by & 15u);
      if constexpr (K == kQ5) {
        const uint8_t* hi = kc + grp_hi_off<K, D>(bg, max_seq, t);
        n |= ((uint32_t(hi[d / 8]) >> (d % 8)) & 1u) << 4;
      }
      code = int(n) - F::kBias;
    }
    const float s =
        h2f(static_cast<const uint16_t*>(ks)[(bg * max_seq + t) * F::kGroups + d / kGroup]);
    return __fmul_rn(float(code), s);
  }
}

// The index of an int8 or group-wise cache: as scan4_build, each key read
// as the cache holds it (cache_key), channel d by thread d < D.
template <int D, int KV>
__global__ void __launch_bounds__(256)
scan4_build_q(const uint8_t* __restrict__ kc, const void* __restrict__ ks,
              const int32_t* __restrict__ pos0, const int32_t* __restrict__ seq_len, int32_t Hkv,
              int32_t max_seq, int32_t max_len, int32_t block, int32_t max_blocks,
              uint8_t* __restrict__ codes4, float* __restrict__ lo_out,
              float* __restrict__ step_out, float* __restrict__ err_out) {
  constexpr int kRow4 = D / 2;
  __shared__ uint8_t cs[kScanBlockMax][D];
  const int32_t g = blockIdx.y, b = blockIdx.z;
  const int32_t L = min(max(seq_len[b], 0), max_len);
  const int32_t p0 = pos0[b];
  const int32_t j = int32_t(blockIdx.x);
  const int32_t nb = (L + block - 1) / block;
  if (p0 < 0 || j < p0 / block || j >= nb) return;
  const int32_t t0 = j * block, t1 = min(t0 + block, L);
  const int64_t bg = int64_t(b) * Hkv + g;
  const int d = threadIdx.x;
  float lo = 0.0f, st = 0.0f, err = 0.0f;
  if (d < D) {
    float mn = INFINITY, mx = -INFINITY;
    for (int32_t t = t0; t < t1; ++t) {
      const float x = cache_key<D, KV>(kc, ks, bg, max_seq, t, d);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    lo = mn;
    st = __fdiv_rn(__fsub_rn(mx, mn), float(kLevels));
    for (int32_t t = t0; t < t1; ++t) {
      const float x = cache_key<D, KV>(kc, ks, bg, max_seq, t, d);
      float c = 0.0f;
      if (st > 0.0f) c = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(x, lo), st)), 0.0f), float(kLevels));
      float prod = st * c;
      asm volatile("" : "+v"(prod));
      const float rec = lo + prod;
      err = fmaxf(err, fabsf(__fsub_rn(x, rec)));
      cs[t - t0][d] = uint8_t(c);
    }
    const int64_t o = (bg * max_blocks + j) * D + d;
    lo_out[o] = lo;
    step_out[o] = st;
    err_out[o] = err;
  }
  __syncthreads();
  const int32_t n = (t1 - t0) * kRow4;
  uint8_t* dst = codes4 + (bg * max_seq + t0) * kRow4;
  for (int32_t e = threadIdx.x; e < n; e += 256) {
    const int32_t t = e / kRow4, i = e % kRow4;
    dst[e] = uint8_t(cs[t][2 * i] | (cs[t][2 * i + 1] << 4));
  }
}

// ------------------------------------------------------------ pass 1: bounds
// 8 nibbles (4 bytes: channels 2i, 2i + 1 per byte) to 8 exact f16 codes
// 0..15 in the order c0 c2 c4 c6 c1 c3 c5 c7: v_perm_b32 puts each nibble
// under a 0x64 high byte (f16 1024 + c), one packed subtraction per pair
// removes the 1024.  kNibPos maps channel s of the 8 to its position.
__device__ __forceinline__ half8_t nibbles_to_half8(uint32_t x) {
  typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
  const uint32_t ev = x & 0x0F0F0F0Fu, od = (x >> 4) & 0x0F0F0F0Fu;
  constexpr uint32_t kSel01 = 0x04010400u;   // (0x64, x1, 0x64, x0)
  constexpr uint32_t kSel23 = 0x04030402u;   // (0x64, x3, 0x64, x2)
  const half2_t off = half2_t{(_Float16)1024.0f, (_Float16)1024.0f};
  const half2_t p0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, ev, kSel01)) - off;
  const half2_t p1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, ev, kSel23)) - off;
  const half2_t p2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, od, kSel01)) - off;
  const half2_t p3 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, od, kSel23)) - off;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
__device__ __forceinline__ constexpr int nib_pos(int s) { return (s & 1) ? 4 + (s >> 1) : (s >> 1); }

// T-token tiles (T = 64 when the block is a multiple of 64, else 32), two in
// flight per wavefront.  The codes go straight from memory into the MFMA
// operand registers: lane (lg, lc) loads the D / 8 bytes of token 16 s + lc
// that hold channels CW lg .. CW lg + CW - 1 (CW = D / 4: 16 B, channels
// 32 lg .. 32 lg + 31 at D = 128), and MFMA kk (kk < D / 32) takes channels
// CW lg + 8 kk .. + 7 as its K index 8 lg .. 8 lg + 7 (the query side uses
// the same assignment, so the dot is over all D channels).  Each tile's
// refill also requests its block's lo, step and err rows (D / 16 bytes of
// each per lane, 12 D bytes per tile), staged through LDS, so no tile waits
// on a separate round trip for its block's operands.
// NW 32-bit words of one lane, as one vector register tuple.
template <int NW>
struct LaneWords {
  typedef unsigned int V __attribute__((ext_vector_type(NW)));
  V w;
};
template <int NW, int AUX>
__device__ __forceinline__ LaneWords<NW> load_words(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  LaneWords<NW> r;
  if constexpr (NW == 1) {
    r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, AUX);
  } else if constexpr (NW == 2) {
    r.w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, AUX));
  } else if constexpr (NW == 4) {
    r.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, AUX));
  } else {
    static_assert(NW == 8, "at most 32 bytes per lane");
    const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, AUX));
    const u32x4 hi =
        __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, AUX));
    r.w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  return r;
}
// NW words to LDS at a 4 NW-byte aligned address, in one store.
template <int NW>
__device__ __forceinline__ void store_words(float* dst, const LaneWords<NW>& v) {
  static_assert(NW == 1 || NW == 2 || NW == 4, "at most 16 bytes per lane");
  *reinterpret_cast<typename LaneWords<NW>::V*>(dst) = v.w;
}
template <int D, int G, int T>
__global__ void __launch_bounds__(kMThreads, D > 128 ? 1 : 2)
scan4_bounds(const uint8_t* __restrict__ codes4, const float* __restrict__ lo_in,
             const float* __restrict__ step_in, const float* __restrict__ err_in,
             const float* __restrict__ q, const int32_t* __restrict__ seq_len, int32_t Hkv,
             int32_t max_seq, int32_t block, int32_t max_blocks, int32_t max_len,
             int32_t n_split, int32_t n_rows, int32_t ups, float* __restrict__ ub_out,
             float* __restrict__ lbmax, int32_t* __restrict__ cand_cnt) {
  constexpr int kSubs = T / 16;                              // 16-token MFMA row blocks
  constexpr int KS = D / 32;                                 // MFMA steps (per 32 channels)
  constexpr int CW = D / 4;                                  // channels per lane group
  constexpr int kCwLog = CW == 16 ? 4 : CW == 32 ? 5 : 6;
  constexpr int kRow4 = D / 2;                               // nibble bytes per token
  constexpr int NPW = D / 64;                                // lo / step / err floats per lane
  __shared__ __attribute__((aligned(16))) float sprm[kMWaves][2][3][D];    // lo, step, err
  // the B operands of the tile's block (f16 high, low) for MFMA lane
  // (lg, lc < G) at entry lg G + lc, and the per-head scalars, written and
  // read by one wavefront
  __shared__ __attribute__((aligned(16))) uint32_t sbw[kMWaves][2][KS][4 * G][4];
  __shared__ float shd[kMWaves][3][16];
  __shared__ float red[kMWaves][16];
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t split = int32_t(slot % uint32_t(n_split));
  const uint32_t row = xcd_row(slot / uint32_t(n_split), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const int32_t H = Hkv * G;
  const int64_t bg = int64_t(b) * Hkv + g;
  const bool hv = lc < G;
  if (split == 0 && threadIdx.x < G) cand_cnt[int64_t(b) * H + g * G + threadIdx.x] = 0;
  const int32_t L_raw = seq_len[b];
  // The per-block operands are computed spread over the wavefront: lane l
  // takes head ph = l / LPH of the group and channels pc .. pc + CPL - 1
  // (LPH = 64 / G lanes per head, CPL = 2 G channels each), instead of every
  // lane computing its own 32 channels for its MFMA column (of which only G
  // of 16 are heads).
  constexpr int LPH = kWave / G, CPL = D / LPH;
  const int ph = lane / LPH, pc = (lane % LPH) * CPL;
  float qd[CPL];
  {
    const float* qp = q + (int64_t(b) * H + g * G + ph) * D + pc;
    if constexpr (CPL == 1) {
      qd[0] = qp[0];
    } else {
#pragma unroll
      for (int e = 0; e < CPL; e += 2) {
        const float2 v2 = *reinterpret_cast<const float2*>(qp + e);
        qd[e] = v2.x;
        qd[e + 1] = v2.y;
      }
    }
  }
  const int32_t L = __builtin_amdgcn_readfirstlane(min(max(L_raw, 0), max_len));
  const ListSeed ls{};
  TileWalk tw = make_walk<T>(ls, nullptr, 0, bg, L, block, split, ups);
  tw.init(wave);
  const uint8_t* cbase = codes4 + bg * int64_t(max_seq) * kRow4;
  const uint8_t* lbase = reinterpret_cast<const uint8_t*>(lo_in + bg * int64_t(max_blocks) * D);
  const uint8_t* sbase = reinterpret_cast<const uint8_t*>(step_in + bg * int64_t(max_blocks) * D);
  const uint8_t* ebase = reinterpret_cast<const uint8_t*>(err_in + bg * int64_t(max_blocks) * D);
  float* urow = ub_out + (int64_t(b) * H + g * G + (hv ? lc : 0)) * int64_t(max_len);
  float lb_run = -INFINITY;
  struct Frag {
    LaneWords<KS> c[kSubs];  // token 16 s + lc, channels CW lg .. CW lg + CW - 1
    LaneWords<NPW> p[3];     // channels NPW lane .. NPW lane + NPW - 1 of lo, step, err
    int32_t r0, nvalid;
  };
  // Every refill issues the same loads, through resources of zero records
  // once the walk is over (they return zeros and touch no memory).
  auto issue = [&](Frag& f) {
    int32_t r0 = 0, nv = 0;
    if (tw.more()) tw.next<T>(r0, nv);
    f.r0 = r0;
    f.nvalid = nv;
    const int bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * kRow4);
    const auto cr = tile_rsrc(cbase + int64_t(r0) * kRow4, bytes);
#pragma unroll
    for (int i = 0; i < kSubs; ++i)
      f.c[i] = load_words<KS, kAuxNontemporal>(
          cr, uint32_t(16 * kRow4 * i + kRow4 * lc + (D / 8) * lg));
    const int pbytes = __builtin_amdgcn_readfirstlane(nv > 0 ? D * 4 : 0);
    const int64_t po = int64_t(r0 / block) * D * 4;
    const uint8_t* bases[3] = {lbase, sbase, ebase};
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const auto pr = tile_rsrc(bases[a] + po, pbytes);
      f.p[a] = load_words<NPW, 0>(pr, 4u * NPW * uint32_t(lane));
    }
  };
  auto process = [&](auto bufc, Frag& fr) {
    constexpr int kBuf = decltype(bufc)::value;
    float(*pm)[D] = sprm[wave][kBuf];
#pragma unroll
    for (int a = 0; a < 3; ++a) store_words<NPW>(&pm[a][NPW * lane], fr.p[a]);
    LaneWords<KS> cv[kSubs];
#pragma unroll
    for (int i = 0; i < kSubs; ++i) cv[i] = fr.c[i];
    const int32_t nvalid = fr.nvalid, r0 = fr.r0;
    issue(fr);
    if (nvalid <= 0) return;               // wave-uniform
    // the LDS stores above precede these reads (one wavefront, in order)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // the block's operands: B = q * step per (head, channel), scaled by a
    // power of two per head so that its largest value lies in [2^13, 2^14)
    // (the f16 low parts stay normal; the MFMA result is scaled back
    // exactly); a_h = sum q lo, r_h = sum |q| err
    float pa = 0.0f, pr = 0.0f, mw = 0.0f;
    float wv[CPL];
    if constexpr (CPL == 1) {
      wv[0] = qd[0] * pm[1][pc];
      mw = fabsf(wv[0]);
      pa = qd[0] * pm[0][pc];
      pr = fabsf(qd[0]) * pm[2][pc];
    } else {
#pragma unroll
      for (int e = 0; e < CPL; e += 2) {
        const float2 s2 = *reinterpret_cast<const float2*>(&pm[1][pc + e]);
        const float2 l2 = *reinterpret_cast<const float2*>(&pm[0][pc + e]);
        const float2 e2 = *reinterpret_cast<const float2*>(&pm[2][pc + e]);
        const float sv[2] = {s2.x, s2.y}, lv[2] = {l2.x, l2.y}, ev[2] = {e2.x, e2.y};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          wv[e + i] = qd[e + i] * sv[i];
          mw = fmaxf(mw, fabsf(wv[e + i]));
          pa += qd[e + i] * lv[i];
          pr += fabsf(qd[e + i]) * ev[i];
        }
      }
    }
    // the head's LPH lanes
#pragma unroll
    for (int o = 1; o < LPH; o <<= 1) {
      mw = fmaxf(mw, __shfl_xor(mw, o));
      pa += __shfl_xor(pa, o);
      pr += __shfl_xor(pr, o);
    }
    {
      const int we = mw > 0.0f ? 14 - __builtin_amdgcn_frexp_expf(mw) : 0;
      // channel c lies in MFMA step (c % CW) / 8 at lane entry G (c / CW) +
      // head, position nib_pos(c % 8) of the 8 f16 (the A side's order):
      // channels c, c + 2 (c % 4 < 2) share one 32-bit word
      auto split = [&](float x, uint16_t& h, uint16_t& l) {
        const float w = ldexpf(x, we);
        const _Float16 hh = (_Float16)w;
        h = __builtin_bit_cast(uint16_t, hh);
        l = __builtin_bit_cast(uint16_t, (_Float16)(w - (float)hh));
      };
      if constexpr (CPL >= 4) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          if ((e & 3) >= 2) continue;
          const int c = pc + e;
          uint16_t h0, l0, h1, l1;
          split(wv[e], h0, l0);
          split(wv[e + 2], h1, l1);
          const int kk = (c >> 3) & (CW / 8 - 1), col = G * (c >> kCwLog) + ph,
                    wd = nib_pos(c & 7) >> 1;
          sbw[wave][0][kk][col][wd] = uint32_t(h0) | (uint32_t(h1) << 16);
          sbw[wave][1][kk][col][wd] = uint32_t(l0) | (uint32_t(l1) << 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const int c = pc + e;
          uint16_t h0, l0;
          split(wv[e], h0, l0);
          const int kk = (c >> 3) & (CW / 8 - 1), col = G * (c >> kCwLog) + ph,
                    pos = nib_pos(c & 7);
          reinterpret_cast<uint16_t*>(&sbw[wave][0][kk][col][0])[pos] = h0;
          reinterpret_cast<uint16_t*>(&sbw[wave][1][kk][col][0])[pos] = l0;
        }
      }
      if (lane % LPH == 0) {
        shd[wave][0][ph] = pa;
        shd[wave][1][ph] = pr;
        shd[wave][2][ph] = __int_as_float(we);
      }
    }
    // the stores above precede these reads (one wavefront, in order)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    half8_t whi[KS], wlo[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      whi[kk] = hv ? *reinterpret_cast<const half8_t*>(&sbw[wave][0][kk][G * lg + (hv ? lc : 0)][0]) : half8_t{};
      wlo[kk] = hv ? *reinterpret_cast<const half8_t*>(&sbw[wave][1][kk][G * lg + (hv ? lc : 0)][0]) : half8_t{};
    }
    const float a_h = hv ? shd[wave][0][lc] : 0.0f;
    const float r_h = hv ? shd[wave][1][lc] : 0.0f;
    const int w_exp = hv ? __float_as_int(shd[wave][2][lc]) : 0;
    const float w_scale = ldexpf(1.0f, -w_exp);
    const bool full = nvalid == T;         // wave-uniform
    float st_max = -INFINITY;
#pragma unroll
    for (int s = 0; s < kSubs; ++s) {
      float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        // token 16 s + lc, channels CW lg + 8 kk .. + 7: 4 bytes of nibbles
        const half8_t a = nibbles_to_half8(cv[s].w[kk]);
        acc = mfma_f16_32(a, whi[kk], acc);
        acc = mfma_f16_32(a, wlo[kk], acc);
      }
      // st = acc 2^-w_exp + a_h in one rounding (the scaling is exact); the
      // tile's LB is its largest st less r_h (subtracting r_h is monotone)
      float st[4], ub[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st[r] = __builtin_fmaf(acc[r], w_scale, a_h);
        ub[r] = st[r] + r_h;
      }
      if (full) {
#pragma unroll
        for (int r = 0; r < 4; ++r) st_max = fmaxf(st_max, st[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st_max = 16 * s + 4 * lg + r < nvalid ? fmaxf(st_max, st[r]) : st_max;
      }
      if (hv) {
        const int32_t t = r0 + 16 * s + 4 * lg;
        if (16 * s + 4 * lg + 3 < nvalid) {
          *reinterpret_cast<float4*>(urow + t) = make_float4(ub[0], ub[1], ub[2], ub[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * s + 4 * lg + r < nvalid) urow[t + r] = ub[r];
        }
      }
    }
    lb_run = fmaxf(lb_run, st_max - r_h);
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
  // the part's largest LB per head: over the 4 lane groups, then the waves
  lb_run = rows_max(lb_run);
  if (lane < 16) red[wave][lane] = lb_run;
  __syncthreads();
  if (threadIdx.x < G) {
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) m = fmaxf(m, red[w][threadIdx.x]);
    lbmax[(int64_t(b) * H + g * G + threadIdx.x) * n_split + split] = m;
  }
}

// ------------------------------------------------------- pass 2: candidates
// One workgroup per (4096-token chunk, query head, sequence): the threshold
// max LB - delta from the parts' maxima, one ballot per 64 tokens, one count
// added per workgroup.
constexpr int kSelectChunk = 4096;
constexpr int kSelectPer = kSelectChunk / 256;     // tokens per thread and chunk
__global__ void __launch_bounds__(256)
scan4_select(const float* __restrict__ ub, const float* __restrict__ lbmax,
             const int32_t* __restrict__ seq_len, int32_t H, int32_t max_len, int32_t n_split,
             float delta, int32_t words, uint32_t* __restrict__ cand,
             int32_t* __restrict__ cand_cnt) {
  __shared__ float thr;
  __shared__ int32_t wc[4];
  const int32_t h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = int64_t(b) * H + h;
  const int32_t L = min(max(seq_len[b], 0), max_len);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int32_t c0 = int32_t(blockIdx.x) * kSelectChunk;
  // every UB value of this thread is requested before the threshold is
  // known (one round trip for both)
  float u[kSelectPer];
#pragma unroll
  for (int i = 0; i < kSelectPer; ++i) {
    const int32_t t = c0 + 256 * i + 64 * wave + lane;
    u[i] = t < L ? ub[bh * max_len + t] : 0.0f;
  }
  if (wave == 0) {
    float m = -INFINITY;
    for (int32_t i = lane; i < n_split; i += kWave) m = fmaxf(m, lbmax[bh * n_split + i]);
    m = wave_max(m);
    if (lane == 0) thr = m - delta;
  }
  __syncthreads();
  const float th = thr;
  int32_t n = 0;
#pragma unroll
  for (int i = 0; i < kSelectPer; ++i) {
    const int32_t t0 = c0 + 256 * i + 64 * wave;
    const bool c = t0 + lane < L && u[i] >= th;
    const uint64_t bal = __ballot(int(c));
    const int32_t w0 = t0 / 32;
    if (t0 < max_len) {
      if (lane == 0 && w0 < words) cand[bh * words + w0] = uint32_t(bal & 0xFFFFFFFFu);
      if (lane == 0 && w0 + 1 < words) cand[bh * words + w0 + 1] = uint32_t(bal >> 32);
    }
    n += int32_t(__popcll(bal));
  }
  if (lane == 0) wc[wave] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t tot = wc[0] + wc[1] + wc[2] + wc[3];
    if (tot != 0) atomicAdd(&cand_cnt[bh], tot);
  }
}

}  // namespace

hipError_t launch_scan4_build(const skv_cache& c, const int32_t* pos0, const int32_t* seq_len,
                              int32_t max_len, uint8_t* codes4, float* lo, float* step,
                              float* err, hipStream_t stream) {
  if (c.block > kScanBlockMax) return hipErrorInvalidValue;
  const int32_t max_blocks = (c.max_seq + c.block - 1) / c.block;
  const int32_t nb = (max_len + c.block - 1) / c.block;
  if (nb == 0) return hipSuccess;
  const dim3 grid(nb, c.n_kv_heads, c.batch);
  if (c.kv_dtype == SKV_F16) {
#define SKV_BUILD(DD)                                                                           \
  scan4_build<DD><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(c.k), pos0, seq_len,   \
                                           c.n_kv_heads, c.max_seq, max_len, c.block,           \
                                           max_blocks, codes4, lo, step, err)
    switch (c.head_dim) {
      case 64: SKV_BUILD(64); break;
      case 128: SKV_BUILD(128); break;
      case 256: SKV_BUILD(256); break;
      default: return hipErrorInvalidValue;
    }
#undef SKV_BUILD
    return hipGetLastError();
  }
#define SKV_BUILD_Q(DD, KV)                                                                     \
  scan4_build_q<DD, KV><<<grid, 256, 0, stream>>>(static_cast<const uint8_t*>(c.k), c.k_scale,  \
                                                 pos0, seq_len, c.n_kv_heads, c.max_seq,        \
                                                 max_len, c.block, max_blocks, codes4, lo,      \
                                                 step, err)
#define SKV_BUILD_QD(KV)                       \
  switch (c.head_dim) {                        \
    case 64: SKV_BUILD_Q(64, KV); break;       \
    case 128: SKV_BUILD_Q(128, KV); break;     \
    case 256: SKV_BUILD_Q(256, KV); break;     \
    default: return hipErrorInvalidValue;      \
  }
  switch (c.kv_dtype) {
    case SKV_I8: SKV_BUILD_QD(SKV_I8); break;
    case SKV_Q8_0: SKV_BUILD_QD(SKV_Q8_0); break;
    case SKV_Q4_0: SKV_BUILD_QD(SKV_Q4_0); break;
    case SKV_Q5_0: SKV_BUILD_QD(SKV_Q5_0); break;
    default: return hipErrorInvalidValue;
  }
#undef SKV_BUILD_QD
#undef SKV_BUILD_Q
  return hipGetLastError();
}

hipError_t launch_scan4(const Scan4Params& p, hipStream_t stream) {
  const skv_cache& c = *p.c;
  const int32_t B = c.batch, H = p.n_heads, S = p.n_split, Hkv = c.n_kv_heads;
  const int G = H / Hkv;
  const int32_t max_blocks = (c.max_seq + c.block - 1) / c.block;
  const int32_t nb_max = (p.max_len + c.block - 1) / c.block;
  int32_t ups = (nb_max + S - 1) / S;
  ups = ups < 1 ? 1 : ups;
  const int64_t n_wg = int64_t(S) * Hkv * B;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  float* ub = p.ws;
  float* lbm = p.ws + size_t(B) * H * p.max_len;
  if (G != 1 && G != 2 && G != 4 && G != 8) return hipErrorInvalidValue;
  if (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256) return hipErrorInvalidValue;
#define SKV_SCAN(DD, GG, TT)                                                                    \
  scan4_bounds<DD, GG, TT><<<dim3(uint32_t(n_wg)), kMThreads, 0, stream>>>(                    \
      p.codes4, p.lo, p.step, p.err, p.q, p.seq_len, Hkv, c.max_seq, c.block, max_blocks,     \
      p.max_len, S, Hkv * B, ups, ub, lbm, p.cand_cnt)
#define SKV_SCAN_T(DD, GG)                                                                      \
  if (c.block % 64 == 0) SKV_SCAN(DD, GG, 64); else SKV_SCAN(DD, GG, 32);
#define SKV_SCAN_G(DD)                         \
  switch (G) {                                 \
    case 1: SKV_SCAN_T(DD, 1); break;          \
    case 2: SKV_SCAN_T(DD, 2); break;          \
    case 4: SKV_SCAN_T(DD, 4); break;          \
    default: SKV_SCAN_T(DD, 8); break;         \
  }
  switch (c.head_dim) {
    case 64: SKV_SCAN_G(64); break;
    case 128: SKV_SCAN_G(128); break;
    default: SKV_SCAN_G(256); break;
  }
#undef SKV_SCAN_G
#undef SKV_SCAN_T
#undef SKV_SCAN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_len == 0) return e;
  const int32_t words = (p.max_len + 31) / 32;
  scan4_select<<<dim3((p.max_len + kSelectChunk - 1) / kSelectChunk, H, B), 256, 0, stream>>>(
      ub, lbm, p.seq_len, H, p.max_len, S, p.delta, words, p.cand, p.cand_cnt);
  return hipGetLastError();
}

}  // namespace skv
