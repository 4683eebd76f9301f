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
// tiles: 16 lanes per block, each lane holding 8 channels (one 16-byte load of
// kmin and one of kmax), a 16-lane DPP sum per head, then the group max.
//
// A decode step may fold its one-token append into this pass
// (launch_append_bounds), which saves a launch and a dependent round trip.
#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int kBoundsThreads = 256;
constexpr int kLanesPerBlock = 16;
constexpr int kBlocksPerWG = kBoundsThreads / kLanesPerBlock;  // 16

enum AppendMode { kNoAppend = 0, kAppendF16 = 1, kAppendI8 = 2 };

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
      uint16_t bmn = x, bmx = x;
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
      uint16_t bmn = f32_to_f16_down(x), bmx = f32_to_f16_up(x);
      if (!fresh) {
        bmn = f16_min_bits(kmin[bo + d], bmn);
        bmx = f16_max_bits(kmax[bo + d], bmx);
      }
      kmin[bo + d] = bmn;
      kmax[bo + d] = bmx;
    }
  }
}

// MODE != kNoAppend: first append one token per sequence at pos0[b] (the
// first workgroup of each (sequence, KV head) writes it) and score its block
// with the merged bounds.  The merge is computed from the new key in
// registers, so it does not matter whether this workgroup reads the side
// cache before or after the append writes it: min/max with the same key is
// idempotent, and a fresh block ignores the old values.
template <int D, int G, int MODE>
__global__ void __launch_bounds__(kBoundsThreads)
bounds_kernel(uint16_t* __restrict__ kmin, uint16_t* __restrict__ kmax,
              const float* __restrict__ q, const int32_t* __restrict__ seq_len,
              float* __restrict__ score, int32_t Hkv, int32_t max_len, int32_t block,
              int32_t max_blocks, int32_t tiles, int32_t n_rows, AppendOne ap) {
  static_assert(D == kLanesPerBlock * 8, "one 16-byte load per lane per bound");
  static_assert(G * D / 4 <= kBoundsThreads, "one 16-byte query load per thread");
  // 1-D grid of tiles x Hkv x batch, row by row (XCD-aware slots: a row's
  // scores are written on the XCD whose L2 its decode parts read them from)
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t tile = int32_t(slot % uint32_t(tiles));
  const uint32_t row = xcd_row(slot / uint32_t(tiles), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int32_t j = tile * kBlocksPerWG + int32_t(threadIdx.x) / kLanesPerBlock;
  const int32_t c = threadIdx.x % kLanesPerBlock;  // channels 8c .. 8c+7
  // Requests issued before anything waits (one round trip): the row length
  // (and append position), the group's G query rows (G * 512 B, one 16-byte
  // load per thread, staged once per workgroup in LDS) and this thread's
  // bounds, read for every block of the launched tile that exists in the
  // side cache; only those below the row's length are scored.
  const int32_t L_raw = seq_len[b];
  int32_t p0 = -1;
  if constexpr (MODE != kNoAppend) p0 = ap.pos0[b];
  const int32_t H = Hkv * G;
  const float* qg = q + (int64_t(b) * H + g * G) * D;
  float4 qreg = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (threadIdx.x < G * D / 4) qreg = reinterpret_cast<const float4*>(qg)[threadIdx.x];
  uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
  if (j < max_blocks) {
    const int64_t off = ((int64_t(b) * Hkv + g) * max_blocks + j) * D + c * 8;
    // read once per step: streaming (nontemporal) loads
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 l4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kmin + off));
    const u32x4 h4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kmax + off));
    lo = make_uint4(l4.x, l4.y, l4.z, l4.w);
    hi = make_uint4(h4.x, h4.y, h4.z, h4.w);
  }
  int32_t jn = -1;
  bool fresh = false;
  if constexpr (MODE != kNoAppend) {
    if (p0 >= 0 && p0 < ap.max_seq) {
      jn = p0 / block;
      fresh = (p0 % block) == 0;
      if (tile == 0) append_one<D, MODE>(ap, kmin, kmax, b, g, Hkv, p0, jn, fresh, max_blocks);
    }
  }
  const int32_t L = min(max(L_raw, 0), max_len);
  const int32_t nb = (L + block - 1) / block;
  if (tile * kBlocksPerWG >= nb) return;   // whole tile past the end

  __shared__ __attribute__((aligned(16))) float qs[G * D];
  if (threadIdx.x < G * D / 4) reinterpret_cast<float4*>(qs)[threadIdx.x] = qreg;
  const bool live = j < nb;
  __syncthreads();
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float4 a = reinterpret_cast<const float4*>(qs + h * D + c * 8)[0];
    const float4 bq = reinterpret_cast<const float4*>(qs + h * D + c * 8)[1];
    qv[h][0] = a.x; qv[h][1] = a.y; qv[h][2] = a.z; qv[h][3] = a.w;
    qv[h][4] = bq.x; qv[h][5] = bq.y; qv[h][6] = bq.z; qv[h][7] = bq.w;
  }
  uint16_t lb[8], hb[8];
  {
    const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w};
    const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lb[2 * i] = uint16_t(lw[i] & 0xFFFFu); lb[2 * i + 1] = uint16_t(lw[i] >> 16);
      hb[2 * i] = uint16_t(hw[i] & 0xFFFFu); hb[2 * i + 1] = uint16_t(hw[i] >> 16);
    }
  }
  if constexpr (MODE != kNoAppend) {
    if (live && j == jn) {
      const int64_t src = (int64_t(b) * Hkv + g) * D + c * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint16_t nmn, nmx;
        if constexpr (MODE == kAppendF16) {
          nmn = nmx = static_cast<const uint16_t*>(ap.k_new)[src + e];
        } else {
          const float x = static_cast<const float*>(ap.k_new)[src + e];
          nmn = f32_to_f16_down(x);
          nmx = f32_to_f16_up(x);
        }
        lb[e] = fresh ? nmn : f16_min_bits(lb[e], nmn);
        hb[e] = fresh ? nmx : f16_max_bits(hb[e], nmx);
      }
    }
  }
  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { mn[e] = h2f(lb[e]); mx[e] = h2f(hb[e]); }
  float best = -INFINITY;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = qv[h][e];
      const float kb = x > 0.0f ? mx[e] : mn[e];
      acc += (x != 0.0f) ? x * kb : 0.0f;
    }
    acc = group16_sum(acc);
    best = fmaxf(best, acc);
  }
  if (live && c == 0) score[(int64_t(b) * Hkv + g) * max_blocks + j] = best;
}

template <int G, int MODE>
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
  bounds_kernel<128, G, MODE><<<grid, kBoundsThreads, 0, stream>>>(
      c.kmin, c.kmax, q, seq_len, score, c.n_kv_heads, max_len, c.block, max_blocks, tiles,
      c.n_kv_heads * c.batch, ap);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_bounds_m(const skv_cache& c, const float* q, int32_t n_heads,
                           const int32_t* seq_len, int32_t max_len, float* score,
                           const AppendOne& ap, hipStream_t stream) {
  switch (n_heads / c.n_kv_heads) {
    case 1: return launch_bounds_g<1, MODE>(c, q, seq_len, max_len, score, ap, stream);
    case 2: return launch_bounds_g<2, MODE>(c, q, seq_len, max_len, score, ap, stream);
    case 4: return launch_bounds_g<4, MODE>(c, q, seq_len, max_len, score, ap, stream);
    case 8: return launch_bounds_g<8, MODE>(c, q, seq_len, max_len, score, ap, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_bounds(const skv_cache& c, const float* q, int32_t n_heads,
                         const int32_t* seq_len, int32_t max_len, float* score,
                         hipStream_t stream) {
  return launch_bounds_m<kNoAppend>(c, q, n_heads, seq_len, max_len, score, AppendOne{}, stream);
}

hipError_t launch_append_bounds(const skv_cache& c, const int32_t* pos0, const void* k_new,
                                const void* v_new, const float* q, int32_t n_heads,
                                const int32_t* seq_len, int32_t max_len, float* score,
                                hipStream_t stream) {
  AppendOne ap{c.k, c.v, c.k_scale, c.v_scale, k_new, v_new, pos0, c.max_seq};
  if (c.kv_dtype == SKV_F16)
    return launch_bounds_m<kAppendF16>(c, q, n_heads, seq_len, max_len, score, ap, stream);
  return launch_bounds_m<kAppendI8>(c, q, n_heads, seq_len, max_len, score, ap, stream);
}

}  // namespace skv
