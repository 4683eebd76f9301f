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
#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int kBoundsThreads = 256;
constexpr int kLanesPerBlock = 16;
constexpr int kBlocksPerWG = kBoundsThreads / kLanesPerBlock;  // 16

template <int D, int G>
__global__ void __launch_bounds__(kBoundsThreads)
bounds_kernel(const uint16_t* __restrict__ kmin, const uint16_t* __restrict__ kmax,
              const float* __restrict__ q, const int32_t* __restrict__ seq_len,
              float* __restrict__ score, int32_t Hkv, int32_t max_len, int32_t block,
              int32_t max_blocks) {
  static_assert(D == kLanesPerBlock * 8, "one 16-byte load per lane per bound");
  const int32_t g = blockIdx.y, b = blockIdx.z;
  const int32_t L = min(max(seq_len[b], 0), max_len);
  const int32_t nb = (L + block - 1) / block;
  const int32_t j = int32_t(blockIdx.x) * kBlocksPerWG + int32_t(threadIdx.x) / kLanesPerBlock;
  const int32_t c = threadIdx.x % kLanesPerBlock;  // channels 8c .. 8c+7
  if (int32_t(blockIdx.x) * kBlocksPerWG >= nb) return;   // whole tile past the end

  // Query slice of the G heads of this group.
  float qv[G][8];
  const int32_t H = Hkv * G;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float4* qp = reinterpret_cast<const float4*>(q + (int64_t(b) * H + g * G + h) * D + c * 8);
    const float4 a = qp[0], bq = qp[1];
    qv[h][0] = a.x; qv[h][1] = a.y; qv[h][2] = a.z; qv[h][3] = a.w;
    qv[h][4] = bq.x; qv[h][5] = bq.y; qv[h][6] = bq.z; qv[h][7] = bq.w;
  }
  const bool live = j < nb;
  uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
  if (live) {
    const int64_t off = ((int64_t(b) * Hkv + g) * max_blocks + j) * D + c * 8;
    lo = *reinterpret_cast<const uint4*>(kmin + off);
    hi = *reinterpret_cast<const uint4*>(kmax + off);
  }
  float mn[8], mx[8];
  const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w};
  const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mn[2 * i] = h2f_lo(lw[i]); mn[2 * i + 1] = h2f_hi(lw[i]);
    mx[2 * i] = h2f_lo(hw[i]); mx[2 * i + 1] = h2f_hi(hw[i]);
  }
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

template <int G>
void launch_bounds_g(const skv_cache& c, const float* q, const int32_t* seq_len,
                     int32_t max_len, float* score, hipStream_t stream) {
  const int32_t max_blocks = (c.max_seq + c.block - 1) / c.block;
  const int32_t nb_max = (max_len + c.block - 1) / c.block;
  const int32_t tiles = (nb_max + kBlocksPerWG - 1) / kBlocksPerWG;
  if (tiles == 0) return;
  dim3 grid(tiles, c.n_kv_heads, c.batch);
  bounds_kernel<128, G><<<grid, kBoundsThreads, 0, stream>>>(
      c.kmin, c.kmax, q, seq_len, score, c.n_kv_heads, max_len, c.block, max_blocks);
}

}  // namespace

hipError_t launch_bounds(const skv_cache& c, const float* q, int32_t n_heads,
                         const int32_t* seq_len, int32_t max_len, float* score,
                         hipStream_t stream) {
  switch (n_heads / c.n_kv_heads) {
    case 1: launch_bounds_g<1>(c, q, seq_len, max_len, score, stream); break;
    case 2: launch_bounds_g<2>(c, q, seq_len, max_len, score, stream); break;
    case 4: launch_bounds_g<4>(c, q, seq_len, max_len, score, stream); break;
    case 8: launch_bounds_g<8>(c, q, seq_len, max_len, score, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace skv
