// combine: merge the split-K partial softmax states of every query head.
//
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i with M = max_i m_i over
// the non-empty parts (m_i = -inf marks an empty part); a head with no
// non-empty part gets zeros.
//
// The merge is latency-bound (a few KiB per head, read right after the decode
// kernel wrote it, often from another XCD's L2), so each thread owns one
// (head, channel) output and issues all of its loads before it uses any of
// them: kBatch parts' numerators, maxima and masses per memory round trip
// (one round trip for up to kBatch parts).  No barriers and no LDS.  The sum
// runs over the parts in index order.
#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int kCombThreads = 128;
constexpr int kBatch = 32;

__global__ void __launch_bounds__(kCombThreads)
combine_kernel(const float* __restrict__ ws_m, const float* __restrict__ ws_l,
               const float* __restrict__ ws_o, int32_t n_split, int32_t D,
               float* __restrict__ out) {
  const int64_t head = blockIdx.x;
  const int d = blockIdx.y * kCombThreads + threadIdx.x;
  if (d >= D) return;
  const float* mp = ws_m + head * n_split;
  const float* lp = ws_l + head * n_split;
  const float* op = ws_o + head * int64_t(n_split) * D + d;
  // One batch of parts per memory round trip: all maxima, masses and
  // numerators of the batch are loaded, then folded into a running max with
  // the accumulators rescaled when it grows (2^(m - M) is exact at m == M).
  float M = -INFINITY, num = 0.0f, den = 0.0f;
  for (int32_t i0 = 0; i0 < n_split; i0 += kBatch) {
    float mv[kBatch], lv[kBatch], ov[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = i0 + j < n_split;
      mv[j] = in ? mp[i0 + j] : -INFINITY;
      lv[j] = in ? lp[i0 + j] : 0.0f;
      ov[j] = in ? op[int64_t(i0 + j) * D] : 0.0f;
    }
    float bm = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) bm = fmaxf(bm, mv[j]);
    if (bm == -INFINITY) continue;
    if (bm > M) {
      const float c = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - bm);
      num *= c;
      den *= c;
      M = bm;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float a = (mv[j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mv[j] - M);
      num = fmaf(a, ov[j], num);
      den = fmaf(a, lv[j], den);
    }
  }
  out[head * D + d] = den > 0.0f ? num / den : 0.0f;
}

}  // namespace

hipError_t launch_combine(const float* ws, int32_t batch, int32_t n_heads, int32_t head_dim,
                          int32_t n_split, float* out, hipStream_t stream) {
  const float* ws_m = ws + ws_m_offset(batch, n_heads, n_split);
  const float* ws_l = ws + ws_l_offset(batch, n_heads, n_split);
  const float* ws_o = ws + ws_o_offset(batch, n_heads, n_split);
  dim3 grid(batch * n_heads, (head_dim + kCombThreads - 1) / kCombThreads);
  combine_kernel<<<grid, kCombThreads, 0, stream>>>(ws_m, ws_l, ws_o, n_split, head_dim, out);
  return hipGetLastError();
}

}  // namespace skv
