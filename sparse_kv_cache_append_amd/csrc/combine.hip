// combine: merge the split-K partial softmax states of every query head.
//
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i with M = max_i m_i over
// the non-empty parts (m_i = -inf marks an empty part); a head with no
// non-empty part gets zeros.
//
// One workgroup per (sequence, query head).  The parts are spread over the
// threads, not walked by one: a block max gives M, each part's weight
// 2^(m_i - M) goes to LDS together with a block sum of the weighted masses,
// then every (channel, part-slice) thread sums its weighted numerators with
// independent loads and the slices are added in a fixed order.
#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int kCombThreads = 256;
constexpr int kCombWaves = kCombThreads / kWave;
constexpr int kMaxSplitLds = 4096;

__global__ void __launch_bounds__(kCombThreads)
combine_kernel(const float* __restrict__ ws_m, const float* __restrict__ ws_l,
               const float* __restrict__ ws_o, int32_t n_split, int32_t D,
               float* __restrict__ out) {
  __shared__ float wts[kMaxSplitLds];
  __shared__ float red[kCombWaves];
  __shared__ float part[kCombThreads];
  const int64_t head = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const float* mp = ws_m + head * n_split;
  const float* lp = ws_l + head * n_split;

  float mx = -INFINITY;
  for (int32_t i = tid; i < n_split; i += kCombThreads) mx = fmaxf(mx, mp[i]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kCombWaves; ++w) M = fmaxf(M, red[w]);
  __syncthreads();

  float den = 0.0f;
  for (int32_t i = tid; i < n_split; i += kCombThreads) {
    const float mi = mp[i];
    const float a = (mi == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mi - M);
    wts[i] = a;
    den = fmaf(a, lp[i], den);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
  if (lane == 0) red[wave] = den;
  __syncthreads();
  den = 0.0f;
#pragma unroll
  for (int w = 0; w < kCombWaves; ++w) den += red[w];

  // threads = (channel slice) x (part slice)
  const int slices = kCombThreads / D > 0 ? kCombThreads / D : 1;
  for (int32_t d0 = 0; d0 < D; d0 += kCombThreads / slices) {
    const int d = d0 + tid % (kCombThreads / slices);
    const int sl = tid / (kCombThreads / slices);
    float num = 0.0f;
    if (d < D && M != -INFINITY) {
      const float* op = ws_o + head * int64_t(n_split) * D + d;
      int32_t i = sl;
      for (; i + 3 * slices < n_split; i += 4 * slices) {
        const float o0 = op[int64_t(i) * D], o1 = op[int64_t(i + slices) * D];
        const float o2 = op[int64_t(i + 2 * slices) * D], o3 = op[int64_t(i + 3 * slices) * D];
        num = fmaf(wts[i], o0, num);
        num = fmaf(wts[i + slices], o1, num);
        num = fmaf(wts[i + 2 * slices], o2, num);
        num = fmaf(wts[i + 3 * slices], o3, num);
      }
      for (; i < n_split; i += slices) num = fmaf(wts[i], op[int64_t(i) * D], num);
    }
    part[tid] = num;
    __syncthreads();
    if (sl == 0 && d < D) {
      float s = 0.0f;
      for (int k = 0; k < slices; ++k) s += part[tid + k * (kCombThreads / slices)];
      out[head * D + d] = den > 0.0f ? s / den : 0.0f;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_combine(const float* ws, int32_t batch, int32_t n_heads, int32_t head_dim,
                          int32_t n_split, float* out, hipStream_t stream) {
  if (n_split > kMaxSplitLds) return hipErrorInvalidValue;
  const float* ws_m = ws + ws_m_offset(batch, n_heads, n_split);
  const float* ws_l = ws + ws_l_offset(batch, n_heads, n_split);
  const float* ws_o = ws + ws_o_offset(batch, n_heads, n_split);
  combine_kernel<<<dim3(batch * n_heads), kCombThreads, 0, stream>>>(ws_m, ws_l, ws_o, n_split,
                                                                    head_dim, out);
  return hipGetLastError();
}

}  // namespace skv
