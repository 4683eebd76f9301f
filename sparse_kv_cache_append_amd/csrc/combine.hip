// combine: merge the split-K partial softmax states of every query head.
//
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i with M = max_i m_i over
// the non-empty parts (m_i = -inf marks an empty part); a head with no
// non-empty part gets zeros.  One workgroup per (sequence, query head), one
// thread per channel.
#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int kCombThreads = 128;

__global__ void __launch_bounds__(kCombThreads)
combine_kernel(const float* __restrict__ ws_m, const float* __restrict__ ws_l,
               const float* __restrict__ ws_o, int32_t n_split, int32_t D,
               float* __restrict__ out) {
  const int64_t head = blockIdx.x;
  const float* mp = ws_m + head * n_split;
  const float* lp = ws_l + head * n_split;
  float M = -INFINITY;
  for (int32_t i = 0; i < n_split; ++i) M = fmaxf(M, mp[i]);
  for (int32_t d = threadIdx.x; d < D; d += kCombThreads) {
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
      for (int32_t i = 0; i < n_split; ++i) {
        const float mi = mp[i];
        if (mi == -INFINITY) continue;
        const float a = __builtin_amdgcn_exp2f(mi - M);
        num = fmaf(a, ws_o[(head * n_split + i) * D + d], num);
        den = fmaf(a, lp[i], den);
      }
    }
    out[head * D + d] = den > 0.0f ? num / den : 0.0f;
  }
}

}  // namespace

hipError_t launch_combine(const float* ws, int32_t batch, int32_t n_heads, int32_t head_dim,
                          int32_t n_split, float* out, hipStream_t stream) {
  const float* ws_m = ws + ws_m_offset(batch, n_heads, n_split);
  const float* ws_l = ws + ws_l_offset(batch, n_heads, n_split);
  const float* ws_o = ws + ws_o_offset(batch, n_heads, n_split);
  combine_kernel<<<dim3(batch * n_heads), kCombThreads, 0, stream>>>(ws_m, ws_l, ws_o, n_split,
                                                                    head_dim, out);
  return hipGetLastError();
}

}  // namespace skv
