// combine: merge the split-K partial softmax states of every query head
// (the merge itself, and its shape, is in combine_core.h).
//
// The merge is latency-bound (a few KiB per head, read right after the decode
// kernel wrote it from every XCD), so it is shaped for few memory round trips
// and short per-lane queues: one workgroup of W wavefronts per head.
#include <algorithm>

#include "combine_core.h"
#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {

// VEC: numerators and outputs 16-byte aligned; VML: so are the maxima and
// masses of every head (n_split % 4 == 0 and aligned bases).
template <bool VEC, bool VML>
__global__ void __launch_bounds__(kCombineMaxWaves * kWave)
combine_kernel(const float* __restrict__ ws_m, const float* __restrict__ ws_l,
               const float* __restrict__ ws_o, int32_t n_split, int32_t D,
               float* __restrict__ out) {
  __shared__ float s_m[kCombineMaxWaves], s_den[kCombineMaxWaves];
  __shared__ float4 s_num[kCombineMaxWaves * 32];
  const int64_t head = xcd_slot(blockIdx.x, gridDim.x);   // heads row by row per XCD
  combine_head<VEC, VML>(ws_m, ws_l, ws_o, n_split, D, out, head, 128 * int(blockIdx.y),
                         int(threadIdx.x / kWave), int(blockDim.x / kWave), true, s_m, s_den,
                         s_num);
}

}  // namespace

hipError_t launch_combine(const float* ws, int32_t batch, int32_t n_heads, int32_t head_dim,
                          int32_t n_split, float* out, hipStream_t stream) {
  const float* ws_m = ws + ws_m_offset(batch, n_heads, n_split);
  const float* ws_l = ws + ws_l_offset(batch, n_heads, n_split);
  const float* ws_o = ws + ws_o_offset(batch, n_heads, n_split);
  const int64_t heads = int64_t(batch) * n_heads;
  if (heads > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<uint32_t>(heads), (head_dim + 127) / 128);
  auto aligned = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const bool vec = aligned(ws_o) && aligned(out) && head_dim % 4 == 0;
  const bool vml = aligned(ws_m) && aligned(ws_l) && n_split % 4 == 0;
  const int W = combine_waves(n_split);
#define SKV_COMBINE(V, M)                                                                     \
  combine_kernel<V, M><<<grid, W * kWave, 0, stream>>>(ws_m, ws_l, ws_o, n_split, head_dim, out)
  if (vec && vml) SKV_COMBINE(true, true);
  else if (vec) SKV_COMBINE(true, false);
  else if (vml) SKV_COMBINE(false, true);
  else SKV_COMBINE(false, false);
#undef SKV_COMBINE
  return hipGetLastError();
}

}  // namespace skv
