// combine: merge the split-K partial softmax states of every query head.
//
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i with M = max_i m_i over
// the non-empty parts (m_i = -inf marks an empty part); a head with no
// non-empty part gets zeros.
//
// The merge is latency-bound (a few KiB per head, read right after the decode
// kernel wrote it from every XCD), so it is shaped for few memory round trips
// and short per-lane queues: W = min(8, ceil(n_split / 16)) wavefronts per
// head, wavefront w taking parts 16 w .. 16 w + 15 of every batch of 16 W
// parts, its two 32-lane halves 8 parts each, lane l covering channels
// 4 (l % 32) .. +3.  Every load of a batch is issued before any is used
// (8 float4 numerators plus the maxima and masses).  The halves meet through
// a lane swap across the two 32-lane halves, the wavefronts through LDS.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {


// Four consecutive floats: one 16-byte load when the launcher has checked the
// 16-byte alignment of the buffers, else four 4-byte loads.
template <bool VEC>
__device__ __forceinline__ float4 load4(const float* p) {
  if constexpr (VEC) return *reinterpret_cast<const float4*>(p);
  else return make_float4(p[0], p[1], p[2], p[3]);
}
template <bool VEC>
__device__ __forceinline__ void store4(float* p, float4 v) {
  if constexpr (VEC) {
    *reinterpret_cast<float4*>(p) = v;
  } else {
    p[0] = v.x; p[1] = v.y; p[2] = v.z; p[3] = v.w;
  }
}

constexpr int kCombineMaxWaves = 8;
constexpr int kCombineHalf = 8;                         // parts per half-wavefront and batch
constexpr int kCombineWavePart = 2 * kCombineHalf;      // parts per wavefront and batch

// VEC: numerators and outputs 16-byte aligned; VML: so are the maxima and
// masses of every head (n_split % 4 == 0 and aligned bases).
template <bool VEC, bool VML>
__global__ void __launch_bounds__(kCombineMaxWaves * kWave)
combine_kernel(const float* __restrict__ ws_m, const float* __restrict__ ws_l,
               const float* __restrict__ ws_o, int32_t n_split, int32_t D,
               float* __restrict__ out) {
  constexpr int HB = kCombineHalf;
  const int64_t head = xcd_slot(blockIdx.x, gridDim.x);   // heads row by row per XCD
  const int lane = threadIdx.x % kWave, half = lane / 32;
  const int wave = threadIdx.x / kWave, W = blockDim.x / kWave;
  const int d4 = 4 * (lane % 32) + 128 * blockIdx.y;   // first of this lane's 4 channels
  const bool ch_ok = d4 < D;
  const float* mp = ws_m + head * n_split;
  const float* lp = ws_l + head * n_split;
  const float* op = ws_o + head * int64_t(n_split) * D;
  float M = -INFINITY, den = 0.0f;
  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int32_t i0 = kCombineWavePart * wave; i0 < n_split; i0 += kCombineWavePart * W) {
    const int32_t p0 = i0 + HB * half;          // this half's first part
    float mv[HB], lv[HB];
    float4 ov[HB];
#pragma unroll
    for (int j = 0; j < HB; j += 4) {
      if (VML && p0 + j + 3 < n_split) {
        const float4 m4 = *reinterpret_cast<const float4*>(mp + p0 + j);
        const float4 l4 = *reinterpret_cast<const float4*>(lp + p0 + j);
        mv[j] = m4.x; mv[j + 1] = m4.y; mv[j + 2] = m4.z; mv[j + 3] = m4.w;
        lv[j] = l4.x; lv[j + 1] = l4.y; lv[j + 2] = l4.z; lv[j + 3] = l4.w;
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bool in = p0 + j + t < n_split;
          mv[j + t] = in ? mp[p0 + j + t] : -INFINITY;
          lv[j + t] = in ? lp[p0 + j + t] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < HB; ++j) {
      const int32_t i = p0 + j;
      ov[j] = (i < n_split && ch_ok) ? load4<VEC>(op + int64_t(i) * D + d4)
                                     : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    // running max over both halves (identical in every lane), then rescale
    float bm = M;
#pragma unroll
    for (int j = 0; j < HB; ++j) bm = fmaxf(bm, mv[j]);
    uint32_t hi;
    const float lo = __uint_as_float(halves_lo(__float_as_uint(bm), hi));
    bm = fmaxf(lo, __uint_as_float(hi));
    if (bm == -INFINITY) continue;
    if (bm > M) {
      const float c = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - bm);
      num.x *= c; num.y *= c; num.z *= c; num.w *= c;
      den *= c;
      M = bm;
    }
#pragma unroll
    for (int j = 0; j < HB; ++j) {
      const float a = (mv[j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mv[j] - M);
      num.x = fmaf(a, ov[j].x, num.x);
      num.y = fmaf(a, ov[j].y, num.y);
      num.z = fmaf(a, ov[j].z, num.z);
      num.w = fmaf(a, ov[j].w, num.w);
      den = fmaf(a, lv[j], den);
    }
  }
  // both halves share M: add the lower half's sums to the upper half's
  uint32_t h;
  float t;
  t = __uint_as_float(halves_lo(__float_as_uint(num.x), h)); num.x = t + __uint_as_float(h);
  t = __uint_as_float(halves_lo(__float_as_uint(num.y), h)); num.y = t + __uint_as_float(h);
  t = __uint_as_float(halves_lo(__float_as_uint(num.z), h)); num.z = t + __uint_as_float(h);
  t = __uint_as_float(halves_lo(__float_as_uint(num.w), h)); num.w = t + __uint_as_float(h);
  t = __uint_as_float(halves_lo(__float_as_uint(den), h)); den = t + __uint_as_float(h);
  if (W > 1) {
    // the wavefronts' states meet in wavefront 0 (a wavefront with no
    // non-empty part has M = -inf and adds nothing)
    __shared__ float s_m[kCombineMaxWaves], s_den[kCombineMaxWaves];
    __shared__ float4 s_num[kCombineMaxWaves][32];
    if (lane == 0) { s_m[wave] = M; s_den[wave] = den; }
    if (half == 0) s_num[wave][lane] = num;
    __syncthreads();
    if (wave != 0) return;
    float Mg = -INFINITY;
    for (int w = 0; w < W; ++w) Mg = fmaxf(Mg, s_m[w]);
    M = Mg;
    den = 0.0f;
    num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (Mg != -INFINITY) {
      for (int w = 0; w < W; ++w) {
        const float a = (s_m[w] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s_m[w] - Mg);
        const float4 nw = s_num[w][lane % 32];
        num.x = fmaf(a, nw.x, num.x);
        num.y = fmaf(a, nw.y, num.y);
        num.z = fmaf(a, nw.z, num.z);
        num.w = fmaf(a, nw.w, num.w);
        den = fmaf(a, s_den[w], den);
      }
    }
  }
  if (half == 0 && ch_ok) {
    float4 o;
    o.x = den > 0.0f ? num.x / den : 0.0f;
    o.y = den > 0.0f ? num.y / den : 0.0f;
    o.z = den > 0.0f ? num.z / den : 0.0f;
    o.w = den > 0.0f ? num.w / den : 0.0f;
    store4<VEC>(out + head * D + d4, o);
  }
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
  const int W = std::min(kCombineMaxWaves, std::max(1, (n_split + kCombineWavePart - 1) /
                                                         kCombineWavePart));
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
