// kv_append: write new tokens into the cache and keep the Quest side cache
// current.
//
// One workgroup per (sequence, KV head, block touched by the append).  The
// workgroup owns every new row of its block, so the block's channel min/max
// is reduced without atomics and then either overwrites the block (a block
// that starts at or after the append position holds no earlier token) or is
// min/max-merged into it (the block that straddles the append position) —
// the incremental fill of sparse_attn.md, "All-KV-types composition", which
// equals recomputing the bounds from scratch because min and max are exact
// and directed rounding is monotone.
//
// f16 cache: rows are copied bit for bit with 16-byte vector moves.
// int8 cache: each row (token, KV head) is quantized by one wavefront: absmax
// by a wave reduction, scale = a / 127, codes = rint(x / scale) (cpu-attn
// kernel card, "Method"); bounds come from the float32 rows, rounded outward
// to f16.
#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int kAppendThreads = 256;

struct AppendGeom {
  int32_t p0, j, t0, t1;
};

__device__ __forceinline__ bool append_rows(const int32_t* pos0, int32_t b, int32_t n_new,
                                            int32_t block, int32_t max_seq, AppendGeom& a) {
  a.p0 = pos0[b];
  if (a.p0 < 0) return false;
  a.j = a.p0 / block + int32_t(blockIdx.x);
  int64_t lo = max(int64_t(a.p0), int64_t(a.j) * block);
  int64_t hi = min(min(int64_t(a.p0) + n_new, int64_t(a.j + 1) * block), int64_t(max_seq));
  if (lo >= hi) return false;
  a.t0 = int32_t(lo);
  a.t1 = int32_t(hi);
  return true;
}

template <int D>
__global__ void __launch_bounds__(kAppendThreads)
append_f16_kernel(uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
                  uint16_t* __restrict__ kmin, uint16_t* __restrict__ kmax,
                  const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
                  const int32_t* __restrict__ pos0, int32_t n_new, int32_t Hkv,
                  int32_t max_seq, int32_t block, int32_t max_blocks) {
  const int32_t g = blockIdx.y, b = blockIdx.z;
  AppendGeom a;
  if (!append_rows(pos0, b, n_new, block, max_seq, a)) return;
  const int32_t nrows = a.t1 - a.t0;
  constexpr int kVecPerRow = D * 2 / 16;
  const uint4* ks = reinterpret_cast<const uint4*>(kn);
  const uint4* vs = reinterpret_cast<const uint4*>(vn);
  uint4* kd = reinterpret_cast<uint4*>(kc);
  uint4* vd = reinterpret_cast<uint4*>(vc);
  for (int32_t i = threadIdx.x; i < nrows * kVecPerRow; i += kAppendThreads) {
    const int32_t r = i / kVecPerRow, col = i % kVecPerRow;
    const int32_t t = a.t0 + r;
    const int64_t src = (int64_t(b) * n_new + (t - a.p0)) * Hkv + g;
    const int64_t dst = (int64_t(b) * Hkv + g) * max_seq + t;
    kd[dst * kVecPerRow + col] = ks[src * kVecPerRow + col];
    vd[dst * kVecPerRow + col] = vs[src * kVecPerRow + col];
  }
  if (kmin == nullptr) return;
  const bool fresh = int64_t(a.j) * block >= a.p0;
  for (int32_t d = threadIdx.x; d < D; d += kAppendThreads) {
    float mn = INFINITY, mx = -INFINITY;
    uint16_t bmn = 0x7C00u, bmx = 0xFC00u;   // +inf, -inf
    for (int32_t t = a.t0; t < a.t1; ++t) {
      const int64_t src = (int64_t(b) * n_new + (t - a.p0)) * Hkv + g;
      const uint16_t x = kn[src * D + d];
      const float xf = h2f(x);
      if (xf < mn) { mn = xf; bmn = x; }
      if (xf > mx) { mx = xf; bmx = x; }
    }
    const int64_t o = ((int64_t(b) * Hkv + g) * max_blocks + a.j) * D + d;
    if (!fresh) {
      bmn = f16_min_bits(kmin[o], bmn);
      bmx = f16_max_bits(kmax[o], bmx);
    }
    kmin[o] = bmn;
    kmax[o] = bmx;
  }
}

template <int D>
__global__ void __launch_bounds__(kAppendThreads)
append_i8_kernel(int8_t* __restrict__ kc, int8_t* __restrict__ vc,
                 float* __restrict__ ksc, float* __restrict__ vsc,
                 uint16_t* __restrict__ kmin, uint16_t* __restrict__ kmax,
                 const float* __restrict__ kn, const float* __restrict__ vn,
                 const int32_t* __restrict__ pos0, int32_t n_new, int32_t Hkv,
                 int32_t max_seq, int32_t block, int32_t max_blocks) {
  static_assert(D % kWave == 0, "D must be a multiple of 64");
  constexpr int E = D / kWave;  // elements per lane
  const int32_t g = blockIdx.y, b = blockIdx.z;
  AppendGeom a;
  if (!append_rows(pos0, b, n_new, block, max_seq, a)) return;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  for (int32_t t = a.t0 + wave; t < a.t1; t += kAppendThreads / kWave) {
    const int64_t src = ((int64_t(b) * n_new + (t - a.p0)) * Hkv + g) * D;
    const int64_t row = (int64_t(b) * Hkv + g) * max_seq + t;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const float* x = (which == 0 ? kn : vn) + src;
      float xv[E];
      float am = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        xv[e] = x[lane * E + e];
        am = fmaxf(am, fabsf(xv[e]));
      }
      am = wave_max(am);
      const float scale = absmax_scale(am);
      int8_t* dst = (which == 0 ? kc : vc) + row * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = int8_t(quant_code(xv[e], scale));
      if (lane == 0) (which == 0 ? ksc : vsc)[row] = scale;
    }
  }
  if (kmin == nullptr) return;
  const bool fresh = int64_t(a.j) * block >= a.p0;
  for (int32_t d = threadIdx.x; d < D; d += kAppendThreads) {
    float mn = INFINITY, mx = -INFINITY;
    for (int32_t t = a.t0; t < a.t1; ++t) {
      const int64_t src = ((int64_t(b) * n_new + (t - a.p0)) * Hkv + g) * D;
      const float x = kn[src + d];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    uint16_t bmn = f32_to_f16_down(mn), bmx = f32_to_f16_up(mx);
    const int64_t o = ((int64_t(b) * Hkv + g) * max_blocks + a.j) * D + d;
    if (!fresh) {
      bmn = f16_min_bits(kmin[o], bmn);
      bmx = f16_max_bits(kmax[o], bmx);
    }
    kmin[o] = bmn;
    kmax[o] = bmx;
  }
}

template <int D>
hipError_t launch_append_d(const skv_cache& c, const int32_t* pos0, int32_t n_new,
                           const void* k_new, const void* v_new, hipStream_t stream) {
  const int32_t max_blocks = (c.max_seq + c.block - 1) / c.block;
  const int32_t n_aff = (n_new + c.block - 2) / c.block + 1;
  dim3 grid(n_aff, c.n_kv_heads, c.batch);
  if (c.kv_dtype == SKV_F16) {
    append_f16_kernel<D><<<grid, kAppendThreads, 0, stream>>>(
        static_cast<uint16_t*>(c.k), static_cast<uint16_t*>(c.v), c.kmin, c.kmax,
        static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), pos0, n_new,
        c.n_kv_heads, c.max_seq, c.block, max_blocks);
  } else {
    append_i8_kernel<D><<<grid, kAppendThreads, 0, stream>>>(
        static_cast<int8_t*>(c.k), static_cast<int8_t*>(c.v), c.k_scale, c.v_scale, c.kmin,
        c.kmax, static_cast<const float*>(k_new), static_cast<const float*>(v_new), pos0, n_new,
        c.n_kv_heads, c.max_seq, c.block, max_blocks);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const skv_cache& c, const int32_t* pos0, int32_t n_new,
                         const void* k_new, const void* v_new, hipStream_t stream) {
  switch (c.head_dim) {
    case 64: return launch_append_d<64>(c, pos0, n_new, k_new, v_new, stream);
    case 128: return launch_append_d<128>(c, pos0, n_new, k_new, v_new, stream);
    case 256: return launch_append_d<256>(c, pos0, n_new, k_new, v_new, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace skv
