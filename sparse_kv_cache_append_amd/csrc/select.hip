// select_topk: fixed top-K block selection per (sequence, KV head).
//
// sparse_attn.md, "Method: Quest-style min/max block bounds" and "Budget
// policy": keep the K highest-bound blocks plus the sink block(s) and the
// recent window.  The forced blocks are a prefix [0, n_sink) and a suffix
// [NB - n_recent, NB), so the candidates are one contiguous range and the
// output (ascending) is: prefix, chosen candidates in index order, suffix.
//
// The K-th largest candidate score is found exactly with a most-significant-
// digit radix select over order-preserving uint32 keys of the float scores
// (-0 canonicalized to +0): four 8-bit passes, each an LDS histogram of the
// keys that still match the digits fixed so far, then a wave scan of the 256
// bins from the top to find the digit where the running count reaches the
// remaining rank.  After the passes the threshold key T and the number of
// T-equal keys to take are known; candidates are selected iff key > T, or
// key == T and fewer than that many T-equal keys precede them (ties go to the
// lower block index).  Two workgroup-wide exclusive scans turn the selection
// flags into ascending output positions.
#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxSelectBlocks = 16384;

// Exclusive scan of one int per thread over the workgroup; also returns the
// total.  `tmp` holds kSelWaves ints of LDS.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int t = tmp[w];
    off += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + x - v;
}

__global__ void __launch_bounds__(kSelThreads)
select_kernel(const float* __restrict__ score, const int32_t* __restrict__ seq_len,
              int32_t Hkv, int32_t max_blocks, int32_t block, const int32_t* __restrict__ k_sel,
              int32_t n_sink, int32_t n_recent, int32_t max_sel, int32_t* __restrict__ sel_idx,
              int32_t* __restrict__ sel_cnt, uint32_t* __restrict__ sel_mask) {
  extern __shared__ uint32_t smem[];
  uint32_t* keys = smem;                           // [max_blocks]
  uint32_t* maskw = smem + max_blocks;             // [ceil(max_blocks / 32)]
  __shared__ uint32_t hist[256];
  __shared__ int scan_tmp[kSelWaves];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_above;

  const int32_t g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t row = int64_t(b) * Hkv + g;
  const int32_t L = min(max(seq_len[b], 0), max_blocks * block);
  const int32_t nb = (L + block - 1) / block;
  const int32_t cs = min(n_sink, nb);                       // candidates [cs, ce)
  const int32_t ce = max(nb - n_recent, cs);
  const int32_t n_cand = ce - cs;
  const int32_t K = min(max(k_sel[b], 0), n_cand);
  const int32_t n_sel = cs + K + (nb - ce);
  const int32_t n_words = (max_blocks + 31) / 32;
  const bool want_mask = sel_mask != nullptr;

  if (want_mask)
    for (int w = tid; w < n_words; w += kSelThreads) maskw[w] = 0u;
  __syncthreads();

  auto emit = [&](int32_t pos, int32_t j) {
    if (pos < max_sel) sel_idx[row * max_sel + pos] = j;
    if (want_mask) atomicOr(&maskw[j >> 5], 1u << (j & 31));
  };

  // Forced prefix and suffix.
  for (int32_t j = tid; j < cs; j += kSelThreads) emit(j, j);
  for (int32_t j = ce + tid; j < nb; j += kSelThreads) emit(cs + K + (j - ce), j);

  if (K == n_cand) {
    for (int32_t j = cs + tid; j < ce; j += kSelThreads) emit(j, j);
  } else if (K > 0) {
    for (int32_t i = tid; i < n_cand; i += kSelThreads)
      keys[i] = float_key(score[row * max_blocks + cs + i]);
    uint32_t prefix = 0u, pmask = 0u;
    int remaining = K;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0u;  // kSelThreads == 256 bins
      __syncthreads();
      for (int32_t i = tid; i < n_cand; i += kSelThreads) {
        const uint32_t k = keys[i];
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < kWave) {
        // lane l owns digits 255-4l .. 252-4l (descending)
        int cnt[4], s = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { cnt[q] = int(hist[255 - 4 * tid - q]); s += cnt[q]; }
        int x = s;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int y = __shfl_up(x, o);
          if (tid >= o) x += y;
        }
        int above = x - s;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above < remaining && remaining <= above + cnt[q]) {
            sh_digit = uint32_t(255 - 4 * tid - q);
            sh_above = above;
          }
          above += cnt[q];
        }
      }
      __syncthreads();
      remaining -= sh_above;
      prefix |= sh_digit << shift;
      pmask |= 255u << shift;
    }
    const uint32_t T = prefix;
    const int need_eq = remaining;   // T-equal keys to take, lowest index first

    // Each thread owns a contiguous run of candidates.
    const int32_t per = (n_cand + kSelThreads - 1) / kSelThreads;
    const int32_t i0 = min(tid * per, n_cand), i1 = min(i0 + per, n_cand);
    int n_eq = 0;
    for (int32_t i = i0; i < i1; ++i) n_eq += (keys[i] == T);
    int tot;
    int eq_rank = wg_exclusive_scan(n_eq, scan_tmp, tot);
    int n_take = 0;
    {
      int r = eq_rank;
      for (int32_t i = i0; i < i1; ++i) {
        const uint32_t k = keys[i];
        if (k > T) ++n_take;
        else if (k == T) { n_take += (r < need_eq); ++r; }
      }
    }
    int pos = wg_exclusive_scan(n_take, scan_tmp, tot) + cs;
    {
      int r = eq_rank;
      for (int32_t i = i0; i < i1; ++i) {
        const uint32_t k = keys[i];
        bool take = false;
        if (k > T) take = true;
        else if (k == T) { take = (r < need_eq); ++r; }
        if (take) emit(pos++, cs + i);
      }
    }
  }
  // Pad the list and publish the count.
  for (int32_t p = n_sel + tid; p < max_sel; p += kSelThreads) sel_idx[row * max_sel + p] = -1;
  if (tid == 0) sel_cnt[row] = n_sel;
  if (want_mask) {
    __syncthreads();
    for (int w = tid; w < n_words; w += kSelThreads) sel_mask[row * n_words + w] = maskw[w];
  }
}

}  // namespace

hipError_t launch_select(const float* score, const int32_t* seq_len, int32_t batch,
                         int32_t n_kv_heads, int32_t max_blocks, int32_t block,
                         const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                         int32_t max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                         uint32_t* sel_mask, hipStream_t stream) {
  const size_t lds = (size_t(max_blocks) + (max_blocks + 31) / 32) * sizeof(uint32_t);
  static bool attr_set[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    const size_t most = (size_t(kMaxSelectBlocks) + kMaxSelectBlocks / 32) * sizeof(uint32_t);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(most));
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  dim3 grid(n_kv_heads, batch);
  select_kernel<<<grid, kSelThreads, lds, stream>>>(score, seq_len, n_kv_heads, max_blocks, block,
                                                    k_sel, n_sink, n_recent, max_sel, sel_idx,
                                                    sel_cnt, sel_mask);
  return hipGetLastError();
}

}  // namespace skv
