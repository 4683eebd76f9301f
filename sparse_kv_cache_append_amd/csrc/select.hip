// select_topk: fixed top-K block selection per (sequence, KV head).
//
// sparse_attn.md, "Method: Quest-style min/max block bounds" and "Budget
// policy": keep the K highest-bound blocks plus the sink block(s) and the
// recent window.  The forced blocks are a prefix [0, n_sink) and a suffix
// [NB - n_recent, NB), so the candidates are one contiguous range and the
// output (ascending) is: prefix, chosen candidates in index order, suffix.
//
// One workgroup per (sequence, KV head): the candidates' keys are loaded into
// registers, sel_cut (select_core.h) finds the cut value, and the index order
// of the taken candidates gives their ascending output positions.
#include "device_common.h"
#include "launch.h"
#include "select_core.h"

namespace skv {
namespace {

constexpr int kMaxSelectBlocks = kSelMaxChunks * kSelThreads;   // 16384

template <int RMAX>
__global__ void __launch_bounds__(kSelThreads)
select_kernel(const float* __restrict__ score, const int32_t* __restrict__ seq_len,
              int32_t Hkv, int32_t max_blocks, int32_t block, const int32_t* __restrict__ k_sel,
              int32_t n_sink, int32_t n_recent, int32_t max_sel, int32_t* __restrict__ sel_idx,
              int32_t* __restrict__ sel_cnt, uint32_t* __restrict__ sel_mask) {
  __shared__ SelectShared sh;
  __shared__ uint32_t maskw[kMaxSelectBlocks / 32];

  // 1-D grid of Hkv x batch rows in the XCD order of the decode's parts
  const uint32_t r = xcd_row(xcd_slot(blockIdx.x, gridDim.x), gridDim.x);
  const int32_t g = int32_t(r % uint32_t(Hkv)), b = int32_t(r / uint32_t(Hkv));
  const int tid = threadIdx.x;
  const int64_t row = int64_t(b) * Hkv + g;
  // The candidates start at n_sink whenever there are any, so their scores
  // are requested together with the row's length and budget.
  const int32_t k_req = k_sel[b];
  SelKeys<RMAX> kk;
  kk.load(score + row * max_blocks + n_sink, max_blocks - n_sink);
  sel_init(sh);
  const int32_t L = min(max(seq_len[b], 0), max_blocks * block);
  const int32_t nb = (L + block - 1) / block;
  const int32_t cs = min(n_sink, nb);                       // candidates [cs, ce)
  const int32_t ce = max(nb - n_recent, cs);
  const int32_t n_cand = ce - cs;
  const int32_t K = min(max(k_req, 0), n_cand);
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
  } else if (K > 0) {                 // then cs == n_sink
    kk.set_count(n_cand);
    const uint64_t cut = sel_cut(kk, K, sh);
    const uint64_t taken = sel_taken_mask(kk, cut);
    const int R = (n_cand + kSelThreads - 1) / kSelThreads;
    const SelOrder o = sel_order_prepare<RMAX>(taken, R, sh);
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r < R) {
        const int pos = sel_order_pos(o, taken, r);
        if ((taken >> r) & 1u) emit(cs + pos, cs + kk.index(r));
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
  if (max_blocks > kMaxSelectBlocks) return hipErrorInvalidValue;
  const int64_t rows = int64_t(n_kv_heads) * batch;
  if (rows > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(rows));
#define SKV_LAUNCH_SELECT(RM)                                                                 \
  select_kernel<RM><<<grid, kSelThreads, 0, stream>>>(score, seq_len, n_kv_heads, max_blocks, \
                                                      block, k_sel, n_sink, n_recent, max_sel, \
                                                      sel_idx, sel_cnt, sel_mask)
  if (max_blocks <= 4 * kSelThreads) SKV_LAUNCH_SELECT(4);
  else if (max_blocks <= 16 * kSelThreads) SKV_LAUNCH_SELECT(16);
  else SKV_LAUNCH_SELECT(64);
#undef SKV_LAUNCH_SELECT
  return hipGetLastError();
}

}  // namespace skv
