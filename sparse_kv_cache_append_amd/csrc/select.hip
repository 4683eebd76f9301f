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
              int32_t* __restrict__ sel_cnt, uint32_t* __restrict__ sel_mask, int32_t n_tok) {
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
  // a chunk of n_tok query tokens: rows are (KV head, token) pairs (Hkv counts
  // them), and token t of the chunk sees the first seq_len - (n_tok - 1 - t)
  // positions
  const int32_t back = n_tok - 1 - g % n_tok;
  const int32_t L = min(max(seq_len[b] - back, 0), max_blocks * block);
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
    if constexpr (RMAX >= 16) {
      // this thread's taken candidates RMAX tid + j, in ascending order
      const SelRank rk = sel_rank_prepare<RMAX>(taken, sh);
      uint64_t bits = rk.bits;
      int32_t pos = cs + rk.base;
      while (bits != 0u) {
        emit(pos++, cs + RMAX * tid + __builtin_ctzll(bits));
        bits &= bits - 1u;
      }
    } else {
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
  }
  // Pad the list and publish the count.
  for (int32_t p = n_sel + tid; p < max_sel; p += kSelThreads) sel_idx[row * max_sel + p] = -1;
  if (tid == 0) sel_cnt[row] = n_sel;
  if (want_mask) {
    __syncthreads();
    for (int w = tid; w < n_words; w += kSelThreads) sel_mask[row * n_words + w] = maskw[w];
  }
}

// The union of a KV head's per-query-head lists (ascending), each block with
// the bits of the heads (within the group) that chose it.  One workgroup per
// (sequence, KV head): the heads' entries set their bit in a byte per block
// (LDS, four blocks per word), then the marked blocks are compacted in
// ascending order with a workgroup prefix sum.
__global__ void __launch_bounds__(kSelThreads)
union_kernel(const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
             int32_t Hkv, int32_t G, int32_t max_sel, int32_t max_blocks, int32_t max_union,
             int32_t* __restrict__ uni_idx, int32_t* __restrict__ uni_cnt,
             uint32_t* __restrict__ uni_mask, int32_t bpr) {
  __shared__ uint32_t hw[kMaxSelectBlocks / 4];
  __shared__ int32_t wsum[kSelThreads / kWave];
  const int32_t row = int32_t(blockIdx.x);
  const int32_t b = row / Hkv, g = row % Hkv;
  const int32_t H = Hkv * G;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int32_t n_words = (max_blocks + 3) / 4;
  for (int32_t w = tid; w < n_words; w += kSelThreads) hw[w] = 0u;
  __syncthreads();
  for (int32_t i = 0; i < G; ++i) {
    const int64_t hrow = int64_t(b) * H + g * G + i;
    const int32_t cnt = min(max(sel_cnt[hrow], 0), max_sel);
    for (int32_t e = tid; e < cnt; e += kSelThreads) {
      const int32_t j = sel_idx[hrow * max_sel + e];
      if (j >= 0 && j < max_blocks) atomicOr(&hw[j >> 2], (1u << i) << (8 * (j & 3)));
    }
  }
  __syncthreads();
  // thread t owns blocks [t * per, (t + 1) * per)
  const int32_t per = (max_blocks + kSelThreads - 1) / kSelThreads;
  const int32_t j0 = tid * per, j1 = min(j0 + per, max_blocks);
  int32_t c = 0;
  for (int32_t j = j0; j < j1; ++j) c += ((hw[j >> 2] >> (8 * (j & 3))) & 0xFFu) != 0u;
  const int32_t incl = wave_incl_scan(c);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int32_t base = 0, total = 0;
  for (int w = 0; w < kSelThreads / kWave; ++w) {
    base += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  int32_t pos = base + incl - c;
  const int64_t out = int64_t(row) * max_union;
  for (int32_t j = j0; j < j1; ++j) {
    const uint32_t m = (hw[j >> 2] >> (8 * (j & 3))) & 0xFFu;
    if (m != 0u) {
      if (pos < max_union) {
        // list i's bit becomes bits [i bpr, (i + 1) bpr) of the mask
        uint32_t mm = m;
        if (bpr > 1) {
          mm = 0u;
          for (int i = 0; i < G; ++i)
            if ((m >> i) & 1u) mm |= ((1u << bpr) - 1u) << (i * bpr);
        }
        uni_idx[out + pos] = j;
        uni_mask[out + pos] = mm;
      }
      ++pos;
    }
  }
  for (int32_t p = total + tid; p < max_union; p += kSelThreads) {
    uni_idx[out + p] = -1;
    uni_mask[out + p] = 0u;
  }
  if (tid == 0) uni_cnt[row] = total;
}

}  // namespace

hipError_t launch_select(const float* score, const int32_t* seq_len, int32_t batch,
                         int32_t n_kv_heads, int32_t max_blocks, int32_t block,
                         const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                         int32_t max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                         uint32_t* sel_mask, hipStream_t stream, int32_t n_tok) {
  if (n_tok < 1 || n_kv_heads % n_tok != 0) return hipErrorInvalidValue;
  if (max_blocks > kMaxSelectBlocks) return hipErrorInvalidValue;
  const int64_t rows = int64_t(n_kv_heads) * batch;
  if (rows > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(rows));
#define SKV_LAUNCH_SELECT(RM)                                                                 \
  select_kernel<RM><<<grid, kSelThreads, 0, stream>>>(score, seq_len, n_kv_heads, max_blocks, \
                                                      block, k_sel, n_sink, n_recent, max_sel, \
                                                      sel_idx, sel_cnt, sel_mask, n_tok)
  if (max_blocks <= 4 * kSelThreads) SKV_LAUNCH_SELECT(4);
  else if (max_blocks <= 16 * kSelThreads) SKV_LAUNCH_SELECT(16);
  else SKV_LAUNCH_SELECT(64);
#undef SKV_LAUNCH_SELECT
  return hipGetLastError();
}

hipError_t launch_union(const int32_t* sel_idx, const int32_t* sel_cnt, int32_t batch,
                        int32_t n_kv_heads, int32_t group, int32_t max_sel, int32_t max_blocks,
                        int32_t max_union, int32_t* uni_idx, int32_t* uni_cnt,
                        uint32_t* uni_mask, hipStream_t stream, int32_t bits_per_list) {
  if (max_blocks > kMaxSelectBlocks || group < 1 || group > 8) return hipErrorInvalidValue;
  if (bits_per_list < 1 || group * bits_per_list > 32) return hipErrorInvalidValue;
  const int64_t rows = int64_t(batch) * n_kv_heads;
  if (rows > 0x7fffffff) return hipErrorInvalidValue;
  union_kernel<<<dim3(uint32_t(rows)), kSelThreads, 0, stream>>>(
      sel_idx, sel_cnt, n_kv_heads, group, max_sel, max_blocks, max_union, uni_idx, uni_cnt,
      uni_mask, bits_per_list);
  return hipGetLastError();
}

}  // namespace skv
