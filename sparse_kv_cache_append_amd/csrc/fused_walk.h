// The block selection in the prologue of an attention kernel (decode_kernels.h
// and decode_grouped.hip): every part of a (sequence, KV head) row computes
// the row's top-K with the select kernel's own code (select_core.h) and walks
// its slice of the ascending list.  Included by the .hip sources only;
// everything here has internal linkage.
#pragma once

#include "decode_core.h"
#include "device_common.h"
#include "launch.h"
#include "select_core.h"

namespace skv {
namespace {

static_assert(kMThreads == kSelThreads, "the selection prologue runs on the whole workgroup");

// The part's walk when the block selection runs in this workgroup's prologue
// (the same selection as skv_select_topk, computed redundantly by every part
// of the row: a workgroup-local job of a few microseconds that replaces a
// launch and a round trip through memory).  All threads call this.  The
// part's slice [u0, u0 + ups) of the ascending list goes to LDS and to the
// published list (the n_split slices cover [0, max_sel), ups being
// ceil(max_sel / n_split)); split 0 also publishes the count.
// (The scores are requested here, after the query has arrived; requesting
// them at kernel entry instead measured no faster.)
// sel_lds: workgroup memory of at least sizeof(SelectShared) bytes, 16-byte
// aligned, that nothing else uses until this returns (the kernel's tile
// buffers: no tile is staged before the walk starts, and after the final
// barrier here only plist, a buffer of its own, is read).
template <int T, int SELR>
__device__ __forceinline__ TileWalk fused_walk(const FusedSelect& fs, int32_t max_sel, int64_t bg,
                                               int32_t b, int32_t L, int32_t L_raw, int32_t block,
                                               int32_t split, int32_t units_per_split,
                                               void* sel_lds) {
  SelectShared& ssh = *reinterpret_cast<SelectShared*>(sel_lds);
  __shared__ int32_t plist[kWave + kSelThreads];   // the slice, then one spare entry per thread
  const int tid = threadIdx.x;
  // The candidates start at n_sink whenever there are any, so their scores
  // are requested before the row's length is used (up to the row's capacity).
  const int32_t k_req = fs.k_sel[b];
  SelKeys<SELR> kk;
  kk.load(fs.score + bg * fs.max_blocks + fs.n_sink, fs.max_blocks - fs.n_sink);
  sel_init(ssh);
  TileWalk tw;
  tw.block = block;
  tw.L = L;
  tw.nb = (L + block - 1) / block;
  tw.tpb = (block + T - 1) / T;
  tw.sel = fs.sel_idx;                     // non-null: sparse walk (entries come from jl)
  tw.u0 = split * units_per_split;
  // the selection sees the length as skv_select_topk clamps it; blocks past
  // this kernel's own length are skipped by the walk, as for a given list
  const int32_t L_sel = min(max(L_raw, 0), fs.max_blocks * block);
  const int32_t nb = (L_sel + block - 1) / block;
  const int32_t cs = min(fs.n_sink, nb);                    // candidates [cs, ce)
  const int32_t ce = max(nb - fs.n_recent, cs);
  const int32_t n_cand = ce - cs;
  const int32_t K = min(max(k_req, 0), n_cand);
  const int32_t n_sel = cs + K + (nb - ce);
  const int32_t u0 = tw.u0, ups = units_per_split;
  int32_t* out_row = fs.sel_idx + bg * max_sel;
  // positions whose block follows from the counts alone
  auto arith = [&](int32_t pos) { return pos < cs || pos >= cs + K || K == n_cand; };
  auto block_at = [&](int32_t pos) { return pos < cs + K ? pos : ce + (pos - cs - K); };
  if (tid < ups) {
    const int32_t pos = u0 + tid;
    if (pos < max_sel) {
      if (pos >= n_sel) {
        out_row[pos] = -1;
      } else if (arith(pos)) {
        const int32_t blk = block_at(pos);
        plist[tid] = blk;
        out_row[pos] = blk;
      }
    }
  }
  if (split == 0 && tid == 0) fs.sel_cnt[bg] = n_sel;
  if (K > 0 && K < n_cand) {          // then cs == n_sink
    kk.set_count(n_cand);
    const uint64_t cut = sel_cut(kk, K, ssh);
    const uint64_t taken = sel_taken_mask(kk, cut);
    if constexpr (SELR >= 16) {
      // this thread's taken candidates SELR tid + j, ascending from position
      // cs + base: the ones in this part's slice go to plist
      const SelRank rk = sel_rank_prepare<SELR>(taken, ssh);
      int32_t pos = cs + rk.base;
      if (pos < u0 + ups && pos + __popcll(rk.bits) > u0) {
        uint64_t bits = rk.bits;
        while (bits != 0u) {
          if (pos >= u0 && pos < u0 + ups) plist[pos - u0] = cs + SELR * tid + __builtin_ctzll(bits);
          ++pos;
          bits &= bits - 1u;
        }
      }
    } else {
      const int R = (n_cand + kSelThreads - 1) / kSelThreads;
      const SelOrder o = sel_order_prepare<SELR>(taken, R, ssh);
      // the taken candidates whose positions fall in this part's slice go to
      // plist; every thread writes once per chunk, the others to a spare
      // entry of their own, so the chunks carry no branch and overlap (chunks
      // past R have no taken bit)
#pragma unroll
      for (int r = 0; r < SELR; ++r) {
        const bool t = (taken >> r) & 1u;
        const uint64_t bal = __ballot(int(t));
        const int32_t pos = cs + __builtin_amdgcn_readlane(o.pre, r) + lanes_below(bal);
        const bool hit = t && pos >= u0 && pos < u0 + ups;
        plist[hit ? pos - u0 : kWave + tid] = cs + kk.index(r);
      }
    }
  }
  __syncthreads();
  // the selected (not arithmetic) entries of the slice, published
  if (tid < ups && K > 0 && K < n_cand) {
    const int32_t pos = u0 + tid;
    if (pos >= cs && pos < cs + K && pos < max_sel) out_row[pos] = plist[tid];
  }
  const int lane = tid % kWave;
  tw.jl = lane < ups ? plist[lane] : -1;
  tw.n_units = __builtin_amdgcn_readfirstlane(max(0, min(ups, min(n_sel, max_sel) - u0)));
  return tw;
}

}  // namespace
}  // namespace skv
