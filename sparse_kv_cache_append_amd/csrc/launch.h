// Internal launchers, one per kernel family.  The C entry points in api.cpp
// validate every argument and then call these; the launchers only size the
// grid and enqueue on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skv.h"

namespace skv {

// Block selection folded into decode_attn's prologue (see skv_decode_step):
// the score row, the budget and the outputs of skv_select_topk.
struct FusedSelect {
  const float* score;
  int32_t max_blocks;
  const int32_t* k_sel;
  int32_t n_sink;
  int32_t n_recent;
  int32_t* sel_idx;
  int32_t* sel_cnt;
};
// Largest candidate row the folded selection handles (keys per thread x 256).
constexpr int kFusedSelR = 16;
constexpr int32_t kFusedSelMaxCand = kFusedSelR * 256;
// Keys per thread of the folded selection for rows of up to n_load scores:
// the smallest of 2, 4, 16 that holds them (a shorter unrolled prologue is
// measurably faster to start: about 1 us per step at 512 blocks).
inline int fused_sel_chunks(int32_t n_load) {
  return n_load <= 2 * 256 ? 2 : n_load <= 4 * 256 ? 4 : kFusedSelR;
}

// The one-token append of a dense decode step, folded into decode_attn (see
// skv_decode_step): rows [batch][1][n_kv_heads][128] of the cache's source
// dtype (f16 for an f16 cache, float32 for an int8 cache) written at pos0[b].
struct FoldedAppend {
  const void* k_new = nullptr;   // nullptr: no append
  const void* v_new = nullptr;
  const int32_t* pos0 = nullptr;
};

struct DecodeParams {
  const skv_cache* c;
  const float* q;
  int32_t n_heads;
  const int32_t* seq_len;
  int32_t max_len;
  const int32_t* sel_idx;  // nullptr = dense
  const int32_t* sel_cnt;
  int32_t max_sel;
  float softmax_scale;
  int32_t n_split;
  float* ws;
  int32_t* dbg_logits;
  int fused_r = 0;          // > 0: select in the prologue from fsel with this many keys
                            // per thread (sel_idx/sel_cnt then receive the list)
  FusedSelect fsel{};
  FoldedAppend app{};       // dense walks only (sel_idx == nullptr, fused_r == 0)
  const uint32_t* sel_hmask = nullptr;   // per-query-head lists: head mask per entry
  int32_t n_tok = 1;        // query tokens per sequence (q [batch][n_tok][n_heads][D])
};

hipError_t launch_append(const skv_cache& c, const int32_t* pos0, int32_t n_new,
                         const void* k_new, const void* v_new, hipStream_t stream);

hipError_t launch_bounds(const skv_cache& c, const float* q, int32_t n_heads,
                         const int32_t* seq_len, int32_t max_len, float* score,
                         hipStream_t stream);

// One new token per sequence ([batch][1][n_kv_heads][head_dim] of the cache's
// source dtype), written at pos0[b], folded into the bounds pass.
struct AppendOne {
  void* k;
  void* v;
  float* ks;
  float* vs;
  const void* k_new;
  const void* v_new;
  const int32_t* pos0;
  int32_t max_seq;
};

hipError_t launch_append_bounds(const skv_cache& c, const int32_t* pos0, const void* k_new,
                                const void* v_new, const float* q, int32_t n_heads,
                                const int32_t* seq_len, int32_t max_len, float* score,
                                hipStream_t stream);

// Per-query-head bounds: score [batch][n_heads][max_blocks], no group max.
hipError_t launch_bounds_heads(const skv_cache& c, const float* q, int32_t n_heads,
                               const int32_t* seq_len, int32_t max_len, float* score,
                               hipStream_t stream);

// Bounds of a chunk of n_tok query tokens per sequence (q [batch][n_tok]
// [n_heads][D]): score [batch][n_kv_heads][n_tok][max_blocks], each token's
// group max.
hipError_t launch_bounds_multi(const skv_cache& c, const float* q, int32_t n_tok,
                               int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                               float* score, hipStream_t stream);

// Union of `group` consecutive lists per (sequence, KV head) (rows
// (b n_kv_heads + g) group + i of sel_idx), list i's blocks tagged with bits
// [i bits_per_list, (i + 1) bits_per_list) of the mask.
hipError_t launch_union(const int32_t* sel_idx, const int32_t* sel_cnt, int32_t batch,
                        int32_t n_kv_heads, int32_t group, int32_t max_sel, int32_t max_blocks,
                        int32_t max_union, int32_t* uni_idx, int32_t* uni_cnt,
                        uint32_t* uni_mask, hipStream_t stream, int32_t bits_per_list = 1);

// n_tok > 1: the rows are (KV head, token) pairs of a query-token chunk
// (n_kv_heads counts the pairs), token t seeing seq_len - (n_tok - 1 - t)
// positions.
hipError_t launch_select(const float* score, const int32_t* seq_len, int32_t batch,
                         int32_t n_kv_heads, int32_t max_blocks, int32_t block,
                         const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                         int32_t max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                         uint32_t* sel_mask, hipStream_t stream, int32_t n_tok = 1);

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
// head dims 64 and 256 (called by launch_decode)
hipError_t launch_decode_dims(const DecodeParams& p, hipStream_t stream);

// Sparse-V decode attention (sparse_v.hip): the q.K pass and the value pass
// over the kept rows, writing the standard partial states for skv_combine.
struct SparseVParams {
  const skv_cache* c;
  const float* q;
  int32_t n_heads;
  const int32_t* seq_len;
  int32_t max_len;
  const int32_t* sel_idx;  // nullptr = dense
  const int32_t* sel_cnt;
  int32_t max_sel;
  float softmax_scale;
  float tau, eps;
  int32_t n_split;
  float* ws;               // layout: sparse_v_workspace_floats
  uint32_t* keep;          // optional keep-bit output
};
// Floats of the sparse-V workspace: the standard partial states, then per
// part the pass-A maximum and denominator ([B][H][S] each) and token count
// ([B][Hkv][S] int32), then the logits [B][H][max_len rounded up to 32] and
// 32 floats of padding.
inline size_t sparse_v_workspace_floats(int32_t B, int32_t H, int32_t Hkv, int32_t D, int32_t S,
                                        int32_t max_len) {
  const size_t bhs = size_t(B) * H * S;
  const size_t lstride = (size_t(max_len) + 31) / 32 * 32;
  return bhs * (size_t(D) + 2) + 2 * bhs + size_t(B) * Hkv * S + size_t(B) * H * lstride + 32;
}
hipError_t launch_sparse_v(const SparseVParams& p, hipStream_t stream);

// Group-wise quantized caches (q8_0, q4_0): append and decode attention
// (decode_grouped.hip; dense walks and given lists).
hipError_t launch_append_grouped(const skv_cache& c, const int32_t* pos0, int32_t n_new,
                                 const void* k_new, const void* v_new, hipStream_t stream);
hipError_t launch_decode_grouped(const DecodeParams& p, hipStream_t stream);
inline bool is_grouped(int32_t kv_dtype) {
  return kv_dtype == SKV_Q8_0 || kv_dtype == SKV_Q4_0 || kv_dtype == SKV_Q5_0;
}

// The 4-bit key index and its GQA-shared scan (scan4.hip).
struct Scan4Params {
  const skv_cache* c;
  const uint8_t* codes4;
  const float* lo;
  const float* step;
  const float* err;
  const float* q;
  int32_t n_heads;
  const int32_t* seq_len;
  int32_t max_len;
  float delta;
  int32_t n_split;
  float* ws;               // UB [B][H][max_len], then the parts' LB maxima [B][H][S]
  uint32_t* cand;
  int32_t* cand_cnt;
};
hipError_t launch_scan4_build(const skv_cache& c, const int32_t* pos0, const int32_t* seq_len,
                              int32_t max_len, uint8_t* codes4, float* lo, float* step,
                              float* err, hipStream_t stream);
hipError_t launch_scan4(const Scan4Params& p, hipStream_t stream);

hipError_t launch_combine(const float* ws, int32_t batch, int32_t n_heads, int32_t head_dim,
                          int32_t n_split, float* out, hipStream_t stream);

// Workspace layout of the split-K partial states (see skv_decode_attn).
inline size_t ws_m_offset(int32_t, int32_t, int32_t) { return 0; }
inline size_t ws_l_offset(int32_t B, int32_t H, int32_t S) { return size_t(B) * H * S; }
inline size_t ws_o_offset(int32_t B, int32_t H, int32_t S) { return 2 * size_t(B) * H * S; }


}  // namespace skv
