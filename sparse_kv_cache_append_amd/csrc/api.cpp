// C entry points: argument validation (host only, before anything is
// enqueued) and dispatch to the kernel launchers.
#include <algorithm>
#include <hip/hip_runtime.h>

#include "launch.h"
#include "skv.h"

namespace {

constexpr int32_t kMaxSplit = 4096;
constexpr int32_t kMaxSelectBlocks = 16384;

bool valid_head_dim(int32_t d) { return d >= 16 && d <= 1024 && d % 16 == 0; }
// Head dims built: 64, 128 and 256 for every call, over every cache type
// each call takes; the folded one-token appends move head dim 128 rows.
constexpr int32_t kFoldDim = 128;
bool built_head_dim(int32_t d) { return d == 64 || d == kFoldDim || d == 256; }
bool supported_group(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8; }
bool supported_tokens(int32_t n) { return n == 1 || n == 2 || n == 4 || n == 8; }

int32_t blocks_of(int32_t n, int32_t block) {
  return int32_t((int64_t(n) + block - 1) / block);
}

// Launch grids are 1-D over (part or block tile) x KV head x sequence; the
// append's grid keeps KV heads and sequences in its y and z dimensions.
constexpr int64_t kMaxGridX = 0x7fffffff;
constexpr int32_t kMaxGridYZ = 65535;
bool grid_fits(int64_t a, int64_t b, int64_t c) { return a * b * c <= kMaxGridX; }

// The kernels move cache rows, bounds, queries and new rows in 16-byte vectors.
bool aligned(const void* p, uintptr_t a = 16) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

skv_status check_cache(const skv_cache* c, bool need_bounds) {
  if (c == nullptr) return SKV_EINVAL;
  if (c->batch < 1 || c->n_kv_heads < 1 || c->max_seq < 1) return SKV_EINVAL;
  if (!valid_head_dim(c->head_dim)) return SKV_EINVAL;
  if (c->block < 16 || c->block % 16 != 0) return SKV_EINVAL;
  if (c->kv_dtype != SKV_F16 && c->kv_dtype != SKV_I8 && !skv::is_grouped(c->kv_dtype))
    return SKV_EINVAL;
  if (c->k == nullptr || c->v == nullptr) return SKV_EINVAL;
  if (c->kv_dtype != SKV_F16 && (c->k_scale == nullptr || c->v_scale == nullptr)) return SKV_EINVAL;
  if ((c->kmin == nullptr) != (c->kmax == nullptr)) return SKV_EINVAL;
  if (need_bounds && c->kmin == nullptr) return SKV_EINVAL;
  if (!aligned(c->k) || !aligned(c->v) || !aligned(c->kmin) || !aligned(c->kmax) ||
      !aligned(c->k_scale, 4) || !aligned(c->v_scale, 4))
    return SKV_EINVAL;
  // element counts must fit comfortably in int64 address arithmetic
  const double elems = double(c->batch) * c->n_kv_heads * double(c->max_seq) * c->head_dim;
  if (elems > 4.0e18) return SKV_ERANGE;
  if (c->batch > kMaxGridYZ || c->n_kv_heads > kMaxGridYZ) return SKV_ERANGE;
  if (!grid_fits(blocks_of(c->max_seq, c->block), c->n_kv_heads, c->batch)) return SKV_ERANGE;
  if (!built_head_dim(c->head_dim)) return SKV_EUNSUPPORTED;
  return SKV_OK;
}

skv_status check_heads(const skv_cache* c, int32_t n_heads) {
  if (n_heads < 1 || n_heads % c->n_kv_heads != 0) return SKV_EINVAL;
  if (!supported_group(n_heads / c->n_kv_heads)) return SKV_EUNSUPPORTED;
  return SKV_OK;
}

skv_status device_status(hipError_t e) { return e == hipSuccess ? SKV_OK : SKV_EDEVICE; }

// The new rows' dtype for a cache: f16 rows for an f16 cache, float32 rows
// for every quantized cache.
skv_status check_src(const skv_cache* c, int32_t src_dtype) {
  const bool ok = (c->kv_dtype == SKV_F16 && src_dtype == SKV_F16) ||
                  (c->kv_dtype != SKV_F16 && src_dtype == SKV_F32);
  if (ok) return SKV_OK;
  return (src_dtype == SKV_F16 || src_dtype == SKV_F32) ? SKV_EUNSUPPORTED : SKV_EINVAL;
}

hipError_t append_any(const skv_cache& c, const int32_t* pos0, int32_t n_new, const void* k_new,
                      const void* v_new, hipStream_t stream) {
  return skv::is_grouped(c.kv_dtype) ? skv::launch_append_grouped(c, pos0, n_new, k_new, v_new, stream)
                                     : skv::launch_append(c, pos0, n_new, k_new, v_new, stream);
}

hipError_t decode_any(const skv::DecodeParams& p, hipStream_t stream) {
  return skv::is_grouped(p.c->kv_dtype) ? skv::launch_decode_grouped(p, stream)
                                        : skv::launch_decode(p, stream);
}

}  // namespace

extern "C" {

int32_t skv_max_blocks(const skv_cache* c) {
  if (c == nullptr || c->block < 1 || c->max_seq < 0) return 0;
  return blocks_of(c->max_seq, c->block);
}

size_t skv_workspace_bytes(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t n_split) {
  if (batch < 1 || n_heads < 1 || !valid_head_dim(head_dim) || n_split < 1 || n_split > kMaxSplit)
    return 0;
  return sizeof(float) * size_t(batch) * size_t(n_heads) * size_t(n_split) * size_t(head_dim + 2);
}

const char* skv_status_str(int32_t s) {
  switch (s) {
    case SKV_OK: return "SKV_OK";
    case SKV_EINVAL: return "SKV_EINVAL: malformed argument";
    case SKV_ERANGE: return "SKV_ERANGE: size out of range";
    case SKV_EWORKSPACE: return "SKV_EWORKSPACE: workspace missing or too small";
    case SKV_EUNSUPPORTED: return "SKV_EUNSUPPORTED: valid but not built in this version";
    case SKV_EDEVICE: return "SKV_EDEVICE: HIP runtime error";
    default: return "unknown skv_status";
  }
}

skv_status skv_kv_append(const skv_cache* c, const int32_t* pos0, int32_t n_new,
                         const void* k_new, const void* v_new, int32_t src_dtype,
                         hipStream_t stream) {
  skv_status st = check_cache(c, false);
  if (st != SKV_OK) return st;
  if (pos0 == nullptr || k_new == nullptr || v_new == nullptr || n_new < 1) return SKV_EINVAL;
  if (!aligned(k_new) || !aligned(v_new)) return SKV_EINVAL;
  if (n_new > c->max_seq) return SKV_ERANGE;
  st = check_src(c, src_dtype);
  if (st != SKV_OK) return st;
  return device_status(append_any(*c, pos0, n_new, k_new, v_new, stream));
}

skv_status skv_block_bounds(const skv_cache* c, const float* q, int32_t n_heads,
                            const int32_t* seq_len, int32_t max_len, float* score,
                            hipStream_t stream) {
  skv_status st = check_cache(c, true);
  if (st != SKV_OK) return st;
  if (q == nullptr || seq_len == nullptr || score == nullptr || !aligned(q)) return SKV_EINVAL;
  st = check_heads(c, n_heads);
  if (st != SKV_OK) return st;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  return device_status(skv::launch_bounds(*c, q, n_heads, seq_len, max_len, score, stream));
}

skv_status skv_select_topk(const float* score, const int32_t* seq_len, int32_t batch,
                           int32_t n_kv_heads, int32_t max_blocks, int32_t block,
                           const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                           int32_t max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                           uint32_t* sel_mask, hipStream_t stream) {
  if (score == nullptr || seq_len == nullptr || k_sel == nullptr || sel_idx == nullptr ||
      sel_cnt == nullptr)
    return SKV_EINVAL;
  if (batch < 1 || n_kv_heads < 1 || max_blocks < 1 || block < 16 || block % 16 != 0)
    return SKV_EINVAL;
  if (n_sink < 0 || n_recent < 0 || max_sel < 1) return SKV_EINVAL;
  if (max_blocks > kMaxSelectBlocks) return SKV_EUNSUPPORTED;
  if (!grid_fits(batch, n_kv_heads, 1)) return SKV_ERANGE;
  return device_status(skv::launch_select(score, seq_len, batch, n_kv_heads, max_blocks, block,
                                          k_sel, n_sink, n_recent, max_sel, sel_idx, sel_cnt,
                                          sel_mask, stream));
}

skv_status skv_decode_attn(const skv_cache* c, const float* q, int32_t n_heads,
                           const int32_t* seq_len, int32_t max_len,
                           const int32_t* sel_idx, const int32_t* sel_cnt, int32_t max_sel,
                           float softmax_scale, int32_t n_split,
                           void* workspace, size_t workspace_bytes,
                           int32_t* dbg_logits, hipStream_t stream) {
  skv_status st = check_cache(c, false);
  if (st != SKV_OK) return st;
  if (q == nullptr || seq_len == nullptr || !aligned(q)) return SKV_EINVAL;
  st = check_heads(c, n_heads);
  if (st != SKV_OK) return st;
  if ((sel_idx == nullptr) != (sel_cnt == nullptr)) return SKV_EINVAL;
  if (sel_idx != nullptr && max_sel < 1) return SKV_EINVAL;
  if (n_split < 1 || n_split > kMaxSplit) return SKV_EINVAL;
  if (!grid_fits(n_split, c->n_kv_heads, c->batch)) return SKV_ERANGE;
  if (!(softmax_scale == softmax_scale) || softmax_scale < 0.0f) return SKV_EINVAL;
  if (dbg_logits != nullptr && c->kv_dtype != SKV_I8) return SKV_EINVAL;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  const size_t need = skv_workspace_bytes(c->batch, n_heads, c->head_dim, n_split);
  if (workspace == nullptr || workspace_bytes < need) return SKV_EWORKSPACE;
  skv::DecodeParams p;
  p.c = c;
  p.q = q;
  p.n_heads = n_heads;
  p.seq_len = seq_len;
  p.max_len = max_len;
  p.sel_idx = sel_idx;
  p.sel_cnt = sel_cnt;
  p.max_sel = max_sel;
  p.softmax_scale = softmax_scale;
  p.n_split = n_split;
  p.ws = static_cast<float*>(workspace);
  p.dbg_logits = dbg_logits;
  return device_status(decode_any(p, stream));
}

skv_status skv_decode_step(const skv_cache* c, const int32_t* pos0, const void* k_new,
                           const void* v_new, int32_t src_dtype, const float* q,
                           int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                           const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                           int32_t max_sel, float* score, int32_t* sel_idx, int32_t* sel_cnt,
                           float softmax_scale, int32_t n_split, void* workspace,
                           size_t workspace_bytes, float* out, hipStream_t stream) {
  const bool quest = k_sel != nullptr;
  skv_status st = check_cache(c, quest);
  if (st != SKV_OK) return st;
  if (q == nullptr || seq_len == nullptr || out == nullptr || !aligned(q)) return SKV_EINVAL;
  st = check_heads(c, n_heads);
  if (st != SKV_OK) return st;
  if (k_new != nullptr) {
    if (pos0 == nullptr || v_new == nullptr || !aligned(k_new) || !aligned(v_new))
      return SKV_EINVAL;
    st = check_src(c, src_dtype);
    if (st != SKV_OK) return st;
  }
  const int32_t max_blocks = blocks_of(c->max_seq, c->block);
  if (quest) {
    if (score == nullptr || sel_idx == nullptr || sel_cnt == nullptr) return SKV_EINVAL;
    if (n_sink < 0 || n_recent < 0 || max_sel < 1) return SKV_EINVAL;
    if (max_blocks > kMaxSelectBlocks) return SKV_EUNSUPPORTED;
  }
  if (n_split < 1 || n_split > kMaxSplit) return SKV_EINVAL;
  if (!grid_fits(n_split, c->n_kv_heads, c->batch)) return SKV_ERANGE;
  if (!grid_fits(c->batch, n_heads, 1)) return SKV_ERANGE;
  if (!(softmax_scale == softmax_scale) || softmax_scale < 0.0f) return SKV_EINVAL;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  const size_t need = skv_workspace_bytes(c->batch, n_heads, c->head_dim, n_split);
  if (workspace == nullptr || workspace_bytes < need) return SKV_EWORKSPACE;

  skv::DecodeParams p;
  p.c = c;
  p.q = q;
  p.n_heads = n_heads;
  p.seq_len = seq_len;
  p.max_len = max_len;
  p.sel_idx = nullptr;
  p.sel_cnt = nullptr;
  p.max_sel = max_sel;
  p.softmax_scale = softmax_scale;
  p.n_split = n_split;
  p.ws = static_cast<float*>(workspace);
  p.dbg_logits = nullptr;
  hipError_t e = hipSuccess;
  const bool grouped = skv::is_grouped(c->kv_dtype);
  // the folded appends move head dim 128 rows
  const bool fold = c->head_dim == kFoldDim;
  if (k_new != nullptr && ((grouped && !quest) || !fold)) {
    // dense steps over group-wise caches, and every step at another head dim:
    // the append runs as its own kernel (else the Quest step folds it into
    // the bounds pass, the dense step into the attention kernel)
    e = append_any(*c, pos0, 1, k_new, v_new, stream);
    if (e != hipSuccess) return SKV_EDEVICE;
  }
  if (quest) {
    e = k_new != nullptr && fold
            ? skv::launch_append_bounds(*c, pos0, k_new, v_new, q, n_heads, seq_len, max_len,
                                        score, stream)
            : skv::launch_bounds(*c, q, n_heads, seq_len, max_len, score, stream);
    if (e != hipSuccess) return SKV_EDEVICE;
    p.sel_idx = sel_idx;
    p.sel_cnt = sel_cnt;
    const int32_t ups = (max_sel + n_split - 1) / n_split;
    if (max_blocks <= skv::kFusedSelMaxCand && ups <= 64) {
      p.fused_r = skv::fused_sel_chunks(std::max(max_blocks - n_sink, 1));
      p.fsel = skv::FusedSelect{score, max_blocks, k_sel, n_sink, n_recent, sel_idx, sel_cnt};
    } else {
      e = skv::launch_select(score, seq_len, c->batch, c->n_kv_heads, max_blocks, c->block,
                             k_sel, n_sink, n_recent, max_sel, sel_idx, sel_cnt, nullptr, stream);
      if (e != hipSuccess) return SKV_EDEVICE;
    }
  } else if (k_new != nullptr && !grouped && fold) {
    p.app = skv::FoldedAppend{k_new, v_new, pos0};   // written by the attention kernel
  }
  e = decode_any(p, stream);
  if (e != hipSuccess) return SKV_EDEVICE;
  return device_status(skv::launch_combine(static_cast<const float*>(workspace), c->batch,
                                           n_heads, c->head_dim, n_split, out, stream));
}

skv_status skv_decode_attn_select(const skv_cache* c, const float* q, int32_t n_heads,
                                  const int32_t* seq_len, int32_t max_len, const float* score,
                                  const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                                  int32_t max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                                  float softmax_scale, int32_t n_split, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  skv_status st = check_cache(c, false);
  if (st != SKV_OK) return st;
  if (q == nullptr || seq_len == nullptr || !aligned(q)) return SKV_EINVAL;
  st = check_heads(c, n_heads);
  if (st != SKV_OK) return st;
  if (score == nullptr || k_sel == nullptr || sel_idx == nullptr || sel_cnt == nullptr)
    return SKV_EINVAL;
  if (n_sink < 0 || n_recent < 0 || max_sel < 1) return SKV_EINVAL;
  const int32_t max_blocks = blocks_of(c->max_seq, c->block);
  if (max_blocks > kMaxSelectBlocks) return SKV_EUNSUPPORTED;
  if (n_split < 1 || n_split > kMaxSplit) return SKV_EINVAL;
  if (!grid_fits(n_split, c->n_kv_heads, c->batch)) return SKV_ERANGE;
  if (!(softmax_scale == softmax_scale) || softmax_scale < 0.0f) return SKV_EINVAL;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  const size_t need = skv_workspace_bytes(c->batch, n_heads, c->head_dim, n_split);
  if (workspace == nullptr || workspace_bytes < need) return SKV_EWORKSPACE;
  skv::DecodeParams p;
  p.c = c;
  p.q = q;
  p.n_heads = n_heads;
  p.seq_len = seq_len;
  p.max_len = max_len;
  p.sel_idx = sel_idx;
  p.sel_cnt = sel_cnt;
  p.max_sel = max_sel;
  p.softmax_scale = softmax_scale;
  p.n_split = n_split;
  p.ws = static_cast<float*>(workspace);
  p.dbg_logits = nullptr;
  const int32_t ups = (max_sel + n_split - 1) / n_split;
  if (max_blocks <= skv::kFusedSelMaxCand && ups <= 64) {
    p.fused_r = skv::fused_sel_chunks(std::max(max_blocks - n_sink, 1));
    p.fsel = skv::FusedSelect{score, max_blocks, k_sel, n_sink, n_recent, sel_idx, sel_cnt};
  } else {
    const hipError_t e = skv::launch_select(score, seq_len, c->batch, c->n_kv_heads, max_blocks,
                                            c->block, k_sel, n_sink, n_recent, max_sel, sel_idx,
                                            sel_cnt, nullptr, stream);
    if (e != hipSuccess) return SKV_EDEVICE;
  }
  return device_status(decode_any(p, stream));
}

skv_status skv_block_bounds_heads(const skv_cache* c, const float* q, int32_t n_heads,
                                  const int32_t* seq_len, int32_t max_len, float* score,
                                  hipStream_t stream) {
  skv_status st = check_cache(c, true);
  if (st != SKV_OK) return st;
  if (q == nullptr || seq_len == nullptr || score == nullptr || !aligned(q)) return SKV_EINVAL;
  st = check_heads(c, n_heads);
  if (st != SKV_OK) return st;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  return device_status(skv::launch_bounds_heads(*c, q, n_heads, seq_len, max_len, score, stream));
}

skv_status skv_select_union(const int32_t* sel_idx, const int32_t* sel_cnt, int32_t batch,
                            int32_t n_heads, int32_t n_kv_heads, int32_t max_sel,
                            int32_t max_blocks, int32_t max_union, int32_t* uni_idx,
                            int32_t* uni_cnt, uint32_t* uni_mask, hipStream_t stream) {
  if (sel_idx == nullptr || sel_cnt == nullptr || uni_idx == nullptr || uni_cnt == nullptr ||
      uni_mask == nullptr)
    return SKV_EINVAL;
  if (batch < 1 || n_kv_heads < 1 || n_heads < 1 || n_heads % n_kv_heads != 0) return SKV_EINVAL;
  if (max_sel < 1 || max_blocks < 1 || max_union < 1) return SKV_EINVAL;
  if (!supported_group(n_heads / n_kv_heads)) return SKV_EUNSUPPORTED;
  if (max_blocks > kMaxSelectBlocks) return SKV_EUNSUPPORTED;
  if (!grid_fits(batch, n_kv_heads, 1)) return SKV_ERANGE;
  return device_status(skv::launch_union(sel_idx, sel_cnt, batch, n_kv_heads,
                                         n_heads / n_kv_heads, max_sel, max_blocks, max_union,
                                         uni_idx, uni_cnt, uni_mask, stream));
}

skv_status skv_decode_attn_heads(const skv_cache* c, const float* q, int32_t n_heads,
                                 const int32_t* seq_len, int32_t max_len,
                                 const int32_t* uni_idx, const int32_t* uni_cnt,
                                 const uint32_t* uni_mask, int32_t max_union,
                                 float softmax_scale, int32_t n_split, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  skv_status st = check_cache(c, false);
  if (st != SKV_OK) return st;
  if (q == nullptr || seq_len == nullptr || !aligned(q)) return SKV_EINVAL;
  if (uni_idx == nullptr || uni_cnt == nullptr || uni_mask == nullptr || max_union < 1)
    return SKV_EINVAL;
  st = check_heads(c, n_heads);
  if (st != SKV_OK) return st;
  if (n_split < 1 || n_split > kMaxSplit) return SKV_EINVAL;
  if (!grid_fits(n_split, c->n_kv_heads, c->batch)) return SKV_ERANGE;
  if (!(softmax_scale == softmax_scale) || softmax_scale < 0.0f) return SKV_EINVAL;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  const size_t need = skv_workspace_bytes(c->batch, n_heads, c->head_dim, n_split);
  if (workspace == nullptr || workspace_bytes < need) return SKV_EWORKSPACE;
  skv::DecodeParams p;
  p.c = c;
  p.q = q;
  p.n_heads = n_heads;
  p.seq_len = seq_len;
  p.max_len = max_len;
  p.sel_idx = uni_idx;
  p.sel_cnt = uni_cnt;
  p.max_sel = max_union;
  p.softmax_scale = softmax_scale;
  p.n_split = n_split;
  p.ws = static_cast<float*>(workspace);
  p.dbg_logits = nullptr;
  p.sel_hmask = uni_mask;
  return device_status(decode_any(p, stream));
}

// ------------------------------------------------------- query-token chunks
skv_status skv_block_bounds_multi(const skv_cache* c, const float* q, int32_t n_tokens,
                                  int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                                  float* score, hipStream_t stream) {
  skv_status st = check_cache(c, true);
  if (st != SKV_OK) return st;
  if (q == nullptr || seq_len == nullptr || score == nullptr || !aligned(q)) return SKV_EINVAL;
  st = check_heads(c, n_heads);
  if (st != SKV_OK) return st;
  if (n_tokens < 1) return SKV_EINVAL;
  if (!supported_tokens(n_tokens) || (n_heads / c->n_kv_heads) * n_tokens > 16)
    return SKV_EUNSUPPORTED;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  return device_status(
      skv::launch_bounds_multi(*c, q, n_tokens, n_heads, seq_len, max_len, score, stream));
}

skv_status skv_select_topk_multi(const float* score, const int32_t* seq_len, int32_t batch,
                                 int32_t n_tokens, int32_t n_kv_heads, int32_t max_blocks,
                                 int32_t block, const int32_t* k_sel, int32_t n_sink,
                                 int32_t n_recent, int32_t max_sel, int32_t* sel_idx,
                                 int32_t* sel_cnt, hipStream_t stream) {
  if (score == nullptr || seq_len == nullptr || k_sel == nullptr || sel_idx == nullptr ||
      sel_cnt == nullptr)
    return SKV_EINVAL;
  if (batch < 1 || n_kv_heads < 1 || n_tokens < 1 || max_blocks < 1 || block < 1) return SKV_EINVAL;
  if (n_sink < 0 || n_recent < 0 || max_sel < 1) return SKV_EINVAL;
  if (!supported_tokens(n_tokens)) return SKV_EUNSUPPORTED;
  if (max_blocks > kMaxSelectBlocks) return SKV_EUNSUPPORTED;
  if (int64_t(max_blocks) * block > 0x7fffffff) return SKV_ERANGE;
  if (!grid_fits(batch, n_kv_heads, n_tokens)) return SKV_ERANGE;
  return device_status(skv::launch_select(score, seq_len, batch, n_kv_heads * n_tokens,
                                          max_blocks, block, k_sel, n_sink, n_recent, max_sel,
                                          sel_idx, sel_cnt, nullptr, stream, n_tokens));
}

skv_status skv_select_union_tokens(const int32_t* sel_idx, const int32_t* sel_cnt,
                                   int32_t batch, int32_t n_tokens, int32_t n_kv_heads,
                                   int32_t group, int32_t max_sel, int32_t max_blocks,
                                   int32_t max_union, int32_t* uni_idx, int32_t* uni_cnt,
                                   uint32_t* uni_mask, hipStream_t stream) {
  if (sel_idx == nullptr || sel_cnt == nullptr || uni_idx == nullptr || uni_cnt == nullptr ||
      uni_mask == nullptr)
    return SKV_EINVAL;
  if (batch < 1 || n_kv_heads < 1 || n_tokens < 1 || group < 1) return SKV_EINVAL;
  if (max_sel < 1 || max_blocks < 1 || max_union < 1) return SKV_EINVAL;
  if (!supported_tokens(n_tokens) || !supported_group(group) || n_tokens * group > 16)
    return SKV_EUNSUPPORTED;
  if (max_blocks > kMaxSelectBlocks) return SKV_EUNSUPPORTED;
  if (!grid_fits(batch, n_kv_heads, 1)) return SKV_ERANGE;
  return device_status(skv::launch_union(sel_idx, sel_cnt, batch, n_kv_heads, n_tokens, max_sel,
                                         max_blocks, max_union, uni_idx, uni_cnt, uni_mask,
                                         stream, group));
}

skv_status skv_decode_attn_multi(const skv_cache* c, const float* q, int32_t n_tokens,
                                 int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                                 const int32_t* uni_idx, const int32_t* uni_cnt,
                                 const uint32_t* uni_mask, int32_t max_union,
                                 float softmax_scale, int32_t n_split, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  skv_status st = check_cache(c, false);
  if (st != SKV_OK) return st;
  if (q == nullptr || seq_len == nullptr || !aligned(q)) return SKV_EINVAL;
  const bool list = uni_idx != nullptr;
  if (list != (uni_cnt != nullptr) || list != (uni_mask != nullptr)) return SKV_EINVAL;
  if (list && max_union < 1) return SKV_EINVAL;
  st = check_heads(c, n_heads);
  if (st != SKV_OK) return st;
  if (n_tokens < 1) return SKV_EINVAL;
  if (!supported_tokens(n_tokens) || (n_heads / c->n_kv_heads) * n_tokens > 16)
    return SKV_EUNSUPPORTED;
  if (n_split < 1 || n_split > kMaxSplit) return SKV_EINVAL;
  if (!grid_fits(n_split, c->n_kv_heads, c->batch)) return SKV_ERANGE;
  if (!(softmax_scale == softmax_scale) || softmax_scale < 0.0f) return SKV_EINVAL;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  const size_t need = skv_workspace_bytes(c->batch, n_tokens * n_heads, c->head_dim, n_split);
  if (workspace == nullptr || workspace_bytes < need) return SKV_EWORKSPACE;
  skv::DecodeParams p;
  p.c = c;
  p.q = q;
  p.n_heads = n_heads;
  p.seq_len = seq_len;
  p.max_len = max_len;
  p.sel_idx = uni_idx;
  p.sel_cnt = uni_cnt;
  p.max_sel = list ? max_union : 0;
  p.softmax_scale = softmax_scale;
  p.n_split = n_split;
  p.ws = static_cast<float*>(workspace);
  p.dbg_logits = nullptr;
  p.sel_hmask = uni_mask;
  p.n_tok = n_tokens;
  return device_status(decode_any(p, stream));
}

skv_status skv_scan4_build(const skv_cache* c, const int32_t* pos0, const int32_t* seq_len,
                           int32_t max_len, uint8_t* codes4, float* lo, float* step, float* err,
                           hipStream_t stream) {
  skv_status st = check_cache(c, false);
  if (st != SKV_OK) return st;
  if (pos0 == nullptr || seq_len == nullptr || codes4 == nullptr || lo == nullptr ||
      step == nullptr || err == nullptr)
    return SKV_EINVAL;
  if (c->block > 256) return SKV_EUNSUPPORTED;
  if (!aligned(lo) || !aligned(step) || !aligned(err)) return SKV_EINVAL;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  return device_status(skv::launch_scan4_build(*c, pos0, seq_len, max_len, codes4, lo, step, err,
                                               stream));
}

size_t skv_scan4_workspace_bytes(int32_t batch, int32_t n_heads, int32_t n_split,
                                 int32_t max_len) {
  if (batch < 1 || n_heads < 1 || n_split < 1 || n_split > kMaxSplit || max_len < 0) return 0;
  return sizeof(float) * (size_t(batch) * n_heads * (size_t(max_len) + size_t(n_split)));
}

skv_status skv_scan4_candidates(const skv_cache* c, const uint8_t* codes4, const float* lo,
                                const float* step, const float* err, const float* q,
                                int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                                float delta, int32_t n_split, void* workspace,
                                size_t workspace_bytes, uint32_t* cand, int32_t* cand_cnt,
                                hipStream_t stream) {
  skv_status st = check_cache(c, false);
  if (st != SKV_OK) return st;
  if (codes4 == nullptr || lo == nullptr || step == nullptr || err == nullptr || q == nullptr ||
      seq_len == nullptr || cand == nullptr || cand_cnt == nullptr || !aligned(q))
    return SKV_EINVAL;
  if (!aligned(codes4) || !aligned(lo) || !aligned(step) || !aligned(err)) return SKV_EINVAL;
  st = check_heads(c, n_heads);
  if (st != SKV_OK) return st;
  if (c->block > 256) return SKV_EUNSUPPORTED;
  if (!(delta >= 0.0f && delta <= 3.4e38f)) return SKV_EINVAL;
  if (n_split < 1 || n_split > kMaxSplit) return SKV_EINVAL;
  if (!grid_fits(n_split, c->n_kv_heads, c->batch)) return SKV_ERANGE;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  const size_t need = skv_scan4_workspace_bytes(c->batch, n_heads, n_split, max_len);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace))
    return SKV_EWORKSPACE;
  skv::Scan4Params p;
  p.c = c;
  p.codes4 = codes4;
  p.lo = lo;
  p.step = step;
  p.err = err;
  p.q = q;
  p.n_heads = n_heads;
  p.seq_len = seq_len;
  p.max_len = max_len;
  p.delta = delta;
  p.n_split = n_split;
  p.ws = static_cast<float*>(workspace);
  p.cand = cand;
  p.cand_cnt = cand_cnt;
  return device_status(skv::launch_scan4(p, stream));
}

size_t skv_sparse_v_workspace_bytes(int32_t batch, int32_t n_heads, int32_t n_kv_heads,
                                    int32_t head_dim, int32_t n_split, int32_t max_len) {
  if (batch < 1 || n_heads < 1 || n_kv_heads < 1 || !valid_head_dim(head_dim) || n_split < 1 ||
      n_split > kMaxSplit || max_len < 0)
    return 0;
  return sizeof(float) *
         skv::sparse_v_workspace_floats(batch, n_heads, n_kv_heads, head_dim, n_split, max_len);
}

skv_status skv_decode_attn_sparse_v(const skv_cache* c, const float* q, int32_t n_heads,
                                    const int32_t* seq_len, int32_t max_len,
                                    const int32_t* sel_idx, const int32_t* sel_cnt,
                                    int32_t max_sel, float softmax_scale, float tau, float eps,
                                    int32_t n_split, void* workspace, size_t workspace_bytes,
                                    uint32_t* keep_mask, hipStream_t stream) {
  skv_status st = check_cache(c, false);
  if (st != SKV_OK) return st;
  if (q == nullptr || seq_len == nullptr || !aligned(q)) return SKV_EINVAL;
  st = check_heads(c, n_heads);
  if (st != SKV_OK) return st;
  if ((sel_idx == nullptr) != (sel_cnt == nullptr)) return SKV_EINVAL;
  if (sel_idx != nullptr && max_sel < 1) return SKV_EINVAL;
  if (n_split < 1 || n_split > kMaxSplit) return SKV_EINVAL;
  if (!grid_fits(n_split, c->n_kv_heads, c->batch)) return SKV_ERANGE;
  if (!(softmax_scale == softmax_scale) || softmax_scale < 0.0f) return SKV_EINVAL;
  // thresholds: finite and >= 0 (NaN fails both comparisons)
  if (!(tau >= 0.0f && tau <= 3.4e38f) || !(eps >= 0.0f && eps <= 3.4e38f)) return SKV_EINVAL;
  if (max_len < 0 || max_len > c->max_seq) return SKV_ERANGE;
  const size_t need = skv_sparse_v_workspace_bytes(c->batch, n_heads, c->n_kv_heads,
                                                   c->head_dim, n_split, max_len);
  if (workspace == nullptr || workspace_bytes < need) return SKV_EWORKSPACE;
  if (!aligned(workspace)) return SKV_EINVAL;
  skv::SparseVParams p;
  p.c = c;
  p.q = q;
  p.n_heads = n_heads;
  p.seq_len = seq_len;
  p.max_len = max_len;
  p.sel_idx = sel_idx;
  p.sel_cnt = sel_cnt;
  p.max_sel = max_sel;
  p.softmax_scale = softmax_scale;
  p.tau = tau;
  p.eps = eps;
  p.n_split = n_split;
  p.ws = static_cast<float*>(workspace);
  p.keep = keep_mask;
  return device_status(skv::launch_sparse_v(p, stream));
}

skv_status skv_combine(const void* workspace, int32_t batch, int32_t n_heads, int32_t head_dim,
                       int32_t n_split, float* out, hipStream_t stream) {
  if (workspace == nullptr || out == nullptr) return SKV_EINVAL;
  if (batch < 1 || n_heads < 1 || !valid_head_dim(head_dim)) return SKV_EINVAL;
  if (n_split < 1 || n_split > kMaxSplit) return SKV_EINVAL;
  if (!grid_fits(batch, n_heads, 1)) return SKV_ERANGE;
  return device_status(skv::launch_combine(static_cast<const float*>(workspace), batch, n_heads,
                                           head_dim, n_split, out, stream));
}

}  // extern "C"
