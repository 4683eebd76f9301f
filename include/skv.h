/*
 * skv.h — decode-step attention over dense, int8 and Quest block-sparse KV
 * caches on AMD MI355X (gfx950).  C ABI.
 *
 * The library computes, for one new query token per sequence, attention of
 * each query head h against the cached keys/values of KV head
 * g = h / (H / Hkv) (grouped-query attention; cpu-attn kernel card, "Usage").
 * Three variants share the same calls:
 *   - dense split-K flash-decode over an f16 cache;
 *   - the same over an int8 cache quantized per token and per head with an
 *     absmax scale at append time, with exact integer q.k logit dots
 *     (cpu-attn kernel card, "Method");
 *   - Quest block-sparse decode: per-(KV head, block) kmin/kmax side cache,
 *     a channel-wise upper bound per block, fixed top-K blocks plus the sink
 *     block(s) and the recent window, attention over the selected blocks only
 *     (opencoti-llamafile sparse_attn.md, "Method: Quest-style min/max block
 *     bounds" and "S2/S3 engineering design").
 *
 * Conventions for every call:
 *   - All tensor arguments are DEVICE pointers to memory the caller allocated
 *     and owns.  The library allocates nothing, keeps no state between calls
 *     and never synchronizes: every call only enqueues kernels on `stream`
 *     (NULL = the default stream) and returns.  Calls on one stream execute in
 *     order, so append -> bounds -> select -> decode -> combine needs no
 *     further synchronization.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed check returns a negative skv_status and enqueues nothing.  No
 *     call aborts.  Values that live in device memory (positions, lengths,
 *     budgets, selected indices) cannot be checked on the host; the kernels
 *     clamp them so that every access stays inside the buffers described
 *     below, and each call documents what it does with out-of-range values.
 *   - Layouts are dense, row-major, with the last dimension contiguous.
 *     f16 means IEEE binary16 bit patterns (uint16_t storage).
 *   - The cache's k, v, kmin, kmax, the queries q and the new rows k_new,
 *     v_new are 16-byte aligned, the int8 scales 4-byte aligned (SKV_EINVAL
 *     otherwise); other buffers need their element's natural alignment.
 *   - Supported in this version: head_dim D = 64, 128 or 256 for every call,
 *     over every cache type (f16, int8, q8_0, q4_0, q5_0) (the cpu-attn
 *     kernel card, "Requirements and limits", admits any multiple of 16 up to
 *     1024);
 *     GQA group size
 *     G = H / Hkv in {1, 2, 4, 8}; block a multiple of 16.  Other values that
 *     are otherwise valid return SKV_EUNSUPPORTED.
 *   - Launch sizes: batch and n_kv_heads up to 65,535, and at most
 *     2^31 - 1 workgroups per launch (n_split x n_kv_heads x batch for
 *     decode, max_blocks x n_kv_heads x batch for the cache, n_kv_heads x
 *     batch for select, batch x n_heads for combine); larger sizes return
 *     SKV_ERANGE.  (A cache that fits in device memory is far inside these.)
 */
#ifndef SKV_H
#define SKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum skv_status {
  SKV_OK = 0,
  SKV_EINVAL = -1,       /* malformed argument: NULL pointer, bad shape, H % Hkv != 0,
                            D not a multiple of 16 or above 1024, negative counts */
  SKV_ERANGE = -2,       /* a size exceeds what the buffers or the cache can hold */
  SKV_EWORKSPACE = -3,   /* workspace missing or smaller than skv_workspace_bytes() */
  SKV_EUNSUPPORTED = -4, /* valid but not built in this version (see above) */
  SKV_EDEVICE = -5       /* the HIP runtime reported an error at launch */
} skv_status;

typedef enum skv_dtype {
  SKV_F16 = 1,
  SKV_F32 = 2,
  SKV_I8 = 3,
  SKV_Q8_0 = 4,   /* group-wise: 32-channel groups, int8 codes, an f16 scale each */
  SKV_Q4_0 = 5,   /* group-wise: 32-channel groups, 4-bit codes, an f16 scale each */
  SKV_Q5_0 = 6    /* group-wise: 32-channel groups, 5-bit codes, an f16 scale each */
} skv_dtype;

/*
 * Cache descriptor (plain data; the caller fills it and owns every buffer).
 *   k, v      : [batch][n_kv_heads][max_seq][head_dim]; f16 when kv_dtype is
 *               SKV_F16, int8 codes when kv_dtype is SKV_I8.
 *   k_scale,
 *   v_scale   : [batch][n_kv_heads][max_seq] float32 absmax scales (SKV_I8
 *               only; ignored for SKV_F16).
 *   kmin, kmax: [batch][n_kv_heads][max_blocks][head_dim] f16, where
 *               max_blocks = ceil(max_seq / block).  The Quest side cache:
 *               channel-wise min and max of the keys of each block, taken
 *               before quantization (sparse_attn.md, "Method" and
 *               "All-KV-types composition").  Both NULL = no side cache
 *               (dense only; appends then skip the bounds update).
 * Group-wise quantized caches (SKV_Q8_0, SKV_Q4_0, SKV_Q5_0; sparse_attn.md,
 * "All-KV-types composition": quantized blocks of 32 values with the side
 * cache filled before quantization; "Method: Quest-style min/max block
 * bounds" names q5_0 and q4_0):
 *   k, v      : [batch][n_kv_heads][max_seq][row] bytes, row = head_dim
 *               (q8_0: int8 codes -127..127) or head_dim / 2 (q4_0: channel
 *               2i in the low nibble of byte i, 2i + 1 in the high nibble,
 *               each code + 8, codes -7..7);
 *               q5_0 (codes -15..15, each stored as code + 16 in five bits):
 *               [batch][n_kv_heads][max_seq * 5 head_dim / 8] bytes, each
 *               (sequence, KV head) holding a plane of max_seq rows of
 *               head_dim / 2 bytes (bits 0..3, laid out as q4_0) followed by
 *               a plane of max_seq rows of head_dim / 8 bytes (bit 4 of
 *               channel c at bit c % 8 of byte c / 8);
 *   k_scale,
 *   v_scale   : f16 bit patterns (uint16_t storage behind the float*
 *               pointers) [batch][n_kv_heads][max_seq][head_dim / 32], the
 *               scale of each group of 32 consecutive channels.
 *   Per group: a = max |x|, scale = f16(a / QMAX) (QMAX 127, 7 or 15), code =
 *   clamp(rint(x / scale), -QMAX, QMAX) against the stored scale (a scale of
 *   0, or beyond f16's range, gives codes 0); a value is scale * code, and
 *   attention runs on those values with the float32 query.
 * Token t of sequence b lives at position t (0-based) of its row.
 */
typedef struct skv_cache {
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t max_seq;
  int32_t block;
  int32_t kv_dtype;
  void* k;
  void* v;
  float* k_scale;
  float* v_scale;
  uint16_t* kmin;
  uint16_t* kmax;
} skv_cache;

/* Number of blocks per sequence row of the side cache: ceil(max_seq/block). */
int32_t skv_max_blocks(const skv_cache* c);

/*
 * skv_kv_append — write n_new consecutive tokens into every sequence.
 * Defines: cpu-attn kernel card, "Method" (int8 cache: per token and per KV
 * head, a = max_d |x_d|, scale = a / 127 in float32, code_d =
 * rint(x_d / scale) clamped to [-127, 127], a == 0 giving scale 0 and codes 0);
 * sparse_attn.md, "All-KV-types composition" and "S2/S3 engineering design"
 * item 1 (side cache: per block, channel min/max of the new pre-quantization
 * keys, min/max-merged into a block that already holds earlier tokens,
 * overwriting a block whose first position is >= pos0).
 *   pos0   : device int32 [batch]; sequence b receives positions
 *            pos0[b] .. pos0[b] + n_new - 1.  Tokens before pos0[b] must
 *            already be in the cache (the bounds merge assumes a filled
 *            prefix).  Rows at positions >= max_seq (or a negative pos0) are
 *            not written.
 *   n_new  : >= 1 tokens per sequence.
 *   k_new,
 *   v_new  : device [batch][n_new][n_kv_heads][head_dim] of src_dtype:
 *            SKV_F16 for an f16 cache (copied bit for bit), SKV_F32 for an
 *            int8, q8_0 or q4_0 cache (quantized; side-cache bounds are the
 *            float32 min rounded toward -inf and max rounded toward +inf into
 *            f16).
 * Errors: SKV_EINVAL (NULL, n_new < 1), SKV_ERANGE (n_new > max_seq),
 * SKV_EUNSUPPORTED (other dtype pairs), SKV_EDEVICE.
 */
skv_status skv_kv_append(const skv_cache* c, const int32_t* pos0, int32_t n_new,
                         const void* k_new, const void* v_new, int32_t src_dtype,
                         hipStream_t stream);

/*
 * skv_block_bounds — Quest upper bound per block, reduced over the GQA group.
 * Defines: sparse_attn.md, "Method" (UB = sum_d max(q_d * kmin_d,
 * q_d * kmax_d)) and "S2/S3 engineering design" item 2 / "Open questions"
 * (max of UB over the query heads of a KV head gives one score per block).
 * A channel with q_d == 0 contributes 0.  Computed in float32.
 *   q       : device float32 [batch][n_heads][head_dim], the query as given
 *             (no softmax scale; the bound only ranks blocks).
 *   seq_len : device int32 [batch]; sequence b has L_b tokens, clamped to
 *             [0, max_len]; blocks j < ceil(L_b / block) are scored.
 *   max_len : host upper bound of every L_b, <= max_seq.
 *   score   : device float32 [batch][n_kv_heads][max_blocks]; entries of
 *             blocks >= ceil(L_b / block) are not written.
 * Errors: SKV_EINVAL (NULL, no side cache, H % Hkv), SKV_ERANGE (max_len),
 * SKV_EUNSUPPORTED, SKV_EDEVICE.
 */
skv_status skv_block_bounds(const skv_cache* c, const float* q, int32_t n_heads,
                            const int32_t* seq_len, int32_t max_len, float* score,
                            hipStream_t stream);

/*
 * skv_select_topk — fixed top-K block selection per (sequence, KV head).
 * Defines: sparse_attn.md, "Method" (top-K_SEL blocks by bound plus the
 * recent window and the attention-sink block) and "Budget policy" (fixed K).
 * Forced blocks F = [0, n_sink) and [NB - n_recent, NB), NB =
 * ceil(L_b / block).  The k_sel[b] highest-scoring blocks among the others are
 * added (scores compare by value, -0 == +0; exact ties go to the lower block
 * index); if k_sel[b] covers every other block, all NB blocks are selected.
 * The selected set is written in ascending block order.
 *   score    : device float32 [batch][n_kv_heads][max_blocks] (from
 *              skv_block_bounds).
 *   seq_len  : device int32 [batch], clamped to [0, max_blocks * block].
 *   k_sel    : device int32 [batch]; negative values count as 0.
 *   max_sel  : capacity of each selected list; should be >= k_sel[b] + n_sink
 *              + n_recent.  At most max_sel indices are written.
 *   sel_idx  : device int32 [batch][n_kv_heads][max_sel]; entries past the
 *              set are filled with -1.
 *   sel_cnt  : device int32 [batch][n_kv_heads]: |S| = min(NB, k + |F|),
 *              reported in full even when it exceeds max_sel (that signals a
 *              truncated list; skv_decode_attn reads at most max_sel).
 *   sel_mask : optional (NULL = none) device uint32
 *              [batch][n_kv_heads][ceil(max_blocks / 32)]: bit (j % 32) of
 *              word j / 32 set iff block j is selected.
 * Errors: SKV_EINVAL (NULL, negative n_sink/n_recent, max_sel < 1),
 * SKV_EUNSUPPORTED (max_blocks > 16384), SKV_EDEVICE.
 */
skv_status skv_select_topk(const float* score, const int32_t* seq_len, int32_t batch,
                           int32_t n_kv_heads, int32_t max_blocks, int32_t block,
                           const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                           int32_t max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                           uint32_t* sel_mask, hipStream_t stream);

/*
 * skv_decode_attn — split-K partial attention (first half of a flash-decode).
 * Defines: for every query head, the softmax over the attended tokens of
 * s_t = (q . k_t) * softmax_scale and the weighted sum of v_t.
 *   f16 cache: s_t from float32 products of the query and the f16 keys;
 *   int8 cache: the query head is quantized with the absmax rule of
 *     skv_kv_append, dot_t = sum_d q_code_d * k_code_{t,d} exactly in int32,
 *     s_t = dot_t * q_scale * k_scale_t * softmax_scale; v_t = v_scale_t *
 *     v_code_t (cpu-attn kernel card, "Method").
 * Softmax and accumulation are float32.  Attended tokens: all of
 * [0, L_b) (dense, sel_idx == NULL), or the tokens of the selected blocks
 * with the last block clipped at L_b (sparse; sparse_attn.md "Method",
 * kernel skip).  Selected indices outside [0, NB) are ignored.
 * The tokens of (sequence, KV head) are cut into n_split contiguous parts
 * (dense: runs of blocks; sparse: runs of the selected list); each part
 * writes one partial state per query head into the workspace:
 *   workspace = float m[batch][n_heads][n_split],
 *               float l[batch][n_heads][n_split],
 *               float o[batch][n_heads][n_split][head_dim]
 *   with, over the part's tokens T: m = max_t s_t * log2(e), l = sum_t
 *   2^(s_t log2 e - m), o = sum_t 2^(s_t log2 e - m) v_t; an empty part has
 *   m = -inf, l = 0, o = 0.
 *   q          : device float32 [batch][n_heads][head_dim].
 *   seq_len    : device int32 [batch], clamped to [0, max_len].
 *   max_len    : host upper bound of every L_b, <= max_seq.
 *   sel_idx,
 *   sel_cnt    : from skv_select_topk, or both NULL for dense.
 *   max_sel    : row length of sel_idx (ignored for dense).
 *   n_split    : 1 .. 4096 parts per (sequence, KV head).
 *   dbg_logits : optional (NULL = none), int8 cache only: device int32
 *                [batch][n_heads][max_len] receiving the exact integer dots
 *                of the attended tokens (others untouched).
 * Errors: SKV_EINVAL, SKV_ERANGE, SKV_EWORKSPACE, SKV_EUNSUPPORTED,
 * SKV_EDEVICE.
 */
skv_status skv_decode_attn(const skv_cache* c, const float* q, int32_t n_heads,
                           const int32_t* seq_len, int32_t max_len,
                           const int32_t* sel_idx, const int32_t* sel_cnt, int32_t max_sel,
                           float softmax_scale, int32_t n_split,
                           void* workspace, size_t workspace_bytes,
                           int32_t* dbg_logits, hipStream_t stream);

/*
 * skv_decode_attn_select — skv_select_topk followed by skv_decode_attn over
 * the selected list, with the selection folded into the attention kernel's
 * prologue: one launch instead of two, and no round trip of the list through
 * memory before the first K/V load.  Defines: sparse_attn.md, "Open
 * questions" (computing the selector as its own small operator or folding it
 * into the attention launch) and "Method" (the selection and the kernel
 * skip).  Every part of a (sequence, KV head) recomputes the row's selection
 * (bit-identical to skv_select_topk's) and walks its share of the list.
 * The results -- the workspace's partial states, sel_idx, sel_cnt -- are
 * bit-identical to
 *     skv_select_topk(score, seq_len, batch, n_kv_heads, max_blocks, block,
 *                     k_sel, n_sink, n_recent, max_sel, sel_idx, sel_cnt, NULL)
 *     skv_decode_attn(c, q, n_heads, seq_len, max_len, sel_idx, sel_cnt,
 *                     max_sel, softmax_scale, n_split, workspace,
 *                     workspace_bytes, NULL)
 * with max_blocks = skv_max_blocks(c).  The fold applies when max_blocks <=
 * 4096 and ceil(max_sel / n_split) <= 64; otherwise the two kernels run one
 * after the other (same results).
 *   Arguments as in skv_select_topk (score, k_sel, n_sink, n_recent,
 *   max_sel, sel_idx, sel_cnt) and skv_decode_attn (the rest).
 * Errors: those of the two calls, checked before any launch.
 */
skv_status skv_decode_attn_select(const skv_cache* c, const float* q, int32_t n_heads,
                                  const int32_t* seq_len, int32_t max_len, const float* score,
                                  const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                                  int32_t max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                                  float softmax_scale, int32_t n_split, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * Per-query-head selection.  sparse_attn.md, "S2/S3 engineering design"
 * item 2 and "Open questions": the group max above gives one block set per KV
 * head; the alternative keeps one set per query head.  Three calls:
 *   skv_block_bounds_heads  each query head's own bound per block;
 *   skv_select_topk         unchanged, called with n_kv_heads = n_heads (one
 *                           row per query head: score [batch][n_heads][...],
 *                           sel_idx [batch][n_heads][max_sel]);
 *   skv_select_union        per KV head, the union of its G heads' lists
 *                           with the heads that chose each block;
 *   skv_decode_attn_heads   attention over the union, each query head over
 *                           its own blocks only; skv_combine as usual.
 * The union's blocks are read once for the whole group.
 */

/*
 * skv_block_bounds_heads — skv_block_bounds without the group max:
 * score[b][h][j] = sum_d max(q_hd * kmin_gjd, q_hd * kmax_gjd), g = h / G.
 *   score : device float32 [batch][n_heads][max_blocks]; entries of blocks
 *           >= ceil(L_b / block) are not written.
 * Other arguments and errors as skv_block_bounds.
 */
skv_status skv_block_bounds_heads(const skv_cache* c, const float* q, int32_t n_heads,
                                  const int32_t* seq_len, int32_t max_len, float* score,
                                  hipStream_t stream);

/*
 * skv_select_union — for each (sequence, KV head), the ascending union of
 * the per-query-head lists of its G = n_heads / n_kv_heads heads.
 *   sel_idx, sel_cnt : from skv_select_topk over per-head rows
 *                      ([batch][n_heads][max_sel], [batch][n_heads]); at most
 *                      min(sel_cnt, max_sel) entries per head are read,
 *                      entries outside [0, max_blocks) are ignored.
 *   uni_idx  : device int32 [batch][n_kv_heads][max_union], ascending, padded
 *              with -1; at most max_union entries are written.
 *   uni_cnt  : device int32 [batch][n_kv_heads], the union's full size
 *              (larger than max_union signals a truncated list; it is at
 *              most min(NB, G * max_sel)).
 *   uni_mask : device uint32 [batch][n_kv_heads][max_union]: bit i set iff
 *              query head g * G + i chose the entry's block (0 on padding).
 * Errors: SKV_EINVAL (NULL, sizes < 1, n_heads % n_kv_heads),
 * SKV_EUNSUPPORTED (G not in {1, 2, 4, 8}, max_blocks > 16384), SKV_ERANGE,
 * SKV_EDEVICE.
 */
skv_status skv_select_union(const int32_t* sel_idx, const int32_t* sel_cnt, int32_t batch,
                            int32_t n_heads, int32_t n_kv_heads, int32_t max_sel,
                            int32_t max_blocks, int32_t max_union, int32_t* uni_idx,
                            int32_t* uni_cnt, uint32_t* uni_mask, hipStream_t stream);

/*
 * skv_decode_attn_heads — skv_decode_attn over a KV head's union list where
 * query head g * G + i attends only the blocks whose uni_mask bit i is set
 * (its own selected set): for every query head, the softmax over exactly its
 * own blocks' tokens (last block clipped at L_b).  Partial states as
 * skv_decode_attn (a part where a head has no block: m = -inf, l = 0, o = 0).
 *   uni_idx, uni_cnt, uni_mask, max_union : from skv_select_union.
 * Every cache type (f16, int8, q8_0, q4_0, q5_0).  Other arguments,
 * workspace and errors as skv_decode_attn.
 */
skv_status skv_decode_attn_heads(const skv_cache* c, const float* q, int32_t n_heads,
                                 const int32_t* seq_len, int32_t max_len,
                                 const int32_t* uni_idx, const int32_t* uni_cnt,
                                 const uint32_t* uni_mask, int32_t max_union,
                                 float softmax_scale, int32_t n_split, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Query-token chunks (sparse_attn.md, "S2/S3 engineering design" item 2 and
 * "Open questions": the selector serves the decode path first; a selector
 * for the prefill path, where one call carries many query tokens, is a later
 * stage whose rule the page leaves open).  A chunk is the last T = n_tokens
 * positions of each sequence, already appended: with L_b = seq_len[b] (the
 * chunk included), token t sits at position L_b - T + t and attends to the
 * positions [0, L_bt), L_bt = L_b - T + 1 + t (a token with L_bt <= 0
 * attends to nothing and gets zeros).  Each token is a decode query of its
 * own: dense over its prefix, or Quest with its own bound (group max over its
 * G heads), its own top-K with the sink and recent blocks counted over its
 * own ceil(L_bt / block) blocks, and attention over its own blocks clipped at
 * L_bt.  The bounds are the side cache's after the chunk's append (a block
 * may hold positions past L_bt: the bound then covers a superset of the keys
 * the token sees and stays sound).  A KV head's K/V are read once for the
 * chunk: its T x G query rows are the columns of one MFMA operand.
 * A chunk step:
 *     skv_block_bounds_multi -> skv_select_topk_multi -> skv_select_union_tokens
 *     -> skv_decode_attn_multi -> skv_combine(ws, batch, T * n_heads, ...)
 * (dense: skv_decode_attn_multi with NULL lists, then skv_combine).
 * q is float32 [batch][T][n_heads][head_dim]; T in {1, 2, 4, 8} with
 * T * G <= 16; head_dim 64, 128 or 256.
 */

/*
 * skv_block_bounds_multi — skv_block_bounds for each token of a chunk, the
 * side cache read once for the chunk.
 *   score : device float32 [batch][n_kv_heads][T][max_blocks]: token t's
 *           group-max bound; blocks >= ceil(L_b / block) are not written.
 * Errors: as skv_block_bounds; SKV_EUNSUPPORTED for T or T * G outside the
 * supported set.
 */
skv_status skv_block_bounds_multi(const skv_cache* c, const float* q, int32_t n_tokens,
                                  int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                                  float* score, hipStream_t stream);

/*
 * skv_select_topk_multi — skv_select_topk for each (sequence, KV head,
 * token) row of skv_block_bounds_multi's score, token t's row taking
 * L_bt = seq_len[b] - T + 1 + t positions (its own blocks, sink and recent
 * window) and the sequence's budget k_sel[b].
 *   sel_idx : device int32 [batch][n_kv_heads][T][max_sel], ascending, -1 pad.
 *   sel_cnt : device int32 [batch][n_kv_heads][T].
 * Errors: as skv_select_topk; SKV_EUNSUPPORTED for T not in {1, 2, 4, 8}.
 */
skv_status skv_select_topk_multi(const float* score, const int32_t* seq_len, int32_t batch,
                                 int32_t n_tokens, int32_t n_kv_heads, int32_t max_blocks,
                                 int32_t block, const int32_t* k_sel, int32_t n_sink,
                                 int32_t n_recent, int32_t max_sel, int32_t* sel_idx,
                                 int32_t* sel_cnt, hipStream_t stream);

/*
 * skv_select_union_tokens — for each (sequence, KV head), the ascending union
 * of its T tokens' lists; an entry's mask has bits [t G, (t + 1) G) set iff
 * token t chose the block (G = group, the query heads per KV head: one bit per
 * MFMA column of skv_decode_attn_multi).
 *   sel_idx, sel_cnt : from skv_select_topk_multi.
 *   uni_idx, uni_cnt, uni_mask, max_union : as skv_select_union.
 * Errors: SKV_EINVAL (NULL, sizes < 1), SKV_EUNSUPPORTED (T or G outside the
 * supported sets, T * G > 16, max_blocks > 16384), SKV_ERANGE, SKV_EDEVICE.
 */
skv_status skv_select_union_tokens(const int32_t* sel_idx, const int32_t* sel_cnt,
                                   int32_t batch, int32_t n_tokens, int32_t n_kv_heads,
                                   int32_t group, int32_t max_sel, int32_t max_blocks,
                                   int32_t max_union, int32_t* uni_idx, int32_t* uni_cnt,
                                   uint32_t* uni_mask, hipStream_t stream);

/*
 * skv_decode_attn_multi — split-K partial attention of a chunk: token t of
 * sequence b, query head h over its positions [0, L_bt), either all of them
 * (uni_idx, uni_cnt, uni_mask all NULL) or those of the union's blocks whose
 * mask has bit t G + (h % G) (its own selected set, from
 * skv_select_union_tokens).  Partial states as skv_decode_attn with
 * T * n_heads query rows per sequence, row t * n_heads + h: the workspace is
 * skv_workspace_bytes(batch, T * n_heads, head_dim, n_split) bytes, and
 * skv_combine(workspace, batch, T * n_heads, head_dim, n_split, out) gives
 * out float32 [batch][T][n_heads][head_dim].
 * Every cache type (f16, int8, q8_0, q4_0, q5_0).
 * Errors: as skv_decode_attn; SKV_EUNSUPPORTED for T or T * G outside the
 * supported set.
 */
skv_status skv_decode_attn_multi(const skv_cache* c, const float* q, int32_t n_tokens,
                                 int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                                 const int32_t* uni_idx, const int32_t* uni_cnt,
                                 const uint32_t* uni_mask, int32_t max_union,
                                 float softmax_scale, int32_t n_split, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * The 4-bit key index and its GQA-shared scan (Certified Sparse Attention via
 * Perturbed Retrieval: the abstract -- a 4-bit scan with deterministic
 * bounds, shared across the GQA group, generates the candidates exactly and
 * reads every key; the appendix layout table -- 4-bit codes of 64 B per token
 * at D = 128, per-block per-channel float32 lo and step).  A token-level
 * candidate generator; the certificate, perturbation and sampling layers of
 * that method are not part of this library.  Every cache type, block <= 256:
 * the keys k are the cache's (f16 values; for an int8 or group-wise cache
 * code x scale, one float32 product).
 *
 * Index, per block of `block` tokens and channel d: lo = min k, step =
 * fl32(fl32(max k - lo) / 15), code = clamp(rint(fl32(fl32(k - lo) / step)),
 * 0, 15) (0 if step == 0), err = max over the block of |fl32(k - fl32(lo +
 * fl32(step * code)))| (single float32 operations), so the reconstruction is
 * within err of every key.  Bounds for query head h and token t (block b):
 * s~ = sum_d q_d (lo_bd + step_bd code_td), r = sum_d |q_d| err_bd,
 * LB = s~ - r <= q . k_t <= UB = s~ + r.
 */

/*
 * skv_scan4_build — (re)build the index of blocks floor(pos0[b] / block) ..
 * ceil(L_b / block) - 1 from the cache's keys (call after an append with its
 * pos0, or with pos0 = 0 for the whole row).  pos0[b] < 0 skips sequence b.
 *   codes4 : device uint8 [batch][n_kv_heads][max_seq][head_dim / 2]: channel
 *            2i in the low nibble of byte i, 2i + 1 in the high nibble.
 *   lo, step, err : device float32 [batch][n_kv_heads][max_blocks][head_dim].
 * Errors: SKV_EINVAL, SKV_ERANGE (max_len), SKV_EUNSUPPORTED (block > 256),
 * SKV_EDEVICE.
 */
skv_status skv_scan4_build(const skv_cache* c, const int32_t* pos0, const int32_t* seq_len,
                           int32_t max_len, uint8_t* codes4, float* lo, float* step, float* err,
                           hipStream_t stream);

/* Bytes of workspace skv_scan4_candidates needs: 4 * batch * n_heads *
 * (max_len + n_split); 0 for invalid arguments. */
size_t skv_scan4_workspace_bytes(int32_t batch, int32_t n_heads, int32_t n_split,
                                 int32_t max_len);

/*
 * skv_scan4_candidates — one scan of the index per (sequence, KV head) for
 * its G query heads: for every head, the tokens whose exact q . k could lie
 * within delta of the largest, C_h = {t < L_b : UB_t >= max_u LB_u - delta}
 * (float32; a token within about 1e-5 relative of the threshold may fall
 * either way).  C_h contains every token with q . k_t >= max_u q . k_u -
 * delta.  delta is in q . k units (no softmax scale); finite, >= 0.
 *   workspace : at least skv_scan4_workspace_bytes(batch, n_heads, n_split,
 *               max_len) bytes, 16-byte aligned; afterwards it holds UB as
 *               float32 [batch][n_heads][max_len] (tokens < L_b), then the
 *               parts' largest LB [batch][n_heads][n_split].
 *   cand      : device uint32 [batch][n_heads][ceil(max_len / 32)]: bit t % 32
 *               of word t / 32 set iff token t is a candidate (every word
 *               written).
 *   cand_cnt  : device int32 [batch][n_heads]: |C_h|.
 * Errors: SKV_EINVAL, SKV_ERANGE, SKV_EWORKSPACE, SKV_EUNSUPPORTED, SKV_EDEVICE.
 */
skv_status skv_scan4_candidates(const skv_cache* c, const uint8_t* codes4, const float* lo,
                                const float* step, const float* err, const float* q,
                                int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                                float delta, int32_t n_split, void* workspace,
                                size_t workspace_bytes, uint32_t* cand, int32_t* cand_cnt,
                                hipStream_t stream);

/*
 * skv_decode_attn_sparse_v — skv_decode_attn that leaves out the value rows
 * of negligible softmax weight.  Defines: sparse_attn.md, "Compose (three
 * sparsity levers, three pipeline stages)" item 3 (inside the attended
 * blocks, skip the value work of positions whose post-softmax weight is
 * negligible), "Stacking with sparse-V" (a static threshold tau) and
 * "Adaptive tau (the eps mode)" (eps times the softmax denominator over the
 * number of positions, so the dropped mass stays below eps; eps = 0 falls
 * back to tau).  For each query head, with p_t the normalized softmax weight
 * of attended token t over all n attended tokens of its (sequence, KV head):
 * token t's value row is used iff p_t >= theta, theta = eps / n if eps > 0
 * else tau; the normalizer still counts every token, so
 *     out = sum over used t of p_t v_t.
 * tau = eps = 0 uses every row (the dense or Quest result).  The weights and
 * the decision are float32 (a token within about 1e-5 relative of theta may
 * fall either way).  Value rows no head of the group uses are not read (for
 * a group-wise cache neither their codes nor their scales).  Every cache
 * type (f16, int8, q8_0, q4_0, q5_0); the "All-KV-types composition"
 * section of the same page composes the levers with every cache type.
 * Two launches (the q.K pass, then the value pass over the kept rows); the
 * workspace then holds the standard partial states at its start, so
 *     skv_combine(workspace, batch, n_heads, head_dim, n_split, out)
 * produces the output.
 *   Arguments as skv_decode_attn, and:
 *   tau, eps   : thresholds, finite and >= 0 (SKV_EINVAL otherwise).
 *   workspace  : at least skv_sparse_v_workspace_bytes(batch, n_heads,
 *                n_kv_heads, head_dim, n_split, max_len) bytes, 16-byte
 *                aligned.  Layout: the skv_decode_attn partial states, then
 *                per part the q.K pass's logit maximum, denominator and
 *                token count, then each query head's base-2 logits.
 *   keep_mask  : optional (NULL = none) device uint32
 *                [batch][n_heads][ceil(max_len / 32)]: bit t % 32 of word
 *                t / 32 is set iff token t's value row was used for the
 *                head; words of tokens that are not attended are not written
 *                (zero the buffer first).
 * Errors: those of skv_decode_attn.
 */
skv_status skv_decode_attn_sparse_v(const skv_cache* c, const float* q, int32_t n_heads,
                                    const int32_t* seq_len, int32_t max_len,
                                    const int32_t* sel_idx, const int32_t* sel_cnt,
                                    int32_t max_sel, float softmax_scale, float tau, float eps,
                                    int32_t n_split, void* workspace, size_t workspace_bytes,
                                    uint32_t* keep_mask, hipStream_t stream);

/* Bytes of workspace skv_decode_attn_sparse_v needs; 0 for invalid arguments. */
size_t skv_sparse_v_workspace_bytes(int32_t batch, int32_t n_heads, int32_t n_kv_heads,
                                    int32_t head_dim, int32_t n_split, int32_t max_len);

/*
 * skv_combine — merge the split-K partial states into the output.
 * Defines: M = max_i m_i; out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i
 * over the non-empty parts: the output as a sum of partial numerators over a
 * sum of partial masses, each part's pair scaled to the common maximum
 * (SCSA: Self-Calibrating Subquadratic Attention, "Mechanism", per-query
 * step 4, forms its output the same way from an exact and a tail part).  A
 * query head whose parts are all empty (L_b == 0) gets zeros.
 *   workspace : as written by skv_decode_attn with the same batch, n_heads,
 *               head_dim, n_split.
 *   out       : device float32 [batch][n_heads][head_dim].
 * Errors: SKV_EINVAL, SKV_EUNSUPPORTED, SKV_EDEVICE.
 */
skv_status skv_combine(const void* workspace, int32_t batch, int32_t n_heads,
                       int32_t head_dim, int32_t n_split, float* out, hipStream_t stream);

/*
 * skv_decode_step — one whole decode step in three kernel launches (Quest)
 * or two (dense).
 * Defines: the composition of the calls above, in the order the pages run
 * them (cpu-attn kernel card, "Usage": append the token, then decode;
 * sparse_attn.md, "S2/S3 engineering design": fill the side cache, select,
 * attend over the selected blocks).  The results -- out, the cache rows,
 * scales and bounds, score, sel_idx, sel_cnt -- are bit-identical to
 *     skv_kv_append(c, pos0, 1, k_new, v_new, src_dtype)        if k_new
 *     skv_block_bounds(c, q, n_heads, seq_len, max_len, score)   if k_sel
 *     skv_select_topk(score, seq_len, batch, n_kv_heads, max_blocks, block,
 *                     k_sel, n_sink, n_recent, max_sel, sel_idx, sel_cnt,
 *                     NULL)                                       if k_sel
 *     skv_decode_attn(c, q, n_heads, seq_len, max_len, sel_idx | NULL,
 *                     sel_cnt | NULL, max_sel, softmax_scale, n_split,
 *                     workspace, workspace_bytes, NULL)
 *     skv_combine(workspace, batch, n_heads, head_dim, n_split, out)
 * with max_blocks = skv_max_blocks(c).  The append runs inside the bounds
 * pass (Quest) or inside the attention kernel (dense: the part whose blocks
 * hold pos0[b] writes the token, and the attention takes the token's row
 * from k_new, v_new, so the cache row's old contents are never read), and
 * the selection inside the attention kernel's prologue
 * (each part of a row recomputes it) when max_blocks <= 4096 and
 * ceil(max_sel / n_split) <= 64; otherwise they run as their own kernels.
 *   pos0, k_new, v_new, src_dtype : as skv_kv_append with n_new = 1
 *            (k_new, v_new: [batch][1][n_kv_heads][head_dim]); k_new == NULL
 *            skips the append (pos0, v_new, src_dtype ignored).
 *   q, n_heads, seq_len, max_len : as skv_decode_attn; seq_len counts the
 *            appended token.
 *   k_sel  : device int32 [batch] Quest budget; NULL = dense decode (then
 *            n_sink, n_recent, max_sel, score, sel_idx, sel_cnt are ignored).
 *   n_sink, n_recent, max_sel, score, sel_idx, sel_cnt : as
 *            skv_block_bounds / skv_select_topk; all required for Quest
 *            (score is scratch the caller owns; sel_idx, sel_cnt are outputs).
 *   softmax_scale, n_split, workspace, workspace_bytes : as skv_decode_attn.
 *   out    : device float32 [batch][n_heads][head_dim].
 * Errors: those of the composed calls (SKV_EINVAL, SKV_ERANGE,
 * SKV_EWORKSPACE, SKV_EUNSUPPORTED, SKV_EDEVICE), checked before any launch.
 */
skv_status skv_decode_step(const skv_cache* c, const int32_t* pos0, const void* k_new,
                           const void* v_new, int32_t src_dtype, const float* q,
                           int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                           const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                           int32_t max_sel, float* score, int32_t* sel_idx, int32_t* sel_cnt,
                           float softmax_scale, int32_t n_split, void* workspace,
                           size_t workspace_bytes, float* out, hipStream_t stream);

/*
 * skv_decode_step_static — skv_decode_step without caller scratch buffers.
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the score
 * row and the split-K workspace come from a fixed array inside the library,
 * skv_static_scratch_bytes() bytes (16 MiB) per GPU, held by each GPU the
 * library runs on from the first call there until the process ends.  The
 * call allocates nothing; the caller still passes every input and output.
 *   Arguments and results are those of skv_decode_step (same kernels, same
 *   bits), without score, workspace and workspace_bytes.
 *   Capacity: 4 * batch * n_heads * n_split * (head_dim + 2) bytes of
 *   workspace, plus (Quest only) 4 * batch * n_kv_heads * max_blocks bytes of
 *   scores rounded up to 256, must fit in the array; larger calls return
 *   SKV_ERANGE before anything is enqueued.
 *   Concurrency: every call on one GPU uses the same array, so calls that may
 *   overlap on one GPU (different streams without ordering between them)
 *   race; calls ordered on one stream are safe.  Nothing in the array needs
 *   clearing between calls: each call writes what it reads.
 * Errors: those of skv_decode_step, SKV_ERANGE for a call beyond the array,
 * SKV_EDEVICE if the array's device address cannot be obtained.
 */
skv_status skv_decode_step_static(const skv_cache* c, const int32_t* pos0, const void* k_new,
                                  const void* v_new, int32_t src_dtype, const float* q,
                                  int32_t n_heads, const int32_t* seq_len, int32_t max_len,
                                  const int32_t* k_sel, int32_t n_sink, int32_t n_recent,
                                  int32_t max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                                  float softmax_scale, int32_t n_split, float* out,
                                  hipStream_t stream);

/* Size in bytes of skv_decode_step_static's per-GPU scratch array. */
size_t skv_static_scratch_bytes(void);

/* Bytes of workspace skv_decode_attn needs: 4 * batch * n_heads * n_split *
 * (head_dim + 2); 0 for invalid arguments. */
size_t skv_workspace_bytes(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t n_split);

/* Static, human-readable name of a status code. */
const char* skv_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* SKV_H */
