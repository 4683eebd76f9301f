// decode_attn for head dims 64 and 256: the kernels of decode_kernels.h at
// that D, dense or over a given or fused-selected list, per-query-head masks
// and query-token chunks, G' = n_tok x G in {1, 2, 4, 8, 16}.  The folded
// one-token append stays at head dim 128 (the step runs the append kernel
// first at the other head dims).
#include "decode_kernels.h"

namespace skv {

namespace {

template <int D>
hipError_t launch_dim(const DecodeParams& p, const DecodeShape& sh, int G, hipStream_t stream) {
  const skv_cache& c = *p.c;
  const int fr = p.fused_r;
  const int32_t nt = p.n_tok;
  const bool hmk = p.sel_hmask != nullptr;
  const AppendArgs aa{};
  if (c.kv_dtype == SKV_F16) {
#define SKV_LAUNCH_F16(GG, SR, HMK)                                                             \
  decode_f16_mfma<D, GG, SR, false, HMK><<<sh.grid, kMThreads, 0, stream>>>(                   \
      static_cast<const uint16_t*>(c.k), static_cast<const uint16_t*>(c.v), p.q, p.seq_len,    \
      p.sel_idx, p.sel_cnt, p.max_sel, c.n_kv_heads, c.max_seq, c.block, p.max_len,           \
      p.n_split, sh.n_rows, sh.ups, sh.scale2, sh.ws_m, sh.ws_l, sh.ws_o, p.fsel, aa,         \
      p.sel_hmask, nt)
#define SKV_F16_G(GG)                                  \
  if (hmk) SKV_LAUNCH_F16(GG, 0, true);                \
  else if (fr == 2) SKV_LAUNCH_F16(GG, 2, false);      \
  else if (fr == 4) SKV_LAUNCH_F16(GG, 4, false);      \
  else if (fr > 0) SKV_LAUNCH_F16(GG, kFusedSelR, false); \
  else SKV_LAUNCH_F16(GG, 0, false)
    switch (G) {
      case 1: SKV_F16_G(1); break;
      case 2: SKV_F16_G(2); break;
      case 4: SKV_F16_G(4); break;
      case 8: SKV_F16_G(8); break;
      case 16:                // 16 columns: query-token chunks only (no fused variants)
        if (hmk) SKV_LAUNCH_F16(16, 0, true);
        else SKV_LAUNCH_F16(16, 0, false);
        break;
      default: return hipErrorInvalidValue;
    }
#undef SKV_F16_G
#undef SKV_LAUNCH_F16
    return hipGetLastError();
  }
  if (c.kv_dtype != SKV_I8) return hipErrorInvalidValue;
#define SKV_LAUNCH_I8(GG, SR, HMK)                                                              \
  decode_i8_mfma<D, GG, SR, false, HMK><<<sh.grid, kMThreads, 0, stream>>>(                    \
      static_cast<const int8_t*>(c.k), static_cast<const int8_t*>(c.v), c.k_scale, c.v_scale,  \
      p.q, p.seq_len, p.sel_idx, p.sel_cnt, p.max_sel, c.n_kv_heads, c.max_seq, c.block,       \
      p.max_len, p.n_split, sh.n_rows, sh.ups, sh.scale2, sh.ws_m, sh.ws_l, sh.ws_o,           \
      p.dbg_logits, p.fsel, aa, p.sel_hmask, nt)
#define SKV_I8_G(GG)                                   \
  if (hmk) SKV_LAUNCH_I8(GG, 0, true);                 \
  else if (fr == 2) SKV_LAUNCH_I8(GG, 2, false);       \
  else if (fr == 4) SKV_LAUNCH_I8(GG, 4, false);       \
  else if (fr > 0) SKV_LAUNCH_I8(GG, kFusedSelR, false); \
  else SKV_LAUNCH_I8(GG, 0, false)
  switch (G) {
    case 1: SKV_I8_G(1); break;
    case 2: SKV_I8_G(2); break;
    case 4: SKV_I8_G(4); break;
    case 8: SKV_I8_G(8); break;
    case 16:
      if (hmk) SKV_LAUNCH_I8(16, 0, true);
      else SKV_LAUNCH_I8(16, 0, false);
      break;
    default: return hipErrorInvalidValue;
  }
#undef SKV_I8_G
#undef SKV_LAUNCH_I8
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_dims(const DecodeParams& p, hipStream_t stream) {
  const skv_cache& c = *p.c;
  if (c.block % 16 != 0) return hipErrorInvalidValue;
  if (p.app.k_new != nullptr) return hipErrorInvalidValue;
  // MFMA columns per KV head: n_tok query tokens x the group's heads
  const int32_t nt = p.n_tok;
  if (nt != 1 && nt != 2 && nt != 4 && nt != 8) return hipErrorInvalidValue;
  const int G = (p.n_heads / c.n_kv_heads) * nt;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return hipErrorInvalidValue;
  if (nt > 1 && p.fused_r > 0) return hipErrorInvalidValue;
  const bool hmk = p.sel_hmask != nullptr;
  if (hmk && (p.sel_idx == nullptr || p.fused_r > 0)) return hipErrorInvalidValue;
  DecodeShape sh;
  if (decode_shape(p, nt, sh) != hipSuccess) return hipErrorInvalidValue;
  switch (c.head_dim) {
    case 64: return launch_dim<64>(p, sh, G, stream);
    case 256: return launch_dim<256>(p, sh, G, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace skv
