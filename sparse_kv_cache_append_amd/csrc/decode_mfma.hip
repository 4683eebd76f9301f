// decode_attn launcher: head dim 128 with every variant (dense, a given
// list, the fused selection, the folded one-token append, per-query-head
// masks, query-token chunks); head dims 64 and 256 go to decode_dims.hip.
// The kernels and their data flow are in decode_kernels.h.
#include "decode_kernels.h"

namespace skv {

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const skv_cache& c = *p.c;
  if (c.head_dim != kD) return launch_decode_dims(p, stream);
  if (c.block % 16 != 0) return hipErrorInvalidValue;
  const int32_t H = p.n_heads, S = p.n_split;
  // MFMA columns per KV head: n_tok query tokens x the group's heads
  const int32_t nt = p.n_tok;
  if (nt != 1 && nt != 2 && nt != 4 && nt != 8) return hipErrorInvalidValue;
  const int G = (H / c.n_kv_heads) * nt;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return hipErrorInvalidValue;
  if (nt > 1 && (p.fused_r > 0 || p.app.k_new != nullptr)) return hipErrorInvalidValue;
  DecodeShape sh;
  if (decode_shape(p, nt, sh) != hipSuccess) return hipErrorInvalidValue;
  const int fr = p.fused_r;
  const bool app = p.app.k_new != nullptr;
  const bool hmk = p.sel_hmask != nullptr;
  if (hmk && (p.sel_idx == nullptr || fr > 0 || app)) return hipErrorInvalidValue;
  AppendArgs aa{};
  if (app) {
    if (p.sel_idx != nullptr || fr > 0 || p.app.v_new == nullptr || p.app.pos0 == nullptr)
      return hipErrorInvalidValue;
    aa = AppendArgs{c.k, c.v, c.k_scale, c.v_scale, c.kmin, c.kmax, p.app.k_new, p.app.v_new,
                    p.app.pos0, (c.max_seq + c.block - 1) / c.block};
  }
  if (c.kv_dtype == SKV_F16) {
#define SKV_LAUNCH_F16(GG, SR, AP, HMK)                                                         \
  decode_f16_mfma<kD, GG, SR, AP, HMK><<<sh.grid, kMThreads, 0, stream>>>(                     \
      static_cast<const uint16_t*>(c.k), static_cast<const uint16_t*>(c.v), p.q, p.seq_len,    \
      p.sel_idx, p.sel_cnt, p.max_sel, c.n_kv_heads, c.max_seq, c.block, p.max_len, S,        \
      sh.n_rows, sh.ups, sh.scale2, sh.ws_m, sh.ws_l, sh.ws_o, p.fsel, aa, p.sel_hmask, nt)
#define SKV_F16_G(GG)                                  \
  if (app) SKV_LAUNCH_F16(GG, 0, true, false);         \
  else if (hmk) SKV_LAUNCH_F16(GG, 0, false, true);    \
  else if (fr == 2) SKV_LAUNCH_F16(GG, 2, false, false); \
  else if (fr == 4) SKV_LAUNCH_F16(GG, 4, false, false); \
  else if (fr > 0) SKV_LAUNCH_F16(GG, kFusedSelR, false, false); \
  else SKV_LAUNCH_F16(GG, 0, false, false)
    switch (G) {
      case 1: SKV_F16_G(1); break;
      case 2: SKV_F16_G(2); break;
      case 4: SKV_F16_G(4); break;
      case 8: SKV_F16_G(8); break;
      default:                // 16 columns: query-token chunks only (no fused variants)
        if (hmk) SKV_LAUNCH_F16(16, 0, false, true);
        else SKV_LAUNCH_F16(16, 0, false, false);
        break;
    }
#undef SKV_F16_G
#undef SKV_LAUNCH_F16
    return hipGetLastError();
  }
  if (c.kv_dtype != SKV_I8) return hipErrorInvalidValue;
#define SKV_LAUNCH_I8(GG, SR, AP, HMK)                                                          \
  decode_i8_mfma<kD, GG, SR, AP, HMK><<<sh.grid, kMThreads, 0, stream>>>(                      \
      static_cast<const int8_t*>(c.k), static_cast<const int8_t*>(c.v), c.k_scale, c.v_scale,  \
      p.q, p.seq_len, p.sel_idx, p.sel_cnt, p.max_sel, c.n_kv_heads, c.max_seq, c.block,       \
      p.max_len, S, sh.n_rows, sh.ups, sh.scale2, sh.ws_m, sh.ws_l, sh.ws_o, p.dbg_logits,     \
      p.fsel, aa, p.sel_hmask, nt)
#define SKV_I8_G(GG)                                   \
  if (app) SKV_LAUNCH_I8(GG, 0, true, false);          \
  else if (hmk) SKV_LAUNCH_I8(GG, 0, false, true);     \
  else if (fr == 2) SKV_LAUNCH_I8(GG, 2, false, false); \
  else if (fr == 4) SKV_LAUNCH_I8(GG, 4, false, false); \
  else if (fr > 0) SKV_LAUNCH_I8(GG, kFusedSelR, false, false); \
  else SKV_LAUNCH_I8(GG, 0, false, false)
  switch (G) {
    case 1: SKV_I8_G(1); break;
    case 2: SKV_I8_G(2); break;
    case 4: SKV_I8_G(4); break;
    case 8: SKV_I8_G(8); break;
    default:
      if (hmk) SKV_LAUNCH_I8(16, 0, false, true);
      else SKV_LAUNCH_I8(16, 0, false, false);
      break;
  }
#undef SKV_I8_G
#undef SKV_LAUNCH_I8
  return hipGetLastError();
}

}  // namespace skv
