// Sparse-V decode attention: inside the attended tokens, the value rows whose
// softmax weight falls below a threshold are neither read nor accumulated
// (opencoti-llamafile sparse_attn.md, "Compose" item 3: skip the value work of
// negligible-weight positions inside the visited blocks; "Stacking with
// sparse-V": a static threshold tau; "Adaptive tau (the eps mode)": eps times
// the softmax denominator over the number of positions).
//
// The threshold is on the normalized weight p_t = 2^(s_t - M) / L of the
// whole attended set (M its maximum base-2 logit, L its denominator), so the
// rule needs M and L before any value row is touched.  Two launches:
//
//   pass A (sv_logits_*): the q.K half of the attention kernel -- K tiles
//     only -- writing each attended token's base-2 logit per query head and,
//     per part, the logit maximum, the denominator relative to it and the
//     token count;
//   pass B (sv_values_*): every part merges the row's pass-A states into M, L
//     and n, then walks its tiles reading each tile's logits two tiles ahead
//     of its value rows, so the keep decision (2^(s - M) >= theta L per head,
//     theta = tau, or eps / n) is known before the rows are requested: a row
//     no head keeps is requested at an out-of-range offset of its buffer
//     resource, which returns zeros without touching memory.  Kept weights
//     2^(s - M) <= 1 feed P.V (f16 high + low parts, as in the dense kernel);
//     the normalizer keeps every token.  Each part writes the standard
//     partial state (m = M, l = its own share of L, o = its kept sum), which
//     skv_combine merges as usual.
//
// Bytes per attended (token, KV head): pass A reads the K row (f16 2 D B,
// int8 D B + a 4-byte scale) and writes G logits; pass B reads the G logits
// and only the kept V rows (f16 2 D B, int8 D B + 4).  Head dims D = 64, 128
// and 256: a tile's 16-byte loads cover 1024 / row-bytes rows per
// instruction, the XOR swizzle runs over the row's 16-byte chunks (capped at
// 16), q.K takes D / 32 (f16) or D / 64 (int8) MFMA steps and P.V D / 16
// channel blocks; at D = 256 one workgroup runs per compute unit.
#include <type_traits>

#include "decode_core.h"
#include "device_common.h"
#include "grouped_core.h"
#include "launch.h"

namespace skv {
namespace {

// Offset past every tile resource's records: the load returns zeros and
// reads nothing.
constexpr uint32_t kSkipOffset = 0x7FFFFFF0u;
// Kept weights are at most 1; P.V takes them times 2^15 (exact), so weights
// down to 2^-18 keep the full precision of the f16 high + low parts.
constexpr int kPwShiftSvF16 = 15;

// Head dim D: workgroups per CU, and the chunk swizzle of a row of CHUNKS
// 16-byte chunks (chunk c of row r at c ^ (r % min(CHUNKS, 16))).
template <int D>
constexpr int sv_occ() { return D > 128 ? 1 : 2; }
template <int CHUNKS>
__device__ __forceinline__ int sv_swz(int row) { return row & ((CHUNKS < 16 ? CHUNKS : 16) - 1); }

// ------------------------------------------------------------ pass A helpers
// Running logit maximum, denominator and token count of one wavefront.
struct TileStats {
  float m = -INFINITY, l = 0.0f;
  int32_t n = 0;

  template <int NT>
  __device__ __forceinline__ void add(const float (&s)[4 * NT], int32_t nvalid) {
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 4 * NT; ++i) mx = fmaxf(mx, s[i]);
    mx = rows_max(mx);
    const float mn = fmaxf(m, mx);
    if (mn != -INFINITY) {
      float ps = 0.0f;
#pragma unroll
      for (int i = 0; i < 4 * NT; ++i) ps += __builtin_amdgcn_exp2f(s[i] - mn);
      ps = rows_sum(ps);
      l = l * __builtin_amdgcn_exp2f(m - mn) + ps;     // exp2(-inf) = 0 while l is 0
      m = mn;
    }
    n += max(nvalid, 0);
  }
};

// Merge the 4 wavefronts' stats of the group's heads and write the part's
// entry (heads < G: maximum, denominator relative to it; the row's count).
template <int G>
__device__ __forceinline__ void finish_stats(const TileStats& ts, float* lds, float* stat_m,
                                             float* stat_l, int32_t* stat_n, int64_t head0,
                                             int64_t bg, int32_t n_split, int32_t split) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  float* lm = lds;                          // [waves][G]
  float* ll = lm + kMWaves * G;
  int32_t* ln = reinterpret_cast<int32_t*>(ll + kMWaves * G);
  __syncthreads();                          // tile buffers are reused
  if (lane < G) { lm[wave * G + lane] = ts.m; ll[wave * G + lane] = ts.l; }
  if (lane == 0) ln[wave] = ts.n;
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) M = fmaxf(M, lm[w * G + h]);
    float sl = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kMWaves; ++w) {
        const float mw = lm[w * G + h];
        sl += mw == -INFINITY ? 0.0f : ll[w * G + h] * __builtin_amdgcn_exp2f(mw - M);
      }
    }
    stat_m[(head0 + h) * n_split + split] = M;
    stat_l[(head0 + h) * n_split + split] = sl;
  }
  if (threadIdx.x == 0) {
    int32_t n = 0;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) n += ln[w];
    stat_n[bg * n_split + split] = n;
  }
}

// ------------------------------------------------------------ pass B helpers
// The row's totals from pass A for this lane's head (lc, clamped into the
// group): M = max over parts, L = denominator relative to M, n = tokens.
// Lane l reduces head l % G over the parts i = l / G, l / G + 64 / G, ...,
// four parts per trip with their loads issued together; the lanes of a head
// then merge with lane swaps, and lane lc hands head lc's totals out.
struct RowTotals {
  float M, L;
  int32_t n;
};
__device__ __forceinline__ void merge_ml(float& M, float& L, float mi, float li) {
  const float mn = fmaxf(M, mi);
  if (mn != -INFINITY) {
    L = (M == -INFINITY ? 0.0f : L * __builtin_amdgcn_exp2f(M - mn)) +
        (mi == -INFINITY ? 0.0f : li * __builtin_amdgcn_exp2f(mi - mn));
    M = mn;
  }
}
template <int G>
__device__ __forceinline__ RowTotals row_totals(const float* stat_m, const float* stat_l,
                                                const int32_t* stat_n, int64_t head0, int64_t bg,
                                                int32_t n_split, int lc) {
  constexpr int kPer = kWave / G;                 // lanes per head
  const int lane = threadIdx.x % kWave;
  const int h = lane % G, s0 = lane / G;
  const float* pm = stat_m + (head0 + h) * n_split;
  const float* pl = stat_l + (head0 + h) * n_split;
  const int32_t* pn = stat_n + bg * n_split;
  float M = -INFINITY, L = 0.0f;
  int32_t n = 0;
  for (int32_t i0 = s0; i0 < n_split; i0 += 4 * kPer) {
    float mi[4], li[4];
    int32_t ni[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t i = i0 + u * kPer;
      const bool ok = i < n_split;
      mi[u] = ok ? pm[i] : -INFINITY;
      li[u] = ok ? pl[i] : 0.0f;
      ni[u] = ok ? pn[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      merge_ml(M, L, mi[u], li[u]);
      n += ni[u];
    }
  }
#pragma unroll
  for (int off = G; off < kWave; off *= 2) {
    const float mo = __shfl_xor(M, off), lo = __shfl_xor(L, off);
    merge_ml(M, L, mo, lo);
    n += __shfl_xor(n, off);
  }
  RowTotals t;
  t.M = __shfl(M, lc % G);
  t.L = __shfl(L, lc % G);
  t.n = n;                                        // the same in every lane
  return t;
}

// Merge the 4 wavefronts' kept sums (one reference M for all: a plain sum)
// and write the part's partial state: m = M, l = the part's own pass-A mass
// relative to M, o = its kept sum.
template <int G, int N>
__device__ __forceinline__ void finish_values(const float4_t (&O)[N], float Mh, float* lds,
                                              const float* stat_m, const float* stat_l,
                                              float* ws_m, float* ws_l, float* ws_o,
                                              int64_t head0, int32_t n_split, int32_t split) {
  constexpr int D = 16 * N;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  float* lo = lds;                          // [waves][G][D]
  float* lm = lds + kMWaves * G * D;        // [G]
  __syncthreads();
  const int g4 = 4 * (lane / 16);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = g4 + r;
    if (h < G) {
#pragma unroll
      for (int n = 0; n < N; ++n) lo[(wave * G + h) * D + 16 * n + lane % 16] = O[n][r];
    }
  }
  if (wave == 0 && lane < G) lm[lane] = Mh;
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kMThreads) {
    const int h = idx / D, d = idx % D;
    float so = 0.0f;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) so += lo[(w * G + h) * D + d];
    const int64_t ps = (head0 + h) * n_split + split;
    ws_o[ps * D + d] = so;
    if (d == 0) {
      const float M = lm[h], mi = stat_m[ps];
      ws_m[ps] = M;
      ws_l[ps] = (M == -INFINITY || mi == -INFINITY) ? 0.0f
                                                     : stat_l[ps] * __builtin_amdgcn_exp2f(mi - M);
    }
  }
}

// The keep decisions of one tile, shared by the lanes that load its value
// rows: each wavefront clears its T flag bytes, lanes set the flags of the
// tokens their heads keep, then every lane reads the flags of its rows (LDS
// executes one wavefront's accesses in order).
template <int T>
__device__ __forceinline__ void clear_flags(uint8_t* fl) {
  const int lane = threadIdx.x % kWave;
  if (lane < T / 4) reinterpret_cast<uint32_t*>(fl)[lane] = 0u;
}

struct SvArgs {
  float* stat_m;       // [B][H][S]
  float* stat_l;       // [B][H][S]
  int32_t* stat_n;     // [B][Hkv][S]
  float* logit;        // [B][H][lstride] (+ 32 floats of padding)
  int32_t lstride;     // max_len rounded up to a multiple of 32
  float* ws_m;
  float* ws_l;
  float* ws_o;
  uint32_t* keep;      // optional [B][H][ceil(max_len / 32)]
  float tau, eps;
};

// ====================================================================== f16
// Pass A: K tiles of 16 tokens, q.K on the matrix cores (query as f16 high +
// low parts, as in the dense kernel), logits and stats out.
template <int D, int G>
__global__ void __launch_bounds__(kMThreads, sv_occ<D>())
sv_logits_f16(const uint16_t* __restrict__ kc, const float* __restrict__ q,
              const int32_t* __restrict__ seq_len, const int32_t* __restrict__ sel_idx,
              const int32_t* __restrict__ sel_cnt, int32_t max_sel, int32_t Hkv,
              int32_t max_seq, int32_t block, int32_t max_len, int32_t n_split, int32_t n_rows,
              int32_t ups, float qscale2, SvArgs sv) {
  constexpr int T = 16;
  const int32_t lstride = sv.lstride;
  constexpr int RB = 2 * D;                                 // bytes per row
  constexpr int kTileBytes = T * RB;                        // 4096 at D = 128
  constexpr int kLoads = kTileBytes / 1024;                 // 16-byte loads per lane
  constexpr int kCpr = RB / 16;                             // chunks per row
  constexpr int kRpl = 1024 / RB;                           // rows per load instruction
  constexpr int KQ = D / 32;                                // q.K steps
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMWaves][2][kTileBytes];
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t split = int32_t(slot % uint32_t(n_split));
  const uint32_t row = xcd_row(slot / uint32_t(n_split), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const int32_t H = Hkv * G;
  const int64_t bg = int64_t(b) * Hkv + g;
  const int32_t L_raw = seq_len[b];
  const ListSeed ls = list_seed(sel_idx, sel_cnt, max_sel, bg, split, ups);
  half8_t qhi[KQ], qlo[KQ];
  const bool hv = lc < G;
  {
    const float* qp = q + (int64_t(b) * H + g * G + (hv ? lc : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(qp + 32 * kk + 8 * lg);
      const float4 c = *reinterpret_cast<const float4*>(qp + 32 * kk + 8 * lg + 4);
      const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float v = hv ? x[s] * qscale2 : 0.0f;
        const _Float16 h = (_Float16)v;
        qhi[kk][s] = h;
        qlo[kk][s] = (_Float16)(v - (float)h);
      }
    }
  }
  const int32_t L = __builtin_amdgcn_readfirstlane(min(max(L_raw, 0), max_len));
  TileWalk tw = make_walk<T>(ls, sel_idx, max_sel, bg, L, block, split, ups);
  tw.init(wave);
  TileStats ts;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(kc + bg * int64_t(max_seq) * D);
  float* lrow = sv.logit + (int64_t(b) * H + g * G + (hv ? lc : 0)) * int64_t(lstride);
  // lane loads row kRpl i + lane / kCpr of the tile, 16-byte chunk lane % kCpr
  struct Frag { int4_t k[kLoads]; int32_t r0, nvalid; };
  auto issue = [&](Frag& f) {
    int32_t r0 = 0, nv = 0;
    if (tw.more()) tw.next<T>(r0, nv);
    f.r0 = r0;
    f.nvalid = nv;
    const uint32_t lo = 16u * uint32_t(lane);
    const int bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * RB);
    const auto kr = tile_rsrc(kbase + int64_t(r0) * RB, bytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) f.k[i] = tile_load(kr, lo + 1024 * i);
  };
  auto process = [&](auto bufc, Frag& fr) {
    constexpr int kBuf = decltype(bufc)::value;
    uint8_t* kt = smem[wave][kBuf];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int rw = kRpl * i + lane / kCpr;
      *reinterpret_cast<int4_t*>(kt + rw * RB + 16 * ((lane % kCpr) ^ sv_swz<kCpr>(rw))) =
          fr.k[i];
    }
    const int32_t nvalid = fr.nvalid, r0 = fr.r0;
    issue(fr);
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const half8_t a = *reinterpret_cast<const half8_t*>(
          kt + lc * RB + 16 * ((lg + 4 * kk) ^ sv_swz<kCpr>(lc)));
      acc = mfma_f16_32(a, qhi[kk], acc);
      acc = mfma_f16_32(a, qlo[kk], acc);
    }
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (4 * lg + r < nvalid) ? acc[r] : -INFINITY;
    ts.add<1>(sc, nvalid);
    if (hv && nvalid > 0) {
      if (nvalid == T) {
        *reinterpret_cast<float4*>(lrow + r0 + 4 * lg) = make_float4(sc[0], sc[1], sc[2], sc[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * lg + r < nvalid) lrow[r0 + 4 * lg + r] = sc[r];
      }
    }
  };
  Frag f0, f1;
  const int32_t n_mine = tw.count();
  issue(f0);
  issue(f1);
  for (int32_t t = 0; t + 1 < n_mine; t += 2) {
    process(std::integral_constant<int, 0>{}, f0);
    process(std::integral_constant<int, 1>{}, f1);
  }
  if (n_mine & 1) process(std::integral_constant<int, 0>{}, f0);
  finish_stats<G>(ts, reinterpret_cast<float*>(&smem[0][0][0]), sv.stat_m, sv.stat_l, sv.stat_n,
                  int64_t(b) * H + g * G, bg, n_split, split);
}

// Pass B: V tiles of 16 tokens, only the rows some head keeps.
template <int D, int G>
__global__ void __launch_bounds__(kMThreads, sv_occ<D>())
sv_values_f16(const uint16_t* __restrict__ vc, const int32_t* __restrict__ seq_len,
              const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
              int32_t max_sel, int32_t Hkv, int32_t max_seq, int32_t block, int32_t max_len,
              int32_t n_split, int32_t n_rows, int32_t ups, int32_t keep_words, SvArgs sv) {
  constexpr int T = 16;
  const int32_t lstride = sv.lstride;
  constexpr int RB = 2 * D;                                 // bytes per row
  constexpr int kTileBytes = T * RB;                        // 4096 at D = 128
  constexpr int kLoads = kTileBytes / 1024;                 // 16-byte loads per lane
  constexpr int kCpr = RB / 16;                             // chunks per row
  constexpr int kRpl = 1024 / RB;                           // rows per load instruction
  constexpr int NB = D / 16;                                // P.V channel blocks
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMWaves][2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t flags[kMWaves][T];
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t split = int32_t(slot % uint32_t(n_split));
  const uint32_t row = xcd_row(slot / uint32_t(n_split), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const int32_t H = Hkv * G;
  const int64_t bg = int64_t(b) * Hkv + g;
  const int32_t L_raw = seq_len[b];
  const ListSeed ls = list_seed(sel_idx, sel_cnt, max_sel, bg, split, ups);
  const bool hl = lc < G;
  const int64_t hrow = int64_t(b) * H + g * G + (hl ? lc : 0);
  const RowTotals rt = row_totals<G>(sv.stat_m, sv.stat_l, sv.stat_n, int64_t(b) * H + g * G,
                                     bg, n_split, lc);
  const float theta = sv.eps > 0.0f ? sv.eps / float(max(rt.n, 1)) : sv.tau;
  const float thr = theta * rt.L;           // keep iff 2^(s - M) >= theta L
  const bool hv = hl && rt.M != -INFINITY;
  const int32_t L = __builtin_amdgcn_readfirstlane(min(max(L_raw, 0), max_len));
  TileWalk tw = make_walk<T>(ls, sel_idx, max_sel, bg, L, block, split, ups);
  tw.init(wave);
  float4_t O[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) O[n] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(vc + bg * int64_t(max_seq) * D);
  const float* lrow = sv.logit + hrow * int64_t(lstride);
  uint16_t* krow = sv.keep != nullptr
                       ? reinterpret_cast<uint16_t*>(sv.keep + hrow * int64_t(keep_words))
                       : nullptr;
  uint8_t* fl = flags[wave];
  // a tile's logits (this lane: tokens 4 lg .. 4 lg + 3 of head lc), requested
  // two tiles ahead of its value rows; the padding past the buffer's rows
  // keeps the whole float4 in bounds
  struct Lgt { float4 s; int32_t r0, nvalid; };
  struct Frag { int4_t v[kLoads]; float p[4]; int32_t r0, nvalid; };
  auto issue_logits = [&](Lgt& lt) {
    int32_t r0 = 0, nv = 0;
    if (tw.more()) tw.next<T>(r0, nv);
    lt.r0 = r0;
    lt.nvalid = nv;
    lt.s = *reinterpret_cast<const float4*>(lrow + (nv > 0 ? r0 + 4 * lg : 0));
  };
  // keep decisions and weights of the tile in lt, then its kept value rows
  auto fill = [&](Frag& f, const Lgt& lt) {
    const int32_t r0 = lt.r0, nv = lt.nvalid;
    f.r0 = r0;
    f.nvalid = nv;
    const float s[4] = {lt.s.x, lt.s.y, lt.s.z, lt.s.w};
    bool keep[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float w = __builtin_amdgcn_exp2f(s[r] - rt.M);
      keep[r] = hv && 4 * lg + r < nv && w >= thr;
      f.p[r] = keep[r] ? w : 0.0f;
    }
    clear_flags<T>(fl);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (f.p[r] > 0.0f) fl[4 * lg + r] = 1;
    if (krow != nullptr && nv > 0) {
      uint64_t bal[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) bal[r] = __ballot(int(keep[r]));
      if (lg == 0 && hl) {
        uint32_t bits = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int r = 0; r < 4; ++r) bits |= uint32_t((bal[r] >> (16 * j + lc)) & 1u) << (4 * j + r);
        }
        krow[r0 / 16] = uint16_t(bits);
      }
    }
    const uint32_t lo = 16u * uint32_t(lane);
    const int bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * RB);
    const auto vr = tile_rsrc(vbase + int64_t(r0) * RB, bytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const bool need = fl[kRpl * i + lane / kCpr] != 0;   // row kRpl i + lane / kCpr
      f.v[i] = tile_load(vr, need ? lo + 1024 * i : kSkipOffset);
    }
  };
  auto process = [&](auto bufc, Frag& fr, Lgt& lt) {
    constexpr int kBuf = decltype(bufc)::value;
    uint8_t* vt = smem[wave][kBuf];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int rw = kRpl * i + lane / kCpr;
      *reinterpret_cast<int4_t*>(vt + rw * RB + 16 * ((lane % kCpr) ^ sv_swz<kCpr>(rw))) =
          fr.v[i];
    }
    float pc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pc[r] = fr.p[r];
    fill(fr, lt);            // the tile two ahead
    issue_logits(lt);        // and the logits of the tile four ahead
    half4_t phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = pc[r] * float(1 << kPwShiftSvF16);
      const _Float16 h = (_Float16)x;
      phi[r] = h;
      plo[r] = (_Float16)(x - (float)h);
    }
    const int tr_row = 4 * lg + (lc >> 2);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int chunk = 2 * n + ((lc & 3) >> 1);
      const int off = tr_row * RB + 16 * (chunk ^ sv_swz<kCpr>(tr_row)) + 8 * (lc & 1);
      const short4_t raw =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((SKV_LDS short4_t*)(vt + off));
      const half4_t bv = __builtin_bit_cast(half4_t, raw);
      O[n] = mfma_f16_16(phi, bv, O[n]);
      O[n] = mfma_f16_16(plo, bv, O[n]);
    }
  };
  Lgt la, lb;
  Frag f0, f1;
  const int32_t n_mine = tw.count();
  issue_logits(la);
  issue_logits(lb);
  fill(f0, la);
  issue_logits(la);
  fill(f1, lb);
  issue_logits(lb);
  for (int32_t t = 0; t + 1 < n_mine; t += 2) {
    process(std::integral_constant<int, 0>{}, f0, la);
    process(std::integral_constant<int, 1>{}, f1, lb);
  }
  if (n_mine & 1) process(std::integral_constant<int, 0>{}, f0, la);
#pragma unroll
  for (int n = 0; n < NB; ++n) {
#pragma unroll
    for (int r = 0; r < 4; ++r) O[n][r] *= 1.0f / float(1 << kPwShiftSvF16);
  }
  finish_values<G>(O, rt.M, reinterpret_cast<float*>(&smem[0][0][0]), sv.stat_m, sv.stat_l,
                   sv.ws_m, sv.ws_l, sv.ws_o, int64_t(b) * H + g * G, n_split, split);
}

// ===================================================================== int8
// Tiles of 32 tokens; token order inside a tile as in the dense int8 kernel:
// lane group lg holds tokens tok(lg, e) = 16 (e / 4) + 4 lg + e % 4.
template <int D, int G>
__global__ void __launch_bounds__(kMThreads, sv_occ<D>())
sv_logits_i8(const int8_t* __restrict__ kc, const float* __restrict__ ksc,
             const float* __restrict__ q, const int32_t* __restrict__ seq_len,
             const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
             int32_t max_sel, int32_t Hkv, int32_t max_seq, int32_t block, int32_t max_len,
             int32_t n_split, int32_t n_rows, int32_t ups, float scale2, SvArgs sv) {
  constexpr int T = 32;
  const int32_t lstride = sv.lstride;
  constexpr int RB = D;                                     // bytes per row
  constexpr int kTileBytes = T * RB;                        // 4096 at D = 128
  constexpr int kLoads = kTileBytes / 1024;                 // 16-byte loads per lane
  constexpr int kCpr = RB / 16;                             // chunks per row
  constexpr int kRpl = 1024 / RB;                           // rows per load instruction
  constexpr int KK = D / 64;                                // q.K steps
  constexpr int kBufBytes = kTileBytes + T * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMWaves][2][kBufBytes];
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t split = int32_t(slot % uint32_t(n_split));
  const uint32_t row = xcd_row(slot / uint32_t(n_split), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const int32_t H = Hkv * G;
  const int64_t bg = int64_t(b) * Hkv + g;
  const int32_t L_raw = seq_len[b];
  const ListSeed ls = list_seed(sel_idx, sel_cnt, max_sel, bg, split, ups);
  const bool hv = lc < G;
  float x[KK][16];
  {
    const float* qp = q + (int64_t(b) * H + g * G + (hv ? lc : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v4 = *reinterpret_cast<const float4*>(qp + 64 * kk + 16 * lg + 4 * i);
        x[kk][4 * i + 0] = v4.x; x[kk][4 * i + 1] = v4.y;
        x[kk][4 * i + 2] = v4.z; x[kk][4 * i + 3] = v4.w;
      }
    }
  }
  int4_t qb[KK];
  float coef;
  i8_query_operand(x, hv, scale2, qb, coef);
  const int32_t L = __builtin_amdgcn_readfirstlane(min(max(L_raw, 0), max_len));
  TileWalk tw = make_walk<T>(ls, sel_idx, max_sel, bg, L, block, split, ups);
  tw.init(wave);
  TileStats ts;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(kc + bg * int64_t(max_seq) * D);
  const float* ksb = ksc + bg * int64_t(max_seq);
  const int32_t last = max(L - 1, 0);
  float* lrow = sv.logit + (int64_t(b) * H + g * G + (hv ? lc : 0)) * int64_t(lstride);
  // lane loads row kRpl i + lane / kCpr of the tile, 16-byte chunk lane % kCpr
  struct Frag { int4_t k[kLoads]; float sc; int32_t r0, nvalid; };
  auto issue = [&](Frag& f) {
    int32_t r0 = 0, nv = 0;
    if (tw.more()) tw.next<T>(r0, nv);
    f.r0 = r0;
    f.nvalid = nv;
    const uint32_t lo = 16u * uint32_t(lane);
    const int bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * RB);
    const auto kr = tile_rsrc(kbase + int64_t(r0) * RB, bytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) f.k[i] = tile_load(kr, lo + 1024 * i);
    f.sc = ksb[min(r0 + lane % 32, last)];
  };
  auto sw = [](int rw, int chunk) { return rw * RB + 16 * (chunk ^ sv_swz<kCpr>(rw)); };
  auto process = [&](auto bufc, Frag& fr) {
    constexpr int kBuf = decltype(bufc)::value;
    uint8_t* kt = smem[wave][kBuf];
    float* st = reinterpret_cast<float*>(kt + kTileBytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int rw = kRpl * i + lane / kCpr;
      *reinterpret_cast<int4_t*>(kt + sw(rw, lane % kCpr)) = fr.k[i];
    }
    if (lane < 32) st[lane] = fr.sc;
    const int32_t nvalid = fr.nvalid, r0 = fr.r0;
    issue(fr);
    int4_t acc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      acc[s] = int4_t{0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int4_t a = *reinterpret_cast<const int4_t*>(kt + sw(16 * s + lc, lg + 4 * kk));
        acc[s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qb[kk], acc[s], 0, 0, 0);
      }
    }
    const float4 ks0 = *reinterpret_cast<const float4*>(st + 4 * lg);
    const float4 ks1 = *reinterpret_cast<const float4*>(st + 16 + 4 * lg);
    const float ks[8] = {ks0.x, ks0.y, ks0.z, ks0.w, ks1.x, ks1.y, ks1.z, ks1.w};
    float sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = 16 * (e / 4) + 4 * lg + e % 4;
      sc[e] = t < nvalid ? float(acc[e / 4][e % 4]) * coef * ks[e] : -INFINITY;
    }
    ts.add<2>(sc, nvalid);
    if (hv && nvalid > 0) {
      if (nvalid == T) {
        *reinterpret_cast<float4*>(lrow + r0 + 4 * lg) = make_float4(sc[0], sc[1], sc[2], sc[3]);
        *reinterpret_cast<float4*>(lrow + r0 + 16 + 4 * lg) =
            make_float4(sc[4], sc[5], sc[6], sc[7]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 16 * (e / 4) + 4 * lg + e % 4;
          if (t < nvalid) lrow[r0 + t] = sc[e];
        }
      }
    }
  };
  Frag f0, f1;
  const int32_t n_mine = tw.count();
  issue(f0);
  issue(f1);
  for (int32_t t = 0; t + 1 < n_mine; t += 2) {
    process(std::integral_constant<int, 0>{}, f0);
    process(std::integral_constant<int, 1>{}, f1);
  }
  if (n_mine & 1) process(std::integral_constant<int, 0>{}, f0);
  finish_stats<G>(ts, reinterpret_cast<float*>(&smem[0][0][0]), sv.stat_m, sv.stat_l, sv.stat_n,
                  int64_t(b) * H + g * G, bg, n_split, split);
}

// The weights of pass B are at most 1 (the whole set's maximum is the
// reference), so P' = p * v_scale * 2^(14 - e), 2^e >= every V scale seen so
// far, stays below 2^14 in f16.
constexpr int kPwShiftSvI8 = 14;

template <int D, int G>
__global__ void __launch_bounds__(kMThreads, sv_occ<D>())
sv_values_i8(const int8_t* __restrict__ vc, const float* __restrict__ vsc,
             const int32_t* __restrict__ seq_len, const int32_t* __restrict__ sel_idx,
             const int32_t* __restrict__ sel_cnt, int32_t max_sel, int32_t Hkv,
             int32_t max_seq, int32_t block, int32_t max_len, int32_t n_split, int32_t n_rows,
             int32_t ups, int32_t keep_words, SvArgs sv) {
  constexpr int T = 32;
  const int32_t lstride = sv.lstride;
  constexpr int RB = D;                                     // bytes per row
  constexpr int kTileBytes = T * RB;                        // 4096 at D = 128
  constexpr int kLoads = kTileBytes / 1024;                 // 16-byte loads per lane
  constexpr int kCpr = RB / 16;                             // chunks per row
  constexpr int kRpl = 1024 / RB;                           // rows per load instruction
  constexpr int NB = D / 16;                                // P.V channel blocks
  constexpr int kBufBytes = kTileBytes + T * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMWaves][2][kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t flags[kMWaves][T];
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t split = int32_t(slot % uint32_t(n_split));
  const uint32_t row = xcd_row(slot / uint32_t(n_split), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const int32_t H = Hkv * G;
  const int64_t bg = int64_t(b) * Hkv + g;
  const int32_t L_raw = seq_len[b];
  const ListSeed ls = list_seed(sel_idx, sel_cnt, max_sel, bg, split, ups);
  const bool hl = lc < G;
  const int64_t hrow = int64_t(b) * H + g * G + (hl ? lc : 0);
  const RowTotals rt = row_totals<G>(sv.stat_m, sv.stat_l, sv.stat_n, int64_t(b) * H + g * G,
                                     bg, n_split, lc);
  const float theta = sv.eps > 0.0f ? sv.eps / float(max(rt.n, 1)) : sv.tau;
  const float thr = theta * rt.L;
  const bool hv = hl && rt.M != -INFINITY;
  const int32_t L = __builtin_amdgcn_readfirstlane(min(max(L_raw, 0), max_len));
  TileWalk tw = make_walk<T>(ls, sel_idx, max_sel, bg, L, block, split, ups);
  tw.init(wave);
  float4_t O[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) O[n] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(vc + bg * int64_t(max_seq) * D);
  const float* vsb = vsc + bg * int64_t(max_seq);
  const float* lrow = sv.logit + hrow * int64_t(lstride);
  uint32_t* krow = sv.keep != nullptr ? sv.keep + hrow * int64_t(keep_words) : nullptr;
  uint8_t* fl = flags[wave];
  auto sw = [](int rw, int chunk) { return rw * RB + 16 * (chunk ^ sv_swz<kCpr>(rw)); };
  // logits of tokens tok(lg, 0..7): two float4 (tokens 4 lg .. and 16 + 4 lg ..)
  struct Lgt { float4 s0, s1; int32_t r0, nvalid; };
  struct Frag { int4_t v[kLoads]; float p[8]; float sc; int32_t r0, nvalid; };
  auto issue_logits = [&](Lgt& lt) {
    int32_t r0 = 0, nv = 0;
    if (tw.more()) tw.next<T>(r0, nv);
    lt.r0 = r0;
    lt.nvalid = nv;
    const float* p = lrow + (nv > 0 ? r0 + 4 * lg : 0);
    lt.s0 = *reinterpret_cast<const float4*>(p);
    lt.s1 = *reinterpret_cast<const float4*>(p + 16);
  };
  auto fill = [&](Frag& f, const Lgt& lt) {
    const int32_t r0 = lt.r0, nv = lt.nvalid;
    f.r0 = r0;
    f.nvalid = nv;
    const float s[8] = {lt.s0.x, lt.s0.y, lt.s0.z, lt.s0.w, lt.s1.x, lt.s1.y, lt.s1.z, lt.s1.w};
    bool keep[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = 16 * (e / 4) + 4 * lg + e % 4;
      const float w = __builtin_amdgcn_exp2f(s[e] - rt.M);
      keep[e] = hv && t < nv && w >= thr;
      f.p[e] = keep[e] ? w : 0.0f;
    }
    clear_flags<T>(fl);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (f.p[e] > 0.0f) fl[16 * (e / 4) + 4 * lg + e % 4] = 1;
    if (krow != nullptr && nv > 0) {
      uint64_t bal[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) bal[e] = __ballot(int(keep[e]));
      if (lg == 0 && hl) {
        uint32_t bits = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            bits |= uint32_t((bal[e] >> (16 * j + lc)) & 1u) << (16 * (e / 4) + 4 * j + e % 4);
        }
        // as two 16-bit halves: a tile of a block that is not a multiple of
        // 32 tokens starts at an odd half, and its second half may belong to
        // the next block's first tile
        uint16_t* kh = reinterpret_cast<uint16_t*>(krow);
        kh[r0 / 16] = uint16_t(bits & 0xFFFFu);
        if (nv > 16) kh[r0 / 16 + 1] = uint16_t(bits >> 16);
      }
    }
    const uint32_t lo = 16u * uint32_t(lane);
    const int bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * RB);
    const auto vr = tile_rsrc(vbase + int64_t(r0) * RB, bytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const bool need = fl[kRpl * i + lane / kCpr] != 0;   // row kRpl i + lane / kCpr
      f.v[i] = tile_load(vr, need ? lo + 1024 * i : kSkipOffset);
    }
    // lanes 0..31: the V scale of token lane, when kept
    const auto sr = tile_rsrc(reinterpret_cast<const uint8_t*>(vsb + r0), max(nv, 0) * 4);
    const bool sneed = lane < 32 && fl[lane % 32] != 0;
    f.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         sr, sneed ? 4u * uint32_t(lane) : kSkipOffset, 0,
                                         kAuxNontemporal));
  };
  constexpr int kExpUnset = -100000;
  int e_run = kExpUnset;
  auto process = [&](auto bufc, Frag& fr, Lgt& lt) {
    constexpr int kBuf = decltype(bufc)::value;
    uint8_t* vt = smem[wave][kBuf];
    float* st = reinterpret_cast<float*>(vt + kTileBytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int rw = kRpl * i + lane / kCpr;
      *reinterpret_cast<int4_t*>(vt + sw(rw, lane % kCpr)) = fr.v[i];
    }
    // V-scale unit 2^e_run >= every kept V scale so far (a power of two: the
    // change of unit of O is exact)
    const float scl = fr.sc;
    const int32_t vbits =
        __builtin_amdgcn_readfirstlane(__float_as_int(wave_max(lane < 32 ? scl : 0.0f)));
    float unit = 1.0f;
    if (vbits > 0) {
      const int32_t ex =
          __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(__int_as_float(vbits)));
      if (e_run == kExpUnset) {
        e_run = ex;
      } else if (ex > e_run) {
        unit = ldexpf(1.0f, e_run - ex);
        e_run = ex;
      }
    }
    const int e_use = e_run == kExpUnset ? 0 : e_run;
    if (lane < 32) st[lane] = ldexpf(scl, kPwShiftSvI8 - e_use);
    float pc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pc[e] = fr.p[e];
    fill(fr, lt);
    issue_logits(lt);
    if (unit != 1.0f) {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) O[n][r] *= unit;
      }
    }
    const float4 vs0 = *reinterpret_cast<const float4*>(st + 4 * lg);
    const float4 vs1 = *reinterpret_cast<const float4*>(st + 16 + 4 * lg);
    const float vs[8] = {vs0.x, vs0.y, vs0.z, vs0.w, vs1.x, vs1.y, vs1.z, vs1.w};
    half8_t phi, plo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pw = pc[e] * vs[e];
      const _Float16 h = (_Float16)pw;
      phi[e] = h;
      plo[e] = (_Float16)(pw - (float)h);
    }
    const int tr_row = 16 * ((lc / 2) / 4) + 4 * lg + (lc / 2) % 4;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int off = sw(tr_row, n) + 8 * (lc & 1);
      const int2_t raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SKV_LDS int2_t*)(vt + off));
      const half8_t bv = widen_codes(raw);
      O[n] = mfma_f16_32(phi, bv, O[n]);
      O[n] = mfma_f16_32(plo, bv, O[n]);
    }
  };
  Lgt la, lb;
  Frag f0, f1;
  const int32_t n_mine = tw.count();
  issue_logits(la);
  issue_logits(lb);
  fill(f0, la);
  issue_logits(la);
  fill(f1, lb);
  issue_logits(lb);
  for (int32_t t = 0; t + 1 < n_mine; t += 2) {
    process(std::integral_constant<int, 0>{}, f0, la);
    process(std::integral_constant<int, 1>{}, f1, lb);
  }
  if (n_mine & 1) process(std::integral_constant<int, 0>{}, f0, la);
  if (e_run != kExpUnset) {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) O[n][r] = ldexpf(O[n][r], e_run - kPwShiftSvI8);
    }
  }
  finish_values<G>(O, rt.M, reinterpret_cast<float*>(&smem[0][0][0]), sv.stat_m, sv.stat_l,
                   sv.ws_m, sv.ws_l, sv.ws_o, int64_t(b) * H + g * G, n_split, split);
}

// ============================================================== group-wise
// q8_0 / q4_0 / q5_0 caches: the group-wise attention kernel's tiles (32
// tokens, codes staged in LDS as one byte per channel, per-(token, group) f16
// scales as float), split into the two passes.  Pass A: q.K per 32-channel
// group on the matrix cores (the codes widened to f16 exactly as A, the
// query as f16 high + low parts as B), each group's dot weighted by its
// scale in float32.  Pass B: the kept rows' V codes, fifth bits and scales
// only, P.V per 16-channel block with the weight times the (token, group) V
// scale in a running power-of-two unit as f16 high + low parts.
template <int G, int K, int D>
__global__ void __launch_bounds__(kMThreads, (GrpFmt<K, D>::kOcc))
sv_logits_grp(const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ksc,
              const float* __restrict__ q, const int32_t* __restrict__ seq_len,
              const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
              int32_t max_sel, int32_t Hkv, int32_t max_seq, int32_t block, int32_t max_len,
              int32_t n_split, int32_t n_rows, int32_t ups, float qscale2, SvArgs sv) {
  using F = GrpFmt<K, D>;
  constexpr bool Q5 = K == kQ5;
  constexpr int KG = F::kGroups;
  constexpr int T = 32;
  constexpr int kCpr = D / 16;                              // LDS chunks per code row
  constexpr int kCodeBytes = T * D;
  constexpr int kBufBytes = kCodeBytes + T * KG * 4;        // codes, K scales [T][KG]
  constexpr int kTileBytes = T * F::kRowBytes;
  constexpr int kLoads = kTileBytes / 1024;
  constexpr int kHcpr = F::kRowBytes / 16;
  constexpr int kHrpl = 1024 / F::kRowBytes;
  constexpr int kSwz = kCpr < 16 ? kCpr : 16;
  constexpr int SPL = KG / 2;
  typedef float floatS __attribute__((ext_vector_type(SPL)));
  const int32_t lstride = sv.lstride;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMWaves][2][kBufBytes];
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t split = int32_t(slot % uint32_t(n_split));
  const uint32_t row = xcd_row(slot / uint32_t(n_split), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const int32_t H = Hkv * G;
  const int64_t bg = int64_t(b) * Hkv + g;
  const int32_t L_raw = seq_len[b];
  const ListSeed ls = list_seed(sel_idx, sel_cnt, max_sel, bg, split, ups);
  const bool hv = lc < G;
  half8_t qhi[KG], qlo[KG];
  {
    const float* qp = q + (int64_t(b) * H + g * G + (hv ? lc : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KG; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(qp + 32 * kk + 8 * lg);
      const float4 c = *reinterpret_cast<const float4*>(qp + 32 * kk + 8 * lg + 4);
      const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = hv ? x[e] * qscale2 : 0.0f;
        const _Float16 h = (_Float16)v;
        qhi[kk][e] = h;
        qlo[kk][e] = (_Float16)(v - (float)h);
      }
    }
  }
  const int32_t L = __builtin_amdgcn_readfirstlane(min(max(L_raw, 0), max_len));
  TileWalk tw = make_walk<T>(ls, sel_idx, max_sel, bg, L, block, split, ups);
  tw.init(wave);
  TileStats ts;
  const uint8_t* kbase = kc + grp_row_off<K, D>(bg, max_seq, 0);
  const uint8_t* khbase = kc + grp_hi_off<K, D>(bg, max_seq, 0);
  const uint8_t* ksb = reinterpret_cast<const uint8_t*>(ksc + bg * int64_t(max_seq) * KG);
  float* lrow = sv.logit + (int64_t(b) * H + g * G + (hv ? lc : 0)) * int64_t(lstride);
  // lane loads as in the group-wise attention kernel: 16-byte chunk
  // lane % kHcpr of row kHrpl i + lane / kHcpr; q5_0 also the fifth bits of
  // those 32 channels; the KG / 2 scales of groups (lane % 2) KG / 2 .. of
  // token lane / 2
  struct Frag {
    int4_t k[kLoads];
    uint32_t kh[kLoads];
    uint2 ks;
    int32_t r0, nvalid;
  };
  auto issue = [&](Frag& f) {
    int32_t r0 = 0, nv = 0;
    if (tw.more()) tw.next<T>(r0, nv);
    f.r0 = r0;
    f.nvalid = nv;
    const uint32_t lo = 16u * uint32_t(lane);
    const int bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * F::kRowBytes);
    const auto kr = tile_rsrc(kbase + int64_t(r0) * F::kRowBytes, bytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) f.k[i] = tile_load(kr, lo + 1024 * i);
    if constexpr (Q5) {
      const int hbytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * F::kHiBytes);
      const auto khr = tile_rsrc(khbase + int64_t(r0) * F::kHiBytes, hbytes);
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
        f.kh[i] = __builtin_amdgcn_raw_buffer_load_b32(khr, 256u * i + 4u * uint32_t(lane), 0,
                                                        kAuxNontemporal);
    }
    const int sbytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * KG * 2);
    const auto ksr = tile_rsrc(ksb + int64_t(r0) * KG * 2, sbytes);
    f.ks = grp_scale_load<KG>(ksr, uint32_t(KG) * uint32_t(lane));
  };
  auto sw = [](int rw, int chunk) { return rw * D + 16 * (chunk ^ (rw & (kSwz - 1))); };
  auto process = [&](auto bufc, Frag& fr) {
    constexpr int kBuf = decltype(bufc)::value;
    uint8_t* kt = smem[wave][kBuf];
    float* stk = reinterpret_cast<float*>(kt + kCodeBytes);          // [T][KG]
    grp_stage<K, D>(kt, fr.k, fr.kh);
    {
      floatS ks4;
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const uint32_t kw = j < 2 ? fr.ks.x : fr.ks.y;
        ks4[j] = (j & 1) ? h2f_hi(kw) : h2f_lo(kw);
      }
      reinterpret_cast<floatS*>(stk)[lane] = ks4;
    }
    const int32_t nvalid = fr.nvalid, r0 = fr.r0;
    issue(fr);
    float sc[8];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float4_t acc[KG];
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
        const int rw = 16 * s + lc;
        const int2_t raw = *reinterpret_cast<const int2_t*>(kt + sw(rw, 2 * kk + lg / 2) +
                                                            8 * (lg & 1));
        const half8_t a = widen_grp<K>(raw);
        acc[kk] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        acc[kk] = mfma_f16_32(a, qhi[kk], acc[kk]);
        acc[kk] = mfma_f16_32(a, qlo[kk], acc[kk]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float* kr = stk + (16 * s + 4 * lg + r) * KG;
        float a = acc[0][r] * kr[0];
#pragma unroll
        for (int kk = 1; kk < KG; ++kk) a += acc[kk][r] * kr[kk];
        sc[4 * s + r] = a;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sc[e] = 16 * (e / 4) + 4 * lg + e % 4 < nvalid ? sc[e] : -INFINITY;
    ts.add<2>(sc, nvalid);
    if (hv && nvalid > 0) {
      if (nvalid == T) {
        *reinterpret_cast<float4*>(lrow + r0 + 4 * lg) = make_float4(sc[0], sc[1], sc[2], sc[3]);
        *reinterpret_cast<float4*>(lrow + r0 + 16 + 4 * lg) =
            make_float4(sc[4], sc[5], sc[6], sc[7]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 16 * (e / 4) + 4 * lg + e % 4;
          if (t < nvalid) lrow[r0 + t] = sc[e];
        }
      }
    }
  };
  Frag f0, f1;
  const int32_t n_mine = tw.count();
  issue(f0);
  issue(f1);
  for (int32_t t = 0; t + 1 < n_mine; t += 2) {
    process(std::integral_constant<int, 0>{}, f0);
    process(std::integral_constant<int, 1>{}, f1);
  }
  if (n_mine & 1) process(std::integral_constant<int, 0>{}, f0);
  finish_stats<G>(ts, reinterpret_cast<float*>(&smem[0][0][0]), sv.stat_m, sv.stat_l, sv.stat_n,
                  int64_t(b) * H + g * G, bg, n_split, split);
}

constexpr int kPwShiftSvGrp = 14;

template <int G, int K, int D>
__global__ void __launch_bounds__(kMThreads, (GrpFmt<K, D>::kOcc))
sv_values_grp(const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vsc,
              const int32_t* __restrict__ seq_len, const int32_t* __restrict__ sel_idx,
              const int32_t* __restrict__ sel_cnt, int32_t max_sel, int32_t Hkv,
              int32_t max_seq, int32_t block, int32_t max_len, int32_t n_split, int32_t n_rows,
              int32_t ups, int32_t keep_words, SvArgs sv) {
  using F = GrpFmt<K, D>;
  constexpr bool Q5 = K == kQ5;
  constexpr int KG = F::kGroups;
  constexpr int T = 32;
  constexpr int kCpr = D / 16;
  constexpr int kCodeBytes = T * D;
  constexpr int kBufBytes = kCodeBytes + T * KG * 4;        // codes, V scales [T][KG]
  constexpr int kTileBytes = T * F::kRowBytes;
  constexpr int kLoads = kTileBytes / 1024;
  constexpr int kHcpr = F::kRowBytes / 16;
  constexpr int kHrpl = 1024 / F::kRowBytes;
  constexpr int kSwz = kCpr < 16 ? kCpr : 16;
  constexpr int SPL = KG / 2;
  typedef float floatS __attribute__((ext_vector_type(SPL)));
  const int32_t lstride = sv.lstride;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMWaves][2][kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t flags[kMWaves][T];
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t split = int32_t(slot % uint32_t(n_split));
  const uint32_t row = xcd_row(slot / uint32_t(n_split), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const int32_t H = Hkv * G;
  const int64_t bg = int64_t(b) * Hkv + g;
  const int32_t L_raw = seq_len[b];
  const ListSeed ls = list_seed(sel_idx, sel_cnt, max_sel, bg, split, ups);
  const bool hl = lc < G;
  const int64_t hrow = int64_t(b) * H + g * G + (hl ? lc : 0);
  const RowTotals rt = row_totals<G>(sv.stat_m, sv.stat_l, sv.stat_n, int64_t(b) * H + g * G,
                                     bg, n_split, lc);
  const float theta = sv.eps > 0.0f ? sv.eps / float(max(rt.n, 1)) : sv.tau;
  const float thr = theta * rt.L;
  const bool hv = hl && rt.M != -INFINITY;
  const int32_t L = __builtin_amdgcn_readfirstlane(min(max(L_raw, 0), max_len));
  TileWalk tw = make_walk<T>(ls, sel_idx, max_sel, bg, L, block, split, ups);
  tw.init(wave);
  float4_t O[2 * KG];
#pragma unroll
  for (int n = 0; n < 2 * KG; ++n) O[n] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const uint8_t* vbase = vc + grp_row_off<K, D>(bg, max_seq, 0);
  const uint8_t* vhbase = vc + grp_hi_off<K, D>(bg, max_seq, 0);
  const uint8_t* vsb = reinterpret_cast<const uint8_t*>(vsc + bg * int64_t(max_seq) * KG);
  const float* lrow = sv.logit + hrow * int64_t(lstride);
  uint32_t* krow = sv.keep != nullptr ? sv.keep + hrow * int64_t(keep_words) : nullptr;
  uint8_t* fl = flags[wave];
  auto sw = [](int rw, int chunk) { return rw * D + 16 * (chunk ^ (rw & (kSwz - 1))); };
  // logits of tokens tok(lg, 0..7): two float4 (tokens 4 lg .. and 16 + 4 lg ..)
  struct Lgt { float4 s0, s1; int32_t r0, nvalid; };
  struct Frag {
    int4_t v[kLoads];
    uint32_t vh[kLoads];
    uint2 vs;
    float p[8];
    int32_t r0, nvalid;
  };
  auto issue_logits = [&](Lgt& lt) {
    int32_t r0 = 0, nv = 0;
    if (tw.more()) tw.next<T>(r0, nv);
    lt.r0 = r0;
    lt.nvalid = nv;
    const float* p = lrow + (nv > 0 ? r0 + 4 * lg : 0);
    lt.s0 = *reinterpret_cast<const float4*>(p);
    lt.s1 = *reinterpret_cast<const float4*>(p + 16);
  };
  auto fill = [&](Frag& f, const Lgt& lt) {
    const int32_t r0 = lt.r0, nv = lt.nvalid;
    f.r0 = r0;
    f.nvalid = nv;
    const float s[8] = {lt.s0.x, lt.s0.y, lt.s0.z, lt.s0.w, lt.s1.x, lt.s1.y, lt.s1.z, lt.s1.w};
    bool keep[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = 16 * (e / 4) + 4 * lg + e % 4;
      const float w = __builtin_amdgcn_exp2f(s[e] - rt.M);
      keep[e] = hv && t < nv && w >= thr;
      f.p[e] = keep[e] ? w : 0.0f;
    }
    clear_flags<T>(fl);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (f.p[e] > 0.0f) fl[16 * (e / 4) + 4 * lg + e % 4] = 1;
    if (krow != nullptr && nv > 0) {
      uint64_t bal[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) bal[e] = __ballot(int(keep[e]));
      if (lg == 0 && hl) {
        uint32_t bits = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            bits |= uint32_t((bal[e] >> (16 * j + lc)) & 1u) << (16 * (e / 4) + 4 * j + e % 4);
        }
        // as two 16-bit halves (a tile may start at an odd half of a word)
        uint16_t* kh = reinterpret_cast<uint16_t*>(krow);
        kh[r0 / 16] = uint16_t(bits & 0xFFFFu);
        if (nv > 16) kh[r0 / 16 + 1] = uint16_t(bits >> 16);
      }
    }
    // the kept rows' codes (and fifth bits), and their scales: rows no head
    // keeps are requested past their resource's records (zeros, no read)
    const uint32_t lo = 16u * uint32_t(lane);
    const int bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * F::kRowBytes);
    const auto vr = tile_rsrc(vbase + int64_t(r0) * F::kRowBytes, bytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const bool need = fl[kHrpl * i + lane / kHcpr] != 0;   // row kHrpl i + lane / kHcpr
      f.v[i] = tile_load(vr, need ? lo + 1024 * i : kSkipOffset);
    }
    if constexpr (Q5) {
      const int hbytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * F::kHiBytes);
      const auto vhr = tile_rsrc(vhbase + int64_t(r0) * F::kHiBytes, hbytes);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const bool need = fl[kHrpl * i + lane / kHcpr] != 0;
        f.vh[i] = __builtin_amdgcn_raw_buffer_load_b32(
            vhr, need ? 256u * i + 4u * uint32_t(lane) : kSkipOffset, 0, kAuxNontemporal);
      }
    }
    const int sbytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * KG * 2);
    const auto vsr = tile_rsrc(vsb + int64_t(r0) * KG * 2, sbytes);
    f.vs = grp_scale_load<KG>(vsr, fl[lane / 2] != 0 ? uint32_t(KG) * uint32_t(lane)
                                                     : kSkipOffset);
  };
  constexpr int kExpUnset = -100000;
  int e_run = kExpUnset;
  auto process = [&](auto bufc, Frag& fr, Lgt& lt) {
    constexpr int kBuf = decltype(bufc)::value;
    uint8_t* vt = smem[wave][kBuf];
    float* stv = reinterpret_cast<float*>(vt + kCodeBytes);          // [T][KG]
    grp_stage<K, D>(vt, fr.v, fr.vh);
    // V-scale unit 2^e_run >= every kept V scale so far (a power of two: the
    // change of unit of O is exact)
    float vv[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const uint32_t vw = j < 2 ? fr.vs.x : fr.vs.y;
      vv[j] = (j & 1) ? h2f_hi(vw) : h2f_lo(vw);
    }
    float vmx = vv[0];
#pragma unroll
    for (int j = 1; j < SPL; ++j) vmx = fmaxf(vmx, vv[j]);
    const int32_t vbits = __builtin_amdgcn_readfirstlane(__float_as_int(wave_max(vmx)));
    float unit = 1.0f;
    if (vbits > 0 && vbits < 0x7F800000) {
      const int32_t ex =
          __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(__int_as_float(vbits)));
      if (e_run == kExpUnset) {
        e_run = ex;
      } else if (ex > e_run) {
        unit = ldexpf(1.0f, e_run - ex);
        e_run = ex;
      }
    }
    const int e_use = e_run == kExpUnset ? 0 : e_run;
    {
      floatS vs4;
#pragma unroll
      for (int j = 0; j < SPL; ++j) vs4[j] = ldexpf(vv[j], kPwShiftSvGrp - e_use);
      reinterpret_cast<floatS*>(stv)[lane] = vs4;
    }
    float pc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pc[e] = fr.p[e];
    fill(fr, lt);
    issue_logits(lt);
    if (unit != 1.0f) {
#pragma unroll
      for (int n = 0; n < 2 * KG; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) O[n][r] *= unit;
      }
    }
    const int tr_row = 16 * ((lc / 2) / 4) + 4 * lg + (lc / 2) % 4;
#pragma unroll
    for (int grp = 0; grp < KG; ++grp) {
      half8_t phi, plo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pw = pc[e] * stv[(16 * (e / 4) + 4 * lg + e % 4) * KG + grp];
        const _Float16 h = (_Float16)pw;
        phi[e] = h;
        plo[e] = (_Float16)(pw - (float)h);
      }
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const int n = 2 * grp + nn;
        const int off = sw(tr_row, n) + 8 * (lc & 1);
        const int2_t raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SKV_LDS int2_t*)(vt + off));
        const half8_t bv = widen_grp<K>(raw);
        O[n] = mfma_f16_32(phi, bv, O[n]);
        O[n] = mfma_f16_32(plo, bv, O[n]);
      }
    }
  };
  Lgt la, lb;
  Frag f0, f1;
  const int32_t n_mine = tw.count();
  issue_logits(la);
  issue_logits(lb);
  fill(f0, la);
  issue_logits(la);
  fill(f1, lb);
  issue_logits(lb);
  for (int32_t t = 0; t + 1 < n_mine; t += 2) {
    process(std::integral_constant<int, 0>{}, f0, la);
    process(std::integral_constant<int, 1>{}, f1, lb);
  }
  if (n_mine & 1) process(std::integral_constant<int, 0>{}, f0, la);
  if (e_run != kExpUnset) {
#pragma unroll
    for (int n = 0; n < 2 * KG; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) O[n][r] = ldexpf(O[n][r], e_run - kPwShiftSvGrp);
    }
  }
  finish_values<G>(O, rt.M, reinterpret_cast<float*>(&smem[0][0][0]), sv.stat_m, sv.stat_l,
                   sv.ws_m, sv.ws_l, sv.ws_o, int64_t(b) * H + g * G, n_split, split);
}

}  // namespace

namespace {

template <int D>
hipError_t launch_sparse_v_d(const SparseVParams& p, int G, const dim3 grid, int32_t n_rows,
                             int32_t ups, float scale2, const SvArgs& sv, int32_t keep_words,
                             hipStream_t stream) {
  const skv_cache& c = *p.c;
  const int32_t S = p.n_split, Hkv = c.n_kv_heads;
  if (c.kv_dtype == SKV_F16) {
    const uint16_t* kc = static_cast<const uint16_t*>(c.k);
    const uint16_t* vc = static_cast<const uint16_t*>(c.v);
#define SKV_SV_F16(GG)                                                                          \
  sv_logits_f16<D, GG><<<grid, kMThreads, 0, stream>>>(kc, p.q, p.seq_len, p.sel_idx,          \
                                                        p.sel_cnt, p.max_sel, Hkv, c.max_seq,   \
                                                        c.block, p.max_len, S, n_rows, ups,     \
                                                        scale2, sv);                            \
  sv_values_f16<D, GG><<<grid, kMThreads, 0, stream>>>(vc, p.seq_len, p.sel_idx, p.sel_cnt,    \
                                                        p.max_sel, Hkv, c.max_seq, c.block,     \
                                                        p.max_len, S, n_rows, ups, keep_words,  \
                                                        sv)
    switch (G) {
      case 1: SKV_SV_F16(1); break;
      case 2: SKV_SV_F16(2); break;
      case 4: SKV_SV_F16(4); break;
      default: SKV_SV_F16(8); break;
    }
#undef SKV_SV_F16
    return hipGetLastError();
  }
  if (is_grouped(c.kv_dtype)) {
    const uint8_t* kc = static_cast<const uint8_t*>(c.k);
    const uint8_t* vc = static_cast<const uint8_t*>(c.v);
    const uint16_t* ksc = reinterpret_cast<const uint16_t*>(c.k_scale);
    const uint16_t* vsc = reinterpret_cast<const uint16_t*>(c.v_scale);
#define SKV_SV_GRP(GG, Q)                                                                       \
  sv_logits_grp<GG, Q, D><<<grid, kMThreads, 0, stream>>>(kc, ksc, p.q, p.seq_len, p.sel_idx,  \
                                                           p.sel_cnt, p.max_sel, Hkv,           \
                                                           c.max_seq, c.block, p.max_len, S,    \
                                                           n_rows, ups, scale2, sv);            \
  sv_values_grp<GG, Q, D><<<grid, kMThreads, 0, stream>>>(vc, vsc, p.seq_len, p.sel_idx,       \
                                                           p.sel_cnt, p.max_sel, Hkv,           \
                                                           c.max_seq, c.block, p.max_len, S,    \
                                                           n_rows, ups, keep_words, sv)
#define SKV_SV_GRP_G(GG)                                          \
  if (c.kv_dtype == SKV_Q4_0) { SKV_SV_GRP(GG, kQ4); }             \
  else if (c.kv_dtype == SKV_Q5_0) { SKV_SV_GRP(GG, kQ5); }        \
  else { SKV_SV_GRP(GG, kQ8); }
    switch (G) {
      case 1: SKV_SV_GRP_G(1); break;
      case 2: SKV_SV_GRP_G(2); break;
      case 4: SKV_SV_GRP_G(4); break;
      default: SKV_SV_GRP_G(8); break;
    }
#undef SKV_SV_GRP_G
#undef SKV_SV_GRP
    return hipGetLastError();
  }
  if (c.kv_dtype != SKV_I8) return hipErrorInvalidValue;
  const int8_t* kc = static_cast<const int8_t*>(c.k);
  const int8_t* vc = static_cast<const int8_t*>(c.v);
#define SKV_SV_I8(GG)                                                                           \
  sv_logits_i8<D, GG><<<grid, kMThreads, 0, stream>>>(kc, c.k_scale, p.q, p.seq_len,           \
                                                       p.sel_idx, p.sel_cnt, p.max_sel, Hkv,    \
                                                       c.max_seq, c.block, p.max_len, S,        \
                                                       n_rows, ups, scale2, sv);                \
  sv_values_i8<D, GG><<<grid, kMThreads, 0, stream>>>(vc, c.v_scale, p.seq_len, p.sel_idx,     \
                                                       p.sel_cnt, p.max_sel, Hkv, c.max_seq,    \
                                                       c.block, p.max_len, S, n_rows, ups,      \
                                                       keep_words, sv)
  switch (G) {
    case 1: SKV_SV_I8(1); break;
    case 2: SKV_SV_I8(2); break;
    case 4: SKV_SV_I8(4); break;
    default: SKV_SV_I8(8); break;
  }
#undef SKV_SV_I8
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_v(const SparseVParams& p, hipStream_t stream) {
  const skv_cache& c = *p.c;
  const int32_t B = c.batch, H = p.n_heads, S = p.n_split, Hkv = c.n_kv_heads;
  const int32_t D = c.head_dim;
  const int G = H / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return hipErrorInvalidValue;
  int32_t ups;
  if (p.sel_idx != nullptr) {
    ups = (p.max_sel + S - 1) / S;
  } else {
    const int32_t nb_max = (p.max_len + c.block - 1) / c.block;
    ups = (nb_max + S - 1) / S;
  }
  ups = ups < 1 ? 1 : ups;
  const int64_t n_wg = int64_t(S) * Hkv * B;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(n_wg));
  const int32_t n_rows = Hkv * B;
  const float scale2 = p.softmax_scale * kLog2e;
  float* ws = p.ws;
  const size_t bhs = size_t(B) * H * S;
  SvArgs sv;
  sv.ws_m = ws;
  sv.ws_l = ws + bhs;
  sv.ws_o = ws + 2 * bhs;
  sv.stat_m = ws + bhs * (2 + size_t(D));
  sv.stat_l = sv.stat_m + bhs;
  sv.stat_n = reinterpret_cast<int32_t*>(sv.stat_l + bhs);
  sv.logit = reinterpret_cast<float*>(sv.stat_n + size_t(B) * Hkv * S);
  sv.lstride = (p.max_len + 31) / 32 * 32;
  sv.keep = p.keep;
  sv.tau = p.tau;
  sv.eps = p.eps;
  const int32_t keep_words = (p.max_len + 31) / 32;
  switch (D) {
    case 64: return launch_sparse_v_d<64>(p, G, grid, n_rows, ups, scale2, sv, keep_words, stream);
    case 128:
      return launch_sparse_v_d<128>(p, G, grid, n_rows, ups, scale2, sv, keep_words, stream);
    case 256:
      return launch_sparse_v_d<256>(p, G, grid, n_rows, ups, scale2, sv, keep_words, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace skv
