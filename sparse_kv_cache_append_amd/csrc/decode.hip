// decode_attn: split-K partial attention of one query token per sequence.
//
// Grid (n_split, Hkv, B); one workgroup of 4 wavefronts per (sequence, KV
// head, part).  A part is a run of `block`-token cache blocks: consecutive
// blocks for dense decode, consecutive entries of the selected-block list for
// Quest decode (sparse_attn.md, "Method", kernel skip: unselected blocks are
// never read).
//
// Streaming: LPR lanes share one cache row (LPR = 8 for G <= 2, 16 for
// G >= 4, which halves the per-lane query and accumulator registers), so one
// wavefront instruction reads 64/LPR full rows.  A workgroup step covers
// 4 * 64 / LPR rows.  Each lane keeps its slice of K and V in registers and
// applies it to all G query heads of the group, so every K/V byte crosses
// HBM once for the whole GQA group.  Loads run P steps ahead of the
// arithmetic through a register ring.  Rows past the end of the part are
// loaded from a clamped in-range row and masked out of the softmax, so the
// loads carry no branches.
//
// Arithmetic per row and head: a partial dot over the lane's channels, an
// LPR-lane DPP sum (identical bits in every lane of the group), then an online
// softmax in base 2 (the query is pre-scaled by softmax_scale * log2 e) whose
// running max/mass/numerator live per lane group; the numerator is rescaled
// only when the running max grows.  int8 rows use exact int32 dot4 products
// of the quantized query and key codes (cpu-attn kernel card, "Method") and
// fold the per-token scales into the logit and the weight.
//
// Epilogue: the lane-group states of the workgroup are merged (shuffles inside
// a wavefront, LDS across wavefronts) into one partial state per query head,
// written to the workspace for skv_combine.
#include "device_common.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kD = 128;  // head_dim built in this version

template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  return LPR == 8 ? group8_sum(x) : group16_sum(x);
}
template <int LPR>
__device__ __forceinline__ int group_sum_i(int x) {
  x = group8_sum_i(x);
  if (LPR == 16) x += dpp_i<kDppRowMirror>(x);
  return x;
}

// The blocks of one part, walked in 32- or 16-row steps by an incremental
// cursor (no division per step).  For Quest decode the part's selected block
// indices are loaded once, one per lane, and read back with readlane, so a
// step's address never waits on a memory load.
struct Part {
  const int32_t* sel;  // row of sel_idx for (b, g); nullptr = dense
  int32_t u0, n_units, spb, block, L, nb, rows_per_step;
  int32_t jl;          // lane k: selected block of unit k (k < 64), sparse only

  __device__ __forceinline__ int32_t n_steps() const { return n_units * spb; }
};

struct Cursor {
  int32_t unit = 0, sub = 0;
  // First row and number of valid rows of the cursor's step; then advance.
  __device__ __forceinline__ void next(const Part& pt, int32_t& r0, int32_t& nvalid) {
    int32_t j = pt.u0 + unit;
    if (pt.sel != nullptr)
      j = unit < kWave ? __builtin_amdgcn_readlane(pt.jl, unit) : pt.sel[j];
    if (j < 0 || j >= pt.nb) {
      r0 = 0;
      nvalid = 0;
    } else {
      r0 = j * pt.block + sub * pt.rows_per_step;
      nvalid = min(min(pt.rows_per_step, pt.block - sub * pt.rows_per_step), pt.L - r0);
    }
    if (++sub == pt.spb) { sub = 0; ++unit; }
  }
};

__device__ __forceinline__ Part make_part(const int32_t* sel_idx, const int32_t* sel_cnt,
                                          int32_t max_sel, int64_t bg, int32_t L, int32_t block,
                                          int32_t split, int32_t units_per_split,
                                          int32_t rows_per_step) {
  Part pt;
  pt.block = block;
  pt.L = L;
  pt.nb = (L + block - 1) / block;
  pt.rows_per_step = rows_per_step;
  pt.spb = (block + rows_per_step - 1) / rows_per_step;
  int32_t total = pt.nb;
  pt.sel = nullptr;
  pt.jl = -1;
  if (sel_idx != nullptr) {
    pt.sel = sel_idx + bg * max_sel;
    total = min(max(sel_cnt[bg], 0), max_sel);
  }
  pt.u0 = split * units_per_split;
  pt.n_units = max(0, min(units_per_split, total - pt.u0));
  if (pt.sel != nullptr) {
    const int lane = threadIdx.x % kWave;
    if (lane < pt.n_units) pt.jl = pt.sel[pt.u0 + lane];
  }
  return pt;
}

// Merge the lane-group softmax states of the workgroup and write the part's
// partial state.  Lanes LPR apart hold the same channels.
template <int G, int LPR, int EPL, typename DMap>
__device__ __forceinline__ void finish_part(float (&m)[G], float (&l)[G], float (&o)[G][EPL],
                                            DMap dmap, float* lds, float* __restrict__ ws_m,
                                            float* __restrict__ ws_l, float* __restrict__ ws_o,
                                            int64_t head0, int32_t n_split, int32_t split) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m2 = __shfl_xor(m[h], off);
      const float l2 = __shfl_xor(l[h], off);
      const float M = fmaxf(m[h], m2);
      const float a1 = (m[h] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m[h] - M);
      const float a2 = (m2 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m2 - M);
      l[h] = l[h] * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float o2 = __shfl_xor(o[h][e], off);
        o[h][e] = o[h][e] * a1 + o2 * a2;
      }
      m[h] = M;
    }
  }
  float* lo = lds;                          // [waves][G][D]
  float* lm = lds + kDecWaves * G * kD;     // [waves][G]
  float* ll = lm + kDecWaves * G;           // [waves][G]
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) lo[(wave * G + h) * kD + dmap(lane, e)] = o[h][e];
      if (lane == 0) { lm[wave * G + h] = m[h]; ll[wave * G + h] = l[h]; }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kD; idx += kDecThreads) {
    const int h = idx / kD, d = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, lm[w * G + h]);
    float so = 0.0f, sl = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = lm[w * G + h];
        const float a = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        so += a * lo[(w * G + h) * kD + d];
        sl += a * ll[w * G + h];
      }
    }
    const int64_t ps = (head0 + h) * n_split + split;
    ws_o[ps * kD + d] = so;
    if (d == 0) { ws_m[ps] = M; ws_l[ps] = sl; }
  }
}

// Online softmax of one row for all G heads (logits s[h] in base 2).  The
// reference max m[h] is raised only when a logit exceeds it by more than
// kLazy (weights stay <= 2^kLazy, far from float32 overflow), and the rescale
// sits behind a wavefront-uniform branch, so it runs only in the rare steps
// where some lane needs it.  The final o / l is unchanged by the choice of
// reference.
constexpr float kLazy = 8.0f;

template <int G, int EPL, bool SCALED, typename VGet>
__device__ __forceinline__ void softmax_rows(const float (&s)[G], bool valid, float wscale,
                                             float (&m)[G], float (&l)[G], float (&o)[G][EPL],
                                             VGet vget) {
  bool need = false;
#pragma unroll
  for (int h = 0; h < G; ++h) need |= valid && (s[h] > m[h] + kLazy);
  if (__ballot(need)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bool r = valid && (s[h] > m[h] + kLazy);
      const float cr = r ? __builtin_amdgcn_exp2f(m[h] - s[h]) : 1.0f;
      m[h] = r ? s[h] : m[h];
      l[h] *= cr;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= cr;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float p = valid ? __builtin_amdgcn_exp2f(s[h] - m[h]) : 0.0f;
    l[h] += p;
    if (SCALED) p *= wscale;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(p, vget(e), o[h][e]);
  }
}

// ------------------------------------------------------------------ f16
template <int G, int LPR, int P>
__global__ void __launch_bounds__(kDecThreads, 2)
decode_f16_kernel(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                  const float* __restrict__ q, const int32_t* __restrict__ seq_len,
                  const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
                  int32_t max_sel, int32_t Hkv, int32_t max_seq, int32_t block, int32_t max_len,
                  int32_t n_split, int32_t units_per_split, float qscale2,
                  float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o) {
  constexpr int EPL = kD / LPR;        // channels per lane
  constexpr int NW = EPL / 2;          // 32-bit words per lane per row (K or V)
  constexpr int NV = NW / 4;           // 16-byte loads per lane per row (K or V)
  constexpr int RPW = kWave / LPR;     // rows per wavefront per step
  __shared__ float lds[kDecWaves * G * kD + 2 * kDecWaves * G];
  const int32_t split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int c = lane % LPR, rsub = wave * RPW + lane / LPR;
  const int32_t H = Hkv * G;
  const int32_t L = min(max(seq_len[b], 0), max_len);
  const int64_t bg = int64_t(b) * Hkv + g;
  const Part pt = make_part(sel_idx, sel_cnt, max_sel, bg, L, block, split, units_per_split,
                            kDecWaves * RPW);
  const int32_t n_steps = pt.n_steps();
  // lane channel map: 16-byte chunk v of a row holds channels 8*(c + LPR*v) .. +7
  auto dmap = [](int cc, int e) { return 8 * (cc + LPR * (e / 8)) + (e % 8); };

  float qv[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qp = q + (int64_t(b) * H + g * G + h) * kD;
#pragma unroll
    for (int k = 0; k < EPL / 8; ++k) {
      const float4* q4 = reinterpret_cast<const float4*>(qp + dmap(c, 8 * k));
      const float4 a = q4[0], bq = q4[1];
      qv[h][8 * k + 0] = a.x * qscale2; qv[h][8 * k + 1] = a.y * qscale2;
      qv[h][8 * k + 2] = a.z * qscale2; qv[h][8 * k + 3] = a.w * qscale2;
      qv[h][8 * k + 4] = bq.x * qscale2; qv[h][8 * k + 5] = bq.y * qscale2;
      qv[h][8 * k + 6] = bq.z * qscale2; qv[h][8 * k + 7] = bq.w * qscale2;
    }
  }
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY; l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
  }

  const uint4* kbase = reinterpret_cast<const uint4*>(kc + bg * max_seq * kD);
  const uint4* vbase = reinterpret_cast<const uint4*>(vc + bg * max_seq * kD);
  const int32_t last = max(L - 1, 0);
  struct Frag { uint32_t k[NW], v[NW]; };
  Cursor cur;
  auto issue = [&](Frag& f, int32_t& nvalid) {
    int32_t r0;
    cur.next(pt, r0, nvalid);
    const int32_t row = min(r0 + rsub, last);
    const uint4* kp = kbase + int64_t(row) * (kD / 8);
    const uint4* vp = vbase + int64_t(row) * (kD / 8);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint4 a = kp[c + LPR * v], bb = vp[c + LPR * v];
      f.k[4 * v] = a.x; f.k[4 * v + 1] = a.y; f.k[4 * v + 2] = a.z; f.k[4 * v + 3] = a.w;
      f.v[4 * v] = bb.x; f.v[4 * v + 1] = bb.y; f.v[4 * v + 2] = bb.z; f.v[4 * v + 3] = bb.w;
    }
  };

  Frag ring[P];
  int32_t rnv[P];
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < n_steps) issue(ring[p], rnv[p]);

  for (int32_t base = 0; base < n_steps; base += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int32_t i = base + p;
      if (i < n_steps) {
        const bool valid = rsub < rnv[p];
        const Frag& f = ring[p];
        auto kget = [&](int e) { return (e & 1) ? h2f_hi(f.k[e >> 1]) : h2f_lo(f.k[e >> 1]); };
        auto vget = [&](int e) { return (e & 1) ? h2f_hi(f.v[e >> 1]) : h2f_lo(f.v[e >> 1]); };
        float sc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float acc = 0.0f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc = fmaf(qv[h][e], kget(e), acc);
          sc[h] = group_sum<LPR>(acc);
        }
        softmax_rows<G, EPL, false>(sc, valid, 1.0f, m, l, o, vget);
        if (i + P < n_steps) issue(ring[p], rnv[p]);
      }
    }
  }
  finish_part<G, LPR, EPL>(m, l, o, dmap, lds, ws_m, ws_l, ws_o, int64_t(b) * H + g * G,
                           n_split, split);
}

// ------------------------------------------------------------------ int8
template <int G, int LPR, int P>
__global__ void __launch_bounds__(kDecThreads, 2)
decode_i8_kernel(const int8_t* __restrict__ kc, const int8_t* __restrict__ vc,
                 const float* __restrict__ ksc, const float* __restrict__ vsc,
                 const float* __restrict__ q, const int32_t* __restrict__ seq_len,
                 const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
                 int32_t max_sel, int32_t Hkv, int32_t max_seq, int32_t block, int32_t max_len,
                 int32_t n_split, int32_t units_per_split, float scale2,
                 float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
                 int32_t* __restrict__ dbg) {
  constexpr int EPL = kD / LPR;        // channels (bytes) per lane
  constexpr int NW = EPL / 4;          // 32-bit words per lane per row
  constexpr int RPW = kWave / LPR;
  __shared__ float lds[kDecWaves * G * kD + 2 * kDecWaves * G];
  const int32_t split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int c = lane % LPR, rsub = wave * RPW + lane / LPR;
  const int32_t H = Hkv * G;
  const int32_t L = min(max(seq_len[b], 0), max_len);
  const int64_t bg = int64_t(b) * Hkv + g;
  const Part pt = make_part(sel_idx, sel_cnt, max_sel, bg, L, block, split, units_per_split,
                            kDecWaves * RPW);
  const int32_t n_steps = pt.n_steps();
  auto dmap = [](int cc, int e) { return EPL * cc + e; };

  // Quantize the G query heads with the cache's absmax rule (one scale per
  // head); every wavefront computes the codes of its lanes' channels.
  int32_t qc[G][NW];
  float coef[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qp = q + (int64_t(b) * H + g * G + h) * kD;
    const float2 two = reinterpret_cast<const float2*>(qp)[lane];
    const float a = wave_max(fmaxf(fabsf(two.x), fabsf(two.y)));
    const float qs = absmax_scale(a);
    const float4* q4 = reinterpret_cast<const float4*>(qp + dmap(c, 0));
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float4 x = q4[w];
      const uint32_t packed = (uint32_t(quant_code(x.x, qs)) & 0xFFu) |
                              ((uint32_t(quant_code(x.y, qs)) & 0xFFu) << 8) |
                              ((uint32_t(quant_code(x.z, qs)) & 0xFFu) << 16) |
                              ((uint32_t(quant_code(x.w, qs)) & 0xFFu) << 24);
      qc[h][w] = int32_t(packed);
    }
    coef[h] = qs * scale2;
  }
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY; l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
  }

  const int8_t* kbase = kc + bg * max_seq * kD;
  const int8_t* vbase = vc + bg * max_seq * kD;
  const float* ksb = ksc + bg * max_seq;
  const float* vsb = vsc + bg * max_seq;
  const int32_t last = max(L - 1, 0);
  struct Frag { uint32_t k[NW], v[NW]; float ks, vs; int32_t row; };
  Cursor cur;
  auto issue = [&](Frag& f, int32_t& nvalid) {
    int32_t r0;
    cur.next(pt, r0, nvalid);
    const int32_t row = min(r0 + rsub, last);
    f.row = r0 + rsub;
    const int8_t* kp = kbase + int64_t(row) * kD + EPL * c;
    const int8_t* vp = vbase + int64_t(row) * kD + EPL * c;
    if constexpr (NW == 4) {
      const uint4 a = *reinterpret_cast<const uint4*>(kp), bb = *reinterpret_cast<const uint4*>(vp);
      f.k[0] = a.x; f.k[1] = a.y; f.k[2] = a.z; f.k[3] = a.w;
      f.v[0] = bb.x; f.v[1] = bb.y; f.v[2] = bb.z; f.v[3] = bb.w;
    } else {
      const uint2 a = *reinterpret_cast<const uint2*>(kp), bb = *reinterpret_cast<const uint2*>(vp);
      f.k[0] = a.x; f.k[1] = a.y;
      f.v[0] = bb.x; f.v[1] = bb.y;
    }
    f.ks = ksb[row];
    f.vs = vsb[row];
  };

  Frag ring[P];
  int32_t rnv[P];
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < n_steps) issue(ring[p], rnv[p]);

  for (int32_t base = 0; base < n_steps; base += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int32_t i = base + p;
      if (i < n_steps) {
        const Frag& f = ring[p];
        const bool valid = rsub < rnv[p];
        auto vget = [&](int e) { return float(int8_t((f.v[e >> 2] >> (8 * (e & 3))) & 0xFFu)); };
        float sc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          int32_t dot = 0;
#pragma unroll
          for (int w = 0; w < NW; ++w)
            dot = __builtin_amdgcn_sdot4(qc[h][w], int32_t(f.k[w]), dot, false);
          dot = group_sum_i<LPR>(dot);
          if (dbg != nullptr && valid && c == 0)
            dbg[(int64_t(b) * H + g * G + h) * max_len + f.row] = dot;
          sc[h] = float(dot) * coef[h] * f.ks;
        }
        softmax_rows<G, EPL, true>(sc, valid, f.vs, m, l, o, vget);
        if (i + P < n_steps) issue(ring[p], rnv[p]);
      }
    }
  }
  finish_part<G, LPR, EPL>(m, l, o, dmap, lds, ws_m, ws_l, ws_o, int64_t(b) * H + g * G,
                           n_split, split);
}

template <int G>
void launch_decode_g(const DecodeParams& p, hipStream_t stream) {
  const skv_cache& c = *p.c;
  const int32_t B = c.batch, H = p.n_heads, S = p.n_split;
  float* ws_m = p.ws + ws_m_offset(B, H, S);
  float* ws_l = p.ws + ws_l_offset(B, H, S);
  float* ws_o = p.ws + ws_o_offset(B, H, S);
  int32_t ups;
  if (p.sel_idx != nullptr) {
    ups = (p.max_sel + S - 1) / S;
  } else {
    const int32_t nb_max = (p.max_len + c.block - 1) / c.block;
    ups = (nb_max + S - 1) / S;
  }
  dim3 grid(S, c.n_kv_heads, B);
  const float scale2 = p.softmax_scale * kLog2e;
  constexpr int LPR = G <= 2 ? 8 : 16;
  if (c.kv_dtype == SKV_F16) {
    constexpr int P = LPR == 8 ? 4 : 5;
    decode_f16_kernel<G, LPR, P><<<grid, kDecThreads, 0, stream>>>(
        static_cast<const uint16_t*>(c.k), static_cast<const uint16_t*>(c.v), p.q, p.seq_len,
        p.sel_idx, p.sel_cnt, p.max_sel, c.n_kv_heads, c.max_seq, c.block, p.max_len, S, ups,
        scale2, ws_m, ws_l, ws_o);
  } else {
    constexpr int P = LPR == 8 ? 6 : 8;
    decode_i8_kernel<G, LPR, P><<<grid, kDecThreads, 0, stream>>>(
        static_cast<const int8_t*>(c.k), static_cast<const int8_t*>(c.v), c.k_scale, c.v_scale,
        p.q, p.seq_len, p.sel_idx, p.sel_cnt, p.max_sel, c.n_kv_heads, c.max_seq, c.block,
        p.max_len, S, ups, scale2, ws_m, ws_l, ws_o, p.dbg_logits);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (launch_decode_mfma(p, stream)) return hipGetLastError();
  switch (p.n_heads / p.c->n_kv_heads) {
    case 1: launch_decode_g<1>(p, stream); break;
    case 2: launch_decode_g<2>(p, stream); break;
    case 4: launch_decode_g<4>(p, stream); break;
    case 8: launch_decode_g<8>(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace skv
