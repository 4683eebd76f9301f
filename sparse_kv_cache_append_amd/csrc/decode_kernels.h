// decode_attn kernels on the matrix cores (gfx950 MFMA), for the launchers in
// decode_mfma.hip (head dim 128, every variant) and decode_dims.hip (64, 256).
//
// The per-step contractions of decode attention for one KV head are small
// dense products: S = K_tile q^T (tokens x GQA heads, reduced over the head
// dimension) and O += P V_tile (heads x channels, reduced over tokens).  Both
// run on MFMA; the vector ALUs only do the online softmax.  The query heads of
// a GQA group fill the N = 16 columns of the MFMA tile (zero-padded past G),
// so every K/V byte is read once for the whole group.
//
// Layouts (verified lane maps of the gfx950 instructions):
//   v_mfma_f32_16x16x32_f16 / _16x16x16f16 / _i32_16x16x64_i8:
//     A: lane l holds row l%16, k-chunk l/16;  B: column l%16, k-chunk l/16;
//     C: column l%16, rows 4*(l/16) .. +3.
//   ds_read_b64_tr_b16: in each 16-lane group, lane j receives element j%4 of
//     the 4-element rows read by lanes j/4, 4+j/4, 8+j/4, 12+j/4.
//   ds_read_b64_tr_b8: lane j receives byte j%8 of the 8-byte rows read by
//     lanes j/8, 2+j/8, ..., 14+j/8.
//
// Data flow per wavefront and tile (f16: 16 tokens, int8: 32 tokens):
//   global -> registers: coalesced 16-byte loads, 4 rows per instruction,
//     raw-buffer loads off a per-tile resource (no vector address
//     arithmetic; its record count is the tile's valid bytes, so rows past
//     the length read as zeros and every refill is the same branch-free
//     load sequence), two tiles in flight per wavefront (each refilled as
//     soon as it is staged in LDS); nontemporal, since every K/V byte is
//     read once per step (the streaming hint raises the read rate of this
//     part by about a tenth);
//   registers -> LDS: row-major tile with the 16-byte chunks of row r XOR-
//     swizzled by r % 16, so both the row reads of the q.K operand and the
//     transposing reads of the P.V operand are free of bank conflicts;
//   q.K: A = K rows from LDS, B = query (f16: split into an f16 high and low
//     part, two MFMAs, ~22-bit query precision; int8: the absmax codes, an
//     exact int32 product);
//   softmax: per-head tile max across the 4 lane groups, running max/mass,
//     one rescale of the accumulators per tile (int8: only on the tiles that
//     move its lazy reference maximum; masks only on a partial tile; the
//     tile walk is wave-uniform, in scalar registers);
//   P.V: A = P (f16 high + low parts, straight from the q.K output registers),
//     B = V^T via the transposing LDS read (int8 codes widened to f16, exact).
#pragma once

#include <type_traits>

#include "decode_core.h"
#include "device_common.h"
#include "fused_walk.h"
#include "launch.h"
#include "select_core.h"

namespace skv {
namespace {

// The weights enter P.V as an f16 high part plus an f16 low part, both taken
// from the weight times 2^kPwShift (exact).  The f16 kernel's weights are at
// most 1 (exact running maximum), so the scaled weights stay below 2^15 and
// every weight down to 2^-18 of the running maximum keeps its full ~22-bit
// precision, weights down to 2^-29 at least 11 bits; without the shift a long
// flat tail of weights below 2^-14 would reach P.V with only a few
// (subnormal) bits while its full mass counts in the normalizer.  O is
// scaled back (exactly) before the partial state is written.
constexpr int kPwShiftF16 = 15;
__device__ __forceinline__ void split_hi_lo4(const float* p, half4_t& hi, half4_t& lo) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float x = p[s] * float(1 << kPwShiftF16);
    const _Float16 h = (_Float16)x;
    hi[s] = h;
    lo[s] = (_Float16)(x - (float)h);
  }
}

// The one-token append of a dense step (APP kernels).  Every wavefront reads
// the new K and V rows (this lane: channels 2 lane, 2 lane + 1) and, when one
// of its tiles holds position pos0[b], writes them over that row of the tile
// staged in LDS, so the attention sees exactly what the separate append would
// have stored there (the cache row itself is stale until this step writes it).
// The part whose blocks hold pos0[b] (the row's last part when pos0 lies past
// every part's blocks) writes the rows, the int8 scales and the block's merged side-cache bounds,
// as skv_kv_append does for one token: wavefront 0, after its walk.  The old
// bounds it merges with are requested before the walk through a buffer
// resource that has records only in that wavefront and only for a block that
// keeps earlier tokens.
struct AppendArgs {
  void* k;
  void* v;
  float* ks;
  float* vs;
  uint16_t* kmin;          // nullptr: the cache has no side cache
  uint16_t* kmax;
  const void* k_new;
  const void* v_new;
  const int32_t* pos0;
  int32_t max_blocks;
};

// Who writes the appended token of row (b, g), and the block's old bounds
// (zeros where not needed).
struct AppendOwner {
  bool own, fresh;
  int32_t jp;
  uint32_t bmn_old, bmx_old;
};
__device__ __forceinline__ AppendOwner append_owner(const AppendArgs& app, int32_t p_new,
                                                    int64_t bg, int32_t max_seq, int32_t block,
                                                    int32_t split, int32_t n_split,
                                                    int32_t units_per_split, int wave) {
  AppendOwner o;
  const bool p_ok = p_new >= 0 && p_new < max_seq;
  o.jp = p_ok ? p_new / block : 0;
  o.fresh = p_ok && o.jp * block == p_new;
  o.own = p_ok && wave == 0 && split == min(o.jp / units_per_split, n_split - 1);
  const bool side = app.kmin != nullptr;
  const int bytes = (o.own && side && !o.fresh) ? kD * 2 : 0;
  const int64_t bo = side ? (bg * app.max_blocks + o.jp) * kD : 0;   // no offset on a null base
  const auto rmn = __builtin_amdgcn_make_buffer_rsrc(app.kmin + bo, (short)0, bytes, kRsrcWord3);
  const auto rmx = __builtin_amdgcn_make_buffer_rsrc(app.kmax + bo, (short)0, bytes, kRsrcWord3);
  const uint32_t lane = threadIdx.x % kWave;
  o.bmn_old = __builtin_amdgcn_raw_buffer_load_b32(rmn, 4u * lane, 0, 0);
  o.bmx_old = __builtin_amdgcn_raw_buffer_load_b32(rmx, 4u * lane, 0, 0);
  return o;
}

// Store this lane's two channels of the new key's bounds (lo, hi: the rounded
// min and max per channel), min/max-merged with the old ones unless the block
// starts at the new token.
__device__ __forceinline__ void store_new_bounds(const AppendArgs& app, const AppendOwner& o,
                                                 int64_t bg, const uint16_t (&mn)[2],
                                                 const uint16_t (&mx)[2]) {
  uint16_t a[2] = {mn[0], mn[1]}, c[2] = {mx[0], mx[1]};
  if (!o.fresh) {
    a[0] = f16_min_bits(uint16_t(o.bmn_old & 0xFFFFu), a[0]);
    a[1] = f16_min_bits(uint16_t(o.bmn_old >> 16), a[1]);
    c[0] = f16_max_bits(uint16_t(o.bmx_old & 0xFFFFu), c[0]);
    c[1] = f16_max_bits(uint16_t(o.bmx_old >> 16), c[1]);
  }
  const int64_t bo = (bg * app.max_blocks + o.jp) * (kD / 2) + threadIdx.x % kWave;
  reinterpret_cast<uint32_t*>(app.kmin)[bo] = uint32_t(a[0]) | (uint32_t(a[1]) << 16);
  reinterpret_cast<uint32_t*>(app.kmax)[bo] = uint32_t(c[0]) | (uint32_t(c[1]) << 16);
}

// Head dimension D (64, 128 or 256): a row is 2 D bytes (f16) or D bytes
// (int8); a tile's 16-byte loads cover 1024 / row-bytes rows per
// instruction; q.K runs D / 32 (f16) or D / 64 (int8) MFMA steps, P.V D / 16
// channel blocks.  At D = 256 the two tiles in flight and the accumulators
// take twice the registers and LDS, so one workgroup runs per CU.  The
// folded append moves two channels per lane: D = 128 only.
template <int D>
struct HeadDim {
  static_assert(D == 64 || D == 128 || D == 256, "head dims 64, 128, 256");
  static constexpr int kNB = D / 16;                     // P.V channel blocks
  static constexpr int kOcc = D > 128 ? 1 : 2;           // workgroups per CU
};
// 16-byte chunk c of row r sits at chunk c ^ (r % C) of its row, C = the
// row's chunk count capped at 16
template <int CHUNKS>
__device__ __forceinline__ int swz_c(int row) { return row & ((CHUNKS < 16 ? CHUNKS : 16) - 1); }

// ------------------------------------------------------------------ f16
// Tile = 16 tokens: K and V tiles are 32 D bytes each (4 KiB at D = 128, 4
// load instructions).
template <int D, int G, int SELR, bool APP, bool HM = false>
__global__ void __launch_bounds__(kMThreads, HeadDim<D>::kOcc)
decode_f16_mfma(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                const float* __restrict__ q, const int32_t* __restrict__ seq_len,
                const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
                int32_t max_sel, int32_t Hkv, int32_t max_seq, int32_t block, int32_t max_len,
                int32_t n_split, int32_t n_rows, int32_t units_per_split, float qscale2,
                float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
                FusedSelect fs, AppendArgs app, const uint32_t* __restrict__ sel_hmask,
                int32_t ntok) {
  static_assert(!APP || D == 128, "the folded append moves two channels per lane");
  constexpr int T = 16;
  constexpr int RB = 2 * D;                                 // bytes per row
  constexpr int kTileBytes = T * RB;                        // 4096 at D = 128
  constexpr int kLoads = kTileBytes / 1024;                 // 16-byte loads per lane
  constexpr int kCpr = RB / 16;                             // chunks per row
  constexpr int kRpl = 1024 / RB;                           // rows per load instruction
  constexpr int KQ = D / 32;                                // q.K steps
  constexpr int NB = HeadDim<D>::kNB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMWaves][2][2 * kTileBytes];
  static_assert(SELR == 0 || sizeof(smem) >= sizeof(SelectShared),
                "the prologue's selection runs in the tile buffers");
  // 1-D grid of n_split x Hkv x batch parts, row by row (XCD-aware slots)
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t split = int32_t(slot % uint32_t(n_split));
  const uint32_t row = xcd_row(slot / uint32_t(n_split), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const QRows qr = make_qrows<G>(ntok, Hkv);
  const int64_t bg = int64_t(b) * Hkv + g;
  // requests issued before anything waits: row length, given list, query
  const int32_t L_raw = seq_len[b];
  ListSeed ls{};
  if constexpr (SELR == 0)
    ls = list_seed(sel_idx, sel_cnt, max_sel, bg, split, units_per_split, HM ? sel_hmask : nullptr);
  // folded append: the position and this lane's two channels of the new rows
  int32_t p_new = -1;
  uint32_t kx = 0u, vx = 0u;
  if constexpr (APP) {
    p_new = app.pos0[b];
    kx = static_cast<const uint32_t*>(app.k_new)[bg * (D / 2) + lane];
    vx = static_cast<const uint32_t*>(app.v_new)[bg * (D / 2) + lane];
  }

  // query as the B operand of q.K: column = head lc, k-chunk = lg; f16 hi + lo
  half8_t qhi[KQ], qlo[KQ];
  {
    const bool hv = lc < G;
    const float* qp = q + qr.row(b, g, hv ? lc : 0) * D;
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
  // wave-uniform (scalar): the walk and its branches stay scalar
  const int32_t L = __builtin_amdgcn_readfirstlane(min(max(L_raw, 0), max_len));
  TileWalk tw;
  if constexpr (SELR > 0)
    tw = fused_walk<T, SELR>(fs, max_sel, bg, b, L, L_raw, block, split, units_per_split,
                            smem);
  else
    tw = make_walk<T>(ls, sel_idx, max_sel, bg, L, block, split, units_per_split);
  if constexpr (HM) tw.hsel = sel_hmask + bg * max_sel;
  tw.init(wave);
  float m_run = -INFINITY, l_run = 0.0f;
  float4_t O[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) O[n] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(kc + bg * int64_t(max_seq) * D);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(vc + bg * int64_t(max_seq) * D);
  struct Frag { int4_t k[kLoads], v[kLoads]; int32_t r0, nvalid; uint32_t hm; };
  // lane loads row kRpl i + lane / kCpr of the tile, 16-byte chunk
  // lane % kCpr (D = 128: row 4 i + lane / 16, chunk lane % 16): byte
  // 1024 i + 16 lane of the tile, through the tile's buffer resource.
  // Its record count is the tile's valid bytes, so the rows of a partial
  // tile past the row's length, and every row once the walk is over, read as
  // zeros without touching memory: one load sequence for every case, no
  // branch (the masked weights of those rows are zero).
  auto issue = [&](Frag& f) {
    int32_t r0 = 0, nv = 0;
    uint32_t hm = ~0u;
    if (tw.more()) tw.next<T, HM>(r0, nv, &hm);
    f.r0 = r0;
    f.nvalid = nv;
    f.hm = hm;
    const uint32_t lo = 16u * uint32_t(lane);
    const int bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * RB);
    const auto kr = tile_rsrc(kbase + int64_t(r0) * RB, bytes);
    const auto vr = tile_rsrc(vbase + int64_t(r0) * RB, bytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      f.k[i] = tile_load(kr, lo + 1024 * i);
      f.v[i] = tile_load(vr, lo + 1024 * i);
    }
  };

  // Process one tile held in registers: stage it in LDS buffer `buf`, refill
  // the fragment with the tile two steps ahead, then q.K, softmax and P.V.
  auto process = [&](auto bufc, Frag& fr) {
    constexpr int kBuf = decltype(bufc)::value;
    uint8_t* kt = smem[wave][kBuf];
    uint8_t* vt = kt + kTileBytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int row = kRpl * i + lane / kCpr;
      const int off = row * RB + 16 * ((lane % kCpr) ^ swz_c<kCpr>(row));
      *reinterpret_cast<int4_t*>(kt + off) = fr.k[i];
      *reinterpret_cast<int4_t*>(vt + off) = fr.v[i];
    }
    if constexpr (APP) {
      // the appended token's row, if this tile holds it (a wave-uniform test;
      // LDS applies the wavefront's writes in order, so these win)
      // (nvalid is negative for the tile slots past the row's end)
      const int32_t prel = p_new - fr.r0;
      if (prel >= 0 && prel < fr.nvalid) {
        const int off = prel * RB + 16 * ((lane >> 2) ^ swz_c<kCpr>(prel)) + 4 * (lane & 3);
        *reinterpret_cast<uint32_t*>(kt + off) = kx;
        *reinterpret_cast<uint32_t*>(vt + off) = vx;
      }
    }
    const int32_t nvalid = fr.nvalid, r0 = fr.r0;
    const uint32_t hm = fr.hm;
    issue(fr);
    // LDS writes above and reads below touch the same array: they stay in
    // program order, and LDS executes one wavefront's accesses in order.
    // q.K: A = K row lc, logical chunk lg + 4kk
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const half8_t a = *reinterpret_cast<const half8_t*>(
          kt + lc * RB + 16 * ((lg + 4 * kk) ^ swz_c<kCpr>(lc)));
      acc = mfma_f16_32(a, qhi[kk], acc);
      acc = mfma_f16_32(a, qlo[kk], acc);
    }
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = acc[r];
    if (nvalid < T || r0 + T > L - ntok + 1) {     // wave-uniform
      // rows past the row's length; with a chunk of query tokens, column lc
      // is token lc >> gsh, which sees the positions below
      // L - (ntok - 1 - token) only
      const int32_t lim = min(nvalid, L - (ntok - 1 - (lc >> qr.gsh)) - r0);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = (4 * lg + r < lim) ? sc[r] : -INFINITY;
    }
    if constexpr (HM) {
      // the heads that did not choose this block leave it out
      const bool off = ((hm >> lc) & 1u) == 0u;
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = off ? -INFINITY : sc[r];
    }
    tile_softmax<G, 1, false>(sc, m_run, l_run, O);
    half4_t phi, plo;
    split_hi_lo4(sc, phi, plo);
    // P.V: B = V^T rows 4lg..4lg+3 via the transposing read; 16 channels per n
    const int tr_row = 4 * lg + (lc >> 2);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int chunk = 2 * n + ((lc & 3) >> 1);
      const int off = tr_row * RB + 16 * (chunk ^ swz_c<kCpr>(tr_row)) + 8 * (lc & 1);
      const short4_t raw =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((SKV_LDS short4_t*)(vt + off));
      const half4_t bv = __builtin_bit_cast(half4_t, raw);
      O[n] = mfma_f16_16(phi, bv, O[n]);
      O[n] = mfma_f16_16(plo, bv, O[n]);
    }
  };

  // Pairs of tiles, then an odd last one: the loop has no exit between its
  // two halves (an exit there gives the compiler a path to the loop head that
  // skips the second refill, and its waits at the head then drain both
  // fragments in flight).
  Frag f0, f1;
  const int32_t n_mine = tw.count();
  issue(f0);
  issue(f1);
  AppendOwner ao{};
  if constexpr (APP) {
    p_new = __builtin_amdgcn_readfirstlane(p_new);
    ao = append_owner(app, p_new, bg, max_seq, block, split, n_split, units_per_split, wave);
  }
  for (int32_t t = 0; t + 1 < n_mine; t += 2) {
    process(std::integral_constant<int, 0>{}, f0);
    process(std::integral_constant<int, 1>{}, f1);
  }
  if (n_mine & 1) process(std::integral_constant<int, 0>{}, f0);
#pragma unroll
  for (int n = 0; n < NB; ++n) {
#pragma unroll
    for (int r = 0; r < 4; ++r) O[n][r] *= 1.0f / float(1 << kPwShiftF16);
  }
  finish_mfma<G>(m_run, l_run, O, reinterpret_cast<float*>(&smem[0][0][0]), ws_m, ws_l, ws_o,
                 qr, b, g, n_split, split);
  if constexpr (APP) {
    if (ao.own) {
      const int64_t row = (bg * max_seq + p_new) * (D / 2) + lane;
      static_cast<uint32_t*>(app.k)[row] = kx;
      static_cast<uint32_t*>(app.v)[row] = vx;
      if (app.kmin != nullptr) {
        // one token's bounds are its own key (a NaN channel keeps +inf / -inf,
        // as the min/max scan of the append kernel leaves it)
        uint16_t mn[2], mx[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint16_t x = uint16_t(kx >> (16 * e));
          const float xf = h2f(x);
          mn[e] = xf < INFINITY ? x : uint16_t(0x7C00u);
          mx[e] = xf > -INFINITY ? x : uint16_t(0xFC00u);
        }
        store_new_bounds(app, ao, bg, mn, mx);
      }
    }
  }
}

// ------------------------------------------------------------------ int8
// Tile = 32 tokens: K and V tiles are 4 KiB each (4 load instructions of 8
// rows) plus their 32 K scales and 32 V scales (one load instruction).
//
// Token order inside a tile.  q.K runs as two 16-token halves, so lane
// (group lg, head lc) holds the logits of tokens 4 lg + r and 16 + 4 lg + r
// (r = 0..3).  P.V contracts all 32 tokens in one 16x16x32 f16 MFMA per 16
// channels, with element e of lane group lg standing for token
// tok(lg, e) = 16 (e / 4) + 4 lg + e % 4 in both operands (a permutation of
// the reduction index leaves the sum unchanged).  The transposing byte read
// delivers that order: lane i of group lg reads the 8 bytes of token
// tok(lg, i / 2) at channel 16 n + 8 (i % 2), and lane j then holds channel
// 16 n + j of tokens tok(lg, 0..7).  The codes are widened to f16 exactly
// (1152 + c is exact in f16, minus 1152).
//
// The V scales are folded into the weights: P' = p * v_scale * 2^(7 - e) with
// 2^e the largest V scale seen so far rounded up to a power of two, so P'
// stays below 2^15 (the softmax's weight bound is 2^8 with its lazy
// reference) and the f16 high + low split keeps its precision whatever the
// scale's magnitude, with 7 bits of headroom for small weights (a weight 2^-10
// of the largest still gets about 18 bits); the accumulator holds
// O * 2^(7 - e), is rescaled (exactly, by a power of two) in the rare tile
// where e grows, and is scaled back at the end.
constexpr int kPwShiftI8 = 7;
template <int D, int G, int SELR, bool APP, bool HM = false>
__global__ void __launch_bounds__(kMThreads, HeadDim<D>::kOcc)
decode_i8_mfma(const int8_t* __restrict__ kc, const int8_t* __restrict__ vc,
               const float* __restrict__ ksc, const float* __restrict__ vsc,
               const float* __restrict__ q, const int32_t* __restrict__ seq_len,
               const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
               int32_t max_sel, int32_t Hkv, int32_t max_seq, int32_t block, int32_t max_len,
               int32_t n_split, int32_t n_rows, int32_t units_per_split, float scale2,
               float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
               int32_t* __restrict__ dbg, FusedSelect fs, AppendArgs app,
               const uint32_t* __restrict__ sel_hmask, int32_t ntok) {
  static_assert(!APP || D == 128, "the folded append moves two channels per lane");
  constexpr int T = 32;
  constexpr int RB = D;                                     // bytes per row
  constexpr int kTileBytes = T * RB;                        // 4096 at D = 128
  constexpr int kLoads = kTileBytes / 1024;                 // 16-byte loads per lane
  constexpr int kCpr = RB / 16;                             // chunks per row
  constexpr int kRpl = 1024 / RB;                           // rows per load instruction
  constexpr int KQ = D / 64;                                // q.K steps
  constexpr int NB = HeadDim<D>::kNB;
  constexpr int kScaleOff = 2 * kTileBytes;                 // 32 K scales, 32 V scales
  constexpr int kBufBytes = 2 * kTileBytes + 2 * T * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMWaves][2][kBufBytes];
  static_assert(SELR == 0 || sizeof(smem) >= sizeof(SelectShared),
                "the prologue's selection runs in the tile buffers");
  // 1-D grid of n_split x Hkv x batch parts, row by row (XCD-aware slots)
  const uint32_t slot = xcd_slot(blockIdx.x, gridDim.x);
  const int32_t split = int32_t(slot % uint32_t(n_split));
  const uint32_t row = xcd_row(slot / uint32_t(n_split), uint32_t(n_rows));
  const int32_t g = int32_t(row % uint32_t(Hkv)), b = int32_t(row / uint32_t(Hkv));
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const QRows qr = make_qrows<G>(ntok, Hkv);
  const int64_t bg = int64_t(b) * Hkv + g;
  // requests issued before anything waits: row length, given list, query
  const int32_t L_raw = seq_len[b];
  ListSeed ls{};
  if constexpr (SELR == 0)
    ls = list_seed(sel_idx, sel_cnt, max_sel, bg, split, units_per_split, HM ? sel_hmask : nullptr);
  // folded append: the position and this lane's two channels of the new rows
  int32_t p_new = -1;
  float2 kf = {0.0f, 0.0f}, vf = {0.0f, 0.0f};
  if constexpr (APP) {
    p_new = app.pos0[b];
    kf = static_cast<const float2*>(app.k_new)[bg * (D / 2) + lane];
    vf = static_cast<const float2*>(app.v_new)[bg * (D / 2) + lane];
  }

  // the query (float32), requested at entry with the row length and list;
  // its codes are computed once the first tiles are in flight
  const bool hv = lc < G;
  float x[KQ][16];
  {
    const float* qp = q + qr.row(b, g, hv ? lc : 0) * D;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v4 = *reinterpret_cast<const float4*>(qp + 64 * kk + 16 * lg + 4 * i);
        x[kk][4 * i + 0] = v4.x; x[kk][4 * i + 1] = v4.y;
        x[kk][4 * i + 2] = v4.z; x[kk][4 * i + 3] = v4.w;
      }
    }
  }
  int4_t qb[KQ];
  float coef;
  // wave-uniform (scalar): the walk and its branches stay scalar
  const int32_t L = __builtin_amdgcn_readfirstlane(min(max(L_raw, 0), max_len));
  TileWalk tw;
  if constexpr (SELR > 0)
    tw = fused_walk<T, SELR>(fs, max_sel, bg, b, L, L_raw, block, split, units_per_split,
                            smem);
  else
    tw = make_walk<T>(ls, sel_idx, max_sel, bg, L, block, split, units_per_split);
  if constexpr (HM) tw.hsel = sel_hmask + bg * max_sel;
  tw.init(wave);
  float m_run = -INFINITY, l_run = 0.0f;
  float4_t O[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) O[n] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(kc + bg * int64_t(max_seq) * D);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(vc + bg * int64_t(max_seq) * D);
  const float* ksb = ksc + bg * int64_t(max_seq);
  const float* vsb = vsc + bg * int64_t(max_seq);
  // optional exact-logit dump (uniform test, so the hot loop only branches once)
  const bool want_dbg = dbg != nullptr;
  int32_t* dbg_h = want_dbg ? dbg + qr.row(b, g, min(lc, G - 1)) * int64_t(max_len) : nullptr;
  const int32_t last = max(L - 1, 0);
  const float* sbase = (lane < 32 ? ksb : vsb) + lane % 32;
  struct Frag { int4_t k[kLoads], v[kLoads]; float sc; int32_t r0, nvalid; uint32_t hm; };
  // lane loads row kRpl i + lane / kCpr of the tile, 16-byte chunk
  // lane % kCpr (D = 128: row 8 i + lane / 8, chunk lane % 8; byte
  // 1024 i + 16 lane of the tile), through the tile's buffer
  // resource whose record count is the valid bytes: rows past the row's
  // length, and every row once the walk is over, read as zeros without
  // touching memory.  Lanes < 32 load the K scale of token lane, the others
  // the V scale of token lane - 32, clamped to the last valid token (finite;
  // the weights of those rows are zero).  One load sequence for every case,
  // no branch.
  auto issue = [&](Frag& f) {
    int32_t r0 = 0, nv = 0;
    uint32_t hm = ~0u;
    if (tw.more()) tw.next<T, HM>(r0, nv, &hm);
    f.r0 = r0;
    f.nvalid = nv;
    f.hm = hm;
    const uint32_t lo = 16u * uint32_t(lane);
    const int bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * RB);
    const auto kr = tile_rsrc(kbase + int64_t(r0) * RB, bytes);
    const auto vr = tile_rsrc(vbase + int64_t(r0) * RB, bytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      f.k[i] = tile_load(kr, lo + 1024 * i);
      f.v[i] = tile_load(vr, lo + 1024 * i);
    }
    f.sc = sbase[min(r0 + lane % 32, last) - lane % 32];
  };
  auto sw = [](int row, int chunk) { return row * RB + 16 * (chunk ^ (row & (kCpr - 1))); };
  constexpr int kExpUnset = -100000;       // no nonzero V scale seen yet
  int e_run = kExpUnset;
  float ks_new = 0.0f, vs_new = 0.0f;      // the appended token's scales and codes
  uint32_t kcode = 0u, vcode = 0u;

  auto process = [&](auto bufc, Frag& fr) {
    constexpr int kBuf = decltype(bufc)::value;
    uint8_t* kt = smem[wave][kBuf];
    uint8_t* vt = kt + kTileBytes;
    float* st = reinterpret_cast<float*>(kt + kScaleOff);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int row = kRpl * i + lane / kCpr;
      *reinterpret_cast<int4_t*>(kt + sw(row, lane % kCpr)) = fr.k[i];
      *reinterpret_cast<int4_t*>(vt + sw(row, lane % kCpr)) = fr.v[i];
    }
    float scl = fr.sc;
    const int32_t nvalid = fr.nvalid, r0 = fr.r0;
    const uint32_t hm = fr.hm;
    if constexpr (APP) {
      // the appended token's codes and scales, if this tile holds it (the
      // scale also where a lane's clamped token is that token)
      const int32_t prel = p_new - r0;
      if (prel >= 0 && prel < nvalid) {          // nvalid < 0 past the row's end
        const int off = sw(prel, lane >> 3) + 2 * (lane & 7);
        *reinterpret_cast<uint16_t*>(kt + off) = uint16_t(kcode);
        *reinterpret_cast<uint16_t*>(vt + off) = uint16_t(vcode);
      }
      scl = min(r0 + lane % 32, last) == p_new ? (lane < 32 ? ks_new : vs_new) : scl;
    }
    // V-scale unit: 2^e_run >= every V scale seen so far; a power of two, so
    // the V scales stored in units of it and the change of unit of O when it
    // grows are exact.  Done before the refill, so the fragment's scale
    // register is free when the refill's scale lands in it (a copy of a
    // register still being loaded would make the wave wait for every load).
    const int32_t vbits =
        __builtin_amdgcn_readfirstlane(__float_as_int(wave_max(lane >= 32 ? scl : 0.0f)));
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
    st[lane] = lane >= 32 ? ldexpf(scl, kPwShiftI8 - e_use) : scl;
    issue(fr);
    // q.K, exact: two 16-token halves, D channels as D / 64 k = 64 steps
    int4_t acc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      acc[s] = int4_t{0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) {
        const int4_t a = *reinterpret_cast<const int4_t*>(kt + sw(16 * s + lc, lg + 4 * kk));
        acc[s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qb[kk], acc[s], 0, 0, 0);
      }
    }
    const float4 ks0 = *reinterpret_cast<const float4*>(st + 4 * lg);
    const float4 ks1 = *reinterpret_cast<const float4*>(st + 16 + 4 * lg);
    const float4 vs0 = *reinterpret_cast<const float4*>(st + 32 + 4 * lg);
    const float4 vs1 = *reinterpret_cast<const float4*>(st + 48 + 4 * lg);
    const float ks[8] = {ks0.x, ks0.y, ks0.z, ks0.w, ks1.x, ks1.y, ks1.z, ks1.w};
    const float vs[8] = {vs0.x, vs0.y, vs0.z, vs0.w, vs1.x, vs1.y, vs1.z, vs1.w};
    if (want_dbg) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 16 * (e / 4) + 4 * lg + e % 4;
        if (lc < G && t < nvalid) dbg_h[r0 + t] = acc[e / 4][e % 4];
      }
    }
    float sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sc[e] = float(acc[e / 4][e % 4]) * coef * ks[e];
    if (nvalid < T || r0 + T > L - ntok + 1) {     // wave-uniform
      // rows past the row's length, and a chunk token's causal limit (as in
      // the f16 kernel)
      const int32_t lim = min(nvalid, L - (ntok - 1 - (lc >> qr.gsh)) - r0);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sc[e] = 16 * (e / 4) + 4 * lg + e % 4 < lim ? sc[e] : -INFINITY;
    }
    if constexpr (HM) {
      // the heads that did not choose this block leave it out
      const bool off = ((hm >> lc) & 1u) == 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = off ? -INFINITY : sc[e];
    }
    // O is kept in units of 2^(e_run - 7); the exact change of unit when e_run
    // grows rides on the softmax rescale of O
    tile_softmax<G, 2, true>(sc, m_run, l_run, O, unit);
    // P' = p * v_scale * 2^(7 - e_run) (the stored V scales are in that unit)
    float pw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pw[e] = sc[e] * vs[e];
    half8_t phi, plo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const _Float16 h = (_Float16)pw[e];
      phi[e] = h;
      plo[e] = (_Float16)(pw[e] - (float)h);
    }
    // P.V: B = V codes of channels 16 n + lc for tokens tok(lg, 0..7)
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

  // Pairs of tiles, then an odd last one: the loop has no exit between its
  // two halves (an exit there gives the compiler a path to the loop head that
  // skips the second refill, and its waits at the head then drain both
  // fragments in flight).
  Frag f0, f1;
  const int32_t n_mine = tw.count();
  issue(f0);
  issue(f1);
  AppendOwner ao{};
  if constexpr (APP) {
    p_new = __builtin_amdgcn_readfirstlane(p_new);
    ao = append_owner(app, p_new, bg, max_seq, block, split, n_split, units_per_split, wave);
    // the new rows quantized as the append kernel does (same reduction order)
    auto quant2 = [](float2 x, float& scale) {
      const float a = wave_max(fmaxf(fmaxf(0.0f, fabsf(x.x)), fabsf(x.y)));
      scale = absmax_scale(a);
      return (uint32_t(quant_code(x.x, scale)) & 0xFFu) |
             ((uint32_t(quant_code(x.y, scale)) & 0xFFu) << 8);
    };
    kcode = quant2(kf, ks_new);
    vcode = quant2(vf, vs_new);
  }
  // Query codes as the B operand of q.K (column = head lc, k-chunk lg): the
  // head's absmax scale over all D channels (the 4 lanes of a column hold
  // D / 4 channels each), then the codes of channels 64 kk + 16 lg + 0..15.
  // (After the first two refills: this is a few hundred vector instructions
  // that would otherwise delay every wavefront's first tile loads.)
  i8_query_operand(x, hv, scale2, qb, coef);
  for (int32_t t = 0; t + 1 < n_mine; t += 2) {
    process(std::integral_constant<int, 0>{}, f0);
    process(std::integral_constant<int, 1>{}, f1);
  }
  if (n_mine & 1) process(std::integral_constant<int, 0>{}, f0);
  if (e_run != kExpUnset) {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) O[n][r] = ldexpf(O[n][r], e_run - kPwShiftI8);
    }
  }
  finish_mfma<G>(m_run, l_run, O, reinterpret_cast<float*>(&smem[0][0][0]), ws_m, ws_l, ws_o,
                 qr, b, g, n_split, split);
  if constexpr (APP) {
    if (ao.own) {
      const int64_t row = bg * max_seq + p_new;
      reinterpret_cast<uint16_t*>(static_cast<int8_t*>(app.k) + row * D)[lane] = uint16_t(kcode);
      reinterpret_cast<uint16_t*>(static_cast<int8_t*>(app.v) + row * D)[lane] = uint16_t(vcode);
      if (lane == 0) {
        app.ks[row] = ks_new;
        app.vs[row] = vs_new;
      }
      if (app.kmin != nullptr) {
        // bounds from the float32 key, rounded outward to f16
        const uint16_t mn[2] = {f32_to_f16_down(fminf(INFINITY, kf.x)),
                                f32_to_f16_down(fminf(INFINITY, kf.y))};
        const uint16_t mx[2] = {f32_to_f16_up(fmaxf(-INFINITY, kf.x)),
                                f32_to_f16_up(fmaxf(-INFINITY, kf.y))};
        store_new_bounds(app, ao, bg, mn, mx);
      }
    }
  }
}


// The launch shape shared by every decode variant: the partial-state regions
// (nt query tokens per sequence: H * nt state rows), the units (blocks, or
// entries of the selected list) per part -- at least one, also for an empty
// cache (max_len == 0), since the folded append divides the new token's block
// index by it to find the part that writes the token -- and the 1-D grid of
// n_split x Hkv x batch parts.
struct DecodeShape {
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int32_t ups, n_rows;
  dim3 grid;
  float scale2;
};
inline hipError_t decode_shape(const DecodeParams& p, int32_t nt, DecodeShape& s) {
  const skv_cache& c = *p.c;
  const int32_t B = c.batch, S = p.n_split;
  const int32_t Hq = p.n_heads * nt;
  s.ws_m = p.ws + ws_m_offset(B, Hq, S);
  s.ws_l = p.ws + ws_l_offset(B, Hq, S);
  s.ws_o = p.ws + ws_o_offset(B, Hq, S);
  int32_t ups;
  if (p.sel_idx != nullptr) {
    ups = (p.max_sel + S - 1) / S;
  } else {
    const int32_t nb_max = (p.max_len + c.block - 1) / c.block;
    ups = (nb_max + S - 1) / S;
  }
  s.ups = ups < 1 ? 1 : ups;
  const int64_t n_wg = int64_t(S) * c.n_kv_heads * B;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  s.n_rows = c.n_kv_heads * B;
  s.grid = dim3(static_cast<uint32_t>(n_wg));
  s.scale2 = p.softmax_scale * kLog2e;
  return hipSuccess;
}

}  // namespace
}  // namespace skv
