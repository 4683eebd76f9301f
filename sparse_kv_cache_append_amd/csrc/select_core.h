// Exact fixed top-K of one row of block scores, computed by one workgroup of
// kSelThreads threads: the selection rule of sparse_attn.md, "Method" (the
// K highest upper bounds) and "Budget policy" (fixed K), with exact ties
// going to the lower block index.
//
// Order.  Candidate i with score key k_i (float_key: order-preserving, -0
// and +0 equal) has the 64-bit order value v_i = k_i * 2^32 + (2^32 - 1 - i):
// a larger score wins, and among equal scores the lower index.  The v_i are
// distinct, so "the K best candidates" is exactly {i : v_i >= V*} for the
// K-th largest value V*; computing V* is the whole selection.
//
// Thread t holds the keys of candidates t, t + 256, ... in registers (RMAX
// of them), loaded in one round trip.  V* is found by
//   * fixing the leading key bits that every candidate shares (a DPP AND/OR
//     reduction): the bounds of one row share sign and most exponent bits,
//     and a histogram of those bits would pile every key into one or two bins;
//   * most-significant-digit radix passes (LDS histogram of 256 bins filled
//     straight from registers, then every wavefront scans the bins itself
//     with a DPP prefix sum, so a pass costs one barrier) fixing 8 more bits
//     of the K-th key each, until at most 64 candidates share its prefix;
//   * gathering those (ballot compaction into per-wavefront rows, no
//     atomics) and narrowing them in every wavefront with ballots, one bit
//     of the order value at a time, to the one of the right rank;
//   * or, if more than 64 keys equal the K-th key exactly, taking its
//     occurrence of the right rank in index order.
// Index order of flagged candidates (ascending output positions) comes from
// per-(chunk, wavefront) ballot counts, published once and scanned by every
// wavefront, and the set ballot bits below each lane.
//
// The per-chunk loops avoid a branch per chunk (exec-mask changes or scalar
// exits) where they can: the chunks are independent, and without branches
// between them their ballots and compares overlap instead of running as one
// dependent chain per chunk (4096 candidates: taken mask and order counts
// 3,600 -> 1,900 cycles, a radix pass 3,200 -> 2,300).  Chunks past the row
// are run too; their keys are invalid and change nothing.
#pragma once

#include "device_common.h"

namespace skv {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelMaxChunks = 64;                 // candidates <= 64 * 256 = 16384

struct __attribute__((aligned(16))) SelectShared {
  uint32_t hist[3][256];                          // rotating radix-pass histograms
  uint64_t slot[kSelWaves][kWave];                // per-wave order values tied on the prefix
  int32_t part[kSelMaxChunks * kSelWaves];        // (chunk, wave) counts, chunk-major
  uint32_t red_and[kSelWaves], red_or[kSelWaves];
  alignas(16) int32_t n_gather[kSelWaves];       // read as one 16-byte load
  uint64_t cut;                                   // the many-equal-keys case only
};

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}
__device__ __forceinline__ uint64_t order_value(uint32_t key, int32_t i) {
  return (uint64_t(key) << 32) | uint64_t(~uint32_t(i));
}

// Clears the first radix pass's histogram.  Call it (whole workgroup) before
// sel_cut, e.g. while the keys are in flight: sel_cut's first barrier orders
// it before the first use.
__device__ __forceinline__ void sel_init(SelectShared& s) {
  s.hist[0][threadIdx.x] = 0u;                    // kSelThreads == 256 bins
}

// Keys of candidates threadIdx.x + 256 r, r < RMAX, of a row of n.
template <int RMAX>
struct SelKeys {
  uint32_t k[RMAX];
  int32_t n;
  __device__ __forceinline__ bool valid(int r) const {
    return int32_t(threadIdx.x) + kSelThreads * r < n;
  }
  // uniform: chunk r holds at least one candidate
  __device__ __forceinline__ bool used(int r) const { return kSelThreads * r < n; }
  __device__ __forceinline__ int32_t index(int r) const {
    return int32_t(threadIdx.x) + kSelThreads * r;
  }
  // Every load is issued before any key is formed (one round trip).  n_load
  // may exceed the final candidate count: set_count() then narrows n (the
  // loads can start before the row's length is known).
  __device__ __forceinline__ void load(const float* __restrict__ score_row, int32_t n_load) {
    n = n_load;
    float v[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) v[r] = valid(r) ? score_row[index(r)] : 0.0f;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) k[r] = used(r) ? float_key(v[r]) : 0u;
  }
  __device__ __forceinline__ void set_count(int32_t n_cand) { n = n_cand; }
};

// Index order of flagged candidates.  Bit r of `flags` flags candidate
// threadIdx.x + 256 r.  sel_order_prepare publishes the per-(chunk, wave)
// flag counts (one barrier) and every wavefront scans all of them itself:
// lane j keeps the number of flagged candidates before (chunk j, this wave).
// sel_order_pos is then a flagged candidate's number of flagged candidates
// with a smaller index.  Called by the whole workgroup (R = chunks in use,
// <= RMAX <= 64; flags has no bit at or above R).  A later writer of s.part
// must be separated from these reads by a barrier.
struct SelOrder {
  int pre;     // lane j: flagged candidates before (chunk j, this wave)
  int total;   // all flagged candidates
};
template <int RMAX>
__device__ __forceinline__ SelOrder sel_order_prepare(uint64_t flags, int R, SelectShared& s) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  // lane r collects chunk r's count by selects, then one write per lane
  int mine = 0;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int c = __popcll(__ballot(int((flags >> r) & 1u)));
    mine = lane == r ? c : mine;
  }
  if (lane < R) s.part[lane * kSelWaves + wave] = mine;
  __syncthreads();
  // lane j holds chunk j's four per-wave counts
  int4 c4 = make_int4(0, 0, 0, 0);
  if (lane < R) c4 = *reinterpret_cast<const int4*>(&s.part[lane * kSelWaves]);
  const int c[kSelWaves] = {c4.x, c4.y, c4.z, c4.w};
  int sum = 0, below = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    sum += c[w];
    below += w < wave ? c[w] : 0;
  }
  const int incl = wave_incl_scan(sum);
  SelOrder o;
  o.pre = incl - sum + below;
  o.total = __builtin_amdgcn_readlane(incl, kWave - 1);
  return o;
}
__device__ __forceinline__ int sel_order_pos(const SelOrder& o, uint64_t flags, int r) {
  const uint64_t bal = __ballot(int((flags >> r) & 1u));
  return __builtin_amdgcn_readlane(o.pre, r) + lanes_below(bal);
}

// 0 < K < n, sel_init(s) called before.  Returns V* in every thread:
// candidate i is among the K best iff order_value(key_i, i) >= V*.
template <int RMAX>
__device__ __forceinline__ uint64_t sel_cut(const SelKeys<RMAX>& kk, int32_t K, SelectShared& s) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int32_t n = kk.n;

  uint32_t a = ~0u, o = 0u;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const bool ok = kk.valid(r);
    a &= ok ? kk.k[r] : ~0u;
    o |= ok ? kk.k[r] : 0u;
  }
  a = wave_and(a);
  o = wave_or(o);
  if (lane == 0) { s.red_and[wave] = a; s.red_or[wave] = o; }
  __syncthreads();
  a = s.red_and[0]; o = s.red_or[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) { a &= s.red_and[w]; o |= s.red_or[w]; }
  const uint32_t diff = a ^ o;
  uint32_t pmask = diff == 0u ? ~0u : (__clz(diff) == 0 ? 0u : ~0u << (32 - __clz(diff)));
  uint32_t prefix = a & pmask;
  int remaining = K;
  int active = n;

  int pass = 0;
  while (active > kWave && pmask != ~0u) {
    const int free_bits = __popc(~pmask);
    const int width = free_bits < 8 ? free_bits : 8;
    const int shift = free_bits - width;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* hist = s.hist[pass % 3];     // zeroed by sel_init or the previous pass
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        const uint32_t k = kk.k[r];
      if (kk.valid(r) && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
    }
    // the next pass's bins: that buffer was last read two passes ago, before
    // every wavefront reached the previous barrier
    s.hist[(pass + 1) % 3][tid] = 0u;
    __syncthreads();
    // every wavefront finds the digit of the remaining-th largest key; lane l
    // owns digits 255-4l .. 252-4l (descending), exactly one lane holds it
    const uint4 h4 = *reinterpret_cast<const uint4*>(&hist[252 - 4 * lane]);
    const int cnt[4] = {int(h4.w), int(h4.z), int(h4.y), int(h4.x)};
    const int sum = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    int above = wave_incl_scan(sum) - sum;
    int hit = -1, hit_above = 0, hit_count = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (above < remaining && remaining <= above + cnt[q]) {
        hit = q;
        hit_above = above;
        hit_count = cnt[q];
      }
      above += cnt[q];
    }
    const int src = __builtin_ctzll(__ballot(hit >= 0));
    const uint32_t digit = uint32_t(255 - 4 * src - __builtin_amdgcn_readlane(hit, src));
    remaining -= __builtin_amdgcn_readlane(hit_above, src);
    active = __builtin_amdgcn_readlane(hit_count, src);
    prefix |= digit << shift;
    pmask |= dmask << shift;
    ++pass;
  }

  if (active <= kWave) {
    // the (at most 64) candidates tied on the prefix: each wavefront packs
    // its own into its slot row (ballot compaction)
    int n_w = 0;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        const uint32_t k = kk.k[r];
      const bool m = kk.valid(r) && (k & pmask) == prefix;
      const uint64_t bal = __ballot(int(m));
      if (m) s.slot[wave][n_w + lanes_below(bal)] = order_value(k, kk.index(r));
      n_w += __popcll(bal);
    }
    if (lane == 0) s.n_gather[wave] = n_w;
    __syncthreads();
    // every wavefront: lane l takes the l-th of the concatenated rows, then
    // the remaining-th largest of the m <= 64 order values by a ballot radix
    // from the highest bit that is not shared, keeping the lanes that can
    // still hold it (values are distinct, so one remains)
    const int m = active;
    uint64_t v = 0u;
    {
      const int4 g4 = *reinterpret_cast<const int4*>(s.n_gather);
      const int gw[kSelWaves] = {g4.x, g4.y, g4.z, g4.w};
      int idx = lane;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) {
        if (idx >= 0 && idx < gw[w]) v = s.slot[w][idx];
        idx -= gw[w];
      }
    }
    uint64_t cand = __ballot(lane < m);
    int r = remaining;
    // Two bits per trip and one uniqueness test per trip (each bit is a
    // chain of dependent scalar instructions, ~150 cycles): a step after the
    // candidate is alone keeps it (r is then 1), and bit -1 has no ones.
    auto step = [&](int bit) {
      const uint64_t ones = bit >= 0 ? __ballot(int((v >> bit) & 1u)) & cand : uint64_t(0);
      const int n1 = __popcll(ones);
      const bool take = n1 >= r;
      r = take ? r : r - n1;
      cand = take ? ones : cand ^ ones;      // ones is a subset of cand
    };
    for (int bit = 63 - __popc(pmask); bit >= 0 && (cand & (cand - 1u)) != 0u; bit -= 2) {
      step(bit);
      step(bit - 1);
    }
    const int win = __builtin_ctzll(cand);
    const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(v >> 32), win);
    const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(v), win);
    return (uint64_t(hi) << 32) | lo;
  }
  // every bit fixed and more than 64 keys equal the K-th key: its occurrence
  // number `remaining` in index order is the cut
  uint64_t eq = 0u;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (kk.valid(r) && kk.k[r] == prefix) eq |= uint64_t(1) << r;
  }
  const int R = (n + kSelThreads - 1) / kSelThreads;
  const SelOrder ord = sel_order_prepare<RMAX>(eq, R, s);
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (r < R) {
      const int pos = sel_order_pos(ord, eq, r);
      if (((eq >> r) & 1u) && pos == remaining - 1) s.cut = order_value(prefix, kk.index(r));
    }
  }
  __syncthreads();                          // also ends the reads of s.part
  return s.cut;
}

// Bit r set iff candidate threadIdx.x + 256 r is among the K best.
template <int RMAX>
__device__ __forceinline__ uint64_t sel_taken_mask(const SelKeys<RMAX>& kk, uint64_t cut) {
  uint64_t m = 0u;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const bool t = kk.valid(r) && order_value(kk.k[r], kk.index(r)) >= cut;
    m |= uint64_t(t) << r;
  }
  return m;
}

}  // namespace skv
