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
// of them; "chunk" r is candidates 256 r .. 256 r + 255), loaded in one
// round trip.  V* is found by
//   * fixing the leading key bits that every candidate shares (a DPP AND/OR
//     reduction): the bounds of one row share sign and most exponent bits,
//     and a histogram of those bits would pile every key into one or two bins;
//   * most-significant-digit radix passes fixing the next bits of the K-th
//     key: an LDS histogram filled straight from registers (10-bit digits in
//     the first pass, which usually leaves a few dozen keys, 8-bit digits
//     after it), then every wavefront scans the bins itself with a DPP prefix
//     sum, so a pass costs one barrier; until at most 64 candidates share the
//     K-th key's prefix;
//   * gathering those (a workgroup prefix sum of per-thread counts gives each
//     its slot) and narrowing them in every wavefront with ballots, one bit
//     of the order value at a time, to the one of the right rank;
//   * or, if more than 64 keys equal the K-th key exactly, taking its
//     occurrence of the right rank in index order.
// The histogram updates and gather stores carry no branch: a key off the
// prefix counts into its lane's own discard word (stores: its thread's
// discard slot), so the chunks' LDS operations issue back to back instead of
// one exec-mask change each.
//
// Index order of flagged candidates (ascending output positions): for a few
// chunks (sel_order_prepare), per-(chunk, wavefront) ballot counts,
// published once and scanned by every wavefront, and the set ballot bits
// below each lane; for many chunks (sel_rank_prepare), the per-chunk ballots
// form the flag bitmap in index order in LDS, thread t then owns candidates
// RMAX t .. RMAX t + RMAX - 1 of that order, and a workgroup prefix sum of
// its flag counts gives the position of its first one.
#pragma once

#include "device_common.h"

namespace skv {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelMaxChunks = 64;                 // candidates <= 64 * 256 = 16384
constexpr int kSelWideBits = 10;                  // first radix pass
constexpr int kSelWide = 1 << kSelWideBits;

struct __attribute__((aligned(16))) SelectShared {
  uint32_t wide[kSelWide];                        // first pass's bins
  uint32_t narrow[3][256];                        // later passes' bins, rotating
  uint32_t discard[kWave];                        // one count word per lane
  uint64_t slot[kWave];                           // order values tied on the prefix
  union {
    uint64_t bits[kSelMaxChunks * kSelWaves];     // flags in index order
    uint64_t spare[kSelThreads];                  // the gather's discard slots
  } u;
  int32_t part[kSelMaxChunks * kSelWaves];        // (chunk, wave) counts, chunk-major
  uint32_t red_and[kSelWaves], red_or[kSelWaves];
  alignas(16) int32_t wtot[2][kSelWaves];         // wavefront totals of two scans
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
  static_assert(kSelWide == 4 * kSelThreads, "one 16-byte store per thread");
  reinterpret_cast<uint4*>(s.wide)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
}

// Exclusive prefix sum of x over the workgroup's threads (in thread order) and
// its total, through wavefront totals buffer `buf`.  Whole workgroup; one
// barrier.  Two calls on one buffer must be separated by another barrier.
__device__ __forceinline__ int sel_wg_scan(int x, int& total, SelectShared& s, int buf) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int incl = wave_incl_scan(x);
  if (lane == kWave - 1) s.wtot[buf][wave] = incl;
  __syncthreads();
  const int4 t4 = *reinterpret_cast<const int4*>(s.wtot[buf]);
  const int w[kSelWaves] = {t4.x, t4.y, t4.z, t4.w};
  int before = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) before += i < wave ? w[i] : 0;
  total = w[0] + w[1] + w[2] + w[3];
  return before + incl - x;
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

// Index order of flagged candidates, the form for a few chunks (RMAX <= 4:
// no barrier beyond one, no bitmap).  Bit r of `flags` flags candidate
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

// Index order of flagged candidates, the form for many chunks (RMAX >= 16).
// Bit r of `flags` flags candidate threadIdx.x + 256 r (no bit for an
// invalid candidate).  Thread t gets
// `bits`, the flags of candidates RMAX t .. RMAX t + RMAX - 1 (bit j for
// candidate RMAX t + j), `base`, the number of flagged candidates before
// RMAX t, and `total`.  Whole workgroup, two barriers; s.u.bits is read
// after the first, so a later writer of it needs another barrier.
struct SelRank {
  uint64_t bits;
  int base;
  int total;
};
template <int RMAX>
__device__ __forceinline__ SelRank sel_rank_prepare(uint64_t flags, SelectShared& s) {
  static_assert(RMAX <= kSelMaxChunks && (RMAX & (RMAX - 1)) == 0, "RMAX: a power of two <= 64");
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  // lane r keeps chunk r's ballot: candidates 256 r + 64 wave + (0 .. 63),
  // which is 64-bit word 4 r + wave of the bitmap in index order
  uint64_t mine = 0u;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const uint64_t bal = __ballot(int((flags >> r) & 1u));
    mine = lane == r ? bal : mine;
  }
  if (lane < RMAX) s.u.bits[kSelWaves * lane + wave] = mine;
  __syncthreads();
  SelRank rk;
  if constexpr (RMAX == 64) {
    rk.bits = s.u.bits[tid];
  } else {
    const int first = RMAX * tid;
    rk.bits = (s.u.bits[first / 64] >> (first % 64)) & ((uint64_t(1) << RMAX) - 1u);
  }
  rk.base = sel_wg_scan(__popcll(rk.bits), rk.total, s, 1);
  return rk;
}

// One radix pass's digit: the histogram `hist` holds 64 P bins (P per lane,
// lane l owning digits 64 P - 1 - P l down to 64 P - P l - P, descending);
// the digit of the remaining-th largest key, the keys above its bin and in it.
template <int P>
__device__ __forceinline__ void sel_find_digit(const uint32_t* hist, int remaining,
                                               uint32_t& digit, int& above_out, int& count_out) {
  const int lane = threadIdx.x % kWave;
  int cnt[P];
#pragma unroll
  for (int i = 0; i < P / 4; ++i) {
    const uint4 h4 = *reinterpret_cast<const uint4*>(&hist[64 * P - P * lane - P + 4 * i]);
    // ascending bins in memory, descending digits in cnt
    cnt[P - 1 - 4 * i] = int(h4.x);
    cnt[P - 2 - 4 * i] = int(h4.y);
    cnt[P - 3 - 4 * i] = int(h4.z);
    cnt[P - 4 - 4 * i] = int(h4.w);
  }
  int sum = 0;
#pragma unroll
  for (int q = 0; q < P; ++q) sum += cnt[q];
  int above = wave_incl_scan(sum) - sum;
  int hit = -1, hit_above = 0, hit_count = 0;
#pragma unroll
  for (int q = 0; q < P; ++q) {
    const bool h = above < remaining && remaining <= above + cnt[q];
    hit = h ? q : hit;
    hit_above = h ? above : hit_above;
    hit_count = h ? cnt[q] : hit_count;
    above += cnt[q];
  }
  const int src = __builtin_ctzll(__ballot(hit >= 0));
  digit = uint32_t(64 * P - 1 - P * src - __builtin_amdgcn_readlane(hit, src));
  above_out = __builtin_amdgcn_readlane(hit_above, src);
  count_out = __builtin_amdgcn_readlane(hit_count, src);
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
    const bool wide = pass == 0 && free_bits >= kSelWideBits;
    const int width = wide ? kSelWideBits : (free_bits < 8 ? free_bits : 8);
    const int shift = free_bits - width;
    const uint32_t dmask = (1u << width) - 1u;
    // the first pass fills s.wide (zeroed by sel_init); pass p >= 1 fills
    // narrow[(p - 1) % 3], zeroed in pass p - 1, whose reads of it (two
    // passes back) ended before that pass's barrier
    uint32_t* hist = pass == 0 ? s.wide : s.narrow[(pass - 1) % 3];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      const uint32_t k = kk.k[r];
      const bool m = kk.valid(r) && (k & pmask) == prefix;
      atomicAdd(m ? &hist[(k >> shift) & dmask] : &s.discard[lane], 1u);
    }
    s.narrow[pass % 3][tid] = 0u;                 // kSelThreads == 256 bins
    __syncthreads();
    uint32_t digit;
    int d_above, d_count;
    if (wide) sel_find_digit<kSelWide / kWave>(hist, remaining, digit, d_above, d_count);
    else sel_find_digit<4>(hist, remaining, digit, d_above, d_count);
    remaining -= d_above;
    active = d_count;
    prefix |= digit << shift;
    pmask |= dmask << shift;
    ++pass;
  }

  if (active <= kWave) {
    // the (at most 64) candidates tied on the prefix, packed in thread order
    int c = 0;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) c += (kk.valid(r) && (kk.k[r] & pmask) == prefix) ? 1 : 0;
    int m_tot;
    int pos = sel_wg_scan(c, m_tot, s, 0);
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      const uint32_t k = kk.k[r];
      const bool m = kk.valid(r) && (k & pmask) == prefix;
      *(m ? &s.slot[pos] : &s.u.spare[tid]) = order_value(k, kk.index(r));
      pos += m ? 1 : 0;
    }
    __syncthreads();
    // every wavefront: lane l takes the l-th, then the remaining-th largest
    // of the m <= 64 order values by a ballot radix from the highest bit
    // that is not shared, keeping the lanes that can still hold it (values
    // are distinct, so one remains)
    const int m = active;
    const uint64_t v = lane < m ? s.slot[lane] : uint64_t(0);
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
  const SelRank rk = sel_rank_prepare<RMAX>(eq, s);
  const int want = remaining - 1 - rk.base;       // rank of the cut among this thread's flags
  if (want >= 0 && want < __popcll(rk.bits)) {
    uint64_t b = rk.bits;
    for (int i = 0; i < want; ++i) b &= b - 1u;
    s.cut = order_value(prefix, RMAX * int32_t(threadIdx.x) + __builtin_ctzll(b));
  }
  __syncthreads();
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
