// Block-wide radix selection of the k-th largest 64-bit key in shared memory.
#pragma once

#include "common.h"

namespace dtv {

constexpr int kRadixBits = 11;                  // digit width of a pass
constexpr int kRadixBins = 1 << kRadixBits;
constexpr int kMaxBlockWaves = 16;             // 1024-thread workgroups

struct RadixSmem {
  int hist[kRadixBins];   // counts of the pass; zero between passes
  int digit, rem, cnt;
  int scan[kMaxBlockWaves];
  unsigned long long red[kMaxBlockWaves];
  unsigned long long red2[kMaxBlockWaves];
};

// Result of radix_topk_cut: the keys k with (k & mask) > prefix are all among the top k;
// of those with (k & mask) == prefix, all are when all_in, else (mask is then all ones and
// prefix the k-th largest key) the first `rem` in the caller's tie order.
struct RadixCut {
  unsigned long long prefix, mask;
  int rem;
  bool all_in;
  bool group;   // stopped at a small group: its `rem` best by (full key desc, tie order) are in
};

// The cut of the top k (k >= 1) of the nonzero keys key[0 .. n) (zero marks an absent
// entry; at least k keys present), by most-significant-digit-first radix selection with
// 11-bit digits that starts at the highest bit where the present keys differ: each pass
// histograms the next digit of the keys sharing the prefix so far (2048 bins, so keys
// packed in a narrow range still spread over many bins and the shared-memory atomics
// rarely collide) and extends the prefix by the digit at which the count from the top
// reaches the number still to take. It stops as soon as the group of keys sharing the
// prefix lies entirely within the top k (then no lower digit matters), or when the whole
// key is resolved. A pass clears the bins it has read, ready for the next one.
// With max_passes, the selection stops after that many passes; the cut is then a prefix
// whose group holds the k-th largest key, so prefix (lower bits zero) still bounds that key
// from below. With group_max > 0 it also stops once the group that holds the k-th largest
// key has at most group_max members and is not taken whole (group set): the caller then
// ranks those members by full key (and its tie order) itself, which costs less than the
// remaining passes. With min_unresolved, the selection also stops once at most that many
// low bits are left unresolved (a bound: the prefix then fixes the key to within 2^that).
// Every thread of the block (NT threads) must call it; all get the same result.
template <int NT = kBlock>
__device__ __forceinline__ RadixCut radix_topk_cut(const unsigned long long* key, int n, int k, RadixSmem& rs,
                                                   int max_passes = 64, int group_max = 0,
                                                   int min_unresolved = 0) {
  static_assert(kRadixBins % NT == 0 && NT / 64 <= kMaxBlockWaves, "whole bins per thread");
  constexpr int kRadixPer = kRadixBins / NT;  // bins owned by a thread in the scan
  unsigned long long kmax = 0ull, kmin = ~0ull;
  for (int e = threadIdx.x; e < n; e += NT) {
    const unsigned long long x = key[e];
    if (x != 0ull) {
      kmax = x > kmax ? x : kmax;
      kmin = x < kmin ? x : kmin;
    }
  }
  kmax = wave_max(kmax);
  kmin = wave_min(kmin);
  if ((threadIdx.x & 63) == 0) {
    rs.red[threadIdx.x >> 6] = kmax;
    rs.red2[threadIdx.x >> 6] = kmin;
  }
#pragma unroll
  for (int q = 0; q < kRadixPer; ++q) rs.hist[threadIdx.x * kRadixPer + q] = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NT / 64; ++q) {
    kmax = rs.red[q] > kmax ? rs.red[q] : kmax;
    kmin = rs.red2[q] < kmin ? rs.red2[q] : kmin;
  }
  const unsigned long long diff = kmax ^ kmin;
  // bits above the highest differing one are shared by every present key
  int unresolved = diff ? 64 - __clzll(static_cast<long long>(diff)) : kRadixBits;
  RadixCut cut;
  cut.mask = unresolved >= 64 ? 0ull : (~0ull << unresolved);
  cut.prefix = kmax & cut.mask;
  cut.rem = k;
  cut.all_in = false;
  cut.group = false;
  const int t = threadIdx.x;
  for (int pass = 0; unresolved > min_unresolved && pass < max_passes; ++pass) {
    const int w = unresolved < kRadixBits ? unresolved : kRadixBits;
    const int shift = unresolved - w;
    const unsigned dmask = (1u << w) - 1u;
    for (int e = t; e < n; e += NT) {
      const unsigned long long x = key[e];
      if (x != 0ull && (x & cut.mask) == cut.prefix) atomicAdd(&rs.hist[(x >> shift) & dmask], 1);
    }
    __syncthreads();
    // thread t owns the kRadixPer digits just below kRadixBins - kRadixPer t, largest first;
    // it reads and clears them, and the thread whose range takes the count from the top
    // past rem records the digit
    int c[kRadixPer];
    int mine = 0;
#pragma unroll
    for (int q = 0; q < kRadixPer; ++q) {
      const int d = kRadixBins - 1 - kRadixPer * t - q;
      c[q] = rs.hist[d];
      rs.hist[d] = 0;
      mine += c[q];
    }
    int tot = 0;
    const int above = block_exclusive_scan<int, NT / 64>(mine, rs.scan, &tot);
    if (above < cut.rem && cut.rem <= above + mine) {
      int acc = above;
#pragma unroll
      for (int q = 0; q < kRadixPer; ++q) {
        if (acc + c[q] >= cut.rem) {
          rs.digit = kRadixBins - 1 - kRadixPer * t - q;
          rs.rem = cut.rem - acc;
          rs.cnt = c[q];
          break;
        }
        acc += c[q];
      }
    }
    __syncthreads();
    cut.prefix |= static_cast<unsigned long long>(rs.digit) << shift;
    cut.mask |= static_cast<unsigned long long>(dmask) << shift;
    cut.rem = rs.rem;
    const int cnt = rs.cnt;
    unresolved = shift;
    // (the next pass writes the result only after its own barriers, which every thread
    // reaches after these reads)
    if (cnt == cut.rem) {   // the whole group is taken
      cut.all_in = true;
      break;
    }
    if (cnt <= group_max && unresolved > 0) {   // a small group: ranked by the caller
      cut.group = true;
      break;
    }
  }
  return cut;
}

}  // namespace dtv
