// Block-wide radix selection of the k-th largest 64-bit key in shared memory.
#pragma once

#include "common.h"

namespace dtv {

struct RadixSmem {
  int hist[256];
  int digit, rem, cnt;
  unsigned long long red[kWaves];
};

// Result of radix_topk_cut: the keys k with (k & mask) > prefix are all among the top k;
// of those with (k & mask) == prefix, all are when all_in, else (mask is then all ones and
// prefix the k-th largest key) the first `rem` in the caller's tie order.
struct RadixCut {
  unsigned long long prefix, mask;
  int rem;
  bool all_in;
};

// The cut of the top k (k >= 1) of the nonzero keys key[0 .. n) (zero marks an absent
// entry; at least k keys present), by most-significant-byte-first radix selection that
// starts at the highest byte where the present keys differ: each pass histograms the next
// byte of the keys sharing the prefix so far and extends the prefix by the byte at which
// the count from the top reaches the number still to take. It stops as soon as the group
// of keys sharing the prefix lies entirely within the top k (then no lower byte matters).
// Every thread of the block must call it; all get the same result.
__device__ __forceinline__ RadixCut radix_topk_cut(const unsigned long long* key, int n, int k, RadixSmem& rs) {
  static_assert(kBlock == 256, "one histogram bin per thread");
  unsigned long long kmax = 0ull, kmin = ~0ull;
  for (int e = threadIdx.x; e < n; e += kBlock) {
    const unsigned long long x = key[e];
    if (x != 0ull) {
      kmax = x > kmax ? x : kmax;
      kmin = x < kmin ? x : kmin;
    }
  }
  kmax = block_max(kmax, rs.red);
  kmin = block_min(kmin, rs.red);
  const unsigned long long diff = kmax ^ kmin;
  int top = 0;
  for (int b = 7; b >= 0; --b)
    if ((diff >> (8 * b)) & 0xFFull) {
      top = b;
      break;
    }
  RadixCut cut;
  cut.mask = top == 7 ? 0ull : (~0ull << (8 * (top + 1)));
  cut.prefix = kmax & cut.mask;
  cut.rem = k;
  cut.all_in = false;
  for (int shift = 8 * top; shift >= 0; shift -= 8) {
    rs.hist[threadIdx.x] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += kBlock) {
      const unsigned long long x = key[e];
      if (x != 0ull && (x & cut.mask) == cut.prefix) atomicAdd(&rs.hist[(x >> shift) & 255u], 1);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l owns digits 255-4l .. 252-4l; find the digit whose cumulative count from
      // the top first reaches rem
      const int l = threadIdx.x;
      const int c0 = rs.hist[255 - 4 * l], c1 = rs.hist[254 - 4 * l];
      const int c2 = rs.hist[253 - 4 * l], c3 = rs.hist[252 - 4 * l];
      const int mine = c0 + c1 + c2 + c3;
      int inc = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o, 64);
        if (l >= o) inc += y;
      }
      const int above = inc - mine;
      if (above < cut.rem && cut.rem <= inc) {
        int acc = above, d = 255 - 4 * l;
        const int cs[4] = {c0, c1, c2, c3};
        for (int q = 0; q < 4; ++q) {
          if (acc + cs[q] >= cut.rem) {
            d = 255 - 4 * l - q;
            break;
          }
          acc += cs[q];
        }
        rs.digit = d;
        rs.rem = cut.rem - acc;
        rs.cnt = rs.hist[d];
      }
    }
    __syncthreads();
    cut.prefix |= static_cast<unsigned long long>(rs.digit) << shift;
    cut.mask |= 0xFFull << shift;
    cut.rem = rs.rem;
    const int cnt = rs.cnt;
    __syncthreads();
    if (cnt == cut.rem) {   // the whole group is taken
      cut.all_in = true;
      break;
    }
  }
  return cut;
}

}  // namespace dtv
