// Vocab-wide statistics of bf16 logit rows on gfx950: log-sum-exp and top-K (value desc,
// index asc) of every row, in parts of 32768 values, one 1024-thread workgroup (16 waves)
// per part. The parts of a row are merged by whichever workgroup finishes the row's last
// part; a row of at most 32768 values is a single part and needs no merge.
//
// Sums of exponentials. For |x| < 256 the float64 exp(x) is at most 1.5e111, so
// sum_x exp(x) over any row is finite and needs no shift by the maximum. Every bf16 value
// with 2^-16 <= |x| < 2^8 has its exp in a compile-time table (bf16_maps.h), copied into
// shared memory by the workgroup's first loads. Two values at a time (one 32-bit word),
// packed 16-bit integer operations turn the raw bits into table addresses, so that a value
// costs about two VALU instructions, one table read and one float64 add; values past the
// row end read the table's 0.0 pair. A wave holding any value outside that range (tiny,
// huge, infinite, NaN) sums exp(x - wave max) directly instead (fexp.h). A wave's partial is
// (shift, sum) with the exponentials summing to sum * exp(shift); table waves have shift 0.
//
// Order. Values are compared by 16-bit keys (bf16_maps.h), also computed two at a time;
// padding has key 0, below every value. The top-K of a part lie among the values >= tau, a
// bound with at least K values at or above it: for K <= 16 the K-th largest of the part's 64
// row maxima (a row is 16 lanes, 512 values; one wave bisects them), which lets through
// barely more than K values; for larger K the largest over the waves of each wave's K-th
// largest lane maximum. Only lanes whose maximum reaches tau look at their values; they
// write them into a region of shared memory of their wave (a prefix sum of the lanes'
// counts, no atomics), and wave 0 ranks them in registers by (key desc, index asc). A wave
// whose region would overflow (ties at tau) sends the part to an exact fallback: every wave
// bisects its own K-th largest key, takes ties in index order, and all candidates are
// ranked by counting.
#pragma once

#include "bf16_maps.h"
#include "common.h"
#include "fexp.h"
#include "rowstats.h"

namespace dtv {

constexpr int kPartThreads = 1024;
constexpr int kPartWaves = kPartThreads / 64;
constexpr int kPartLoads = 4;                                 // 16-byte loads per thread
constexpr int kPartWords = 4 * kPartLoads;                    // bf16 pairs per thread
constexpr int kPartValues = 2 * kPartWords * kPartThreads;    // 32768
constexpr int kPartVecs = kPartValues / 8;                    // 16-byte vectors per part
constexpr int kPartSlots = 64;                                // candidate slots per wave
constexpr int kPartMergeCap = kPartWaves * kPartSlots;        // list entries a row merge holds
constexpr int kPartMaxParts = 64;
constexpr int kPartRowBoundK = 16;   // K up to this: threshold from the part's 64 row maxima

__host__ __device__ constexpr int parts_of(int V) { return (V + kPartValues - 1) / kPartValues; }

// One part's share of a row, kept in the row's chunk-statistics slots.
struct PartStat {
  float shift;   // the part's exponentials sum to sum * exp(shift)
  int cnt;       // entries in the part's list
  double sum;
};
static_assert(sizeof(PartStat) <= sizeof(ChunkStat), "a part's record fits a chunk slot");

__constant__ const ExpBf16Table kExpBf16Dev = kExpBf16Tab;
__constant__ const Exp2Table kExp2Dev = kExp2Tab;

struct alignas(16) PartSmem {
  double tab[kExpBf16Entries];   // exp of the bf16 values in range, then a 1.0 pair and a 0.0 pair
  double e64[64];                // 2^(j/64) for fexp.h
  unsigned long long slot[kPartWaves][kPartSlots];   // each wave's candidates; the merge's lists
  unsigned long long cand[64];     // the candidates packed, for wave 0's rank
  double wsum[kPartWaves];
  float wshift[kPartWaves];
  uint32_t wtau[kPartWaves];
  uint32_t rmax[4 * kPartWaves];   // row maxima (rows of 16 lanes)
  uint32_t cmk[kPartWaves][2];     // each wave's maximum keys of the part's 8192-value chunks, two per word
  uint32_t tau;                    // the part's bound (row maxima)
  int wcnt[kPartWaves];            // candidates of each wave (beyond kPartSlots: overflow)
  int ncand2;                      // entries of the exact fallback (packed from slot[0][0])
  int pcnt[kPartMaxParts];
  float pshift[kPartMaxParts];
  double psum[kPartMaxParts];
  int flag;
};
static_assert((sizeof(double) * kExpBf16Entries) % 16 == 0, "the table is copied in 16-byte pieces");

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2, w); }
__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Order keys of the two bf16 values of w (bf16_order_key of each half).
__device__ __forceinline__ uint32_t bf16x2_keys(uint32_t w) {
  const u16x2 mag = as_u16x2(w & 0x7FFF7FFFu);
  const u16x2 neg = __builtin_bit_cast(u16x2, __builtin_bit_cast(s16x2, as_u16x2(w)) >> (short)15);
  return as_u32(((mag ^ neg) - neg) + (unsigned short)0x8000);
}

// Byte offsets into the table of the two values of w (low half in bits 0..15); out-of-range
// magnitudes go to the 1.0 pair. `acc` collects, per half, the largest magnitude offset
// seen (wrapped below the range): a half >= kExpBf16Mags means a value outside the table.
__device__ __forceinline__ uint32_t bf16x2_tab_offsets(uint32_t w, uint32_t& acc) {
  const u16x2 rel = as_u16x2(w & 0x7FFF7FFFu) - (unsigned short)kExpBf16Lo;
  acc = as_u32(__builtin_elementwise_max(as_u16x2(acc), rel));
  const u16x2 rc = __builtin_elementwise_min(rel, (u16x2)(unsigned short)kExpBf16Mags);
  return (as_u32(rc) << 4) | ((w >> 12) & 0x00080008u);
}

__device__ __forceinline__ float bf16_key_value(uint32_t k) { return __uint_as_float(bf16_key_bits(k) << 16); }
__device__ __forceinline__ uint32_t f32_bf16_key(float v) { return bf16_order_key(__float_as_uint(v) >> 16); }

__device__ __forceinline__ unsigned long long part_sort_key(uint32_t key, int idx) {
  return (static_cast<unsigned long long>(key) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(idx));
}
__device__ __forceinline__ int part_key_index(unsigned long long k) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull));
}
__device__ __forceinline__ float part_key_value(unsigned long long k) {
  return bf16_key_value(static_cast<uint32_t>(k >> 32));
}

// The half (0: low, 1: high) of word j of a thread's part data, and its element index: word
// j = 4 i + q holds values 2q and 2q + 1 of the thread's i-th 16-byte vector.
__device__ __forceinline__ uint32_t key_half(uint32_t k2, int h) { return h ? (k2 >> 16) : (k2 & 0xFFFFu); }
__device__ __forceinline__ int part_index(int vbase, int j, int h) {
  return (vbase + (j >> 2) * kPartThreads + static_cast<int>(threadIdx.x)) * 8 + (j & 3) * 2 + h;
}

// Copies the tables into shared memory with direct loads (no registers); the caller waits
// for its loads (drain) and passes a barrier before reading them.
__device__ __forceinline__ void part_tables_issue(PartSmem& sm) {
  typedef __attribute__((address_space(3))) void lds_void_t;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int kPieces = static_cast<int>(sizeof(double) * kExpBf16Entries / 16);
  const char* src = reinterpret_cast<const char*>(kExpBf16Dev.v);
  char* dst = reinterpret_cast<char*>(sm.tab);
  for (int p0 = 64 * w; p0 < kPieces; p0 += kPartThreads) {
    if (p0 + lane < kPieces)
      __builtin_amdgcn_global_load_lds(src + 16 * (p0 + lane), (lds_void_t*)(dst + 16 * p0), 16, 0, 0);
  }
  if (w == kPartWaves - 1 && lane < 32)
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(kExp2Dev.v) + 16 * lane,
                                     (lds_void_t*)(reinterpret_cast<char*>(sm.e64)), 16, 0, 0);
}

// The raw words of one part of a row: word j = 4 i + q of a thread is word q of the
// thread's i-th vector (vector vbase + i * 1024 + thread). Vectors past the row's last full
// vector are loaded from that vector (valid memory) and are masked by the callers. Rows that
// are not 16-byte aligned, or hold no full vector, are loaded value by value.
struct PartData {
  uint32_t w[kPartWords];
};

__device__ __forceinline__ void part_load(const uint16_t* row, int V, int vbase, bool vec, PartData& d) {
  const int vfull = V / 8;
  if (vec) {
#pragma unroll
    for (int i = 0; i < kPartLoads; ++i) {
      const int vi = min(vbase + i * kPartThreads + static_cast<int>(threadIdx.x), vfull - 1);
      const uint4 q = *reinterpret_cast<const uint4*>(row + static_cast<size_t>(vi) * 8);
      d.w[4 * i] = q.x;
      d.w[4 * i + 1] = q.y;
      d.w[4 * i + 2] = q.z;
      d.w[4 * i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPartWords; ++j) {
      const int i0 = part_index(vbase, j, 0);
      const uint32_t lo = i0 < V ? row[i0] : 0u;
      const uint32_t hi = i0 + 1 < V ? row[i0 + 1] : 0u;
      d.w[j] = lo | (hi << 16);
    }
  }
}

// Per-wave reduction of a part. Writes the wave's keys (padding 0), lane maximum, and its
// (shift, sum) partial. `clean`: every value of the wave is in the row (vector path).
// In a wave that is not clean, the values of the vector that straddles the row end are
// re-read one by one into d, so that d holds every in-row value.
// Also the lane's key maximum over each group of 4 words (g, both halves) and overall.
__device__ __forceinline__ void part_keys(PartData& d, bool clean, const uint16_t* row, int V, int vbase,
                                          bool vec, uint32_t (&k2)[kPartWords], uint32_t (&g)[kPartLoads],
                                          uint32_t& lmax) {
  const int vfull = V / 8;
  if (clean) {
#pragma unroll
    for (int j = 0; j < kPartWords; ++j) k2[j] = bf16x2_keys(d.w[j]);
  } else {
#pragma unroll
    for (int j = 0; j < kPartWords; ++j) {
      uint32_t kk = 0u, ww = 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ix = part_index(vbase, j, h);
        const int vi = ix >> 3;
        uint32_t b = (d.w[j] >> (16 * h)) & 0xFFFFu;
        if (vec && vi >= vfull && ix < V) b = row[ix];   // the vector that straddles the row end
        const uint32_t key = ix < V ? bf16_order_key(b) : 0u;
        kk |= key << (16 * h);
        ww |= b << (16 * h);
      }
      k2[j] = kk;
      d.w[j] = ww;
    }
  }
  const auto pmax = [](uint32_t a, uint32_t b) { return as_u32(__builtin_elementwise_max(as_u16x2(a), as_u16x2(b))); };
#pragma unroll
  for (int i = 0; i < kPartLoads; ++i)
    g[i] = pmax(pmax(k2[4 * i], k2[4 * i + 1]), pmax(k2[4 * i + 2], k2[4 * i + 3]));
  const uint32_t m2 = pmax(pmax(g[0], g[1]), pmax(g[2], g[3]));
  lmax = max(m2 & 0xFFFFu, m2 >> 16);
}

// Table offsets of the two values of word j of a wave that holds padding: a value past the
// row end reads the 0.0 pair and does not count as out of range.
__device__ __forceinline__ uint32_t bf16x2_tab_offsets_padded(uint32_t w, int ix0, int V, uint32_t& acc) {
  constexpr uint32_t kZero = 16u * (kExpBf16Mags + 1u);   // byte offset of the 0.0 pair
  const bool p0 = ix0 >= V, p1 = ix0 + 1 >= V;
  w = p0 ? (w & 0xFFFF0000u) | kExpBf16Lo : w;
  w = p1 ? (w & 0x0000FFFFu) | (kExpBf16Lo << 16) : w;
  uint32_t a = bf16x2_tab_offsets(w, acc);
  a = p0 ? (a & 0xFFFF0000u) | kZero : a;
  a = p1 ? (a & 0x0000FFFFu) | (kZero << 16) : a;
  return a;
}

// sum_x exp(x) of the wave's values from the table, a value outside it counted as 1.0;
// false if there is any (wave-uniform). PAD: the wave holds values past the row end, which
// add nothing.
template <bool PAD>
__device__ __forceinline__ bool part_table_sum(const PartData& d, const PartSmem& sm, int vbase, int V, double& sum) {
  const char* tb = reinterpret_cast<const char*>(sm.tab);
  uint32_t acc = 0u;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
#pragma unroll
  for (int j = 0; j < kPartWords; j += 2) {
    const uint32_t a0 = PAD ? bf16x2_tab_offsets_padded(d.w[j], part_index(vbase, j, 0), V, acc)
                            : bf16x2_tab_offsets(d.w[j], acc);
    const uint32_t a1 = PAD ? bf16x2_tab_offsets_padded(d.w[j + 1], part_index(vbase, j + 1, 0), V, acc)
                            : bf16x2_tab_offsets(d.w[j + 1], acc);
    s0 += *reinterpret_cast<const double*>(tb + (a0 & 0xFFFFu));
    s1 += *reinterpret_cast<const double*>(tb + (a0 >> 16));
    s2 += *reinterpret_cast<const double*>(tb + (a1 & 0xFFFFu));
    s3 += *reinterpret_cast<const double*>(tb + (a1 >> 16));
  }
  sum = (s0 + s1) + (s2 + s3);
  const bool out = (acc & 0xFFFFu) >= kExpBf16Mags || (acc >> 16) >= kExpBf16Mags;
  return __ballot(out) == 0ull;
}

// The correction of a table sum for the values outside the table (each was counted as
// 1.0): sum over them of exp(x) - 1, the exp as in fexp.h (x < 256 here: the wave holds no
// larger value). Values past the row end (PAD) are skipped. Per lane; waves with any such
// value only.
template <bool PAD>
__device__ __forceinline__ double part_table_fixup(const PartData& d, int vbase, int V, const double* e64) {
  double c = 0.0;
#pragma unroll
  for (int j = 0; j < kPartWords; ++j) {
    const u16x2 rel = as_u16x2(d.w[j] & 0x7FFF7FFFu) - (unsigned short)kExpBf16Lo;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bool out = rel[h] >= kExpBf16Mags;
      if (PAD) out = out && part_index(vbase, j, h) < V;
      if (__ballot(out) == 0ull) continue;
      if (out) {
        const float x = __uint_as_float(((d.w[j] >> (16 * h)) & 0xFFFFu) << 16);
        c += exp_nonpos(static_cast<double>(x), e64) - 1.0;
      }
    }
  }
  return c;
}

// sum_x exp(x - m) of the wave's values (padding: key 0, no term), m the wave's largest
// value. A maximum of +inf or NaN makes the sum, like the log-sum-exp itself, non-finite.
__device__ __forceinline__ double part_shifted_sum(const uint32_t (&k2)[kPartWords], float m, const double* e64) {
  float x[2 * kPartWords];
#pragma unroll
  for (int j = 0; j < kPartWords; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t k = key_half(k2[j], h);
      x[2 * j + h] = k ? bf16_key_value(k) : -INFINITY;
    }
  }
  return exp_nonpos_sum<2 * kPartWords>(x, static_cast<double>(m), e64);
}

// The wave's (shift, sum) partial, in every lane: the table sum (with the correction for
// values outside the table) when every value is below 256, else the sum shifted by the wave
// maximum (key km). Wave-uniform control flow.
__device__ __forceinline__ void part_wave_exp(const PartData& d, const uint32_t (&k2)[kPartWords], uint32_t km,
                                              bool clean, int vbase, int V, const PartSmem& sm, double& sum,
                                              float& shift) {
  sum = 0.0;
  shift = 0.0f;
  const bool huge = km >= bf16_order_key(0x4380u);   // some value >= 256 (or +inf, NaN)
  if (!huge) {   // the table, and for a value outside it (|x| < 2^-16 or x <= -256) exp(x) - 1
    if (clean) {
      if (!part_table_sum<false>(d, sm, vbase, V, sum)) sum += part_table_fixup<false>(d, vbase, V, sm.e64);
    } else {
      if (!part_table_sum<true>(d, sm, vbase, V, sum)) sum += part_table_fixup<true>(d, vbase, V, sm.e64);
    }
  } else if (km != 0u) {
    const float m = bf16_key_value(km);
    if (m != -INFINITY) {
      shift = m;
      sum = part_shifted_sum(k2, m, sm.e64);
    }
  }
  sum = wave_sum(sum);
}

// Number of the wave's values with key >= thr (wave-uniform).
__device__ __forceinline__ int part_count_ge(const uint32_t (&k2)[kPartWords], uint32_t thr) {
  int n = 0;
#pragma unroll
  for (int j = 0; j < kPartWords; ++j) {
    n += __popcll(__ballot((k2[j] & 0xFFFFu) >= thr));
    n += __popcll(__ballot((k2[j] >> 16) >= thr));
  }
  return n;
}

// The wave's own top-min(K, valid) by bisection of the key space, ties at the threshold in
// index order, appended to out (a range reserved with one atomic on *ctr). K <= 64.
__device__ __forceinline__ void part_wave_exact(const uint32_t (&k2)[kPartWords], uint32_t km, int K, int vbase,
                                                unsigned long long* out, int* ctr) {
  const int nv = part_count_ge(k2, 1u);
  const int kw = K < nv ? K : nv;
  if (kw <= 0) return;
  int taken = 0;
  if ((threadIdx.x & 63) == 0) taken = atomicAdd(ctr, kw);
  taken = __builtin_amdgcn_readfirstlane(taken);
  uint32_t lo = 1u, hi = km + 1u;   // count(>= lo) >= kw > count(>= hi)
  while (hi - lo > 1u) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (part_count_ge(k2, mid) >= kw) lo = mid; else hi = mid;
  }
  const uint32_t tau = lo;
  const int cnt_gt = part_count_ge(k2, tau + 1u);
  const int need = kw - cnt_gt;   // ties at tau to take, lowest index first
  // index order inside the wave: vector i, then lane, then value within the vector
  int ties = 0;
#pragma unroll
  for (int i = 0; i < kPartLoads; ++i) {
    int below = 0, tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned long long m = __ballot(key_half(k2[4 * i + q], h) == tau);
        below += lanes_below(m);
        tot += __popcll(m);
      }
    int own = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = 4 * i + q;
        const uint32_t k = key_half(k2[j], h);
        bool take = k > tau;
        if (k == tau) {
          take = ties + below + own < need;
          ++own;
        }
        const unsigned long long m = __ballot(take);
        if (take) out[taken + lanes_below(m)] = part_sort_key(k, part_index(vbase, j, h));
        taken += __popcll(m);
      }
    ties += tot;
  }
}

// The rank of `me` among the n distinct sort keys keys[0..n) in shared memory (keys
// descending): a loop of broadcast reads, the same address in every lane.
__device__ __forceinline__ int lds_rank(const unsigned long long* keys, int n, unsigned long long me) {
  int r = 0, e = 0;
  for (; e + 8 <= n; e += 8) {   // eight reads issued before the first compare
    ulonglong2 k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = reinterpret_cast<const ulonglong2*>(keys + e)[u];
#pragma unroll
    for (int u = 0; u < 4; ++u) r += (k[u].x > me ? 1 : 0) + (k[u].y > me ? 1 : 0);
  }
  for (; e < n; ++e) r += keys[e] > me ? 1 : 0;
  return r;
}

// Reductions over lanes 0..15 (one DPP row), the result in every lane.
template <typename T, typename Op>
__device__ __forceinline__ T row16_reduce(T v, Op op) {
  v = op(v, dpp_move<0xB1>(v));
  v = op(v, dpp_move<0x4E>(v));
  v = op(v, dpp_move<0x141>(v));
  v = op(v, dpp_move<0x140>(v));
  return read_lane(v, 0);
}

// The (shift, sum) of partials (sq, hq) held by the lanes of one wave (sum 0: no values),
// in every lane: exponentials sum to S * exp(M). ROW: only lanes 0..15 hold partials.
template <bool ROW>
__device__ __forceinline__ void merge_partials(double sq, float hq, const double* e64, float& M, double& S) {
  const auto fmax2 = [](float a, float b) { return b > a ? b : a; };
  const auto add = [](double a, double b) { return a + b; };
  const float h = sq > 0.0 ? hq : -INFINITY;
  const float M0 = ROW ? row16_reduce(h, fmax2) : wave_max(h);
  M = M0 == -INFINITY ? 0.0f : M0;
  const double term = sq > 0.0 ? sq * exp_nonpos(static_cast<double>(hq) - static_cast<double>(M), e64) : 0.0;
  S = ROW ? row16_reduce(term, add) : wave_sum(term);
}

// Merges the np <= 16 parts of one row (their lists and records written with st_cc by
// other workgroups) when np * K <= 64, in one wave: lane e holds list entry e, lane q part
// q's record. Writes the row's log-sum-exp, list length and top min(K, entries) into rv/ri.
__device__ __forceinline__ void part_merge_wave(const PartStat* ps, const float* pval, const int* pidx, int np,
                                                int K, double* lse, float* rv, int* ri, int* rcnt, PartSmem& sm) {
  const int lane = threadIdx.x & 63;
  const int n = np * K;
  // one round of loads (lanes past n or np load entry 0 and drop it)
  const int le = lane < n ? lane : 0, lp = lane < np ? lane : 0;
  const float v = ld_cc(&pval[le]);
  const int ix = ld_cc(&pidx[le]);
  int pc = ld_cc(&ps[lp].cnt);
  const float ph = ld_cc(&ps[lp].shift);
  double pm = ld_cc(&ps[lp].sum);
  if (lane >= np) {
    pc = 0;
    pm = 0.0;
  }
  if (lane < np) sm.pcnt[lane] = pc;
  int mypart = 0;   // lane / K, without a division
  for (int q = 1; q < np; ++q) mypart += lane >= q * K ? 1 : 0;
  __builtin_amdgcn_wave_barrier();
  const int mycnt = lane < n ? sm.pcnt[mypart] : 0;
  const unsigned long long me = (lane < n && lane - mypart * K < mycnt) ? part_sort_key(f32_bf16_key(v), ix) : 0ull;
  if (lane < n) sm.cand[lane] = me;
  __builtin_amdgcn_wave_barrier();
  const int r = lds_rank(sm.cand, n, me);
  const int total = row16_reduce(pc, [](int a, int b) { return a + b; });
  const int kk = K < total ? K : total;
  if (me != 0ull && r < kk) {
    rv[r] = part_key_value(me);
    ri[r] = part_key_index(me);
  }
  float M;
  double S;
  merge_partials<true>(pm, ph, sm.e64, M, S);
  if (lane == 0) {
    *lse = static_cast<double>(M) + log(S);
    *rcnt = kk;
  }
}

// With poll_ok (a caller whose chunk-list area holds nothing else between calls, so that the
// slots below are zero whenever a call starts), rows of np parts with np * (K + 2) <= 64
// (and np <= 16) merge without a ticket: every part publishes
// its list as K 64-bit sort keys (the empty marker 1 past its length; a real key is at least
// 2^32) and its record as two 64-bit words ((count << 32) | shift bits, and the complement
// of the sum's bits), each store a value that no unwritten (zero) slot holds. The row's last
// part in launch order (p = np - 1) then polls all np * (K + 2) words in one wave until none
// is zero, merges them and zeroes them for the next call. The parts it waits for come
// earlier in launch order, so they are resident or done while it polls.
constexpr long kPartSpinLimit = 2000000;   // polls (each a memory round trip) before a timeout

__device__ __forceinline__ unsigned long long* part_poll_slots(float* pval0) {
  // the row's chunk-list area holds np * K 64-bit slots (np * K * 8 + 4 <= nch * K * 4 bytes
  // for every row of two or more parts); the slots start at its first 8-byte boundary
  const uintptr_t a = (reinterpret_cast<uintptr_t>(pval0) + 7u) & ~static_cast<uintptr_t>(7u);
  return reinterpret_cast<unsigned long long*>(a);
}

__device__ __forceinline__ bool part_poll_merge(unsigned long long* slots, PartStat* ps, int np, int K, double* lse,
                                                float* rv, int* ri, int* rcnt, int* err, PartSmem& sm) {
  const int lane = threadIdx.x & 63;
  const int n = np * K, nw = np * (K + 2);
  unsigned long long* src = nullptr;
  if (lane < n) src = slots + lane;
  else if (lane < nw) src = reinterpret_cast<unsigned long long*>(&ps[(lane - n) >> 1]) + ((lane - n) & 1);
  unsigned long long v = 1ull;
  long polls = 0;
  if (src != nullptr) {
    v = ld_cc(src);
    while (v == 0ull && ++polls <= kPartSpinLimit) {
      __builtin_amdgcn_s_sleep(1);
      v = ld_cc(src);
    }
  }
  if (__ballot(v == 0ull) != 0ull) {   // a part never reported
    if (lane == 0) {
      if (err != nullptr) atomicExch(err, kErrTimeout);
      *rcnt = 0;
    }
    return false;
  }
  if (src != nullptr) st_cc(src, 0ull);   // ready for the next call
  if (lane >= n && lane < nw) {
    const int q = (lane - n) >> 1;
    if (((lane - n) & 1) == 0) {
      sm.pcnt[q] = static_cast<int>(v >> 32);
      sm.pshift[q] = __uint_as_float(static_cast<uint32_t>(v));
    } else {
      sm.psum[q] = __longlong_as_double(static_cast<long long>(~v));
    }
  }
  const unsigned long long me = (lane < n && v != 1ull) ? v : 0ull;
  if (lane < n) sm.cand[lane] = me;
  __builtin_amdgcn_wave_barrier();
  const int pc = lane < np ? sm.pcnt[lane] : 0;
  const int total = row16_reduce(pc, [](int a, int b) { return a + b; });
  const int kk = K < total ? K : total;
  const int r = lds_rank(sm.cand, n, me);
  if (me != 0ull && r < kk) {
    rv[r] = part_key_value(me);
    ri[r] = part_key_index(me);
  }
  float M;
  double S;
  merge_partials<true>(lane < np ? sm.psum[lane] : 0.0, lane < np ? sm.pshift[lane] : 0.0f, sm.e64, M, S);
  if (lane == 0) {
    *lse = static_cast<double>(M) + log(S);
    *rcnt = kk;
  }
  return true;
}

// The same for any np * K <= kPartMergeCap (= kPartThreads), by the whole workgroup.
__device__ __forceinline__ void part_merge_wide(const PartStat* ps, const float* pval, const int* pidx, int np,
                                                int K, double* lse, float* rv, int* ri, int* rcnt, PartSmem& sm) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  unsigned long long* key = &sm.slot[0][0];
  for (int q = threadIdx.x; q < np; q += kPartThreads) {
    sm.pcnt[q] = ld_cc(&ps[q].cnt);
    sm.pshift[q] = ld_cc(&ps[q].shift);
    sm.psum[q] = ld_cc(&ps[q].sum);
  }
  const int n = np * K;
  const int e = threadIdx.x;
  float v = 0.0f;
  int ix = 0;
  if (e < n) {
    v = ld_cc(&pval[e]);
    ix = ld_cc(&pidx[e]);
  }
  __syncthreads();
  if (e < n) key[e] = (e % K) < sm.pcnt[e / K] ? part_sort_key(f32_bf16_key(v), ix) : 0ull;
  int total = 0;
  for (int q = 0; q < np; ++q) total += sm.pcnt[q];
  const int kk = K < total ? K : total;
  if (w == 0) {
    float M;
    double S;
    merge_partials<false>(lane < np ? sm.psum[lane] : 0.0, lane < np ? sm.pshift[lane] : 0.0f, sm.e64, M, S);
    if (lane == 0) {
      *lse = static_cast<double>(M) + log(S);
      *rcnt = kk;
    }
  }
  __syncthreads();
  if (e < n && key[e] != 0ull) {   // rank by counting
    const unsigned long long me = key[e];
    int r = 0;
    for (int e2 = 0; e2 < n; ++e2) r += key[e2] > me ? 1 : 0;
    if (r < kk) {
      rv[r] = part_key_value(me);
      ri[r] = part_key_index(me);
    }
  }
}

// Reduces part p of the np parts of a row of V bf16 values (every thread of the 1024 calls
// it). A one-part row is written directly: its log-sum-exp, list length and top min(K, V)
// into lse, rcnt, rv/ri. Otherwise the part's list and record go to pval/pidx (K slots) and
// ps[p] (st_cc), the part counts itself in `ticket` (zero between calls; the last part
// resets it), and the workgroup of the row's last part merges the row's parts (pval0/pidx0:
// part 0's slots, part q's at q * K; ps: part 0's record) into lse, rcnt, rv/ri.
// `cmax`, if given, receives the largest value of each of the row's 8192-value chunks that
// the part holds (chunk 4 p + i is the part's i-th load; -inf for a chunk of padding only).
//
// part_row_reduce_loaded takes the part's words already requested (part_load) after the
// tables (part_tables_issue), and calls `next` once every wave's table pieces and the
// part's words have landed: a caller may request its next part's words there, so that they
// arrive while this part is reduced. Waves that have no more to do return early; no block
// barrier follows such a return, so a caller may place one after the call.
template <typename Next>
__device__ __forceinline__ void part_row_reduce_loaded(PartData& d, const uint16_t* row, int V, int p, int np, int K,
                                                       float* pval0, int* pidx0, PartStat* ps, unsigned* ticket,
                                                       double* lse, float* rv, int* ri, int* rcnt, PartSmem& sm,
                                                       float* cmax, int* err, bool poll_ok, Next&& next) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int vbase = p * kPartVecs;
  const int vfull = V / 8;
  const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) && vfull > 0;
  // the wave's values all lie in the row (its last vector is a full one)
  const bool clean = vec && vbase + (kPartLoads - 1) * kPartThreads + 64 * w + 63 < vfull;
  uint32_t k2[kPartWords];
  uint32_t g4[kPartLoads];
  uint32_t lm;
  part_keys(d, clean, row, V, vbase, vec, k2, g4, lm);
  // the wave's four row maxima (rows of 16 lanes, 512 values each) and its maximum
  uint32_t rm = lm;
  rm = max(rm, dpp_move<0xB1>(rm));
  rm = max(rm, dpp_move<0x4E>(rm));
  rm = max(rm, dpp_move<0x141>(rm));
  rm = max(rm, dpp_move<0x140>(rm));
  const uint32_t km = max(max(read_lane(rm, 0), read_lane(rm, 16)), max(read_lane(rm, 32), read_lane(rm, 48)));
  if (cmax != nullptr) {   // the wave's maximum key of each load, two loads per packed reduction
    const auto pmax = [](uint32_t x, uint32_t y) { return as_u32(__builtin_elementwise_max(as_u16x2(x), as_u16x2(y))); };
    const auto hmax = [](uint32_t g) { return max(g & 0xFFFFu, g >> 16); };
    const uint32_t m01 = wave_reduce(hmax(g4[0]) | (hmax(g4[1]) << 16), pmax);
    const uint32_t m23 = wave_reduce(hmax(g4[2]) | (hmax(g4[3]) << 16), pmax);
    if (lane == 0) {
      sm.cmk[w][0] = m01;
      sm.cmk[w][1] = m23;
    }
  }
  // A lower bound of the part's K-th largest value. K <= 16: the K-th largest of the part's
  // 64 row maxima. Larger K: the largest over the waves of each wave's K-th largest lane
  // maximum. Either way at least K values reach it.
  const bool by_rows = K <= kPartRowBoundK;
  if (by_rows) {
    if ((lane & 15) == 0) sm.rmax[4 * w + (lane >> 4)] = rm;
  } else {
    uint32_t tau_w = 1u;
    if (__popcll(__ballot(lm != 0u)) >= K) {
      uint32_t hi = km + 1u;
      while (hi - tau_w > 1u) {
        const uint32_t mid = tau_w + ((hi - tau_w) >> 1);
        if (__popcll(__ballot(lm >= mid)) >= K) tau_w = mid; else hi = mid;
      }
    }
    if (lane == 0) sm.wtau[w] = tau_w;
  }
  if (threadIdx.x == 0) sm.ncand2 = 0;
  drain();          // this wave's table pieces have landed
  __syncthreads();  // every wave's have, and the row maxima are visible
  if (cmax != nullptr && w == kPartWaves - 1 && lane < kPartLoads) {
    uint32_t m = 0u;
#pragma unroll
    for (int q = 0; q < kPartWaves; ++q) {
      const uint32_t pk = sm.cmk[q][lane >> 1];
      m = max(m, (lane & 1) ? pk >> 16 : pk & 0xFFFFu);
    }
    const int c = p * kPartLoads + lane;
    if (c * (kPartValues / kPartLoads) < V) cmax[c] = m != 0u ? bf16_key_value(m) : -INFINITY;
  }
  next();

  // ---- the bound: wave 0 bisects the 64 row maxima (one per lane) before its own sum
  if (by_rows && w == 0) {
    const uint32_t v = sm.rmax[lane];
    uint32_t lo = 1u;
    if (__popcll(__ballot(v != 0u)) >= K) {   // count(>= lo) >= K > count(>= hi)
      lo = wave_min(v != 0u ? v : 0xFFFFFFFFu);
      uint32_t hi = wave_max(v) + 1u;
      while (hi - lo > 1u) {
        const uint32_t mid = lo + ((hi - lo) >> 1);
        if (__popcll(__ballot(v >= mid)) >= K) lo = mid; else hi = mid;
      }
    }
    if (lane == 0) sm.tau = lo;
  }

  // ---- the wave's exponentials: table, else shifted by the wave maximum
  double sum;
  float shift;
  part_wave_exp(d, k2, km, clean, vbase, V, sm, sum, shift);
  if (by_rows) __syncthreads();   // the bound is visible
  const uint32_t tau = by_rows ? sm.tau : wave_max(lane < kPartWaves ? sm.wtau[lane] : 0u);

  // ---- candidates: values >= tau, looked for only in the lanes whose maximum reaches it
  // (a word is looked at only if one of its two values reaches tau in some lane), written
  // into the wave's slots at ballot prefix counts
  int cnt = 0;
  if (__ballot(lm >= tau) != 0ull) {
#pragma unroll
    for (int i = 0; i < kPartLoads; ++i) {
      if (__ballot(max(g4[i] & 0xFFFFu, g4[i] >> 16) >= tau) == 0ull) continue;   // a group of 4 words
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = 4 * i + q;
        const uint32_t lo = k2[j] & 0xFFFFu, hi = k2[j] >> 16;
        if (__ballot(max(lo, hi) >= tau) == 0ull) continue;
        const bool t0 = lo >= tau, t1 = hi >= tau;
        const unsigned long long m0 = __ballot(t0), m1 = __ballot(t1);
        const int c0 = __popcll(m0);
        const int p0 = cnt + lanes_below(m0), p1 = cnt + c0 + lanes_below(m1);
        if (t0 && p0 < kPartSlots) sm.slot[w][p0] = part_sort_key(lo, part_index(vbase, j, 0));
        if (t1 && p1 < kPartSlots) sm.slot[w][p1] = part_sort_key(hi, part_index(vbase, j, 1));
        cnt += c0 + __popcll(m1);
      }
    }
  }

  if (lane == 0) {
    sm.wsum[w] = sum;
    sm.wshift[w] = shift;
    sm.wcnt[w] = cnt;
  }
  __syncthreads();

  // ---- rank
  const bool whole = np == 1;
  const bool wide = !whole && (np * K > 64 || np > 16);   // the row merge needs the whole workgroup
  const bool poll = poll_ok && !whole && np <= 16 && np * (K + 2) <= 64;   // merged without a ticket
  unsigned long long* const pslot = poll ? part_poll_slots(pval0) + static_cast<size_t>(p) * K : nullptr;
  const int nvalid = min(max(V - p * kPartValues, 0), kPartValues);
  const int kk = K < nvalid ? K : nvalid;
  float* const ov = whole ? rv : pval0 + static_cast<size_t>(p) * K;
  int* const oi = whole ? ri : pidx0 + static_cast<size_t>(p) * K;
  // the counts of all waves (lane q < 16 of every wave holds wave q's)
  const int cq = lane < kPartWaves ? sm.wcnt[lane] : 0;
  int n = row16_reduce(cq, [](int a, int b) { return a + b; });
  const bool over = row16_reduce(cq, [](int a, int b) { return b > a ? b : a; }) > kPartSlots;
  const unsigned long long* packed = sm.cand;
  if (over) {   // ties overflowed a wave's slots: exact per-wave lists, packed from slot 0
    __syncthreads();   // every wave has read the counts before the slots are rewritten
    part_wave_exact(k2, km, K, vbase, &sm.slot[0][0], &sm.ncand2);
    __syncthreads();
    n = sm.ncand2;
    packed = &sm.slot[0][0];
  }
  // Wave 0 ranks and stores the list while wave 1 forms the part's (shift, sum): for a row
  // of one part its log-sum-exp and count, else its record.
  if (n <= 64) {   // wave 0: a candidate per lane
    if (w > 1 && !wide) return;
    if (w == 0) {
      unsigned long long me = 0ull;
      if (over) {
        me = lane < n ? packed[lane] : 0ull;
      } else {
        const int c4 = sm.wcnt[lane >> 2];
        if (__ballot((lane & 3) == 0 && c4 > 4) == 0ull) {   // at most 4 per wave: slot lane & 3 of wave lane >> 2
          me = (lane & 3) < c4 ? sm.slot[lane >> 2][lane & 3] : 0ull;
          const unsigned long long m = __ballot(me != 0ull);
          if (me != 0ull) sm.cand[lanes_below(m)] = me;
        } else {
          int b = 0, src = 0;
#pragma unroll
          for (int q = 0; q < kPartWaves; ++q) {
            const int c = sm.wcnt[q];
            if (lane >= b && lane < b + c) src = q * kPartSlots + lane - b;
            b += c;
          }
          me = lane < n ? (&sm.slot[0][0])[src] : 0ull;
          sm.cand[lane] = me;
        }
        __builtin_amdgcn_wave_barrier();
      }
      const int r = lds_rank(packed, n, me);
      if (me != 0ull && r < kk) {
        if (whole) {
          ov[r] = part_key_value(me);
          oi[r] = part_key_index(me);
        } else if (poll) {
          st_cc(&pslot[r], me);
        } else {
          st_cc(&ov[r], part_key_value(me));
          st_cc(&oi[r], part_key_index(me));
        }
      }
      if (poll && lane >= kk && lane < K) st_cc(&pslot[lane], 1ull);   // the empty marker
    }
  } else {   // rank by counting, a candidate per thread, over every wave's slots
    const int* cnts = sm.wcnt;
    const unsigned long long* mine = over ? &sm.slot[0][0] + threadIdx.x : &sm.slot[w][lane];
    const bool have = over ? static_cast<int>(threadIdx.x) < n : lane < min(cnts[w], kPartSlots);
    if (have) {
      const unsigned long long me = *mine;
      int r = 0;
      if (over) {
        r = lds_rank(&sm.slot[0][0], n, me);
      } else {
        for (int q2 = 0; q2 < kPartWaves; ++q2) r += lds_rank(sm.slot[q2], min(cnts[q2], kPartSlots), me);
      }
      if (r < kk) {
        if (poll) {
          st_cc(&pslot[r], me);
        } else {
          st_cc(&ov[r], part_key_value(me));
          st_cc(&oi[r], part_key_index(me));
        }
      }
    }
    if (poll && static_cast<int>(threadIdx.x) >= kk && static_cast<int>(threadIdx.x) < K)
      st_cc(&pslot[threadIdx.x], 1ull);   // the empty marker
    drain();
    __syncthreads();   // every list entry is stored
    if (w > 1 && !wide) return;
  }
  if (w == 1) {
    float M;
    double S;
    merge_partials<true>(lane < kPartWaves ? sm.wsum[lane] : 0.0, lane < kPartWaves ? sm.wshift[lane] : 0.0f,
                         sm.e64, M, S);
    if (lane == 0) {
      if (whole) {
        *lse = static_cast<double>(M) + log(S);
        *rcnt = kk;
      } else if (poll) {
        unsigned long long* rw = reinterpret_cast<unsigned long long*>(&ps[p]);
        st_cc(&rw[0], (static_cast<unsigned long long>(kk) << 32) | __float_as_uint(M));
        st_cc(&rw[1], ~static_cast<unsigned long long>(__double_as_longlong(S)));
      } else {
        st_cc(&ps[p].shift, M);
        st_cc(&ps[p].cnt, kk);
        st_cc(&ps[p].sum, S);
      }
    }
  }
  if (whole) return;
  if (poll) {   // the row's last part merges; its own words are polled like the others'
    if (p != np - 1 || w != 0) return;
    part_poll_merge(part_poll_slots(pval0), ps, np, K, lse, rv, ri, rcnt, err, sm);
    return;
  }
  if (!wide) {   // waves 0 and 1 (the others have ended): their stores complete, then wave 0's ticket
    drain();
    __syncthreads();
    if (w != 0) return;
    unsigned prev = 0u;
    if (lane == 0) prev = atomic_add_cc(ticket, 1u);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != static_cast<unsigned>(np - 1)) return;
    acquire_cc();
    part_merge_wave(ps, pval0, pidx0, np, K, lse, rv, ri, rcnt, sm);
    if (lane == 0) st_cc(ticket, 0u);   // after the merge: the acquire need not wait for it
    return;
  }
  if (last_arrival(ticket, np, &sm.flag)) part_merge_wide(ps, pval0, pidx0, np, K, lse, rv, ri, rcnt, sm);
}

__device__ __forceinline__ void part_row_reduce(const uint16_t* row, int V, int p, int np, int K, float* pval0,
                                                int* pidx0, PartStat* ps, unsigned* ticket, double* lse, float* rv,
                                                int* ri, int* rcnt, PartSmem& sm, float* cmax = nullptr,
                                                int* err = nullptr, bool poll_ok = false) {
  // the tables first: the keys wait for the data loads, which are issued after them
  part_tables_issue(sm);
  PartData d;
  part_load(row, V, p * kPartVecs, ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) && V / 8 > 0, d);
  part_row_reduce_loaded(d, row, V, p, np, K, pval0, pidx0, ps, ticket, lse, rv, ri, rcnt, sm, cmax, err, poll_ok,
                         [] {});
}

}  // namespace dtv
