// Vocab-wide row statistics on gfx950: max, argmax, log-sum-exp and top-K of logit rows.
//
// A row of V logits is cut into chunks of kBlock * kLoads * VEC elements (8192 bf16 or
// 4096 fp32); one 256-thread workgroup reads a chunk with coalesced 16-byte loads, keeps
// it in registers, and reduces it to a ChunkStat plus its sorted top-K list. The chunks of
// a row are then merged (by whichever workgroup finishes the row last). Everything that
// orders values uses exact order-preserving integer keys of the stored values, so argmax
// and top-K are exact; log-sum-exp accumulates exp(x - max) in float64.
#pragma once

#include "common.h"
#include "fexp.h"

namespace dtv {

struct ChunkStat {
  float maxv;      // largest value of the chunk
  int argmax;      // lowest index holding it
  double sumexp;   // sum over the chunk of exp(x - maxv), float64
  int cnt;         // entries in the chunk's top-K list
  int pad;
};

template <int DT>  // 0: fp32 rows, 1: bf16 rows
struct RowT {
  static constexpr int VEC = DT ? 8 : 4;           // values per 16-byte load
  static constexpr int E = kLoads * VEC;            // values per thread per chunk
  static constexpr int CHUNK = kBlock * E;          // values per chunk
  static constexpr int KEYBITS = DT ? 16 : 32;      // bits of the exact ordering key
  static constexpr int ESIZE = DT ? 2 : 4;
};

template <int DT>
__host__ __device__ constexpr int chunks_of(int V) {
  return (V + RowT<DT>::CHUNK - 1) / RowT<DT>::CHUNK;
}

// Shared-memory scratch used by the chunk routines.
struct RowSmem {
  double redd[kWaves];
  float redf[kWaves];
  unsigned redu[kWaves];
  int redi[kWaves];
  // per-wave partial results of chunk_reduce
  double wse[kWaves];
  float wmax[kWaves];
  uint32_t wkey[kWaves];
  int warg[kWaves];
  int wcnt[kWaves];
  uint32_t wtau[kWaves];
  int ncand;
  int flag;
  double exptab[64];  // table of exp_nonpos; filled by row_smem_init
};

// Must run in every thread at kernel start, followed by __syncthreads().
__device__ __forceinline__ void row_smem_init(RowSmem& sm) { exp_table_load(sm.exptab); }

// The same without registers, so that the table shares the round trip of the loads that
// follow it: wave 0 copies the table straight into shared memory with two direct loads
// (lane l moves bytes 4l .. 4l+3 of each 256-byte half). Every thread must then wait for its
// loads (drain) and pass __syncthreads() before the table is read.
__device__ __forceinline__ void row_smem_issue(RowSmem& sm) {
  typedef __attribute__((address_space(3))) void lds_void_t;
  if (threadIdx.x < 64) {
    const char* src = reinterpret_cast<const char*>(kExp2_64) + 4 * threadIdx.x;
    char* dst = reinterpret_cast<char*>(sm.exptab);
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 4, 0, 0);
    __builtin_amdgcn_global_load_lds(src + 256, (lds_void_t*)(dst + 256), 4, 0, 0);
  }
}

constexpr int kCandCap = 512;   // candidate slots of the small-K selection (sortbuf entries)

// Loads chunk `c` of `row` into registers. Out-of-range elements get key 0 and -inf.
// For a 16-byte aligned row every thread issues its four 16-byte loads back to back
// before using any: a vector past the row end is loaded from the row's last full vector
// (valid memory) and masked, and only the one vector that straddles the row end (V not a
// multiple of VEC) re-reads its valid elements one by one. Unaligned rows take scalar
// loads throughout.
template <int DT>
__device__ __forceinline__ void load_chunk(const void* row, int V, int c, float (&x)[RowT<DT>::E],
                                           uint32_t (&key)[RowT<DT>::E]) {
  using R = RowT<DT>;
  const int t = threadIdx.x;
  const int base = c * R::CHUNK;
  const int vfull = V / R::VEC;   // full 16-byte vectors in the row
  const bool aligned = ((reinterpret_cast<uintptr_t>(row) & 15u) == 0);
  if (aligned && vfull > 0) {
    uint4 raw[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int vi = (base + i * kBlock * R::VEC) / R::VEC + t;
      const int vc = vi < vfull ? vi : vfull - 1;
      raw[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(row) + static_cast<size_t>(vc) * 16);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int vi = (base + i * kBlock * R::VEC) / R::VEC + t;
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int e = 0; e < R::VEC; ++e) {
        float f;
        if (DT)
          f = bf16_to_f32(static_cast<uint16_t>((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu));
        else
          f = __uint_as_float(w[e]);
        const bool ok = vi < vfull;
        x[i * R::VEC + e] = ok ? f : -INFINITY;
        key[i * R::VEC + e] = ok ? (f32_key(f) >> (32 - R::KEYBITS)) : 0u;
      }
      if (vi == vfull && vfull * R::VEC < V) {   // the straddling vector
#pragma unroll
        for (int e = 0; e < R::VEC; ++e) {
          const int ix = vi * R::VEC + e;
          if (ix < V) {
            const float f = DT ? bf16_to_f32(static_cast<const uint16_t*>(row)[ix])
                               : static_cast<const float*>(row)[ix];
            x[i * R::VEC + e] = f;
            key[i * R::VEC + e] = f32_key(f) >> (32 - R::KEYBITS);
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int i0 = base + i * kBlock * R::VEC + t * R::VEC;
#pragma unroll
    for (int e = 0; e < R::VEC; ++e) {
      const int ix = i0 + e;
      if (ix < V) {
        const float f = DT ? bf16_to_f32(static_cast<const uint16_t*>(row)[ix])
                           : static_cast<const float*>(row)[ix];
        x[i * R::VEC + e] = f;
        key[i * R::VEC + e] = f32_key(f) >> (32 - R::KEYBITS);
      } else {
        x[i * R::VEC + e] = -INFINITY;
        key[i * R::VEC + e] = 0u;
      }
    }
  }
}

// The 16-byte loads of one chunk, held in registers so that a loop over chunks can issue
// the next chunk's loads before working on the current one (vector path of load_chunk:
// the row must be 16-byte aligned and hold at least one full vector).
struct RawChunk {
  uint4 r0, r1, r2, r3;   // named members keep them in registers
};
static_assert(kLoads == 4, "RawChunk holds kLoads vectors");

template <int DT>
__device__ __forceinline__ void raw_chunk_load(const void* row, int V, int c, RawChunk& rc) {
  using R = RowT<DT>;
  const int vfull = V / R::VEC;
  const int v0 = c * R::CHUNK / R::VEC + static_cast<int>(threadIdx.x);
  const char* b = static_cast<const char*>(row);
  rc.r0 = *reinterpret_cast<const uint4*>(b + static_cast<size_t>(min(v0, vfull - 1)) * 16);
  rc.r1 = *reinterpret_cast<const uint4*>(b + static_cast<size_t>(min(v0 + kBlock, vfull - 1)) * 16);
  rc.r2 = *reinterpret_cast<const uint4*>(b + static_cast<size_t>(min(v0 + 2 * kBlock, vfull - 1)) * 16);
  rc.r3 = *reinterpret_cast<const uint4*>(b + static_cast<size_t>(min(v0 + 3 * kBlock, vfull - 1)) * 16);
}

// Values of a chunk loaded by raw_chunk_load, as load_chunk gives them (-inf past the row
// end; the one vector straddling the row end re-reads its valid elements).
template <int DT>
__device__ __forceinline__ void raw_chunk_decode(const void* row, int V, int c, const RawChunk& rc,
                                                 float (&x)[RowT<DT>::E]) {
  using R = RowT<DT>;
  const int vfull = V / R::VEC;
  const int v0 = c * R::CHUNK / R::VEC + static_cast<int>(threadIdx.x);
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const uint4 q = i == 0 ? rc.r0 : i == 1 ? rc.r1 : i == 2 ? rc.r2 : rc.r3;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    const int vi = v0 + i * kBlock;
#pragma unroll
    for (int e = 0; e < R::VEC; ++e) {
      const float f = DT ? bf16_to_f32(static_cast<uint16_t>((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu))
                         : __uint_as_float(w[e]);
      x[i * R::VEC + e] = vi < vfull ? f : -INFINITY;
    }
    if (vi == vfull && vfull * R::VEC < V) {
#pragma unroll
      for (int e = 0; e < R::VEC; ++e) {
        const int ix = vi * R::VEC + e;
        if (ix < V)
          x[i * R::VEC + e] = DT ? bf16_to_f32(static_cast<const uint16_t*>(row)[ix])
                                 : static_cast<const float*>(row)[ix];
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ int elem_index(int c, int i, int e) {
  using R = RowT<DT>;
  return c * R::CHUNK + (i * kBlock + static_cast<int>(threadIdx.x)) * R::VEC + e;
}

// Sort `n` (a power of two) 64-bit keys in shared memory, descending.
__device__ __forceinline__ void bitonic_sort_desc(unsigned long long* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kBlock) {
        const int p = i ^ j;
        if (p > i) {
          const unsigned long long x = a[i], y = a[p];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            a[i] = y;
            a[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ unsigned long long sort_key(float v, int idx) {
  return (static_cast<unsigned long long>(f32_key(v)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(idx));
}
__device__ __forceinline__ int sort_key_index(unsigned long long k) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull));
}
__device__ __forceinline__ float sort_key_value(unsigned long long k) {
  return key_to_f32(static_cast<uint32_t>(k >> 32));
}

__host__ __device__ constexpr int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Number of chunk elements (of this wave) whose key is >= thr; wave-uniform, scalar.
template <int DT>
__device__ __forceinline__ int wave_count_ge(const uint32_t (&key)[RowT<DT>::E], uint32_t thr) {
  int n = 0;
#pragma unroll
  for (int j = 0; j < RowT<DT>::E; ++j) n += __popcll(__ballot(key[j] >= thr));
  return n;
}

__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__device__ __forceinline__ float bf16key_to_f32(uint32_t k16) {
  return bf16_to_f32(static_cast<uint16_t>((k16 & 0x8000u) ? (k16 & 0x7FFFu) : (~k16 & 0xFFFFu)));
}

// Reduces the chunk in registers. Writes *st and, when K > 0, the chunk's top-K (value,
// index) sorted by (value desc, index asc) into out_val/out_idx (global, st_cc). The
// argmax (largest value, lowest index) is the list's first entry when K > 0; only for
// K = 0 is it looked for separately. `cmax`, if given, receives the chunk's maximum too.
//
// Per wave, without block barriers: maximum (and, for K = 0, its lowest index), float64 sum
// of exp(x - wave max), valid count. Top-K, for K <= 32: every wave takes the K-th largest of
// its 64 lane maxima (bisection with one ballot per step); the largest of those, tau, is a
// lower bound of the chunk's K-th largest value (that wave alone has K values >= tau), so
// the chunk's top-K are among the values >= tau, usually barely more than K of them. They
// are gathered in shared memory and ranked exactly by (value desc, index asc). If ties make
// the candidates overflow, or K > 32, each wave instead bisects the key space for its own
// K-th largest value (ballot counts over all its elements), resolves ties at the threshold
// in index order with lane-prefix counts, and the <= 4K wave candidates are ranked (K <= 32)
// or sorted. `sortbuf` holds at least max(kCandCap, pow2_at_least(4 * K)) entries.
template <int DT>
__device__ void chunk_reduce(const float (&x)[RowT<DT>::E], const uint32_t (&key)[RowT<DT>::E], int c,
                             int V, int K, ChunkStat* st, float* out_val, int* out_idx,
                             unsigned long long* sortbuf, RowSmem& sm, float* cmax = nullptr) {
  using R = RowT<DT>;
  const int w = threadIdx.x >> 6;
  // ---- wave max, lowest index of the max, sum of exp, valid count
  uint32_t lmk = 0;
#pragma unroll
  for (int j = 0; j < R::E; ++j) lmk = key[j] > lmk ? key[j] : lmk;
  const uint32_t km = wave_max(lmk);
  int am = 0x7FFFFFFF;
  if (K == 0) {   // with a list, its first entry (value desc, index asc) is the argmax
#pragma unroll
    for (int i = kLoads - 1; i >= 0; --i)
#pragma unroll
      for (int e = R::VEC - 1; e >= 0; --e)
        if (key[i * R::VEC + e] == km) am = elem_index<DT>(c, i, e);
    am = wave_min(am);
  }
  // in-range elements of the chunk (padding has key 0; a stored -inf does not)
  const int nvalid = min(max(V - c * R::CHUNK, 0), R::CHUNK);
  const float mw = (km == 0u) ? -INFINITY : (DT ? bf16key_to_f32(km) : key_to_f32(km));
  double se = 0.0;
  if (km != 0u) {  // wave-uniform; padding elements hold -inf and contribute exp(-inf) = 0
    se = exp_nonpos_sum<R::E>(x, static_cast<double>(mw), sm.exptab);
  }
  se = wave_sum(se);
  const bool small = K <= 32;
  if (small && K > 0) {  // K-th largest lane maximum of this wave
    uint32_t lo = 1u;
    if (__popcll(__ballot(lmk != 0u)) >= K) {
      uint32_t hi = km + 1u;
      while (hi - lo > 1u) {
        const uint32_t mid = lo + ((hi - lo) >> 1);
        if (__popcll(__ballot(lmk >= mid)) >= K) lo = mid; else hi = mid;
      }
    }
    if ((threadIdx.x & 63) == 0) sm.wtau[w] = lo;
  }
  if ((threadIdx.x & 63) == 0) {
    sm.wkey[w] = km;
    sm.warg[w] = am;
    sm.wse[w] = se;
    sm.wmax[w] = mw;
    sm.wcnt[w] = 0;
  }
  if (threadIdx.x == 0) sm.ncand = 0;
  __syncthreads();

  // ---- chunk results, read by the workgroup that merges the row: lane q of the last wave
  //      holds wave q's partials
  const int kk = K < nvalid ? K : nvalid;
  if (w == kWaves - 1) {
    const int q = threadIdx.x & 63;
    const uint32_t kq = q < kWaves ? sm.wkey[q] : 0u;
    const uint32_t KM = wave_max(kq);
    const float M = (KM == 0u) ? -INFINITY : (DT ? bf16key_to_f32(KM) : key_to_f32(KM));
    const int AM = wave_min(q < kWaves && kq == KM ? sm.warg[q] : 0x7FFFFFFF);
    double term = 0.0;
    if (q < kWaves && kq != 0u)
      term = sm.wse[q] * exp_nonpos(static_cast<double>(sm.wmax[q]) - static_cast<double>(M), sm.exptab);
    const double S = wave_sum(term);
    if (q == 0) {
      st_cc(&st->maxv, M);
      if (cmax != nullptr) st_cc(cmax, M);
      if (K == 0) st_cc(&st->argmax, AM);   // else written with the list's first entry
      st_cc(&st->sumexp, S);
      st_cc(&st->cnt, kk);
    }
  }
  if (kk <= 0) {
    __syncthreads();
    return;
  }

  if (small) {
    uint32_t tau = 1u;
    for (int q = 0; q < kWaves; ++q) tau = sm.wtau[q] > tau ? sm.wtau[q] : tau;
    // the candidates (keys >= tau) are packed without per-element atomics: a ballot pass
    // counts the wave's candidates and notes which element slots hold any, one shared-memory
    // atomic reserves the wave's range, and only those slots (usually a handful) write their
    // candidates, each at its lane's rank within the wave
    int wn = 0;
    uint32_t slots = 0u;   // wave-uniform
#pragma unroll
    for (int j = 0; j < R::E; ++j) {
      const int cj = __popcll(__ballot(key[j] >= tau));
      wn += cj;
      slots |= (cj != 0 ? 1u : 0u) << j;
    }
    int pos = 0;
    if ((threadIdx.x & 63) == 0 && wn > 0) pos = atomicAdd(&sm.ncand, wn);
    pos = __builtin_amdgcn_readfirstlane(pos);
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
#pragma unroll
      for (int e = 0; e < R::VEC; ++e) {
        if (slots & (1u << (i * R::VEC + e))) {
          const bool take = key[i * R::VEC + e] >= tau;
          const unsigned long long m = __ballot(take);
          const int p = pos + lanes_below(m);
          if (take && p < kCandCap) sortbuf[p] = sort_key(x[i * R::VEC + e], elem_index<DT>(c, i, e));
          pos += __popcll(m);
        }
      }
    __syncthreads();
    const int n = sm.ncand;
    if (n <= kCandCap) {
      for (int e = threadIdx.x; e < n; e += kBlock) {
        const unsigned long long me = sortbuf[e];
        int rank = 0;
        for (int e2 = 0; e2 < n; ++e2) rank += sortbuf[e2] > me ? 1 : 0;
        if (rank < kk) {
          st_cc(&out_val[rank], sort_key_value(me));
          st_cc(&out_idx[rank], sort_key_index(me));
          if (rank == 0) st_cc(&st->argmax, sort_key_index(me));
        }
      }
      __syncthreads();
      return;
    }
    __syncthreads();  // too many ties at tau: exact per-wave selection below
  }

  const int P2 = pow2_at_least(kWaves * K);
  const bool big = kWaves * K > 128;
  if (big) {
    for (int i = threadIdx.x; i < P2; i += kBlock) sortbuf[i] = 0ull;
    __syncthreads();
  }
  // ---- the wave's own top-K by bisection of the key space
  int nv = 0;   // in-range elements of this wave
#pragma unroll
  for (int j = 0; j < R::E; ++j) nv += __popcll(__ballot(key[j] != 0u));
  const int kw = K < nv ? K : nv;
  if (kw > 0) {
    uint32_t lo = 1u, hi = km + 1u;  // count(>= lo) >= kw > count(>= hi)
    while (hi - lo > 1u) {
      const uint32_t mid = lo + ((hi - lo) >> 1);
      if (wave_count_ge<DT>(key, mid) >= kw) lo = mid; else hi = mid;
    }
    const uint32_t tau = lo;
    const int cnt_gt = wave_count_ge<DT>(key, tau + 1u);
    const int cnt_eq = wave_count_ge<DT>(key, tau) - cnt_gt;
    const int need = kw - cnt_gt;   // ties at tau to take, lowest index first
    int base = 0;                   // ties of this wave in earlier loads
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      int below = 0, tot = 0;
      if (cnt_eq > need) {
#pragma unroll
        for (int e = 0; e < R::VEC; ++e) {
          const unsigned long long m = __ballot(key[i * R::VEC + e] == tau);
          below += lanes_below(m);
          tot += __popcll(m);
        }
      }
      int own = 0;
#pragma unroll
      for (int e = 0; e < R::VEC; ++e) {
        const uint32_t k = key[i * R::VEC + e];
        bool take = k > tau;
        if (k == tau) {
          take = (cnt_eq > need) ? (base + below + own < need) : true;
          ++own;
        }
        if (take) {
          const int pos = atomicAdd(&sm.wcnt[w], 1);
          sortbuf[w * K + pos] = sort_key(x[i * R::VEC + e], elem_index<DT>(c, i, e));
        }
      }
      base += tot;
    }
  }
  __syncthreads();
  if (!big) {
    // rank of each wave candidate among all of them (keys are unique)
    for (int e = threadIdx.x; e < kWaves * K; e += kBlock) {
      const int q = e / K, j = e % K;
      if (j >= sm.wcnt[q]) continue;
      const unsigned long long me = sortbuf[e];
      int rank = 0;
      for (int q2 = 0; q2 < kWaves; ++q2)
        for (int j2 = 0; j2 < sm.wcnt[q2]; ++j2) rank += sortbuf[q2 * K + j2] > me ? 1 : 0;
      if (rank < kk) {
        st_cc(&out_val[rank], sort_key_value(me));
        st_cc(&out_idx[rank], sort_key_index(me));
        if (rank == 0) st_cc(&st->argmax, sort_key_index(me));
      }
    }
  } else {
    bitonic_sort_desc(sortbuf, P2);
    for (int i = threadIdx.x; i < kk; i += kBlock) {
      st_cc(&out_val[i], sort_key_value(sortbuf[i]));
      st_cc(&out_idx[i], sort_key_index(sortbuf[i]));
      if (i == 0) st_cc(&st->argmax, sort_key_index(sortbuf[0]));
    }
  }
  __syncthreads();
}

// Shared staging area of row_merge: CAP entries of all chunk lists together.
constexpr int kMergeMaxChunks = 64;

constexpr int kMergeFast = 64;   // candidates of the thresholded merge (one per lane of a wave)

template <int CAP>
struct MergeSmem {
  unsigned long long key[CAP];  // sort keys of every chunk's list, list c at c*K
  unsigned long long cand[kMergeFast];   // entries at or above the threshold (fast path)
  int ncand;
  int cnt[kMergeMaxChunks];
  float maxv[kMergeMaxChunks];
  int argmax[kMergeMaxChunks];
  double sumexp[kMergeMaxChunks];
};

// Merges the ChunkStats and sorted top-K lists of the `nch` chunks of one row (written by
// other workgroups with st_cc). The lists are first copied into shared memory (one
// parallel pass of coherent loads). The last wave forms the log-sum-exp while wave 0 looks
// for a bound T: the kout-th largest of the lists' first ceil(kout / nch) entries, which
// has at least kout entries at or above it, so only entries >= T can be among the top;
// wave 0 gathers those (usually a few more than kout) and ranks them in registers. When
// the bound cannot be formed that way or more than 64 entries reach it, every entry's rank
// is the count of entries of all lists that precede it (counting for <= 1024 entries, else
// binary search in the sorted lists).
// Outputs: maxv, argmax, lse (last wave); the top kout (default K) entries (value, index)
// into rv/ri, all written with st_cc. Requires nch <= 64 and nch * K <= CAP.
// Returns min(kout, entries).
template <int CAP>
__device__ int row_merge(const ChunkStat* st, const float* cval, const int* cidx, int nch, int K,
                         float* maxv, int* argmax, double* lse, float* rv, int* ri, RowSmem& sm,
                         MergeSmem<CAP>& ms, int kout = -1) {
  // one parallel round of loads: the chunk statistics and every list slot (slots past a
  // chunk's count are read too and ignored, so no load waits for a count)
  for (int c = threadIdx.x; c < nch; c += kBlock) {
    ms.cnt[c] = ld_cc(&st[c].cnt);
    ms.maxv[c] = ld_cc(&st[c].maxv);
    ms.argmax[c] = ld_cc(&st[c].argmax);
    ms.sumexp[c] = ld_cc(&st[c].sumexp);
  }
  for (int e = threadIdx.x; e < nch * K; e += kBlock) ms.key[e] = sort_key(ld_cc(&cval[e]), ld_cc(&cidx[e]));
  if (threadIdx.x == 0) ms.ncand = 0;
  __syncthreads();
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (w == kWaves - 1) {  // the last wave: lane c holds chunk c (nch <= 64)
    const int c = lane;
    const float mc = c < nch ? ms.maxv[c] : -INFINITY;
    const float M = wave_max(mc);
    // chunks are in index order: the first chunk reaching the maximum has the lowest index
    const int first = wave_min(c < nch && mc == M ? c : 0x7FFFFFFF);
    double term = 0.0;
    if (c < nch && mc != -INFINITY)
      term = ms.sumexp[c] * exp_nonpos(static_cast<double>(mc) - static_cast<double>(M), sm.exptab);
    const double s = wave_sum(term);
    if (c == 0) {
      if (maxv) st_cc(maxv, M);
      if (argmax) st_cc(argmax, ms.argmax[first < nch ? first : 0]);
      if (lse) st_cc(lse, static_cast<double>(M) + log(s));
    }
  }
  int total = 0;
  for (int c = 0; c < nch; ++c) total += ms.cnt[c];
  const int want = kout < 0 ? K : kout;   // entries of the merged list (chunk lists hold K)
  const int kk = want < total ? want : total;
  if (kk <= 0) {
    __syncthreads();
    return 0;
  }
  const int n = nch * K;
  // Fast path (wave 0): a bound T with at least `want` entries at or above it, so that the
  // merged list is among the entries >= T. Every list is sorted, so T is taken among the
  // lists' first h = ceil(want / nch) entries: the want-th largest of those. Wave 0 gathers
  // the entries >= T (usually a few more than want) and ranks them in registers.
  const int h = (want + nch - 1) / nch;
  if (w == 0 && n <= 1024 && h <= K && nch * h <= 64) {
    bool fast = false;
    const int hc = lane / h, hj = lane % h;
    const unsigned long long hk = (lane < nch * h && hj < ms.cnt[hc]) ? ms.key[hc * K + hj] : 0ull;
    if (__popcll(__ballot(hk != 0ull)) >= want) {   // keys are unique and never 0
      int r = 0;
      for (int q = 0; q < nch * h; ++q) r += read_lane(hk, q) > hk ? 1 : 0;
      const unsigned long long sel = __ballot(hk != 0ull && r == want - 1);
      const unsigned long long T = read_lane(hk, static_cast<int>(__builtin_ctzll(sel)));
      int base = 0;
      for (int e0 = 0; e0 < n; e0 += 64) {
        const int e = e0 + lane;
        const int c = e / K, j = e % K;
        const unsigned long long k = e < n ? ms.key[e] : 0ull;
        const bool in = e < n && j < ms.cnt[c] && k >= T;
        const unsigned long long m = __ballot(in);
        const int pos = base + lanes_below(m);
        if (in && pos < kMergeFast) ms.cand[pos] = k;
        base += __popcll(m);
      }
      fast = base <= kMergeFast;
      if (fast) {
        __builtin_amdgcn_wave_barrier();
        const unsigned long long me = lane < base ? ms.cand[lane] : 0ull;
        int rank = 0;
        for (int q = 0; q < base; ++q) rank += read_lane(me, q) > me ? 1 : 0;
        if (lane < base && rank < kk) {
          st_cc(&rv[rank], sort_key_value(me));
          st_cc(&ri[rank], sort_key_index(me));
        }
      }
    }
    if (lane == 0) ms.ncand = fast ? 1 : 0;
  }
  __syncthreads();
  if (ms.ncand != 0) {
    __syncthreads();   // every wave has read ncand before the next merge may reset it
    return kk;
  }
  // ---- general path: every entry's rank among all lists
  if (n <= 1024) {  // absent entries count as key 0, below every real key
    for (int e = threadIdx.x; e < n; e += kBlock)
      if ((e % K) >= ms.cnt[e / K]) ms.key[e] = 0ull;
    __syncthreads();
  }
  for (int e = threadIdx.x; e < n; e += kBlock) {
    const int c = e / K, j = e % K;
    if (j >= ms.cnt[c]) continue;
    const unsigned long long me = ms.key[e];
    int rank = 0;
    if (n <= 1024) {
      // count the larger keys of all lists (keys are unique); independent broadcast reads
      for (int e2 = 0; e2 < n; ++e2) rank += ms.key[e2] > me ? 1 : 0;
    } else {
      rank = j;
      for (int c2 = 0; c2 < nch; ++c2) {
        if (c2 == c) continue;
        int a = 0, b = ms.cnt[c2];  // entries of list c2 greater than me (binary search)
        const unsigned long long* l2 = ms.key + c2 * K;
        while (a < b) {
          const int m = (a + b) >> 1;
          if (l2[m] > me) a = m + 1; else b = m;
        }
        rank += a;
      }
    }
    if (rank < kk) {
      st_cc(&rv[rank], sort_key_value(me));
      st_cc(&ri[rank], sort_key_index(me));
    }
  }
  __syncthreads();
  return kk;
}

}  // namespace dtv
