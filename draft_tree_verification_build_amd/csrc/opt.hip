// OPT-Tree draft-tree construction on gfx950 (OPT-Tree summary, section 3).
//
// Every layer, each frontier node proposes its most probable children, scored with the
// product of draft probabilities along the path (a float64 sum of logs); the layer keeps
// the n best candidates (ties: lower frontier position, then lower rank in the row), which
// become the next frontier in (parent position, rank) order. E_l, the sum of the scores of
// the best n nodes drafted so far, stops the drafting when it grows by less than delta.
// The final tree is those best n nodes.
//
// The exact top-n of W rows x n children per layer (262144 candidates at n = 512) is found
// without sorting them: each row only reports m = max(8, ceil(n / W)) of its best entries
// (the best of its chunks' top ceil(m / chunks) lists) and its log-sum-exp; the n-th best
// score among those W*m reported candidates is a lower bound `lo` of the layer's n-th best
// score (a subset of the candidates reaches it n times). A second pass over
// the rows gathers every candidate whose score is >= lo (a few hundred at the shapes of the
// pages), and one workgroup selects exactly among them in shared memory.
//
// Launches per layer (the host loop knows the frontier width W, which depends only on n
// and V): opt_rows (W x chunks workgroups), opt_bound (1 per sequence), opt_collect
// (W x chunks), opt_select (1 per sequence); then opt_finalize once. A sequence whose
// drafting has stopped makes every later launch return at once.
#include "dtv_internal.h"
#include "rows_bf16.h"
#include "rowstats.h"
#include "select.h"

namespace dtv {

constexpr int kOptMergeCap = 8192;  // chunks * K of one row merge
constexpr int kOptMaxWords = 16;    // ancestor-mask words of a tree of at most 1024 slots
constexpr int kOptLdsCand = 4096;   // candidates selected in shared memory

struct OptCand {
  double score;   // log path score
  uint32_t fj;    // (frontier position of the parent << 22) | token
  float x;        // the token's draft logit
};

// Frontier-order key of a candidate: (parent position asc, logit desc, token asc), i.e. a
// parent's children in their row's rank order. Also breaks ties between equal scores.
__device__ __forceinline__ unsigned long long front_key(const OptCand& c) {
  return (static_cast<unsigned long long>(c.fj >> 22) << 54) |
         (static_cast<unsigned long long>(~f32_key(c.x)) << 22) | (c.fj & 0x3FFFFFu);
}

// In-place bitonic sort of n (power of two) elements of shared memory by `before`.
template <int NT = kBlock, typename T, typename Cmp>
__device__ void bitonic_sort(T* a, int n, Cmp before) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += NT) {
        const int p = i ^ j;
        if (p > i) {
          const T x = a[i], y = a[p];
          const bool up = (i & k) == 0;  // this block is ordered by `before`
          if (up ? before(y, x) : before(x, y)) {
            a[i] = y;
            a[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int row_of(const OptArgs& a, int f) {
  if (a.row_base >= 0) return a.row_base + f;   // the call's own frontier rows, in frontier order
  return a.layer == 1 ? 0 : 1 + (a.layer - 2) * a.n + f;
}

__device__ __forceinline__ double parent_score(const OptArgs& a, int s, int f) {
  return a.layer == 1 ? 0.0 : a.lscore[(static_cast<size_t>(s) * a.max_layers + (a.layer - 2)) * a.n + f];
}

// ------------------------------------------------------------------ 1. frontier rows

// BIG: lists of up to 1024 per chunk (the root layer, K up to n); otherwise K <= 32, which
// needs far less shared memory and lets several workgroups share a compute unit.
template <int DT, bool BIG>
__global__ __launch_bounds__(kBlock, 4) void opt_rows_kernel(OptArgs a) {
  constexpr int kMergeCap = BIG ? kOptMergeCap : 2048;
  constexpr int kSort = BIG ? 4 * 1024 : kCandCap;
  __shared__ RowSmem rs;
  __shared__ MergeSmem<kMergeCap> ms;
  __shared__ unsigned long long sortbuf[kSort];
  using Rw = RowT<DT>;
  int bid = blockIdx.x;
  const int c = bid % a.nch;
  bid /= a.nch;
  const int f = bid % a.W;
  const int s = bid / a.W;
  // the stop flag was set by an earlier launch: a plain load sees it (a stopped sequence
  // must not stream its rows, so the chunk waits for it)
  if (a.done[s]) return;
  const char* row = static_cast<const char*>(a.draft) +
                    (static_cast<size_t>(s) * a.R + row_of(a, f)) * static_cast<size_t>(a.V) * Rw::ESIZE;
  // the exp table and the chunk in one round trip
  row_smem_issue(rs);
  float x[Rw::E];
  uint32_t key[Rw::E];
  load_chunk<DT>(row, a.V, c, x, key);
  drain();
  __syncthreads();
  const size_t rf = static_cast<size_t>(s) * a.Wcap + f;
  const size_t ci = rf * a.nch + c;
  // each chunk reports its top Kc (nch * Kc >= K): the row's merged K are then the best of
  // those, a subset of the row's candidates, which is all the lower bound needs
  chunk_reduce<DT>(x, key, c, a.V, a.Kc, &a.st[ci], a.cval + ci * a.Kc, a.cidx + ci * a.Kc, sortbuf, rs,
                   &a.cmax[ci]);
  if (!last_arrival(&a.tickets[rf], a.nch, &rs.flag)) return;
  const int n = row_merge(a.st + rf * a.nch, a.cval + rf * a.nch * a.Kc, a.cidx + rf * a.nch * a.Kc, a.nch, a.Kc,
                          nullptr, nullptr, &a.rlse[rf], a.rv + rf * a.K, a.ri + rf * a.K, rs, ms, a.K);
  if (threadIdx.x == 0) st_cc(&a.rcnt[rf], n);
}

// bf16 rows in 32768-value parts (rows_bf16.h): the row's log-sum-exp and top-K as above,
// and the maximum of each of its 8192-value chunks for the gathering pass. K <= 64. Rows of
// one part go two to a 1024-thread workgroup (one workgroup of 16 waves fills a compute
// unit's registers): the second row's words are requested once the first row's have landed,
// and arrive while the first is reduced; the exp table is copied once for both. Longer rows
// take one workgroup per part.
__global__ __launch_bounds__(kPartThreads) void opt_rows_bf16_kernel(OptArgs a) {
  __shared__ PartSmem sm;
  const int np = parts_of(a.V);
  const int K = a.K;
  const auto row_ptr = [&](int s, int f) {
    return static_cast<const uint16_t*>(a.draft) + (static_cast<size_t>(s) * a.R + row_of(a, f)) * static_cast<size_t>(a.V);
  };
  if (np == 1) {
    const int pairs = (a.W + 1) >> 1;
    const int s = blockIdx.x / pairs;
    const int f0 = 2 * (blockIdx.x % pairs);
    if (a.done[s]) return;
    const bool two = f0 + 1 < a.W;
    const uint16_t* r0 = row_ptr(s, f0);
    const uint16_t* r1 = row_ptr(s, two ? f0 + 1 : f0);
    const bool vec1 = ((reinterpret_cast<uintptr_t>(r1) & 15u) == 0) && a.V / 8 > 0;
    part_tables_issue(sm);
    PartData d0, d1;
    part_load(r0, a.V, 0, ((reinterpret_cast<uintptr_t>(r0) & 15u) == 0) && a.V / 8 > 0, d0);
    const size_t rf0 = static_cast<size_t>(s) * a.Wcap + f0;
    part_row_reduce_loaded(d0, r0, a.V, 0, 1, K, nullptr, nullptr, nullptr, nullptr, &a.rlse[rf0], a.rv + rf0 * K,
                           a.ri + rf0 * K, &a.rcnt[rf0], sm, a.cmax + rf0 * a.nch, &a.hdr->err, false,
                           [&] { if (two) part_load(r1, a.V, 0, vec1, d1); });
    if (!two) return;
    __syncthreads();   // the first row's waves are done with shared memory
    const size_t rf1 = rf0 + 1;
    part_row_reduce_loaded(d1, r1, a.V, 0, 1, K, nullptr, nullptr, nullptr, nullptr, &a.rlse[rf1], a.rv + rf1 * K,
                           a.ri + rf1 * K, &a.rcnt[rf1], sm, a.cmax + rf1 * a.nch, &a.hdr->err, false, [] {});
    return;
  }
  int bid = blockIdx.x;
  const int p = bid % np;
  bid /= np;
  const int f = bid % a.W;
  const int s = bid / a.W;
  if (a.done[s]) return;
  const size_t rf = static_cast<size_t>(s) * a.Wcap + f;
  const size_t ci = rf * a.nch;   // the row's chunk slots hold its parts' records
  part_row_reduce(row_ptr(s, f), a.V, p, np, K, a.cval + ci * K, a.cidx + ci * K,
                  reinterpret_cast<PartStat*>(a.st + ci), &a.tickets[rf], &a.rlse[rf], a.rv + rf * K, a.ri + rf * K,
                  &a.rcnt[rf], sm, a.cmax + ci, &a.hdr->err);
}

// ------------------------------------------------------------------ 1'. the root layer in one launch
//
// Layer 1 expands the root alone: its frontier is the root row's n best entries by (logit
// desc, token asc), each scored logit - lse, and the best list is that frontier. One launch
// does all of it. Each chunk workgroup reduces its chunk (max, float64 sum of exp) and, in
// every wave whose lanes all hold in-range elements, takes the Kw-th largest of the 64 lane
// maxima: that wave holds at least Kw elements at or above it, so the minimum over such
// waves bounds the row's n-th largest key from below once their count times Kw reaches n.
// The last chunk workgroup to finish forms the log-sum-exp, re-reads the row gathering every
// element at or above the bound (somewhat more than n) and ranks them exactly through value
// buckets: an entry's rank is the number of entries in higher buckets plus the members of
// its own bucket with a larger sort key ((value key, index) keys are unique). Entries ranked
// below n are the layer.

constexpr int kRootCand = 4096;      // gathered elements at or above the bound
constexpr int kRootBuckets = 1024;

struct OptRootSmem {
  RowSmem rs;
  unsigned long long cand[kRootCand];
  int kbs[kRootCand];          // (bucket << 16) | place within the bucket
  unsigned long long mkey[kRootCand];   // keys of the gathered entries grouped by bucket
  double ksc[1024];            // score of the entry at each rank
  int bcnt[kRootBuckets];      // entries per bucket
  int bbase[kRootBuckets];     // entries in higher buckets
  float cmax[kMergeMaxChunks];
  double csum[kMergeMaxChunks];
  uint32_t ctau[kMergeMaxChunks];
  uint32_t wtau[kWaves];
  unsigned long long red64[kWaves];
  int scan[kWaves];
  double red[kWaves];
  int ncand;
  uint32_t lokey;
  double lse;
};

// Appends this thread's elements of chunk c at or above the bound: one shared-memory atomic
// per wave, placed by the lanes' prefix counts.
template <int DT>
__device__ __forceinline__ void root_gather(const float (&xv)[RowT<DT>::E], int c, int V, uint32_t lok,
                                            OptRootSmem& sm) {
  using Rw = RowT<DT>;
  static_assert(Rw::E <= 32, "one predicate bit per element");
  uint32_t bits = 0u;
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
#pragma unroll
    for (int e = 0; e < Rw::VEC; ++e) {
      const int j = i * Rw::VEC + e;
      const uint32_t k = f32_key(xv[j]) >> (32 - Rw::KEYBITS);
      if (elem_index<DT>(c, i, e) < V && k != 0u && k >= lok) bits |= 1u << j;
    }
  const int lane = threadIdx.x & 63;
  const int cnt = __popc(bits);
  const int incl = wave_inclusive_scan(cnt);
  int base = 0;
  if (lane == 63) base = atomicAdd(&sm.ncand, incl);
  base = read_lane(base, 63);
  int pos = base + incl - cnt;
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
#pragma unroll
    for (int e = 0; e < Rw::VEC; ++e) {
      const int j = i * Rw::VEC + e;
      if ((bits >> j) & 1u) {
        if (pos < kRootCand) sm.cand[pos] = sort_key(xv[j], elem_index<DT>(c, i, e));
        ++pos;
      }
    }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void opt_root_kernel(OptArgs a) {
  __shared__ OptRootSmem sm;
  using Rw = RowT<DT>;
  const int c = blockIdx.x % a.nch;
  const int s = blockIdx.x / a.nch;
  const char* row = static_cast<const char*>(a.draft) +
                    static_cast<size_t>(s) * a.R * static_cast<size_t>(a.V) * Rw::ESIZE;   // row 0: the root
  const size_t cb = static_cast<size_t>(s) * a.Wcap * a.nch;   // chunk statistics of (s, f = 0)
  {
    // the exp table and the chunk in one round trip
    row_smem_issue(sm.rs);
    float x[Rw::E];
    uint32_t key[Rw::E];
    load_chunk<DT>(row, a.V, c, x, key);
    drain();
    __syncthreads();
    chunk_reduce<DT>(x, key, c, a.V, 0, &a.st[cb + c], nullptr, nullptr, sm.cand, sm.rs);
    // the Kw-th largest lane maximum of every full wave
    const int w = threadIdx.x >> 6;
    uint32_t lmk = 0u;
#pragma unroll
    for (int j = 0; j < Rw::E; ++j) lmk = key[j] > lmk ? key[j] : lmk;
    const long last = static_cast<long>(c) * Rw::CHUNK +
                      static_cast<long>((kLoads - 1) * kBlock + 64 * w + 63) * Rw::VEC + Rw::VEC - 1;
    uint32_t tau = 0xFFFFFFFFu;
    if (last < a.V) {   // wave-uniform: every lane holds in-range elements only
      unsigned long long lo = 1ull, hi = static_cast<unsigned long long>(wave_max(lmk)) + 1ull;
      if (__popcll(__ballot(lmk >= 1u)) >= a.Kw) {
        while (hi - lo > 1ull) {
          const unsigned long long mid = lo + ((hi - lo) >> 1);
          if (__popcll(__ballot(lmk >= mid)) >= a.Kw) lo = mid; else hi = mid;
        }
        tau = static_cast<uint32_t>(lo);
      } else {
        tau = 1u;   // keys of 0 (absent) in a full wave: no bound from it
      }
    }
    if ((threadIdx.x & 63) == 0) sm.wtau[w] = tau;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t t = 0xFFFFFFFFu;
      for (int q = 0; q < kWaves; ++q) t = sm.wtau[q] < t ? sm.wtau[q] : t;
      st_cc(&a.st[cb + c].pad, static_cast<int>(t));
    }
  }
  if (!last_arrival(&a.tickets[static_cast<size_t>(s) * a.Wcap], a.nch, &sm.rs.flag)) return;

  // ---- the last chunk workgroup: the first four chunks of the row are requested before the
  //      chunk statistics, so that both round trips overlap
  const int vfull = a.V / Rw::VEC;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(row) & 15u) == 0 && vfull > 0;
  RawChunk rq[4];
  if (vec_ok) {
#pragma unroll
    for (int u = 0; u < 4; ++u) raw_chunk_load<DT>(row, a.V, u < a.nch ? u : a.nch - 1, rq[u]);
  }
  for (int q = threadIdx.x; q < a.nch; q += kBlock) {
    sm.cmax[q] = ld_cc(&a.st[cb + q].maxv);
    sm.csum[q] = ld_cc(&a.st[cb + q].sumexp);
    sm.ctau[q] = static_cast<uint32_t>(ld_cc(&a.st[cb + q].pad));
  }
  for (int b = threadIdx.x; b < kRootBuckets; b += kBlock) sm.bcnt[b] = 0;
  if (threadIdx.x == 0) sm.ncand = 0;
  __syncthreads();
  // log-sum-exp (as the row merge forms it) and the bound
  if (threadIdx.x < 64) {   // lane q holds chunk q (nch <= 64)
    const int q = threadIdx.x;
    const float mc = q < a.nch ? sm.cmax[q] : -INFINITY;
    const float M = wave_max(mc);
    double term = 0.0;
    if (q < a.nch && mc != -INFINITY)
      term = sm.csum[q] * exp_nonpos(static_cast<double>(mc) - static_cast<double>(M), sm.rs.exptab);
    const double S = wave_sum(term);
    const uint32_t lk = wave_min(q < a.nch ? sm.ctau[q] : 0xFFFFFFFFu);
    if (q == 0) {
      sm.lse = static_cast<double>(M) + log(S);
      sm.lokey = lk;
    }
  }
  __syncthreads();
  const uint32_t lok = sm.lokey;
  // ---- every element at or above the bound, four chunks' loads in flight at a time
  if (vec_ok) {
    for (int c0 = 0; c0 < a.nch; c0 += 4) {
      if (c0 > 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) raw_chunk_load<DT>(row, a.V, c0 + u < a.nch ? c0 + u : a.nch - 1, rq[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (c0 + u < a.nch) {
          float xv[Rw::E];
          raw_chunk_decode<DT>(row, a.V, c0 + u, rq[u], xv);
          root_gather<DT>(xv, c0 + u, a.V, lok, sm);
        }
      }
    }
  } else {
    for (int c0 = 0; c0 < a.nch; ++c0) {
      float xv[Rw::E];
      uint32_t kv[Rw::E];
      load_chunk<DT>(row, a.V, c0, xv, kv);
      root_gather<DT>(xv, c0, a.V, lok, sm);
    }
  }
  __syncthreads();
  const int C = sm.ncand;
  const int n = a.n;
  if (C > kRootCand) {   // far more entries tie at the bound than the buffer holds: refuse
    if (threadIdx.x == 0) {
      atomicExch(&a.hdr->err, kErrCapacity);
      a.done[s] = 1;
    }
    return;
  }
  const int kept = C < n ? C : n;
  // ---- exact ranks: buckets of the value-key range, largest values first
  unsigned long long vmax = 0ull, vmin = ~0ull;
  for (int e = threadIdx.x; e < C; e += kBlock) {
    const unsigned long long v = sm.cand[e] >> 32;
    vmax = v > vmax ? v : vmax;
    vmin = v < vmin ? v : vmin;
  }
  vmax = block_max(vmax, sm.red64);
  vmin = block_min(vmin, sm.red64);
  const unsigned long long range = vmax - vmin + 1ull;
  for (int e = threadIdx.x; e < C; e += kBlock) {
    const unsigned long long v = sm.cand[e] >> 32;
    const int b = static_cast<int>(((vmax - v) * kRootBuckets) / range);
    sm.kbs[e] = (b << 16) | atomicAdd(&sm.bcnt[b], 1);
  }
  __syncthreads();
  {
    constexpr int per = kRootBuckets / kBlock;
    const int b0 = threadIdx.x * per;
    int loc = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) loc += sm.bcnt[b0 + q];
    int tot = 0;
    int run = block_exclusive_scan(loc, sm.scan, &tot);
#pragma unroll
    for (int q = 0; q < per; ++q) {
      sm.bbase[b0 + q] = run;
      run += sm.bcnt[b0 + q];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < C; e += kBlock) {
    const int kb = sm.kbs[e];
    sm.mkey[sm.bbase[kb >> 16] + (kb & 0xFFFF)] = sm.cand[e];
  }
  __syncthreads();
  const double lse = sm.lse;
  const size_t lb = static_cast<size_t>(s) * a.max_layers * n;   // layer 1 of sequence s
  const size_t bb = static_cast<size_t>(s) * n;
  for (int e = threadIdx.x; e < C; e += kBlock) {
    const unsigned long long me = sm.cand[e];
    const int b = sm.kbs[e] >> 16;
    const int b0 = sm.bbase[b], bn = sm.bcnt[b];
    if (b0 >= n) continue;   // the whole bucket ranks at or past n
    int r = b0;
    for (int q = 0; q < bn; ++q) r += sm.mkey[b0 + q] > me ? 1 : 0;
    if (r >= n) continue;
    const double sc = 0.0 + (static_cast<double>(sort_key_value(me)) - lse);
    a.lscore[lb + r] = sc;
    a.lparent[lb + r] = 0;
    a.ltoken[lb + r] = sort_key_index(me);
    a.bscore[bb + r] = sc;
    a.blayer[bb + r] = 1;
    a.bpos[bb + r] = r;
    sm.ksc[r] = sc;
  }
  __syncthreads();
  // E_1 = sum of exp(score) over the best list, each thread over ranks t, t + kBlock, ...
  double part = 0.0;
  for (int r = threadIdx.x; r < kept; r += kBlock) part += exp(sm.ksc[r]);
  const double E = block_sum(part, sm.red);
  if (threadIdx.x == 0) {
    a.bcount[s] = kept;
    const double gain = E - a.Eprev[s];
    a.Eprev[s] = E;
    a.nlayers[s] = 1;
    if (gain < a.delta || 1 >= a.max_layers) a.done[s] = 1;
  }
}

// ------------------------------------------------------------------ 1''. the bf16 root layer in one workgroup
//
// A bf16 root row of at most 32768 values fits one 1024-thread workgroup in registers, 32
// values a lane (rows_bf16.h's part layout). The exp table gives the log-sum-exp. A lane
// whose maximum reaches a threshold holds at least one value at or above it, so the n-th
// largest of the 1024 lane maxima bounds the row's n-th largest value from below (wave 0
// bisects it while the other waves sum); for logits of a smooth distribution about 1.5 n
// values reach it. They are gathered and ranked exactly through buckets of their 16-bit
// value keys, one key a bucket when the keys span at most 1024 (else equal slices of the
// span): an entry's rank is the count of entries in higher buckets plus the members of its
// own bucket with a larger (key, index) sort key. Entries ranked below n are layer 1, which
// is also the first best list; the workgroup sets the sequence's per-call state. Applies
// when lanes 0..n-1 all hold values, i.e. ceil(V / 8) >= n.

constexpr int kRootPartCand = 4096;   // gathered entries at or above the bound
constexpr int kRootPartBuckets = kPartThreads;

struct OptRootPartSmem {
  PartSmem ps;                            // tables; after the sums, the grouped keys and the kept scores
  uint32_t lmax[kPartThreads];            // every lane's largest key
  unsigned long long cand[kRootPartCand];
  int kbs[kRootPartCand];                 // (bucket << 16) | place within the bucket
  int bcnt[kRootPartBuckets];
  int bbase[kRootPartBuckets];
  int wred[kPartWaves];
  double dred[kPartWaves];
  uint32_t tau, kmax;
  int ncand;
  double lse;
};
static_assert(sizeof(double) * kExpBf16Entries >= sizeof(unsigned long long) * kRootPartCand + sizeof(double) * 1024,
              "the grouped keys and the kept scores fit the table's space");

bool opt_root_one_workgroup(int V, int n, int dtype) {
  return dtype == 1 && V <= kPartValues && (V + 7) / 8 >= n && n <= 1024;
}

__global__ __launch_bounds__(kPartThreads) void opt_root_bf16_kernel(OptArgs a) {
  __shared__ OptRootPartSmem sm;
  const int s = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int V = a.V, n = a.n;
  const uint16_t* row = static_cast<const uint16_t*>(a.draft) + static_cast<size_t>(s) * a.R * static_cast<size_t>(V);
  const int vfull = V / 8;
  const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) && vfull > 0;
  part_tables_issue(sm.ps);
  PartData d;
  part_load(row, V, 0, vec, d);
  const bool clean = vec && (kPartLoads - 1) * kPartThreads + 64 * w + 63 < vfull;
  uint32_t k2[kPartWords], g4[kPartLoads], lm;
  part_keys(d, clean, row, V, 0, vec, k2, g4, lm);
  sm.lmax[threadIdx.x] = lm;
  const uint32_t km = wave_max(lm);
  sm.bcnt[threadIdx.x] = 0;
  if (lane == 0) sm.ps.wtau[w] = km;
  if (threadIdx.x == 0) sm.ncand = 0;
  drain();          // this wave's table pieces have landed
  __syncthreads();  // every wave's have, and the lane maxima are visible

  // ---- wave 0: the n-th largest lane maximum (lanes 0..n-1 hold values: count(>= 1) >= n)
  if (w == 0) {
    uint32_t v[kPartWaves];
#pragma unroll
    for (int q = 0; q < kPartWaves; ++q) v[q] = sm.lmax[64 * q + lane];
    const uint32_t KM = wave_max(lane < kPartWaves ? sm.ps.wtau[lane] : 0u);
    uint32_t lo = 1u, hi = KM + 1u;   // count(>= lo) >= n > count(>= hi)
    while (hi - lo > 1u) {
      const uint32_t mid = lo + ((hi - lo) >> 1);
      int c = 0;
#pragma unroll
      for (int q = 0; q < kPartWaves; ++q) c += __popcll(__ballot(v[q] >= mid));
      if (c >= n) lo = mid; else hi = mid;
    }
    if (lane == 0) {
      sm.tau = lo;
      sm.kmax = KM;
    }
  }
  double sum;
  float shift;
  part_wave_exp(d, k2, km, clean, 0, V, sm.ps, sum, shift);
  if (lane == 0) {
    sm.ps.wsum[w] = sum;
    sm.ps.wshift[w] = shift;
  }
  __syncthreads();   // the bound and the partials

  // ---- every value at or above the bound; wave 1 forms the log-sum-exp meanwhile
  const uint32_t tau = sm.tau;
  if (__ballot(lm >= tau) != 0ull) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < kPartWords; ++j) c += ((k2[j] & 0xFFFFu) >= tau ? 1 : 0) + ((k2[j] >> 16) >= tau ? 1 : 0);
    const int incl = wave_inclusive_scan(c);
    int base = 0;
    if (lane == 63) base = atomicAdd(&sm.ncand, incl);
    base = read_lane(base, 63);
    int pos = base + incl - c;
#pragma unroll
    for (int j = 0; j < kPartWords; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t k = key_half(k2[j], h);
        if (k >= tau) {
          if (pos < kRootPartCand) sm.cand[pos] = part_sort_key(k, part_index(0, j, h));
          ++pos;
        }
      }
  }
  if (w == 1) {
    float M;
    double S;
    merge_partials<true>(lane < kPartWaves ? sm.ps.wsum[lane] : 0.0, lane < kPartWaves ? sm.ps.wshift[lane] : 0.0f,
                         sm.ps.e64, M, S);
    if (lane == 0) sm.lse = static_cast<double>(M) + log(S);
  }
  __syncthreads();
  const int C = sm.ncand;
  if (C > kRootPartCand) {   // far more entries tie at the bound than the buffer holds: refuse
    if (threadIdx.x == 0) {
      atomicExch(&a.hdr->err, kErrCapacity);
      a.done[s] = 1;
      a.bcount[s] = 0;
      a.nlayers[s] = 0;
    }
    return;
  }
  // ---- exact ranks through buckets of the value keys, largest first
  const uint32_t KM = sm.kmax;
  const uint32_t span = KM - tau + 1u;
  const bool exact = span <= static_cast<uint32_t>(kRootPartBuckets);
  for (int e = threadIdx.x; e < C; e += kPartThreads) {
    const uint32_t k = static_cast<uint32_t>(sm.cand[e] >> 32);
    const int b = static_cast<int>(exact ? KM - k : ((KM - k) * static_cast<uint32_t>(kRootPartBuckets)) / span);
    sm.kbs[e] = (b << 16) | atomicAdd(&sm.bcnt[b], 1);
  }
  __syncthreads();
  {
    const int x = sm.bcnt[threadIdx.x];
    const int incl = wave_inclusive_scan(x);
    if (lane == 63) sm.wred[w] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int q = 0; q < kPartWaves; ++q) before += q < w ? sm.wred[q] : 0;
    sm.bbase[threadIdx.x] = before + incl - x;
  }
  __syncthreads();
  unsigned long long* mkey = reinterpret_cast<unsigned long long*>(sm.ps.tab);   // the table is no longer read
  double* ksc = sm.ps.tab + kRootPartCand;
  for (int e = threadIdx.x; e < C; e += kPartThreads) {
    const int kb = sm.kbs[e];
    mkey[sm.bbase[kb >> 16] + (kb & 0xFFFF)] = sm.cand[e];
  }
  __syncthreads();
  const double lse = sm.lse;
  const size_t lb = static_cast<size_t>(s) * a.max_layers * n;   // layer 1 of sequence s
  const size_t bb = static_cast<size_t>(s) * n;
  for (int e = threadIdx.x; e < C; e += kPartThreads) {
    const unsigned long long me = sm.cand[e];
    const int b = sm.kbs[e] >> 16;
    const int b0 = sm.bbase[b], bn = sm.bcnt[b];
    if (b0 >= n) continue;   // the whole bucket ranks at or past n
    int r = b0;
    for (int q = 0; q < bn; ++q) r += mkey[b0 + q] > me ? 1 : 0;
    if (r >= n) continue;
    const double sc = 0.0 + (static_cast<double>(part_key_value(me)) - lse);
    a.lscore[lb + r] = sc;
    a.lparent[lb + r] = 0;
    a.ltoken[lb + r] = part_key_index(me);
    a.bscore[bb + r] = sc;
    a.blayer[bb + r] = 1;
    a.bpos[bb + r] = r;
    ksc[r] = sc;
  }
  __syncthreads();
  // E_1 = sum of exp(score) over the best list (C >= n: each of lanes 0..n-1 reaches tau)
  double E = static_cast<int>(threadIdx.x) < n ? exp(ksc[threadIdx.x]) : 0.0;
  E = wave_sum(E);
  if (lane == 0) sm.dred[w] = E;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int q = 0; q < kPartWaves; ++q) t += sm.dred[q];
    a.bcount[s] = n;
    a.Eprev[s] = t;
    a.nlayers[s] = 1;
    a.ccount[s] = 0u;
    a.done[s] = (t < a.delta || 1 >= a.max_layers) ? 1 : 0;   // gain over the empty tree
  }
}

// ------------------------------------------------------------------ 2. lower bound

struct OptBoundSmem {
  unsigned long long key[8192];
  int off[1024];
  int cnt[1024];
  double ps[1024];    // parent score of each frontier row
  double lse[1024];   // its log-sum-exp
  int wsum[kMaxBlockWaves];
  RadixSmem rs;
};

template <int NT>
__global__ __launch_bounds__(NT) void opt_bound_kernel(OptArgs a) {
  __shared__ OptBoundSmem sm;
  const int s = blockIdx.x;
  if (a.done[s]) return;
  // the reported candidates: the top-m of every row (m = K), packed row after row
  // per row: list length (scanned to offsets), parent score and log-sum-exp, read once
  int carry = 0;
  for (int f0 = 0; f0 < a.W; f0 += NT) {
    const int f = f0 + threadIdx.x;
    const int fc = f < a.W ? f : a.W - 1;
    const size_t rf = static_cast<size_t>(s) * a.Wcap + fc;
    const int cnt = (f < a.W) ? a.rcnt[rf] : 0;
    const double ps = parent_score(a, s, fc);
    const double lse = a.rlse[rf];
    int tot = 0;
    const int ex = block_exclusive_scan<int, NT / 64>(cnt, sm.wsum, &tot);
    if (f < a.W) {
      sm.off[f] = carry + ex;
      sm.cnt[f] = cnt;
      sm.ps[f] = ps;
      sm.lse[f] = lse;
    }
    carry += tot;
  }
  const int total = carry;
  __syncthreads();   // offsets of every row before the keys are placed
  // the score of an entry is formed exactly as the collection forms it. A thread takes
  // whole rows: their list values are loaded unconditionally (all addresses are in the
  // workspace), eight at a time in flight, and placed after the row's earlier entries
  const int K = a.K;
  for (int f = threadIdx.x; f < a.W; f += NT) {
    const float* rv = a.rv + (static_cast<size_t>(s) * a.Wcap + f) * K;
    const double ps = sm.ps[f], lse = sm.lse[f];
    const int cnt = sm.cnt[f], off = sm.off[f];
    for (int j0 = 0; j0 < K; j0 += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = rv[min(j0 + u, K - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        if (j < cnt) sm.key[off + j] = dkey(ps + (static_cast<double>(x[u]) - lse));
      }
    }
  }
  __syncthreads();
  // the n-th largest reported score bounds the layer's n-th best score from below, and so
  // does anything below it: radix passes narrow the n-th largest key down to a prefix that
  // fixes at least the exponent and 8 mantissa bits (one pass when the reported scores share
  // their sign and upper exponent bits, two when they span, say, (-1, -8]), and the lowest
  // key under that prefix is the bound: it lies within 2^-8 (relative) of the n-th score,
  // so a few more candidates pass it than pass the exact n-th score, for a fraction of the
  // selection's passes
  double lo = -INFINITY;
  if (total >= a.n) {
    const RadixCut cut = radix_topk_cut<NT>(sm.key, total, a.n, sm.rs, 64, 0, 52 - 8);
    const unsigned long long k = cut.prefix;
    const unsigned long long u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    lo = __longlong_as_double(static_cast<long long>(u));
    if (lo != lo) lo = -INFINITY;   // a bucket floor past -inf (the n-th score is -inf)
  }
  if (threadIdx.x == 0) {
    a.lo[s] = lo;
    a.ccount[s] = 0u;
  }
}

// ------------------------------------------------------------------ 3. gather candidates

template <int DT>
__global__ __launch_bounds__(kBlock) void opt_collect_kernel(OptArgs a) {
  using Rw = RowT<DT>;
  int bid = blockIdx.x;
  const int c = bid % a.nch;
  bid /= a.nch;
  const int f = bid % a.W;
  const int s = bid / a.W;
  // the stop flag, the bound and the row's values in one round of loads (valid memory
  // whether or not the sequence has stopped)
  const int done = a.done[s];
  const double lo = a.lo[s];
  const size_t rf = static_cast<size_t>(s) * a.Wcap + f;
  const double base = parent_score(a, s, f);
  const double lse = a.rlse[rf];
  const float cmax = a.cmax[rf * a.nch + c];
  if (done) return;
  // a chunk whose largest logit cannot reach lo has no candidate: skip reading it
  if (!(base + (static_cast<double>(cmax) - lse) >= lo)) return;
  const char* row = static_cast<const char*>(a.draft) +
                    (static_cast<size_t>(s) * a.R + row_of(a, f)) * static_cast<size_t>(a.V) * Rw::ESIZE;
  float x[Rw::E];
  uint32_t key[Rw::E];
  load_chunk<DT>(row, a.V, c, x, key);
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
#pragma unroll
    for (int e = 0; e < Rw::VEC; ++e) {
      if (key[i * Rw::VEC + e] == 0u) continue;
      const double sc = base + (static_cast<double>(x[i * Rw::VEC + e]) - lse);
      if (sc >= lo) {
        const unsigned pos = atomicAdd(&a.ccount[s], 1u);
        if (pos < static_cast<unsigned>(a.ccap)) {
          OptCand* out = a.cand + static_cast<size_t>(s) * a.ccap + pos;
          out->score = sc;
          out->fj = (static_cast<uint32_t>(f) << 22) | static_cast<uint32_t>(elem_index<DT>(c, i, e));
          out->x = x[i * Rw::VEC + e];
        }
      }
    }
}

// ------------------------------------------------------------------ 4. exact selection
//
// One workgroup per sequence. The layer keeps its n best gathered candidates (radix cut of
// the score keys; candidates tied at a full key go in frontier order). Their positions in
// the next frontier, (parent position, logit desc, token), come from grouping them by
// parent (count, scan, scatter) and counting, within a group, the members before each one
// (a bitonic sort when one group is large, as at the root layer). The best n so far are a
// second radix cut over the old best list and this layer's nodes, by (score desc, layer
// asc, position asc); that list is kept unordered.

struct OptKept {
  unsigned long long key;   // frontier key, then unused
  double score;
  int pos;                  // frontier position
  int pad;
};
struct OptBest {
  double score;
  int layer, pos;
};

constexpr int kOptBucketMax = 128;   // largest parent group ranked by counting
constexpr int kOptGroupMax = 64;     // boundary groups ranked directly instead of more radix passes

struct OptSelectSmem {
  union {
    struct {
      OptCand c[kOptLdsCand];                // gathered candidates
      unsigned long long key[kOptLdsCand];   // their score keys
    } in;
    struct {
      OptKept k[1024];      // kept candidates (frontier numbering by bitonic sort)
    } srt;
    struct {
      unsigned long long key[2048];   // score keys of the old best list and this layer
      double score[2048];
      int info[2048];                 // (layer << 16) | position
    } best;
  } u;
  unsigned long long tkey[1024];   // entries tied at a cut: tie-order keys
  int tidx[1024];
  unsigned long long gkey[kOptGroupMax];   // a small boundary group's score keys
  int keep_idx[1024];              // indices of the kept candidates
  unsigned long long fkey[1024];   // frontier keys of the kept candidates
  int cntp[1024];                  // kept candidates per parent
  int basep[1024];                 // first frontier position of each parent's group
  int memb[1024];                  // kept candidates grouped by parent
  int kslot[1024];                 // a kept candidate's slot in its parent's group
  double kscore[1024];             // a kept candidate's score, by frontier position
  int scan[kMaxBlockWaves];
  double red[kMaxBlockWaves];
  RadixSmem rs;
  int ntie, nkept, nout;
};

template <int NT>
__global__ __launch_bounds__(NT) void opt_select_kernel(OptArgs a) {
  __shared__ OptSelectSmem sm;
  const int s = blockIdx.x;
  if (a.done[s]) return;
  const int C = static_cast<int>(a.ccount[s]);
  const int n = a.n;
  if (C > kOptLdsCand || C > a.ccap) {  // far more candidates than the bound allows: refuse
    if (threadIdx.x == 0) {
      atomicExch(&a.hdr->err, kErrCapacity);
      a.done[s] = 1;
    }
    return;
  }
  // (unrolled so that a thread's global loads are all in flight before its first store)
#pragma unroll 8
  for (int e = threadIdx.x; e < C; e += NT) {
    const OptCand cd = a.cand[static_cast<size_t>(s) * a.ccap + e];
    sm.u.in.c[e] = cd;
    sm.u.in.key[e] = dkey(cd.score);
  }
  if (threadIdx.x == 0) {
    sm.ntie = 0;
    sm.nkept = 0;
  }
  __syncthreads();
  // ---- the layer's n best
  const int kept = C < n ? C : n;
  if (C > n) {
    // radix cut of the n best: a boundary group taken whole needs no tie order; a small
    // one (or the keys tied at the n-th full key) is ranked by (score desc, frontier order)
    const RadixCut cut = radix_topk_cut<NT>(sm.u.in.key, C, n, sm.rs, 64, kOptGroupMax);
    const unsigned long long T = cut.prefix;
    const int rem = cut.all_in ? 0 : cut.rem;
    for (int e = threadIdx.x; e < C; e += NT) {
      const unsigned long long k = sm.u.in.key[e];
      const unsigned long long km = k & cut.mask;
      if (cut.all_in ? (km >= T) : (km > T)) {
        sm.keep_idx[atomicAdd(&sm.nkept, 1)] = e;
      } else if (!cut.all_in && km == T) {
        const int t = atomicAdd(&sm.ntie, 1);
        if (t < 1024) {
          sm.tkey[t] = front_key(sm.u.in.c[e]);
          sm.tidx[t] = e;
          if (t < kOptGroupMax) sm.gkey[t] = k;
        }
      }
    }
    __syncthreads();
    if (sm.ntie > 1024) {   // more than 1024 candidates share the n-th best score: refuse
      if (threadIdx.x == 0) {
        atomicExch(&a.hdr->err, kErrCapacity);
        a.done[s] = 1;
      }
      return;
    }
    const int nt = sm.ntie;
    const int above = sm.nkept;   // = n - rem
    for (int t = threadIdx.x; t < nt; t += NT) {
      const unsigned long long me = sm.tkey[t];
      int before = 0;
      if (cut.group) {   // full score key desc, then frontier order
        const unsigned long long mk = sm.gkey[t];
        for (int t2 = 0; t2 < nt; ++t2) {
          const unsigned long long ok2 = sm.gkey[t2];
          before += (ok2 > mk || (ok2 == mk && sm.tkey[t2] < me)) ? 1 : 0;
        }
      } else {           // all at the same full key: frontier order
        for (int t2 = 0; t2 < nt; ++t2) before += sm.tkey[t2] < me ? 1 : 0;
      }
      if (before < rem) sm.keep_idx[above + before] = sm.tidx[t];
    }
  } else {
    for (int e = threadIdx.x; e < C; e += NT) sm.keep_idx[e] = e;
  }
  __syncthreads();
  // ---- frontier order (parent position asc, logit desc, token asc) numbers the next
  //      frontier. Kept candidates are grouped by parent (count, scan, scatter); within a
  //      group, a candidate's position is the count of its group's members before it. A
  //      group larger than kOptBucketMax (the root layer) is numbered by a bitonic sort.
  const int l0 = a.layer - 1;
  const size_t lb = (static_cast<size_t>(s) * a.max_layers + l0) * n;
  for (int f = threadIdx.x; f < a.W; f += NT) sm.cntp[f] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < kept; i += NT) {
    const OptCand cd = sm.u.in.c[sm.keep_idx[i]];
    sm.fkey[i] = front_key(cd);
    sm.kslot[i] = atomicAdd(&sm.cntp[cd.fj >> 22], 1);
  }
  __syncthreads();
  {
    int mb = 0;
    for (int f = threadIdx.x; f < a.W; f += NT) mb = max(mb, sm.cntp[f]);
    mb = block_max<int, NT / 64>(mb, sm.scan);
    if (mb > kOptBucketMax) {
      // one large group: sort all kept candidates by frontier key
      const int P2 = pow2_at_least(kept > 0 ? kept : 1);   // <= 1024
      constexpr int kPer = 1024 / NT;   // entries a thread holds (kept <= n <= 1024)
      OptKept mine[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int i = threadIdx.x + q * NT;
        mine[q].key = i < kept ? sm.fkey[i] : ~0ull;
        mine[q].score = i < kept ? sm.u.in.c[sm.keep_idx[i]].score : -INFINITY;
        mine[q].pos = i;
      }
      __syncthreads();   // the sort area overlaps the candidates
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int i = threadIdx.x + q * NT;
        if (i < P2) sm.u.srt.k[i] = mine[q];
      }
      __syncthreads();
      bitonic_sort<NT>(sm.u.srt.k, P2, [](const OptKept& x, const OptKept& y) { return x.key < y.key; });
      for (int r = threadIdx.x; r < kept; r += NT) {
        const OptKept k = sm.u.srt.k[r];
        a.lscore[lb + r] = k.score;
        a.lparent[lb + r] = static_cast<int>(k.key >> 54);
        a.ltoken[lb + r] = static_cast<int>(k.key & 0x3FFFFFull);
        sm.kscore[r] = k.score;
      }
    } else {
      int carry = 0;
      for (int f0 = 0; f0 < a.W; f0 += NT) {
        const int f = f0 + threadIdx.x;
        int tot = 0;
        const int ex = block_exclusive_scan<int, NT / 64>(f < a.W ? sm.cntp[f] : 0, sm.scan, &tot);
        if (f < a.W) sm.basep[f] = carry + ex;
        carry += tot;
      }
      __syncthreads();
      for (int i = threadIdx.x; i < kept; i += NT) {
        const int f = static_cast<int>(sm.fkey[i] >> 54);
        sm.memb[sm.basep[f] + sm.kslot[i]] = i;
      }
      __syncthreads();
      for (int i = threadIdx.x; i < kept; i += NT) {
        const unsigned long long me = sm.fkey[i];
        const int f = static_cast<int>(me >> 54);
        const int b0 = sm.basep[f], bn = sm.cntp[f];
        int r = b0;
        for (int q = 0; q < bn; ++q) r += sm.fkey[sm.memb[b0 + q]] < me ? 1 : 0;
        const double sc = sm.u.in.c[sm.keep_idx[i]].score;
        a.lscore[lb + r] = sc;
        a.lparent[lb + r] = f;
        a.ltoken[lb + r] = static_cast<int>(me & 0x3FFFFFull);
        sm.kscore[r] = sc;
      }
    }
  }
  __syncthreads();   // the candidate area is reused from here on
  // ---- the best n so far by (score desc, layer asc, position asc): the old best list
  //      and this layer's nodes, cut by radix selection (the list is kept unordered)
  const int nb = a.bcount[s];
  const size_t bb = static_cast<size_t>(s) * n;
#pragma unroll 4
  for (int e = threadIdx.x; e < nb; e += NT) {
    const double sc = a.bscore[bb + e];
    sm.u.best.score[e] = sc;
    sm.u.best.key[e] = dkey(sc);
    sm.u.best.info[e] = (a.blayer[bb + e] << 16) | a.bpos[bb + e];
  }
  for (int r = threadIdx.x; r < kept; r += NT) {
    const double sc = sm.kscore[r];
    sm.u.best.score[nb + r] = sc;
    sm.u.best.key[nb + r] = dkey(sc);
    sm.u.best.info[nb + r] = (a.layer << 16) | r;
  }
  if (threadIdx.x == 0) {
    sm.ntie = 0;
    sm.nout = 0;
  }
  __syncthreads();
  const int M2 = nb + kept;
  const int nnew = M2 < n ? M2 : n;
  double part = 0.0;
  auto emit = [&](int e) {
    const int o = atomicAdd(&sm.nout, 1);
    const double sc = sm.u.best.score[e];
    a.bscore[bb + o] = sc;
    a.blayer[bb + o] = sm.u.best.info[e] >> 16;
    a.bpos[bb + o] = sm.u.best.info[e] & 0xFFFF;
    part += exp(sc);
  };
  if (M2 <= n) {
    for (int e = threadIdx.x; e < M2; e += NT) emit(e);
  } else {
    const RadixCut cut = radix_topk_cut<NT>(sm.u.best.key, M2, n, sm.rs, 64, kOptGroupMax);
    for (int e = threadIdx.x; e < M2; e += NT) {
      const unsigned long long k = sm.u.best.key[e];
      const unsigned long long km = k & cut.mask;
      if (cut.all_in ? (km >= cut.prefix) : (km > cut.prefix)) {
        emit(e);
      } else if (!cut.all_in && km == cut.prefix) {
        const int t = atomicAdd(&sm.ntie, 1);
        if (t < 1024) {
          sm.tkey[t] = static_cast<unsigned long long>(sm.u.best.info[e]);
          sm.tidx[t] = e;
          if (t < kOptGroupMax) sm.gkey[t] = k;
        }
      }
    }
    __syncthreads();
    if (sm.ntie > 1024) {   // more than 1024 entries share the n-th best score: refuse
      if (threadIdx.x == 0) {
        atomicExch(&a.hdr->err, kErrCapacity);
        a.done[s] = 1;
      }
      return;
    }
    const int nt = sm.ntie;
    for (int t = threadIdx.x; t < nt; t += NT) {
      const unsigned long long me = sm.tkey[t];
      int before = 0;
      if (cut.group) {   // full score key desc, then (layer, position)
        const unsigned long long mk = sm.gkey[t];
        for (int t2 = 0; t2 < nt; ++t2) {
          const unsigned long long ok2 = sm.gkey[t2];
          before += (ok2 > mk || (ok2 == mk && sm.tkey[t2] < me)) ? 1 : 0;
        }
      } else {
        for (int t2 = 0; t2 < nt; ++t2) before += sm.tkey[t2] < me ? 1 : 0;
      }
      if (before < cut.rem) emit(sm.tidx[t]);
    }
  }
  const double E = block_sum<double, NT / 64>(part, sm.red);
  if (threadIdx.x == 0) {
    a.bcount[s] = nnew;
    const double gain = E - a.Eprev[s];
    a.Eprev[s] = E;
    a.nlayers[s] = a.layer;
    if (gain < a.delta || a.layer >= a.max_layers) a.done[s] = 1;
  }
}

// ------------------------------------------------------------------ 5. the final tree

struct OptFinalSmem {
  unsigned bits[64 * 1024 / 32];   // presence of (layer, position), bit (layer-1)*1024 + position
  int wpre[64 * 1024 / 32];        // chosen nodes in earlier words
  int lp[1024];      // (layer << 16) | position of each chosen node, sorted
  short par[1025];
  int scan[kMaxBlockWaves];
};

template <int NT>
__global__ __launch_bounds__(NT) void opt_finalize_kernel(OptArgs a) {
  __shared__ OptFinalSmem sm;
  const int s = blockIdx.x;
  // layer by layer: a sequence is written once, by the first call after its drafting stopped
  if (a.fin != nullptr) {
    const int d = a.done[s], f = a.fin[s];
    if (!d || f) return;
    __syncthreads();   // every thread has read fin before it is set
    if (threadIdx.x == 0) a.fin[s] = 1;
  }
  const int n = a.n;
  const int nb = a.bcount[s];
  const size_t bb = static_cast<size_t>(s) * n;
  // the chosen nodes by (layer, position): a presence bitmap over (layer, position) and
  // prefix counts of its words give every node its rank (the keys are distinct)
  const int nwords = a.max_layers * 32;
  for (int w = threadIdx.x; w < nwords; w += NT) sm.bits[w] = 0u;
  __syncthreads();
  for (int e = threadIdx.x; e < nb; e += NT) {
    const int b = (a.blayer[bb + e] - 1) * 1024 + a.bpos[bb + e];
    atomicOr(&sm.bits[b >> 5], 1u << (b & 31));
  }
  __syncthreads();
  {
    const int per = (nwords + NT - 1) / NT;   // contiguous words per thread
    const int w0 = threadIdx.x * per;
    int loc = 0;
    for (int q = 0; q < per; ++q)
      if (w0 + q < nwords) loc += __popc(sm.bits[w0 + q]);
    int tot = 0;
    int run = block_exclusive_scan<int, NT / 64>(loc, sm.scan, &tot);
    for (int q = 0; q < per; ++q)
      if (w0 + q < nwords) {
        sm.wpre[w0 + q] = run;
        run += __popc(sm.bits[w0 + q]);
      }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nb; e += NT) {
    const int layer = a.blayer[bb + e], pos = a.bpos[bb + e];
    const int b = (layer - 1) * 1024 + pos;
    const int r = sm.wpre[b >> 5] + __popc(sm.bits[b >> 5] & ((1u << (b & 31)) - 1u));
    sm.lp[r] = (layer << 16) | pos;
  }
  __syncthreads();
  const size_t tb = static_cast<size_t>(s) * a.tree.n_cap;
  const int words = a.tree.words;
  if (threadIdx.x == 0) {
    sm.par[0] = -1;
    a.tree.parent[tb] = -1;
    a.tree.token[tb] = -1;
    a.tree.depth[tb] = 0;
    a.tree.row[tb] = 0;
    a.tree.score[tb] = 0.0;
    a.tree.n_nodes[s] = nb + 1;
    a.tree.layers[s] = a.nlayers[s];
  }
  for (int e = threadIdx.x; e < nb; e += NT) {
    const int layer = sm.lp[e] >> 16, pos = sm.lp[e] & 0xFFFF;
    const size_t lb = (static_cast<size_t>(s) * a.max_layers + (layer - 1)) * n + pos;
    int pslot = 0;
    if (layer > 1) {  // the parent (layer-1, its frontier position) is chosen too
      const int want = ((layer - 1) << 16) | a.lparent[lb];
      int lo = 0, hi = nb;
      while (lo < hi) {
        const int m = (lo + hi) >> 1;
        if (sm.lp[m] < want) lo = m + 1; else hi = m;
      }
      pslot = (lo < nb && sm.lp[lo] == want) ? lo + 1 : -1;
      if (pslot < 0) atomicExch(&a.hdr->err, kErrBadTree);
    }
    const int slot = e + 1;
    sm.par[slot] = static_cast<short>(pslot < 0 ? 0 : pslot);
    const size_t o = tb + slot;
    a.tree.parent[o] = pslot;
    a.tree.token[o] = a.ltoken[lb];
    a.tree.depth[o] = layer;
    a.tree.row[o] = 1 + (layer - 1) * n + pos;
    a.tree.score[o] = a.lscore[lb];
  }
  __syncthreads();
  // every node's ancestor-or-self mask, built in registers from the parents in shared memory
  // and stored once
  for (int i = threadIdx.x; i <= nb; i += NT) {
    uint64_t acc[kOptMaxWords];
#pragma unroll
    for (int w = 0; w < kOptMaxWords; ++w) acc[w] = 0ull;
    for (int j = i; j >= 0; j = (j > 0) ? sm.par[j] : -1) {
#pragma unroll
      for (int u = 0; u < kOptMaxWords; ++u)
        if (u == (j >> 6)) acc[u] |= 1ull << (j & 63);
    }
    uint64_t* an = a.tree.anc + (tb + i) * words;
#pragma unroll
    for (int w = 0; w < kOptMaxWords; ++w)
      if (w < words) an[w] = acc[w];
  }
}

// ------------------------------------------------------------------ per-call state

__global__ void opt_init_kernel(OptArgs a) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < a.S) {
    if (a.fin) a.fin[s] = 0;
    a.done[s] = 0;
    a.bcount[s] = 0;
    a.nlayers[s] = 0;
    a.Eprev[s] = 0.0;
    a.ccount[s] = 0u;
  }
}

// ------------------------------------------------------------------ launches

// Layer by layer: the next frontier's width and the done flags, for the caller.
__global__ void opt_report_kernel(OptArgs a) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < a.S) {
    const int d = a.done[s];
    a.w_out[s] = d ? 0 : a.w_next;
    a.done_out[s] = d ? 1 : 0;
  }
}

int launch_opt_report(const OptArgs& a, hipStream_t st) {
  DTV_LAUNCH(opt_report_kernel, dim3((a.S + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_opt_init(const OptArgs& a, hipStream_t st) {
  DTV_LAUNCH(opt_init_kernel, dim3((a.S + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}


// bf16 rows go through the part kernel when its lists and merge hold them.
static bool opt_part_rows(const OptArgs& a) {
  const int np = parts_of(a.V);
  return a.K <= 64 && np <= a.nch && np <= kPartMaxParts && np * a.K <= kPartMergeCap;
}

int launch_opt_layer(OptArgs a, int dtype, hipStream_t st) {
  const dim3 rows(a.S * a.W * a.nch);
  const bool big = a.Kc > 32;
  if (dtype == 1 && opt_part_rows(a)) {
    const int np = parts_of(a.V);
    const int wg = np == 1 ? a.S * ((a.W + 1) / 2) : a.S * a.W * np;   // rows of one part go in pairs
    DTV_LAUNCH(opt_rows_bf16_kernel, dim3(wg), dim3(kPartThreads), 0, st, a);
  } else if (dtype == 1) {
    if (big)
      DTV_LAUNCH((opt_rows_kernel<1, true>), rows, dim3(kBlock), 0, st, a);
    else
      DTV_LAUNCH((opt_rows_kernel<1, false>), rows, dim3(kBlock), 0, st, a);
  } else {
    if (big)
      DTV_LAUNCH((opt_rows_kernel<0, true>), rows, dim3(kBlock), 0, st, a);
    else
      DTV_LAUNCH((opt_rows_kernel<0, false>), rows, dim3(kBlock), 0, st, a);
  }
  if (hipGetLastError() != hipSuccess) return -1;
  DTV_LAUNCH(opt_bound_kernel<kPartThreads>, dim3(a.S), dim3(kPartThreads), 0, st, a);
  if (hipGetLastError() != hipSuccess) return -1;
  if (dtype == 1)
    DTV_LAUNCH(opt_collect_kernel<1>, rows, dim3(kBlock), 0, st, a);
  else
    DTV_LAUNCH(opt_collect_kernel<0>, rows, dim3(kBlock), 0, st, a);
  if (hipGetLastError() != hipSuccess) return -1;
  DTV_LAUNCH(opt_select_kernel<kPartThreads>, dim3(a.S), dim3(kPartThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Lane maxima per full wave for the one-launch root layer (0: that path does not apply):
// a wave is full when its 64 lanes hold in-range elements only, and the bound needs
// (full waves) * Kw >= n with Kw <= 64.
int opt_root_wave_quota(int V, int n, int dtype) {
  const int vec = dtype == 1 ? RowT<1>::VEC : RowT<0>::VEC;
  const int chunk = dtype == 1 ? RowT<1>::CHUNK : RowT<0>::CHUNK;
  const int nch = (V + chunk - 1) / chunk;
  if (nch > kMergeMaxChunks || n > 1023) return 0;
  long full = 0;
  for (int c = 0; c < nch; ++c)
    for (int w = 0; w < kWaves; ++w) {
      const long last = static_cast<long>(c) * chunk + static_cast<long>((kLoads - 1) * kBlock + 64 * w + 63) * vec + vec - 1;
      if (last < V) ++full;
    }
  if (full == 0) return 0;
  const long kw = (n + full - 1) / full;
  return kw <= 64 ? static_cast<int>(kw) : 0;
}

int launch_opt_root(const OptArgs& a, int dtype, hipStream_t st) {
  if (opt_root_one_workgroup(a.V, a.n, dtype)) {
    DTV_LAUNCH(opt_root_bf16_kernel, dim3(a.S), dim3(kPartThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const dim3 grid(a.S * a.nch);
  if (dtype == 1)
    DTV_LAUNCH(opt_root_kernel<1>, grid, dim3(kBlock), 0, st, a);
  else
    DTV_LAUNCH(opt_root_kernel<0>, grid, dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_opt_finalize(const OptArgs& a, hipStream_t st) {
  DTV_LAUNCH(opt_finalize_kernel<kPartThreads>, dim3(a.S), dim3(kPartThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace dtv
