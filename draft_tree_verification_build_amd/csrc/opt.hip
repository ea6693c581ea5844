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
// without sorting them: each row only reports its top-m (m = max(8, ceil(n / W))) and its
// log-sum-exp; the n-th best score among those W*m reported candidates is a lower bound
// `lo` of the layer's n-th best score (n reported candidates reach it). A second pass over
// the rows gathers every candidate whose score is >= lo (a few hundred at the shapes of the
// pages), and one workgroup selects exactly among them in shared memory.
//
// Launches per layer (the host loop knows the frontier width W, which depends only on n
// and V): opt_rows (W x chunks workgroups), opt_bound (1 per sequence), opt_collect
// (W x chunks), opt_select (1 per sequence); then opt_finalize once. A sequence whose
// drafting has stopped makes every later launch return at once.
#include "dtv_internal.h"
#include "rowstats.h"

namespace dtv {

constexpr int kOptMergeCap = 8192;  // chunks * K of one row merge
constexpr int kOptLdsCand = 4096;   // candidates selected in shared memory

struct OptCand {
  double score;
  int f;   // frontier position of the parent
  int j;   // vocabulary index (the token)
};

// (score desc, parent position asc, token asc): ranks candidates of one layer. Within a
// row, equal logits rank by token index, so this is also (score desc, parent, rank).
__device__ __forceinline__ bool cand_before(const OptCand& a, const OptCand& b) {
  if (a.score != b.score) return a.score > b.score;
  if (a.f != b.f) return a.f < b.f;
  return a.j < b.j;
}


// In-place bitonic sort of n (power of two) elements of shared memory by `before`.
template <typename T, typename Cmp>
__device__ void bitonic_sort(T* a, int n, Cmp before) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kBlock) {
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
  return a.layer == 1 ? 0 : 1 + (a.layer - 2) * a.n + f;
}

__device__ __forceinline__ double parent_score(const OptArgs& a, int s, int f) {
  return a.layer == 1 ? 0.0 : a.lscore[(static_cast<size_t>(s) * a.max_layers + (a.layer - 2)) * a.n + f];
}

// ------------------------------------------------------------------ 1. frontier rows

template <int DT>
__global__ __launch_bounds__(kBlock) void opt_rows_kernel(OptArgs a) {
  __shared__ RowSmem rs;
  __shared__ MergeSmem<kOptMergeCap> ms;
  __shared__ unsigned long long sortbuf[4 * 1024];
  using Rw = RowT<DT>;
  int bid = blockIdx.x;
  const int c = bid % a.nch;
  bid /= a.nch;
  const int f = bid % a.W;
  const int s = bid / a.W;
  if (ld_cc(&a.done[s])) return;
  row_smem_init(rs);
  __syncthreads();
  const char* row = static_cast<const char*>(a.draft) +
                    (static_cast<size_t>(s) * a.R + row_of(a, f)) * static_cast<size_t>(a.V) * Rw::ESIZE;
  float x[Rw::E];
  uint32_t key[Rw::E];
  load_chunk<DT>(row, a.V, c, x, key);
  const size_t rf = static_cast<size_t>(s) * a.Wcap + f;
  const size_t ci = rf * a.nch + c;
  chunk_reduce<DT>(x, key, c, a.V, a.K, &a.st[ci], a.cval + ci * a.K, a.cidx + ci * a.K, sortbuf, rs);
  if (!last_arrival(&a.tickets[rf], a.nch, &rs.flag)) return;
  const int n = row_merge(a.st + rf * a.nch, a.cval + rf * a.nch * a.K, a.cidx + rf * a.nch * a.K, a.nch, a.K,
                          nullptr, nullptr, &a.rlse[rf], a.rv + rf * a.K, a.ri + rf * a.K, rs, ms);
  if (threadIdx.x == 0) st_cc(&a.rcnt[rf], n);
}

// ------------------------------------------------------------------ 2. lower bound

struct OptBoundSmem {
  unsigned long long key[8192];
  int off[1024];
  int wsum[kWaves];
};

__global__ __launch_bounds__(kBlock) void opt_bound_kernel(OptArgs a) {
  __shared__ OptBoundSmem sm;
  const int s = blockIdx.x;
  if (a.done[s]) return;
  // the reported candidates: the top-m of every row (m = K), packed row after row
  int carry = 0;
  for (int f0 = 0; f0 < a.W; f0 += kBlock) {
    const int f = f0 + threadIdx.x;
    const int cnt = (f < a.W) ? a.rcnt[static_cast<size_t>(s) * a.Wcap + f] : 0;
    int tot = 0;
    const int ex = block_exclusive_scan(cnt, sm.wsum, &tot);
    if (f < a.W) sm.off[f] = carry + ex;
    carry += tot;
  }
  const int total = carry;
  const int P2 = pow2_at_least(total > 0 ? total : 1);
  for (int e = threadIdx.x; e < P2; e += kBlock) sm.key[e] = 0ull;
  __syncthreads();
  for (int e = threadIdx.x; e < a.W * a.K; e += kBlock) {
    const int f = e / a.K, j = e % a.K;
    const size_t rf = static_cast<size_t>(s) * a.Wcap + f;
    if (j < a.rcnt[rf]) {
      const double sc = parent_score(a, s, f) + (static_cast<double>(a.rv[rf * a.K + j]) - a.rlse[rf]);
      sm.key[sm.off[f] + j] = dkey(sc);
    }
  }
  __syncthreads();
  // descending sort of the keys; the n-th largest bounds the layer's n-th best score
  bitonic_sort(sm.key, P2, [](unsigned long long x, unsigned long long y) { return x > y; });
  if (threadIdx.x == 0) {
    double lo = -INFINITY;
    if (total >= a.n) {
      const unsigned long long k = sm.key[a.n - 1];
      const unsigned long long u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
      lo = __longlong_as_double(static_cast<long long>(u));
    }
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
  if (a.done[s]) return;
  const double lo = a.lo[s];
  const size_t rf = static_cast<size_t>(s) * a.Wcap + f;
  const double base = parent_score(a, s, f);
  const double lse = a.rlse[rf];
  // a chunk whose largest logit cannot reach lo has no candidate: skip reading it
  const float cmax = a.st[rf * a.nch + c].maxv;
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
          out->f = f;
          out->j = elem_index<DT>(c, i, e);
        }
      }
    }
}

// ------------------------------------------------------------------ 4. exact selection

struct OptSelectSmem {
  OptCand c[kOptLdsCand];
  OptCand merged[1024];
  int pos[1024];
  double red[kWaves];
  int ired[kWaves];
  int flag;
};

// Rank of candidate x in a list sorted by `before` (number of list entries before it).
template <typename Cmp>
__device__ __forceinline__ int rank_in(const OptCand* list, int n, const OptCand& x, Cmp before) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int m = (lo + hi) >> 1;
    if (before(list[m], x)) lo = m + 1; else hi = m;
  }
  return lo;
}

__global__ __launch_bounds__(kBlock) void opt_select_kernel(OptArgs a) {
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
  const int P2 = pow2_at_least(C > 0 ? C : 1);
  for (int e = threadIdx.x; e < P2; e += kBlock) {
    if (e < C) {
      sm.c[e] = a.cand[static_cast<size_t>(s) * a.ccap + e];
    } else {
      sm.c[e].score = -INFINITY;
      sm.c[e].f = 0x7FFFFFFF;
      sm.c[e].j = 0x7FFFFFFF;
    }
  }
  __syncthreads();
  bitonic_sort(sm.c, P2, cand_before);     // best first
  const int kept = C < n ? C : n;          // the layer keeps its best n
  // frontier order of the kept candidates: (parent position, rank) = (f, score desc, j)
  // written to the layer record; scores to the best-so-far merge below
  const int l0 = a.layer - 1;
  const size_t lb = (static_cast<size_t>(s) * a.max_layers + l0) * n;
  // position of each kept candidate in frontier order = number of kept candidates before it
  for (int e = threadIdx.x; e < kept; e += kBlock) {
    const OptCand me = sm.c[e];
    int pos = 0;
    for (int e2 = 0; e2 < kept; ++e2) {
      const OptCand o = sm.c[e2];
      const bool before = (o.f < me.f) || (o.f == me.f && (o.score > me.score || (o.score == me.score && o.j < me.j)));
      pos += before ? 1 : 0;
    }
    a.lscore[lb + pos] = me.score;
    a.lparent[lb + pos] = me.f;
    a.ltoken[lb + pos] = me.j;
    sm.pos[e] = pos;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kept; e += kBlock) sm.c[e].f = sm.pos[e];  // now: position in the layer
  __syncthreads();
  // best n of all layers so far: merge the previous best (sorted by score desc, layer asc,
  // position asc) with this layer's kept nodes (sorted by score desc, position asc)
  const int nb = a.bcount[s];
  const size_t bb = static_cast<size_t>(s) * n;
  for (int e = threadIdx.x; e < nb + kept; e += kBlock) {
    OptCand me;
    int r;
    if (e < nb) {
      me.score = a.bscore[bb + e];
      me.j = a.blayer[bb + e];
      me.f = a.bpos[bb + e];
      // entries of this layer before me (previous layers win ties)
      int lo = 0, hi = kept;
      while (lo < hi) {
        const int m = (lo + hi) >> 1;
        if (sm.c[m].score > me.score) lo = m + 1; else hi = m;
      }
      r = e + lo;
    } else {
      const int q = e - nb;
      me.score = sm.c[q].score;
      me.j = a.layer;
      me.f = sm.c[q].f;
      int lo = 0, hi = nb;  // previous entries with score >= mine come first
      while (lo < hi) {
        const int m = (lo + hi) >> 1;
        if (a.bscore[bb + m] >= me.score) lo = m + 1; else hi = m;
      }
      // this layer's entries before me: q (the kept list is sorted by score desc, position asc)
      r = q + lo;
    }
    if (r < n) sm.merged[r] = me;
  }
  __syncthreads();
  const int nnew = (nb + kept) < n ? (nb + kept) : n;
  double part = 0.0;
  for (int e = threadIdx.x; e < nnew; e += kBlock) {
    a.bscore[bb + e] = sm.merged[e].score;
    a.blayer[bb + e] = sm.merged[e].j;
    a.bpos[bb + e] = sm.merged[e].f;
    part += exp(sm.merged[e].score);
  }
  const double E = block_sum(part, sm.red);
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
  int lp[1024];      // (layer << 16) | position of each chosen node, sorted
  short par[1025];
  int flag;
};

__global__ __launch_bounds__(kBlock) void opt_finalize_kernel(OptArgs a) {
  __shared__ OptFinalSmem sm;
  const int s = blockIdx.x;
  const int n = a.n;
  const int nb = a.bcount[s];
  const size_t bb = static_cast<size_t>(s) * n;
  const int P2 = pow2_at_least(nb > 0 ? nb : 1);
  for (int e = threadIdx.x; e < P2; e += kBlock)
    sm.lp[e] = (e < nb) ? ((a.blayer[bb + e] << 16) | a.bpos[bb + e]) : 0x7FFFFFFF;
  __syncthreads();
  bitonic_sort(sm.lp, P2, [](int x, int y) { return x < y; });   // by (layer, position)
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
  for (int e = threadIdx.x; e < nb; e += kBlock) {
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
  for (int i = threadIdx.x; i <= nb; i += kBlock) {
    uint64_t* an = a.tree.anc + (tb + i) * words;
    for (int w = 0; w < words; ++w) an[w] = 0ull;
    for (int j = i; j >= 0; j = (j > 0) ? sm.par[j] : -1) an[j >> 6] |= 1ull << (j & 63);
  }
}

// ------------------------------------------------------------------ per-call state

__global__ void opt_init_kernel(OptArgs a) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < a.S) {
    a.done[s] = 0;
    a.bcount[s] = 0;
    a.nlayers[s] = 0;
    a.Eprev[s] = 0.0;
    a.ccount[s] = 0u;
  }
}

// ------------------------------------------------------------------ launches

int launch_opt_init(const OptArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(opt_init_kernel, dim3((a.S + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}


int launch_opt_layer(OptArgs a, int dtype, hipStream_t st) {
  const dim3 rows(a.S * a.W * a.nch);
  if (dtype == 1)
    hipLaunchKernelGGL(opt_rows_kernel<1>, rows, dim3(kBlock), 0, st, a);
  else
    hipLaunchKernelGGL(opt_rows_kernel<0>, rows, dim3(kBlock), 0, st, a);
  if (hipGetLastError() != hipSuccess) return -1;
  hipLaunchKernelGGL(opt_bound_kernel, dim3(a.S), dim3(kBlock), 0, st, a);
  if (hipGetLastError() != hipSuccess) return -1;
  if (dtype == 1)
    hipLaunchKernelGGL(opt_collect_kernel<1>, rows, dim3(kBlock), 0, st, a);
  else
    hipLaunchKernelGGL(opt_collect_kernel<0>, rows, dim3(kBlock), 0, st, a);
  if (hipGetLastError() != hipSuccess) return -1;
  hipLaunchKernelGGL(opt_select_kernel, dim3(a.S), dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_opt_finalize(const OptArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(opt_finalize_kernel, dim3(a.S), dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace dtv
