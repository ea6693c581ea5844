// Draft-tree builders on gfx950: given shapes and TALON budget-driven expansion.
//
// TALON (TALON page, sections 5.1-5.2) grows the tree layer by layer: the root layer is
// the Top-K of the root's draft distribution; every later layer pools the Top-K children
// of each node of the previous layer, scores them with the product of draft
// probabilities along the path (kept as a sum of logs), keeps those within a factor
// alpha of the best (the anchor) and, if more pass than budget remains, the best by
// score. The whole layer loop is one cooperative launch: every workgroup reduces chunks
// of the frontier's draft rows (phase A), a grid barrier publishes the row results, and
// every workgroup then runs the same deterministic selection (phase B) so that all of
// them know the next frontier without a second barrier; workgroup 0 writes the nodes.
#include "dtv_internal.h"
#include "rowstats.h"

namespace dtv {

// ------------------------------------------------------------------ given trees

constexpr int kMaxWords = 16;  // n_cap <= 1024

__global__ __launch_bounds__(kBlock) void given_tree_kernel(TreeArgs t, WsHeader* hdr) {
  const int s = blockIdx.x;
  const int cap = t.n_cap;
  const int N = t.n_nodes[s];
  if (N < 1 || N > cap) {
    if (threadIdx.x == 0) atomicExch(&hdr->err, kErrCapacity);
    return;
  }
  const size_t base = static_cast<size_t>(s) * cap;
  for (int i = threadIdx.x; i < N; i += kBlock) {
    uint64_t acc[kMaxWords];
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w) acc[w] = 0;
    int depth = 0;
    int j = i;
    bool ok = true;
    while (j > 0) {
      const int w = j >> 6;
#pragma unroll
      for (int u = 0; u < kMaxWords; ++u)
        if (u == w) acc[u] |= 1ull << (j & 63);
      const int p = t.parent[base + j];
      if (p < 0 || p >= j) {
        ok = false;
        break;
      }
      j = p;
      ++depth;
    }
    acc[0] |= 1ull;
    if (!ok) atomicExch(&hdr->err, kErrBadTree);
    t.depth[base + i] = depth;
    t.row[base + i] = i;
    t.score[base + i] = 0.0;
    uint64_t* a = t.anc + (base + i) * t.words;
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w)
      if (w < t.words) a[w] = acc[w];
  }
  if (threadIdx.x == 0) t.layers[s] = 0;
}

int launch_given(const TreeArgs& t, int S, WsHeader* hdr, hipStream_t st) {
  hipLaunchKernelGGL(given_tree_kernel, dim3(S), dim3(kBlock), 0, st, t, hdr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------ TALON

constexpr int kTalonMaxK = 64;
constexpr int kTalonMaxPool = 4096;
constexpr int kTalonMaxS = 64;
constexpr int kTalonMergeCap = 2048;  // chunks_of(V) * K must not exceed this
constexpr int kTalonTreeCap = 2048;   // S * n_cap must not exceed this

struct TalonSmem {
  RowSmem rs;
  MergeSmem<kTalonMergeCap> ms;
  unsigned long long sortbuf[pow2_at_least(kWaves * kTalonMaxK) > kCandCap ? pow2_at_least(kWaves * kTalonMaxK)
                                                                           : kCandCap];
  double pool[kTalonMaxPool];     // scores of the candidate pool of one sequence
  int ptok[kTalonMaxPool];        // tokens of the candidate pool
  double tscore[kTalonTreeCap];   // every node's log path score, all sequences
  short tpar[kTalonTreeCap];      // every node's parent slot, all sequences
  int gated[1024];                // per frontier row: entries passing the gate
  int kept[1024];                 // per frontier row: entries kept
  int scan[kBlock];
  int cnt[kTalonMaxS], start[kTalonMaxS], width[kTalonMaxS], done[kTalonMaxS], nlayers[kTalonMaxS];
  int flag;
};

template <int DT>
__global__ __launch_bounds__(kBlock) void talon_kernel(TalonArgs a) {
  __shared__ TalonSmem sm;
  using Rw = RowT<DT>;
  const int nch = a.nch;
  const int K = a.K;
  const int B = a.B;
  const int cap = a.tree.n_cap;
  const size_t row_bytes = static_cast<size_t>(a.V) * Rw::ESIZE;

  row_smem_init(sm.rs);
  for (int s = threadIdx.x; s < a.S; s += kBlock) {
    sm.cnt[s] = 0;
    sm.start[s] = 0;
    sm.width[s] = 1;
    sm.done[s] = 0;
    sm.nlayers[s] = 0;
    sm.tscore[s * cap] = 0.0;
    sm.tpar[s * cap] = -1;
  }
  __syncthreads();

  float x[Rw::E];
  uint32_t key[Rw::E];
  int layer = 0;
  bool ok = true;
  for (;;) {
    ++layer;
    // ---------------- phase A: reduce the frontier rows chunk by chunk
    int total = 0;
    for (int s = 0; s < a.S; ++s) total += sm.done[s] ? 0 : sm.width[s] * nch;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
      int rest = item, s = 0;
      for (; s < a.S; ++s) {
        const int n = sm.done[s] ? 0 : sm.width[s] * nch;
        if (rest < n) break;
        rest -= n;
      }
      const int f = rest / nch, c = rest % nch;
      const int slot = sm.start[s] + f;              // rows are keyed by slot
      const char* row = static_cast<const char*>(a.draft) +
                        (static_cast<size_t>(s) * a.R + slot) * row_bytes;
      load_chunk<DT>(row, a.V, c, x, key);
      const size_t rf = static_cast<size_t>(s) * B + f;
      const size_t ci = rf * nch + c;
      chunk_reduce<DT>(x, key, c, a.V, K, &a.st[ci], a.cval + ci * K, a.cidx + ci * K, sm.sortbuf, sm.rs);
      if (last_arrival(&a.tickets[rf], nch, &sm.flag)) {
        const int n = row_merge(a.st + rf * nch, a.cval + rf * nch * K, a.cidx + rf * nch * K, nch, K,
                                nullptr, nullptr, &a.rlse[rf], a.rv + rf * K, a.ri + rf * K, sm.rs, sm.ms);
        if (threadIdx.x == 0) st_cc(&a.rcnt[rf], n);
      }
    }
    if (!grid_barrier(a.hdr->bar, gridDim.x, &a.hdr->err, kErrTimeout, &sm.flag)) {
      ok = false;
      break;
    }

    // ---------------- phase B: the same selection in every workgroup
    int all_done = 1;
    for (int s = 0; s < a.S; ++s) {
      if (sm.done[s]) continue;
      const int W = sm.width[s];
      const int cnt = sm.cnt[s];
      const int room = B - cnt;
      const size_t rf0 = static_cast<size_t>(s) * B;
      const size_t tb = static_cast<size_t>(s) * cap;
      // pool scores: s(c) = s(parent) + log p_d(token | parent)
      for (int e = threadIdx.x; e < W * K; e += kBlock) {
        const int f = e / K, j = e % K;
        double v = -INFINITY;
        int tok = -1;
        if (j < ld_cc(&a.rcnt[rf0 + f])) {
          v = sm.tscore[tb + sm.start[s] + f] +
              (static_cast<double>(ld_cc(&a.rv[(rf0 + f) * K + j])) - ld_cc(&a.rlse[rf0 + f]));
          tok = ld_cc(&a.ri[(rf0 + f) * K + j]);
        }
        sm.pool[e] = v;
        sm.ptok[e] = tok;
      }
      __syncthreads();
      if (layer == 1) {
        // robust initialisation: the root's Top-K, at most the budget, no gate
        if (threadIdx.x == 0) {
          const int n = ld_cc(&a.rcnt[rf0]);
          sm.kept[0] = n < room ? n : room;
        }
        __syncthreads();
      } else {
        double mx = -INFINITY;
        for (int f = threadIdx.x; f < W; f += kBlock) mx = fmax(mx, sm.pool[f * K]);
        const double anchor = block_max(mx, sm.rs.redd);
        const double thr = a.log_alpha + anchor;
        int tg = 0;
        for (int f = threadIdx.x; f < W; f += kBlock) {
          int g = 0;
          while (g < K && sm.pool[f * K + g] >= thr) ++g;
          sm.gated[f] = g;
          tg += g;
        }
        tg = block_sum(tg, sm.rs.redi);
        if (tg <= room) {
          for (int f = threadIdx.x; f < W; f += kBlock) sm.kept[f] = sm.gated[f];
          __syncthreads();
        } else {
          // budget respect: keep the `room` best gated candidates, ordered by
          // (score desc, parent slot asc, rank asc); kept entries of a row are a prefix
          for (int f = threadIdx.x; f < W; f += kBlock) sm.kept[f] = 0;
          __syncthreads();
          for (int e = threadIdx.x; e < W * K; e += kBlock) {
            const int f = e / K, j = e % K;
            if (j >= sm.gated[f]) continue;
            const double v = sm.pool[e];
            int rank = j;
            for (int f2 = 0; f2 < W && rank < room; ++f2) {
              if (f2 == f) continue;
              const int g2 = sm.gated[f2];
              int c2 = 0;
              if (f2 < f) {
                while (c2 < g2 && sm.pool[f2 * K + c2] >= v) ++c2;
              } else {
                while (c2 < g2 && sm.pool[f2 * K + c2] > v) ++c2;
              }
              rank += c2;
            }
            if (rank < room) atomicAdd(&sm.kept[f], 1);
          }
          __syncthreads();
        }
      }
      // new slots in (parent slot, rank) order; every workgroup records parents and
      // scores in shared memory, workgroup 0 also writes the node arrays
      int carry = 0;
      for (int f0 = 0; f0 < W; f0 += kBlock) {
        const int f = f0 + threadIdx.x;
        const int mine = (f < W) ? sm.kept[f] : 0;
        int tot = 0;
        const int ex = block_exclusive_scan(mine, sm.scan, &tot);
        if (f < W) {
          const int parent = sm.start[s] + f;
          for (int j = 0; j < mine; ++j) {
            const int slot = cnt + 1 + carry + ex + j;
            const double sc = sm.pool[f * K + j];
            sm.tscore[tb + slot] = sc;
            sm.tpar[tb + slot] = static_cast<short>(parent);
            if (blockIdx.x == 0) {
              const size_t o = tb + slot;
              a.tree.parent[o] = parent;
              a.tree.token[o] = sm.ptok[f * K + j];
              a.tree.depth[o] = layer;
              a.tree.row[o] = slot;
              a.tree.score[o] = sc;
            }
          }
        }
        carry += tot;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        sm.start[s] = cnt + 1;
        sm.width[s] = carry;
        sm.cnt[s] = cnt + carry;
        sm.nlayers[s] = layer;
        if (sm.cnt[s] >= B || carry == 0) sm.done[s] = 1;
        if (carry == 0) atomicExch(&a.hdr->err, kErrCapacity);
      }
      __syncthreads();
      if (!sm.done[s]) all_done = 0;
    }
    if (all_done) break;
  }

  // ---------------- outputs of workgroup 0: root, counts and ancestor masks
  if (blockIdx.x != 0 || !ok) return;
  for (int s = threadIdx.x; s < a.S; s += kBlock) {
    const size_t b = static_cast<size_t>(s) * cap;
    a.tree.parent[b] = -1;
    a.tree.token[b] = -1;
    a.tree.depth[b] = 0;
    a.tree.row[b] = 0;
    a.tree.score[b] = 0.0;
    a.tree.n_nodes[s] = sm.cnt[s] + 1;
    a.tree.layers[s] = sm.nlayers[s];
  }
  const int words = a.tree.words;
  for (int e = threadIdx.x; e < a.S * cap; e += kBlock) {
    const int s = e / cap, i = e % cap;
    if (i > sm.cnt[s]) continue;
    uint64_t acc[kMaxWords];
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w) acc[w] = 0;
    for (int j = i; j >= 0; j = (j > 0) ? sm.tpar[s * cap + j] : -1) {
#pragma unroll
      for (int u = 0; u < kMaxWords; ++u)
        if (u == (j >> 6)) acc[u] |= 1ull << (j & 63);
    }
    uint64_t* an = a.tree.anc + static_cast<size_t>(e) * words;
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w)
      if (w < words) an[w] = acc[w];
  }
}

// ------------------------------------------------------------------ GOOSE spine trees
//
// GOOSE page, section 2A: a deep chain of context-match tokens (the spine) with wide,
// shallow branches forking at spine nodes. Slots 1..n_spine hold the spine (slot k has
// parent k-1); fork f (slot f, the root or a spine node) then gets width[f] depth-1
// branches, the most probable tokens of its draft row that are not its spine child's token,
// in slots 1 + n_spine + offset[f] + j. The spine holds the lowest slots, which is what
// lets a greedy walk that prefers low slots follow the spine first (section 2C).
//
// One workgroup per (sequence, fork, chunk of the fork's draft row); the workgroup that
// completes a fork row merges its chunks and writes that fork's branch nodes. Branch
// scores are log p_d(token | fork) (spine nodes carry no draft score).

constexpr int kSpineMaxK = 65;

template <int DT>
__global__ __launch_bounds__(kBlock) void spine_kernel(SpineArgs a) {
  __shared__ RowSmem rs;
  __shared__ MergeSmem<kTalonMergeCap> ms;
  __shared__ unsigned long long sortbuf[pow2_at_least(kWaves * 128) > kCandCap ? pow2_at_least(kWaves * 128)
                                                                              : kCandCap];
  using Rw = RowT<DT>;
  row_smem_init(rs);
  __syncthreads();
  const int nch = a.nch;
  const int K = a.K;
  const int cap = a.tree.n_cap;
  int bid = blockIdx.x;
  const int c = bid % nch;
  bid /= nch;
  const int f = bid % a.F;
  const int s = bid / a.F;
  const size_t tb = static_cast<size_t>(s) * cap;
  const int words = a.tree.words;

  if (f == 0 && c == 0) {  // root and spine chain of sequence s
    for (int k = threadIdx.x; k <= a.n_spine; k += kBlock) {
      const size_t o = tb + k;
      a.tree.parent[o] = k - 1;
      a.tree.token[o] = (k == 0) ? -1 : a.spine[static_cast<size_t>(s) * a.n_spine + k - 1];
      a.tree.depth[o] = k;
      a.tree.row[o] = k;
      a.tree.score[o] = 0.0;
      uint64_t* an = a.tree.anc + o * words;
      for (int w = 0; w < words; ++w) {  // bits 0..k
        const int lo = w * 64;
        const int nb = k + 1 - lo;
        an[w] = nb <= 0 ? 0ull : (nb >= 64 ? ~0ull : ((1ull << nb) - 1ull));
      }
    }
    if (threadIdx.x == 0) {
      a.tree.n_nodes[s] = a.n_nodes;
      a.tree.layers[s] = 1;
    }
  }
  const int wf = a.width[f];
  if (wf <= 0) return;
  const int kf = wf + 1 < a.V ? wf + 1 : a.V;   // one spare for the skipped spine token
  const char* row = static_cast<const char*>(a.draft) +
                    (static_cast<size_t>(s) * a.R + f) * static_cast<size_t>(a.V) * Rw::ESIZE;
  float x[Rw::E];
  uint32_t key[Rw::E];
  load_chunk<DT>(row, a.V, c, x, key);
  const size_t rf = static_cast<size_t>(s) * a.F + f;
  const size_t ci = rf * nch + c;
  chunk_reduce<DT>(x, key, c, a.V, kf, &a.st[ci], a.cval + ci * K, a.cidx + ci * K, sortbuf, rs);
  if (!last_arrival(&a.tickets[rf], nch, &rs.flag)) return;
  // the chunk lists were written with stride K; merge with that stride, keep kf entries
  const int n = row_merge(a.st + rf * nch, a.cval + rf * nch * K, a.cidx + rf * nch * K, nch, K,
                          nullptr, nullptr, &a.rlse[rf], a.rv + rf * K, a.ri + rf * K, rs, ms);
  if (threadIdx.x == 0) {
    const double lse = ld_cc(&a.rlse[rf]);
    const int skip = (f < a.n_spine) ? a.spine[static_cast<size_t>(s) * a.n_spine + f] : -1;
    int j = 0;
    for (int r = 0; r < n && r < kf && j < wf; ++r) {
      const int tok = ld_cc(&a.ri[rf * K + r]);
      if (tok == skip) continue;
      const int slot = 1 + a.n_spine + a.offset[f] + j;
      const size_t o = tb + slot;
      a.tree.parent[o] = f;
      a.tree.token[o] = tok;
      a.tree.depth[o] = f + 1;
      a.tree.row[o] = slot;
      a.tree.score[o] = static_cast<double>(ld_cc(&a.rv[rf * K + r])) - lse;
      uint64_t* an = a.tree.anc + o * words;
      for (int w = 0; w < words; ++w) {  // bits 0..f plus the node itself
        const int lo = w * 64;
        const int nb = f + 1 - lo;
        uint64_t bits = nb <= 0 ? 0ull : (nb >= 64 ? ~0ull : ((1ull << nb) - 1ull));
        if ((slot >> 6) == w) bits |= 1ull << (slot & 63);
        an[w] = bits;
      }
      ++j;
    }
  }
}

int launch_spine(const SpineArgs& a, int dtype, hipStream_t st) {
  const dim3 grid(a.S * a.F * a.nch);
  if (dtype == 1)
    hipLaunchKernelGGL(spine_kernel<1>, grid, dim3(kBlock), 0, st, a);
  else
    hipLaunchKernelGGL(spine_kernel<0>, grid, dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_talon(const TalonArgs& a, int dtype, int grid, hipStream_t st) {
  void* args[] = {const_cast<TalonArgs*>(&a)};
  hipError_t e;
  if (dtype == 1)
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&talon_kernel<1>), dim3(grid),
                                   dim3(kBlock), args, 0, st);
  else
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&talon_kernel<0>), dim3(grid),
                                   dim3(kBlock), args, 0, st);
  return e == hipSuccess ? 0 : -1;
}

int talon_max_grid(int dtype) {
  // one workgroup per compute unit; queried once per device and dtype
  static int cached[64][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  int& c = cached[dev][dtype ? 1 : 0];
  if (c > 0) return c;
  int ncu = 0, per = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  hipError_t e = (dtype == 1)
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(&talon_kernel<1>), kBlock, 0)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(&talon_kernel<0>), kBlock, 0);
  if (e != hipSuccess || per < 1) return -1;
  c = ncu;
  return c;
}

}  // namespace dtv
