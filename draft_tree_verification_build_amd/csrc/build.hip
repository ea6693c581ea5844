// Draft-tree builders on gfx950: given shapes and TALON budget-driven expansion.
//
// TALON (TALON page, sections 5.1-5.2) grows the tree layer by layer: the root layer is
// the Top-K of the root's draft distribution; every later layer pools the Top-K children
// of each node of the previous layer, scores them with the product of draft
// probabilities along the path (kept as a sum of logs), keeps those within a factor
// alpha of the best (the anchor) and, if more pass than budget remains, the best by
// score. Rows are keyed by slot, and only slots 0..B-1 can ever be expanded (the node in
// slot B completes the budget), so the vocab-wide part does not depend on the tree: one
// data-parallel launch reduces draft rows 0..B-1 of every sequence (Top-K and log-sum-exp
// per row, one workgroup per row chunk), and a second launch runs the whole layer loop
// of one sequence inside one workgroup on those small per-row lists.
#include "dtv_internal.h"
#include "rows_bf16.h"
#include "rowstats.h"
#include "select.h"

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
  // the parents in shared memory first (all loads in flight together), so that each node's
  // walk to the root is a chain of shared-memory reads, not of global loads
  __shared__ int par[kMaxWords * 64];
  constexpr int kPer = kMaxWords * 64 / kBlock;
  int pv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) pv[u] = t.parent[base + min(static_cast<int>(threadIdx.x) + u * kBlock, N - 1)];
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (static_cast<int>(threadIdx.x) + u * kBlock < N) par[threadIdx.x + u * kBlock] = pv[u];
  __syncthreads();
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
      const int p = par[j];
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
  DTV_LAUNCH(given_tree_kernel, dim3(S), dim3(kBlock), 0, st, t, hdr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------ TALON

constexpr int kTalonMaxK = 64;
constexpr int kTalonMaxPool = 4096;
constexpr int kTalonMergeCap = 2048;  // chunks_of(V) * K must not exceed this

// Phase 1: one workgroup per (sequence, row f < B, chunk). The workgroup that completes a
// row merges its chunks into the row's Top-K (value, token), count and log-sum-exp.
template <int DT>
__global__ __launch_bounds__(kBlock, 4) void talon_rows_kernel(TalonArgs a) {
  __shared__ RowSmem rs;
  __shared__ MergeSmem<kTalonMergeCap> ms;
  __shared__ unsigned long long sortbuf[pow2_at_least(kWaves * kTalonMaxK) > kCandCap
                                            ? pow2_at_least(kWaves * kTalonMaxK) : kCandCap];
  using Rw = RowT<DT>;
  const int nch = a.nch;
  const int K = a.K;
  const int c = blockIdx.x % nch;
  const int rf = blockIdx.x / nch;         // s * Wr + f
  const int s = rf / a.Wr, f = rf % a.Wr;  // row f of sequence s is draft row f
  if (a.state != nullptr && a.layer > 1) {  // layer by layer: the frontier's rows only
    const int* st = a.state + 8 * s;
    if (st[4] != 0 || f >= st[2]) return;
  }
  const char* row = static_cast<const char*>(a.draft) +
                    (static_cast<size_t>(s) * a.R + f) * static_cast<size_t>(a.V) * Rw::ESIZE;
  // the exp table and the chunk in one round trip
  row_smem_issue(rs);
  float x[Rw::E];
  uint32_t key[Rw::E];
  load_chunk<DT>(row, a.V, c, x, key);
  drain();
  __syncthreads();
  const size_t ci = static_cast<size_t>(rf) * nch + c;
  chunk_reduce<DT>(x, key, c, a.V, K, &a.st[ci], a.cval + ci * K, a.cidx + ci * K, sortbuf, rs);
  if (last_arrival(&a.tickets[rf], nch, &rs.flag)) {
    const size_t rb = static_cast<size_t>(rf) * nch;
    const int n = row_merge(a.st + rb, a.cval + rb * K, a.cidx + rb * K, nch, K, nullptr, nullptr,
                            &a.rlse[rf], a.rv + static_cast<size_t>(rf) * K, a.ri + static_cast<size_t>(rf) * K,
                            rs, ms);
    if (threadIdx.x == 0) a.rcnt[rf] = n;
  }
}

// Phase 1 for bf16 rows: one 1024-thread workgroup per (sequence, row f < B, part of 32768
// values). The workgroup that completes a row merges its parts into the row's Top-K (value,
// token), count and log-sum-exp; a row of one part is complete on its own.
__global__ __launch_bounds__(kPartThreads) void talon_rows_bf16_kernel(TalonArgs a) {
  __shared__ PartSmem sm;
  const int np = parts_of(a.V);
  const int p = blockIdx.x % np;
  const int rf = blockIdx.x / np;          // s * Wr + f
  const int s = rf / a.Wr, f = rf % a.Wr;  // row f of sequence s is draft row f
  if (a.state != nullptr && a.layer > 1) {  // layer by layer: the frontier's rows only
    const int* st = a.state + 8 * s;
    if (st[4] != 0 || f >= st[2]) return;
  }
  const uint16_t* row = static_cast<const uint16_t*>(a.draft) + (static_cast<size_t>(s) * a.R + f) * static_cast<size_t>(a.V);
  const int K = a.K;
  float* rv = a.rv + static_cast<size_t>(rf) * K;
  int* ri = a.ri + static_cast<size_t>(rf) * K;
  const size_t ci = static_cast<size_t>(rf) * a.nch;   // the row's chunk slots hold its parts
  part_row_reduce(row, a.V, p, np, K, a.cval + ci * K, a.cidx + ci * K, reinterpret_cast<PartStat*>(a.st + ci),
                  &a.tickets[rf], &a.rlse[rf], rv, ri, &a.rcnt[rf], sm, nullptr, &a.hdr->err, true);
}

struct TalonSelSmem {
  double redd[kWaves];
  int redi[kWaves];
  RadixSmem rs;
  double lp[kTalonMaxPool];     // log p_d of every row's list entries, row f at f*K
  int tok[kTalonMaxPool];       // their tokens
  double csc[kTalonMaxPool];    // scores of the current layer's candidates, e = f*K + j
  unsigned long long ckey[kTalonMaxPool];   // their order keys while selecting (0: not gated)
  int rcnt[1024];               // list length of every row
  double tscore[1024];          // log path score of every slot
  short tpar[1024];             // parent of every slot
  int gated[1024];              // per frontier row: candidates passing the gate
  int kept[1024];               // per frontier row: candidates kept
  int rowbase[1024];            // per frontier row: first new slot - (cnt + 1)
  int scan[kBlock];
  int cnt, start, width, layers, carry;
};

// Keeps the `room` best candidates (ckey[e] != 0) by (key desc, e asc) and counts them per
// frontier row into kept[]. Radix selection narrows the boundary to a key prefix: either
// every key with that prefix is taken (the keys above the prefix and that whole group), or
// the prefix is the full room-th largest key T and, of the keys equal to T, those with the
// lowest e are taken. Requires more than `room` candidates.
//
// With at most 64 frontier rows and a small room, wave 0 merges the rows' sorted lists
// instead: lane f holds the head of row f's gated prefix (keys do not increase along a row,
// and e grows with f and with the rank), and each of `room` steps takes the largest head,
// the lowest row among equal ones, and advances that row. No block barrier is needed until
// the counts are written; the radix passes cost several barriers each.
constexpr int kTalonHeadMergeRoom = 16;

__device__ void talon_budget_select(TalonSelSmem& sm, int n, int K, int W, int room) {
  if (W <= 64 && room <= kTalonHeadMergeRoom) {
    if (threadIdx.x < 64) {
      const int f = threadIdx.x;
      const int g = f < W ? sm.gated[f] : 0;
      int j = 0;
      unsigned long long head = g > 0 ? sm.ckey[f * K] : 0ull;
      for (int t = 0; t < room; ++t) {   // more than `room` candidates: a head is never 0 here
        const unsigned long long top = wave_max(head);
        const int win = __builtin_ctzll(__ballot(head == top));
        if (f == win) {
          ++j;
          head = j < g ? sm.ckey[f * K + j] : 0ull;
        }
      }
      if (f < W) sm.kept[f] = j;
    }
    __syncthreads();
    return;
  }
  const RadixCut cut = radix_topk_cut(sm.ckey, n, room, sm.rs);
  for (int f = threadIdx.x; f < W; f += kBlock) sm.kept[f] = 0;
  __syncthreads();
  if (cut.all_in) {   // every key of the boundary group is taken: no tie order needed
    for (int e = threadIdx.x; e < n; e += kBlock) {
      const unsigned long long k = sm.ckey[e];
      if (k != 0ull && (k & cut.mask) >= cut.prefix) atomicAdd(&sm.kept[e / K], 1);
    }
    __syncthreads();
    return;
  }
  const unsigned long long T = cut.prefix;   // the full key: ties at T go by e
  int carry_eq = 0;
  for (int e0 = 0; e0 < n; e0 += kBlock) {
    const int e = e0 + threadIdx.x;
    const unsigned long long k = e < n ? sm.ckey[e] : 0ull;
    const int eq = (k != 0ull && k == T) ? 1 : 0;
    int tot = 0;
    const int before = carry_eq + block_exclusive_scan(eq, sm.scan, &tot);
    if (k != 0ull && (k > T || (eq && before < cut.rem))) atomicAdd(&sm.kept[e / K], 1);
    carry_eq += tot;
  }
  __syncthreads();
}

// One layer of TALON's loop for sequence s on the state in shared memory: sm.cnt draft
// nodes so far, the frontier (slots sm.start .. sm.start + sm.width - 1), their scores in
// sm.tscore and every frontier row's list (log p_d and token of its best entries, sorted)
// at sm.lp / sm.tok[slot * K + rank], sm.rcnt[slot]. Every step of the layer (scores, anchor,
// gate, cap, slot numbering) is a parallel pass over its candidates e = f*K + j (frontier
// row f, rank j), so no thread walks a dependent chain of shared-memory reads. Writes the
// new nodes to the tree and advances the state.
__device__ void talon_layer(TalonSelSmem& sm, const TalonArgs& a, int layer, size_t tb) {
  const int K = a.K;
  const int W = sm.width, cnt = sm.cnt, start = sm.start;
  const int room = a.B - cnt;
  const int n = W * K;
  // candidate scores s(c) = s(parent) + log p_d(token | parent); frontier row f is slot start + f
  for (int e = threadIdx.x; e < n; e += kBlock) {
    const int f = e / K, j = e % K, r = start + f;
    sm.csc[e] = j < sm.rcnt[r] ? sm.tscore[r] + sm.lp[r * K + j] : -INFINITY;
  }
  __syncthreads();
  if (layer == 1) {
    // robust initialisation: the root's Top-K, at most the budget, no gate
    if (threadIdx.x == 0) sm.kept[0] = sm.rcnt[0] < room ? sm.rcnt[0] : room;
    __syncthreads();
  } else {
    double mx = -INFINITY;
    for (int f = threadIdx.x; f < W; f += kBlock) mx = fmax(mx, sm.csc[f * K]);
    const double anchor = block_max(mx, sm.redd);
    const double thr = a.log_alpha + anchor;
    // row lists are sorted, so the gated entries of a row are a prefix of it
    int tg = 0;
    for (int f = threadIdx.x; f < W; f += kBlock) {
      int g = 0;
      for (int j = 0; j < K; ++j) g += sm.csc[f * K + j] >= thr ? 1 : 0;
      sm.gated[f] = g;
      tg += g;
    }
    tg = block_sum(tg, sm.redi);
    if (tg <= room) {
      for (int f = threadIdx.x; f < W; f += kBlock) sm.kept[f] = sm.gated[f];
      __syncthreads();
    } else {
      // budget respect: the `room` best gated candidates by (score desc, parent slot
      // asc, rank asc) = (key desc, e asc)
      for (int e = threadIdx.x; e < n; e += kBlock)
        sm.ckey[e] = (e % K) < sm.gated[e / K] ? dkey(sm.csc[e]) : 0ull;
      __syncthreads();
      talon_budget_select(sm, n, K, W, room);
    }
  }
  // new slots in (parent slot, rank) order: row f's kept entries follow those of rows < f
  int carry = 0;
  for (int f0 = 0; f0 < W; f0 += kBlock) {
    const int f = f0 + threadIdx.x;
    int tot = 0;
    const int ex = block_exclusive_scan(f < W ? sm.kept[f] : 0, sm.scan, &tot);
    if (f < W) sm.rowbase[f] = carry + ex;
    carry += tot;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n; e += kBlock) {
    const int f = e / K, j = e % K;
    if (j >= sm.kept[f]) continue;
    const int parent = start + f;
    const int slot = cnt + 1 + sm.rowbase[f] + j;
    const double sc = sm.csc[e];
    sm.tscore[slot] = sc;
    sm.tpar[slot] = static_cast<short>(parent);
    const size_t o = tb + slot;
    a.tree.parent[o] = parent;
    a.tree.token[o] = sm.tok[parent * K + j];
    a.tree.depth[o] = layer;
    a.tree.row[o] = slot;
    a.tree.score[o] = sc;
  }
  if (threadIdx.x == 0) {
    sm.start = cnt + 1;
    sm.width = carry;
    sm.cnt = cnt + carry;
    sm.layers = layer;
    sm.carry = carry;
    if (carry == 0) atomicExch(&a.hdr->err, kErrCapacity);
  }
  __syncthreads();
}

// The root's arrays, the node count and every node's ancestor-or-self mask from the parents
// in sm.tpar (slots 0 .. sm.cnt).
__device__ void talon_finish(TalonSelSmem& sm, const TalonArgs& a, int s, size_t tb) {
  const int nn = sm.cnt + 1;
  if (threadIdx.x == 0) {
    a.tree.parent[tb] = -1;
    a.tree.token[tb] = -1;
    a.tree.depth[tb] = 0;
    a.tree.row[tb] = 0;
    a.tree.score[tb] = 0.0;
    a.tree.n_nodes[s] = nn;
    a.tree.layers[s] = sm.layers;
  }
  const int words = a.tree.words;
  for (int i = threadIdx.x; i < nn; i += kBlock) {
    uint64_t acc[kMaxWords];
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w) acc[w] = 0;
    for (int j = i; j >= 0; j = (j > 0) ? sm.tpar[j] : -1) {
#pragma unroll
      for (int u = 0; u < kMaxWords; ++u)
        if (u == (j >> 6)) acc[u] |= 1ull << (j & 63);
    }
    uint64_t* an = a.tree.anc + (tb + i) * words;
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w)
      if (w < words) an[w] = acc[w];
  }
}

__device__ __forceinline__ void talon_state_root(TalonSelSmem& sm) {
  if (threadIdx.x == 0) {
    sm.cnt = 0;
    sm.start = 0;
    sm.width = 1;
    sm.layers = 0;
    sm.tscore[0] = 0.0;
    sm.tpar[0] = -1;
  }
}

// Phase 2 of the whole-table build: the layer loop of sequence blockIdx.x in one
// workgroup, on the row lists of phase 1 (visible after the kernel boundary), copied into
// shared memory in one parallel pass.
__global__ __launch_bounds__(kBlock) void talon_select_kernel(TalonArgs a) {
  __shared__ TalonSelSmem sm;
  const int s = blockIdx.x;
  const int K = a.K;
  const int B = a.B;
  const size_t rf0 = static_cast<size_t>(s) * B;
  const size_t tb = static_cast<size_t>(s) * a.tree.n_cap;
  for (int f = threadIdx.x; f < B; f += kBlock) sm.rcnt[f] = a.rcnt[rf0 + f];
  for (int e = threadIdx.x; e < B * K; e += kBlock) {
    const int f = e / K;
    sm.lp[e] = static_cast<double>(a.rv[rf0 * K + e]) - a.rlse[rf0 + f];
    sm.tok[e] = a.ri[rf0 * K + e];
  }
  talon_state_root(sm);
  __syncthreads();
  for (int layer = 1;; ++layer) {
    talon_layer(sm, a, layer, tb);
    if (sm.cnt >= B || sm.carry == 0) break;
  }
  talon_finish(sm, a, s, tb);
}

// One layer of the layer-by-layer build for sequence blockIdx.x: the state of the earlier
// layers comes from the workspace (counts) and the tree (scores and parents of the nodes
// so far); this call's frontier lists (call rows f < width, reduced by talon_rows_kernel)
// go to the frontier slots start + f. A finished sequence is left as it is.
__global__ __launch_bounds__(kBlock) void talon_layer_kernel(TalonArgs a) {
  __shared__ TalonSelSmem sm;
  const int s = blockIdx.x;
  const int K = a.K;
  const size_t tb = static_cast<size_t>(s) * a.tree.n_cap;
  int* st = a.state + 8 * s;
  if (a.layer == 1) {
    talon_state_root(sm);
  } else if (threadIdx.x == 0) {
    sm.cnt = st[0];
    sm.start = st[1];
    sm.width = st[2];
    sm.layers = st[3];
    sm.carry = st[4];   // done
  }
  __syncthreads();
  if (a.layer > 1 && sm.carry != 0) return;
  const int W = sm.width, start = sm.start;
  if (W > a.Wr) {   // the call brought fewer rows than the frontier has nodes
    if (threadIdx.x == 0) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  const size_t rf0 = static_cast<size_t>(s) * a.Wr;
  for (int f = threadIdx.x; f < W; f += kBlock) {
    sm.rcnt[start + f] = a.rcnt[rf0 + f];
    if (a.layer > 1) sm.tscore[start + f] = a.tree.score[tb + start + f];
  }
  for (int e = threadIdx.x; e < W * K; e += kBlock) {
    const int f = e / K;
    sm.lp[(start + f) * K + e % K] = static_cast<double>(a.rv[rf0 * K + e]) - a.rlse[rf0 + f];
    sm.tok[(start + f) * K + e % K] = a.ri[rf0 * K + e];
  }
  __syncthreads();
  talon_layer(sm, a, a.layer, tb);
  const bool done = sm.cnt >= a.B || sm.carry == 0;
  if (threadIdx.x == 0) {
    st[0] = sm.cnt;
    st[1] = sm.start;
    st[2] = sm.width;
    st[3] = sm.layers;
    st[4] = done ? 1 : 0;
    a.w_out[s] = done ? 0 : sm.width;
    a.done_out[s] = done ? 1 : 0;
  }
  if (!done) return;
  for (int i = 1 + threadIdx.x; i <= sm.cnt; i += kBlock) sm.tpar[i] = static_cast<short>(a.tree.parent[tb + i]);
  if (threadIdx.x == 0) sm.tpar[0] = -1;
  __syncthreads();
  talon_finish(sm, a, s, tb);
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

// The root and the spine chain of sequence s (nt threads of one workgroup).
__device__ __forceinline__ void spine_chain(const SpineArgs& a, int s, size_t tb, int nt) {
  const int words = a.tree.words;
  for (int k = threadIdx.x; k <= a.n_spine; k += nt) {
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

constexpr int kSpineMaxK = 65;

template <int DT>
__global__ __launch_bounds__(kBlock, 4) void spine_kernel(SpineArgs a) {
  __shared__ RowSmem rs;
  __shared__ MergeSmem<kTalonMergeCap> ms;
  __shared__ unsigned long long sortbuf[pow2_at_least(kWaves * 128) > kCandCap ? pow2_at_least(kWaves * 128)
                                                                              : kCandCap];
  using Rw = RowT<DT>;
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
  const char* row = static_cast<const char*>(a.draft) +
                    (static_cast<size_t>(s) * a.R + f) * static_cast<size_t>(a.V) * Rw::ESIZE;
  // the exp table and the fork row's chunk in one round trip
  row_smem_issue(rs);
  float x[Rw::E];
  uint32_t key[Rw::E];
  load_chunk<DT>(row, a.V, c, x, key);
  drain();
  __syncthreads();

  if (f == 0 && c == 0) spine_chain(a, s, tb, kBlock);   // root and spine chain of sequence s
  const int wf = a.width[f];
  if (wf <= 0) return;
  const int kf = wf + 1 < a.V ? wf + 1 : a.V;   // one spare for the skipped spine token
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

// bf16 fork rows of at most one part (V <= 32768): one 1024-thread workgroup per (sequence,
// fork) reduces the whole row with the part reducer (rows_bf16.h: table-driven float64
// exponentials, packed 16-bit keys), so no chunk merge and no ticket are needed, and then
// writes the fork's branch nodes itself.
__global__ __launch_bounds__(kPartThreads) void spine_bf16_kernel(SpineArgs a) {
  __shared__ PartSmem sm;
  __shared__ int list_len;
  const int f = blockIdx.x % a.F;
  const int s = blockIdx.x / a.F;
  const int cap = a.tree.n_cap;
  const size_t tb = static_cast<size_t>(s) * cap;
  const int words = a.tree.words;
  if (f == 0) spine_chain(a, s, tb, kPartThreads);   // root and spine chain of sequence s
  const int wf = a.width[f];
  if (wf <= 0) return;
  const int kf = wf + 1 < a.V ? wf + 1 : a.V;   // one spare for the skipped spine token
  const size_t rf = static_cast<size_t>(s) * a.F + f;
  const uint16_t* row = static_cast<const uint16_t*>(a.draft) + (static_cast<size_t>(s) * a.R + f) * static_cast<size_t>(a.V);
  float* const rv = a.rv + rf * a.K;
  int* const ri = a.ri + rf * a.K;
  part_row_reduce(row, a.V, 0, 1, kf, nullptr, nullptr, nullptr, nullptr, &a.rlse[rf], rv, ri, &list_len, sm);
  __syncthreads();   // the row's list, log-sum-exp and length are in
  // list entry r becomes branch j = r, or r - 1 after the skipped spine token
  const int r = threadIdx.x;
  if (r >= kf || r >= list_len) return;
  const int skip = (f < a.n_spine) ? a.spine[static_cast<size_t>(s) * a.n_spine + f] : -1;
  const int tok = ri[r];
  if (tok == skip) return;
  int j = r;
  for (int q = 0; q < r; ++q) j -= ri[q] == skip ? 1 : 0;
  if (j >= wf) return;
  const int slot = 1 + a.n_spine + a.offset[f] + j;
  const size_t o = tb + slot;
  a.tree.parent[o] = f;
  a.tree.token[o] = tok;
  a.tree.depth[o] = f + 1;
  a.tree.row[o] = slot;
  a.tree.score[o] = static_cast<double>(rv[r]) - a.rlse[rf];
  uint64_t* an = a.tree.anc + o * words;
  for (int w = 0; w < words; ++w) {  // bits 0..f plus the node itself
    const int lo = w * 64;
    const int nb = f + 1 - lo;
    uint64_t bits = nb <= 0 ? 0ull : (nb >= 64 ? ~0ull : ((1ull << nb) - 1ull));
    if ((slot >> 6) == w) bits |= 1ull << (slot & 63);
    an[w] = bits;
  }
}

int launch_spine(const SpineArgs& a, int dtype, hipStream_t st) {
  if (dtype == 1 && parts_of(a.V) == 1 && a.K <= kPartSlots) {
    DTV_LAUNCH(spine_bf16_kernel, dim3(a.S * a.F), dim3(kPartThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const dim3 grid(a.S * a.F * a.nch);
  if (dtype == 1)
    DTV_LAUNCH(spine_kernel<1>, grid, dim3(kBlock), 0, st, a);
  else
    DTV_LAUNCH(spine_kernel<0>, grid, dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The row phase: bf16 rows in parts (rows_bf16.h), fp32 rows in chunks (rowstats.h).
static int launch_talon_rows(const TalonArgs& a, int dtype, hipStream_t st) {
  if (dtype == 1) {
    const int np = parts_of(a.V);
    // a row's parts live in its chunk slots, and a merge stages every part's list at once
    if (np > a.nch || np > kPartMaxParts || np * a.K > kPartMergeCap) return -1;
    DTV_LAUNCH(talon_rows_bf16_kernel, dim3(a.S * a.Wr * np), dim3(kPartThreads), 0, st, a);
  } else {
    DTV_LAUNCH(talon_rows_kernel<0>, dim3(a.S * a.Wr * a.nch), dim3(kBlock), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_talon_layer(const TalonArgs& a, int dtype, hipStream_t st) {
  if (launch_talon_rows(a, dtype, st) != 0) return -1;
  DTV_LAUNCH(talon_layer_kernel, dim3(a.S), dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_talon(const TalonArgs& a, int dtype, hipStream_t st) {
  if (launch_talon_rows(a, dtype, st) != 0) return -1;
  DTV_LAUNCH(talon_select_kernel, dim3(a.S), dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace dtv
