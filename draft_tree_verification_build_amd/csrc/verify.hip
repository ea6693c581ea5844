// Greedy verification on gfx950 (OPT-Tree summary, section 2; GOOSE page, section 2C).
//
// One workgroup per (sequence, node, chunk of the node's target row) finds the chunk's
// largest value and its lowest index and publishes them as one 64-bit key
// ((value key << 32) | ~index: larger value wins, then lower index) in a slot of its own
// (an agent-scope store; a slot is never 0 once written, and the workspace keeps every slot
// 0 between calls). The sequence's last workgroup in launch order walks: it loads the tree,
// polls the slots of the sequence's nodes (all of them at once, spread over its threads)
// until every chunk has reported, reduces each node's chunks to its argmax, clears the
// slots for the next call, and walks the tree: node c matches when its
// token equals the argmax at its parent; a node is accepted when every node on its root
// path matches (parent links in shared memory); the deepest accepted node, lowest slot
// first, ends the path. No workgroup waits on a counter or a fence.
#include "dtv_internal.h"
#include "rows_bf16.h"
#include "rowstats.h"

namespace dtv {

constexpr int kVerifyMaxNodes = 1024;
constexpr int kVerifyMaxWords = 16;
constexpr long kGreedySpinLimit = 2000000;   // poll rounds (each a memory round trip) before a timeout

// ------------------------------------------------------------------ compaction by the walk
//
// KV compaction of sequence s along its accepted path (spath[k], k < L, in shared memory),
// concept page, "The protocol", step 4: cache[P + k] <- cache[P + spath[k]] for the (KV
// head, tensor) pairs pair0, pair0 + pstep, ... Each pair is memory of its own, and within
// a pair the rows are taken in increasing k, in batches whose reads all precede their
// writes; a node at depth k has slot >= k, so no later source row is an earlier
// destination. Every thread of the workgroup calls it. Returns false, touching nothing,
// when P and the tree do not fit the cache.
template <int NT = kBlock>
__device__ bool walk_compact(const KvCompactView& c, int s, int n_cap, const int* spath, int L, int pair0,
                             int pstep) {
  const int P = c.P[s];
  if (L < 1 || L > n_cap || P < 0 || P + n_cap > c.P_cap) return false;
  const int vpr = c.D * c.esize / 16;   // 16-byte vectors per row
  const size_t row_bytes = static_cast<size_t>(c.D) * c.esize;
  const int npairs = pair0 < 2 * c.Hkv ? (2 * c.Hkv - pair0 + pstep - 1) / pstep : 0;
  const int per_pair = L * vpr;
  const int total = npairs * per_pair;
  // four 16-byte vectors per thread and batch, all loaded before any store (named registers,
  // so that they stay in registers across the barrier)
  auto src_dst = [&](int v, char*& dst) -> const uint4* {
    const int vc = min(v, total - 1);
    const int pi = vc / per_pair, rem = vc % per_pair;
    const int k = rem / vpr, ch = rem % vpr;
    const int pair = pair0 + pi * pstep;
    char* base = ((pair & 1) ? c.v : c.k) + (static_cast<size_t>(s) * c.Hkv + (pair >> 1)) * c.P_cap * row_bytes;
    dst = base + static_cast<size_t>(P + k) * row_bytes + ch * 16;
    return reinterpret_cast<const uint4*>(base + static_cast<size_t>(P + spath[k]) * row_bytes + ch * 16);
  };
  for (int b0 = 0; b0 < total; b0 += NT * 4) {
    const int v0 = b0 + static_cast<int>(threadIdx.x);
    char *d0, *d1, *d2, *d3;
    uint4 x0, x1, x2, x3;   // loads past the end are not issued
    const uint4* s0 = src_dst(v0, d0);
    const uint4* s1 = src_dst(v0 + NT, d1);
    const uint4* s2 = src_dst(v0 + 2 * NT, d2);
    const uint4* s3 = src_dst(v0 + 3 * NT, d3);
    if (v0 < total) x0 = *s0;
    if (v0 + NT < total) x1 = *s1;
    if (v0 + 2 * NT < total) x2 = *s2;
    if (v0 + 3 * NT < total) x3 = *s3;
    __syncthreads();
    if (v0 < total) *reinterpret_cast<uint4*>(d0) = x0;
    if (v0 + NT < total) *reinterpret_cast<uint4*>(d1) = x1;
    if (v0 + 2 * NT < total) *reinterpret_cast<uint4*>(d2) = x2;
    if (v0 + 3 * NT < total) *reinterpret_cast<uint4*>(d3) = x3;
    __syncthreads();
  }
  return true;
}

struct VerifySmem {
  int a[kVerifyMaxNodes];       // target argmax at every node
  short par[kVerifyMaxNodes];   // parent slot
  short dep[kVerifyMaxNodes];   // depth
  int tok[kVerifyMaxNodes];     // drafted token
  unsigned char bad[kVerifyMaxNodes];   // 1: token differs from the argmax at the parent
  unsigned long long best[kVerifyMaxNodes];   // largest chunk key of every node
  unsigned long long redu[16];   // per-wave partials (up to 16 waves)
  int flag;
};

// The walk of sequence s by the 256 threads of one workgroup (every other thread of it has
// ended): the tree is loaded first, so that its loads are in flight with the first polls;
// every thread then polls its share of the N * nslot slots (node-major, nslot per node), up
// to 8 at once, until all have reported, folds them into its node's maximum in shared memory
// and clears them for the next call; then the tree walk and the compaction.
template <int NT = kBlock>
__device__ void greedy_walk(const VerifyArgs& a, int s, int N, int cap, int nch, unsigned long long* slots,
                            VerifySmem& sm) {
  const size_t tb = static_cast<size_t>(s) * cap;
  if (threadIdx.x == 0) sm.flag = 0;
  __syncthreads();
  for (int v = threadIdx.x; v < N; v += NT) {
    sm.best[v] = 0ull;
    sm.tok[v] = a.tree.token[tb + v];
    sm.par[v] = static_cast<short>(v == 0 ? -1 : a.tree.parent[tb + v]);
    sm.dep[v] = static_cast<short>(a.tree.depth[tb + v]);
    const int r = a.tree.row[tb + v];
    const int dv = sm.dep[v];
    // the path is written at the nodes' depths: they must lie inside the tree
    if (r < 0 || r >= a.R || dv < 0 || dv >= N || (v == 0 && dv != 0)) sm.flag = 1;
  }
  __syncthreads();
  int ok = 1;
  const int total = N * nch;
  for (int j0 = 0; j0 < total; j0 += NT * 8) {
    unsigned long long b[8];
    long polls = 0;
    for (;;) {
      bool all = true;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q * NT + static_cast<int>(threadIdx.x);
        b[q] = j < total ? ld_cc(&slots[j]) : 1ull;
        all = all && b[q] != 0ull;
      }
      if (all) break;
      if (++polls > kGreedySpinLimit) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = j0 + q * NT + static_cast<int>(threadIdx.x);
      if (j < total) {
        atomicMax(&sm.best[j / nch], b[q]);
        slots[j] = 0ull;   // ready for the next call
      }
    }
  }
  __syncthreads();
  if (sm.flag) {   // a row outside the table or a depth outside the tree: no path
    if (threadIdx.x == 0) {
      atomicExch(&a.hdr->err, kErrBadRow);
      a.path_len[s] = 0;
      a.bonus[s] = -1;
      if (a.kvc.k != nullptr) a.kvc.P_new[s] = -1;
    }
    return;
  }
  for (int v = threadIdx.x; v < N; v += NT) {
    const int am = sort_key_index(sm.best[v]);
    sm.a[v] = am;
    if (a.argmax_out) a.argmax_out[tb + v] = am;
  }
  if (!ok) atomicExch(&a.hdr->err, kErrTimeout);
  __syncthreads();
  // a node is bad when its token is not the target argmax at its parent (or its parent
  // link is not an earlier slot, which also bounds every walk below)
  for (int v = threadIdx.x; v < N; v += NT) {
    const int p = sm.par[v];
    sm.bad[v] = (v > 0 && (p < 0 || p >= v || sm.tok[v] != sm.a[p])) ? 1 : 0;
  }
  __syncthreads();
  // deepest accepted node, lowest slot among equals: maximise (depth << 20) | (2^20 - 1 - slot);
  // node v is accepted when no node on its root path is bad (slots grow away from the root)
  unsigned long long pick = 0;
  for (int v = threadIdx.x; v < N; v += NT) {
    bool clean = true;
    for (int u = v; u > 0 && clean; u = sm.par[u]) clean = !sm.bad[u];
    if (clean) {
      const unsigned long long key2 = (static_cast<unsigned long long>(sm.dep[v]) << 20) |
                                      static_cast<unsigned long long>(0xFFFFF - v);
      pick = key2 > pick ? key2 : pick;
    }
  }
  {   // the largest pick over the NT / 64 waves
    pick = wave_max(pick);
    if ((threadIdx.x & 63) == 0) sm.redu[threadIdx.x >> 6] = pick;
    __syncthreads();
    for (int q = 0; q < NT / 64; ++q) pick = sm.redu[q] > pick ? sm.redu[q] : pick;
  }
  const int vstar = 0xFFFFF - static_cast<int>(pick & 0xFFFFFull);
  const int A = static_cast<int>(pick >> 20);
  if (threadIdx.x == 0) {
    for (int u = vstar; u >= 0; u = sm.par[u]) {
      a.path[tb + sm.dep[u]] = u;
      sm.tok[sm.dep[u]] = u;   // the path, for the compaction (tokens are no longer read)
    }
    a.path_len[s] = A + 1;
    a.bonus[s] = sm.a[vstar];
  }
  if (a.kvc.k != nullptr) {
    __syncthreads();
    const bool done = walk_compact<NT>(a.kvc, s, cap, sm.tok, A + 1, 0, 1);
    if (threadIdx.x == 0) a.kvc.P_new[s] = done ? a.kvc.P[s] + A + 1 : -1;
  }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void verify_greedy_kernel(VerifyArgs a) {
  __shared__ VerifySmem sm;
  using Rw = RowT<DT>;
  const int nch = a.nch;
  const int cap = a.tree.n_cap;
  const int s = blockIdx.x / (cap * nch);
  const int rest = blockIdx.x % (cap * nch);
  const int i = rest / nch, c = rest % nch;
  const size_t tb = static_cast<size_t>(s) * cap;
  // the node count and this node's row in one round of loads (slot i < n_cap is valid
  // memory; its row is used only when i < N)
  const int N = a.tree.n_nodes[s];
  const int r_slot = a.tree.row[tb + i];
  if (N > cap || N < 1) {  // n_nodes is device data: refuse rather than read past the tree
    if (threadIdx.x == 0 && i == 0 && c == 0) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  unsigned long long* slots = a.cbest + tb * nch;   // [node][chunk]
  if (i < N && (r_slot < 0 || r_slot >= a.R)) {
    // a row outside the table is never read: the chunk reports the smallest non-empty key,
    // so the walker's polls end, and the walker refuses the tree
    if (threadIdx.x == 0) {
      atomicExch(&a.hdr->err, kErrBadRow);
      st_cc(&slots[static_cast<size_t>(i) * nch + c], 1ull);
    }
  } else if (i < N) {
    const int r = r_slot;
    const char* row = static_cast<const char*>(a.target) +
                      (static_cast<size_t>(s) * a.R + r) * static_cast<size_t>(a.V) * Rw::ESIZE;
    float x[Rw::E];
    uint32_t key[Rw::E];
    load_chunk<DT>(row, a.V, c, x, key);
    // this thread's largest value (32-bit order keys, 0 = absent) and, of its entries
    // holding it, the first in index order (a thread's entries ascend with (ii, e))
    uint32_t km = 0u;
#pragma unroll
    for (int j = 0; j < Rw::E; ++j) km = key[j] > km ? key[j] : km;
    int jm = 0;
    float xm = 0.f;
#pragma unroll
    for (int j = Rw::E - 1; j >= 0; --j) {
      const bool hit = key[j] == km;
      jm = hit ? j : jm;
      xm = hit ? x[j] : xm;
    }
    unsigned long long best = 0;
    if (km != 0u) best = sort_key(xm, elem_index<DT>(c, jm / Rw::VEC, jm % Rw::VEC));
    best = block_max(best, sm.redu);
    // every chunk holds an element (c < nch), and a key from an element is never 0
    if (threadIdx.x == 0) st_cc(&slots[static_cast<size_t>(i) * nch + c], best);
  }
  if (i != cap - 1 || c != nch - 1) return;
  greedy_walk(a, s, N, cap, nch, slots, sm);
}

// bf16 target rows: one 1024-thread workgroup per (sequence, node, part of 32768 values of
// the node's target row, rows_bf16.h). The part's largest key is found from packed keys and
// lane maxima; only the lanes that hold it look for its lowest index. The part publishes
// (key << 32 | ~index) in its slot; the sequence's last workgroup in launch order then walks
// on 256 of its threads.
struct VerifyBf16Smem {
  VerifySmem v;
  uint32_t wmax[kPartWaves];
  int wmin[kPartWaves];
};

__global__ __launch_bounds__(kPartThreads) void verify_greedy_bf16_kernel(VerifyArgs a) {
  __shared__ VerifyBf16Smem sm;
  const int np = parts_of(a.V);
  const int cap = a.tree.n_cap;
  const int s = blockIdx.x / (cap * np);
  const int rest = blockIdx.x % (cap * np);
  const int i = rest / np, p = rest % np;
  const size_t tb = static_cast<size_t>(s) * cap;
  const int N = a.tree.n_nodes[s];
  const int r_slot = a.tree.row[tb + i];
  if (N > cap || N < 1) {  // n_nodes is device data: refuse rather than read past the tree
    if (threadIdx.x == 0 && i == 0 && p == 0) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  unsigned long long* slots = a.cbest + tb * np;   // [node][part]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (i < N && (r_slot < 0 || r_slot >= a.R)) {
    // a row outside the table is never read: the part reports the smallest non-empty key
    if (threadIdx.x == 0) {
      atomicExch(&a.hdr->err, kErrBadRow);
      st_cc(&slots[static_cast<size_t>(i) * np + p], 1ull);
    }
  } else if (i < N) {
    const uint16_t* row = static_cast<const uint16_t*>(a.target) + (static_cast<size_t>(s) * a.R + r_slot) * static_cast<size_t>(a.V);
    const int vbase = p * kPartVecs;
    const int vfull = a.V / 8;
    const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) && vfull > 0;
    PartData d;
    part_load(row, a.V, vbase, vec, d);
    const bool clean = vec && vbase + (kPartLoads - 1) * kPartThreads + 64 * w + 63 < vfull;
    uint32_t k2[kPartWords], g4[kPartLoads], lm;
    part_keys(d, clean, row, a.V, vbase, vec, k2, g4, lm);
    const uint32_t km = wave_max(lm);
    if (lane == 0) sm.wmax[w] = km;
    __syncthreads();
    uint32_t M = lane < kPartWaves ? sm.wmax[lane] : 0u;
    M = row16_reduce(M, [](uint32_t x, uint32_t y) { return y > x ? y : x; });
    // the lowest index holding M: a lane's values ascend in index with (word, half)
    int idx = 0x7FFFFFFF;
    if (lm == M) {
#pragma unroll
      for (int j = 0; j < kPartWords; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (idx == 0x7FFFFFFF && key_half(k2[j], h) == M) idx = part_index(vbase, j, h);
    }
    idx = wave_min(idx);
    if (lane == 0) sm.wmin[w] = idx;
    __syncthreads();
    int I = lane < kPartWaves ? sm.wmin[lane] : 0x7FFFFFFF;
    I = row16_reduce(I, [](int x, int y) { return y < x ? y : x; });
    // every part holds a value of the row (p * 32768 < V), so M != 0 and the key is never 0
    if (threadIdx.x == 0) st_cc(&slots[static_cast<size_t>(i) * np + p], part_sort_key(M, I));
  }
  if (i != cap - 1 || p != np - 1) return;
  if (threadIdx.x >= kBlock) return;   // the walk runs on 256 threads
  greedy_walk<kBlock>(a, s, N, cap, np, slots, sm.v);
}

// ------------------------------------------------------------------ rejection sampling
//
// Concept page, "The protocol", step 3: accept a drafted token x with probability
// min(1, p(x)/q(x)); on rejection draw the correction from (p - q)+ normalised. On a tree,
// the children of the current node are tried in slot order with the uniforms u_acc, the
// residual p <- norm((p - q)+) replacing p after each rejection (kept if it sums to 0);
// the walk moves to the first accepted child; when none is accepted (or the node is a
// leaf) the bonus token is drawn from the current p by inverse CDF with u_res.
//
// Work split: one launch. The walk of a sequence is shared by G workgroups, each owning a
// slice of the vocabulary. p and q are needed only at the nodes the walk visits (about
// A + 1 per sequence), so their normalisers are computed there, not for every node of the
// tree: on arriving at a node, every workgroup reduces its slice of the node's target and
// draft rows to (max, float64 sum of exp) and the group exchanges those. A first try then
// needs only the two row values at the child's token; each rejection costs one residual
// pass over the slices (kept in shared memory when they fit) and one exchange of slice
// sums; the bonus draw is one prefix-sum pass in the workgroup that holds the target mass.

struct SampleSmem {
  RowSmem rs;
  short par[kSampleMaxNodes];
  int tok[kSampleMaxNodes];
  int kids[kSampleMaxNodes];
  int spath[kSampleMaxNodes];   // the accepted path so far (every workgroup of the group)
  uint32_t uacc[kSampleMaxNodes];   // every node's acceptance uniform
  uint32_t ures[kSampleMaxNodes];   // every node's residual (bonus) uniform
  unsigned long long kmask[kWaves];   // per-wave ballots of a node's children
  double lsev[4 * kSampleMaxGroup];   // the node's slice statistics of every workgroup
  double wpair[kWaves][4];            // per-wave (max, sum) pairs of the two rows
  double wsum[kWaves];
  int iwsum[kWaves];
  int flag;
  int first;
  int pick;
  int accept;
};

template <int DT>
__device__ __forceinline__ float row_value(const void* row, int j) {
  return DT ? bf16_to_f32(static_cast<const uint16_t*>(row)[j]) : static_cast<const float*>(row)[j];
}

// The VEC logits of 16-byte vector vi of a row (VEC = 8 bf16 or 4 fp32).
template <int DT>
__device__ __forceinline__ void row_vec(const void* row, int vi, float (&x)[RowT<DT>::VEC]) {
  const uint4 raw = reinterpret_cast<const uint4*>(row)[vi];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int e = 0; e < RowT<DT>::VEC; ++e)
    x[e] = DT ? bf16_to_f32(static_cast<uint16_t>((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu)) : __uint_as_float(w[e]);
}

template <int DT>
__device__ __forceinline__ void unit_decode(const uint4 raw, float (&x)[RowT<DT>::VEC]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int e = 0; e < RowT<DT>::VEC; ++e)
    x[e] = DT ? bf16_to_f32(static_cast<uint16_t>((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu)) : __uint_as_float(w[e]);
}

// The walk's view of the current distribution p at node v: softmax of the target row
// (pc null) or the normalised residual pc / zc; q is the softmax of the draft row. A
// "unit" is a 16-byte vector of VEC consecutive logits when `vec` (rows 16-byte aligned,
// V a multiple of VEC), else a single entry. pc and the q cache qc hold this workgroup's
// entries only, entry j at index j - base; they live in shared memory when the slice
// fits, else in the workspace, and only this workgroup ever reads what it wrote there.
// Hence p(j) with pc set and the unit accessors take only entries of this workgroup's
// slice, while q(j) (any entry: the acceptance test reads the child's token) always
// evaluates the draft row; the cache holds the same values, computed the same way.
template <int DT>
struct WalkDist {
  static constexpr int VEC = RowT<DT>::VEC;
  const void* trow;
  const void* drow;
  double lt, ld;
  const double* pc;
  double zc;
  double* qc;
  bool qvalid;
  int base;
  const double* tab;
  bool vec;
  const uint4* tst;   // this workgroup's units of the target / draft row in shared memory
  const uint4* dst;   // (unit u at index u - u0), or null: read the rows in memory
  int u0;

  __device__ int width() const { return vec ? VEC : 1; }
  __device__ double p(int j) const {
    return pc ? pc[j - base] / zc : exp_nonpos(static_cast<double>(row_value<DT>(trow, j)) - lt, tab);
  }
  __device__ double q(int j) const {
    return exp_nonpos(static_cast<double>(row_value<DT>(drow, j)) - ld, tab);
  }
  // p of the entries of unit a into out[0 .. width)
  __device__ void p_unit(int a, double (&out)[VEC]) const {
    if (!vec) {
      out[0] = p(a);
      return;
    }
    if (pc) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) out[e] = pc[a * VEC + e - base] / zc;
    } else {
      float x[VEC];
      if (tst)
        unit_decode<DT>(tst[a - u0], x);
      else
        row_vec<DT>(trow, a, x);
#pragma unroll
      for (int e = 0; e < VEC; ++e) out[e] = exp_nonpos(static_cast<double>(x[e]) - lt, tab);
    }
  }
  // q of the entries of unit a; the first pass at a node computes them and fills the cache
  __device__ void q_unit(int a, double (&out)[VEC]) const {
    if (!vec) {
      if (qvalid) {
        out[0] = qc[a - base];
      } else {
        out[0] = q(a);
        qc[a - base] = out[0];
      }
      return;
    }
    if (qvalid) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) out[e] = qc[a * VEC + e - base];
      return;
    }
    float x[VEC];
    if (dst)
      unit_decode<DT>(dst[a - u0], x);
    else
      row_vec<DT>(drow, a, x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      out[e] = exp_nonpos(static_cast<double>(x[e]) - ld, tab);
      qc[a * VEC + e - base] = out[e];
    }
  }
};

// The G workgroups of a sequence share every V-wide pass: workgroup gi owns units
// [u0, u1). Every exchange uses a slot of its own: entries n gi .. n gi + n-1 receive
// workgroup gi's n values, entries n G and n G + 1 two values from the owner of the next
// child's token (see the walk). A value is stored as the complement of its bits, so that
// an entry of all zero bits, which no stored value takes, means "not yet written": the
// workspace starts zero-filled, and the last workgroup of a sequence to finish its walk
// zeroes the slots the walk used, ready for the next call. Each entry is written once per
// call, and the readers poll the entries they need until none is zero, so an exchange
// costs one store and the polls, with no counter and no fence: the values are the signal.
// Every workgroup then combines the values in workgroup order, so all of them see
// identical totals and take identical decisions.
constexpr long kSpinLimit = 2000000;    // polls (each a memory round trip) before a timeout

__device__ __forceinline__ unsigned long long xch_encode(double v) {
  return ~static_cast<unsigned long long>(__double_as_longlong(v));
}
__device__ __forceinline__ double xch_decode(unsigned long long b) {
  return __longlong_as_double(static_cast<long long>(~b));
}

struct WalkGroup {
  int gi, G;
  int u0, u1;                 // this workgroup's units
  unsigned long long* xch;    // [max_pass][kXchStride] exchange slots
  int max_pass;
  int* err;
  int pass;                   // exchanges so far
};

// Publishes this workgroup's n values (thread 0's `mine`; from the owner also e0 / e1 into
// entries n G and n G + 1), waits until the group's n G values (and the owner's two when
// `extra`) are in and copies them into sm_vals. Returns false on a timeout or when the
// slots are exhausted.
__device__ bool group_exchange(WalkGroup& g, const double* mine, int n, bool owner, double e0, double e1,
                               bool extra, double* sm_vals, int* flag) {
  if (g.pass >= g.max_pass) {
    if (threadIdx.x == 0) atomicExch(g.err, kErrCapacity);
    return false;
  }
  unsigned long long* slot = g.xch + static_cast<size_t>(g.pass) * kXchStride;
  if (threadIdx.x == 0) {
    for (int j = 0; j < n; ++j) st_cc(&slot[g.gi * n + j], xch_encode(mine[j]));
    if (owner) {
      st_cc(&slot[n * g.G], xch_encode(e0));
      st_cc(&slot[n * g.G + 1], xch_encode(e1));
    }
  }
  ++g.pass;
  const int nv = n * g.G + (extra ? 2 : 0);
  if (threadIdx.x < 64) {   // wave 0: lane k waits for entries k, k + 64, ...
    int ok = 1;
    for (int k = threadIdx.x; k < nv && ok; k += 64) {
      unsigned long long bits = ld_cc(&slot[k]);
      long polls = 0;
      while (bits == 0ull) {
        __builtin_amdgcn_s_sleep(1);
        if (++polls > kSpinLimit) {
          ok = 0;
          break;
        }
        bits = ld_cc(&slot[k]);
      }
      sm_vals[k] = xch_decode(bits);
    }
    if (!ok) atomicExch(g.err, kErrTimeout);
    const unsigned long long good = __ballot(ok);
    if (threadIdx.x == 0) *flag = (good == ~0ull) ? 1 : 0;
  }
  __syncthreads();
  return *flag != 0;
}

// (max, float64 sum of exp(x - max)) of this workgroup's units of nr <= 2 rows, in one pass
// over memory: every thread loads its share of both rows together, the block takes each
// row's maximum (one barrier), then every thread sums exp(x - max) over its values and the
// block sums those (a second barrier). With 16-byte units a thread takes half units (8
// bytes), so that a slice of a few hundred units keeps all four waves busy. A slice larger
// than one batch (kStatUnits per thread) is folded batch by batch, rescaling the running sum
// when a later batch raises the maximum. Thread 0 receives the pairs in out[2 r],
// out[2 r + 1] (max -inf and sum 0 for an empty slice or r >= nr).
constexpr int kStatUnits = 2;   // values groups per thread and batch

template <int DT>
__device__ __forceinline__ void half_decode(const uint2 raw, float (&x)[RowT<DT>::VEC / 2]) {
  const uint32_t w2[2] = {raw.x, raw.y};
#pragma unroll
  for (int e = 0; e < RowT<DT>::VEC / 2; ++e)
    x[e] = DT ? bf16_to_f32(static_cast<uint16_t>((w2[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu)) : __uint_as_float(w2[e]);
}

template <int DT>
__device__ void slice_stats(const void* row0, const void* row1, const uint4* st0, const uint4* st1, int nr,
                            const WalkGroup& g, bool vec, const double* tab, double (*wred)[4], double* out) {
  constexpr int HV = RowT<DT>::VEC / 2;   // values per half unit
  const int w = vec ? HV : 1;            // values per item: a half unit, or one entry
  const int i0 = vec ? 2 * g.u0 : g.u0, i1 = vec ? 2 * g.u1 : g.u1;   // this workgroup's items
  const void* rows[2] = {row0, row1};
  const uint4* sts[2] = {st0, st1};
  const int wv = threadIdx.x >> 6;
  double M[2] = {-INFINITY, -INFINITY}, S[2] = {0.0, 0.0};
  for (int b0 = i0; b0 < i1; b0 += kBlock * kStatUnits) {   // block-uniform batches
    float x[2][kStatUnits][HV];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int q = 0; q < kStatUnits; ++q) {
        const int it = b0 + q * kBlock + static_cast<int>(threadIdx.x);
        const bool in = r < nr && it < i1;
        if (vec) {
          if (in) {
            const uint2 raw = sts[r] != nullptr ? reinterpret_cast<const uint2*>(sts[r])[it - i0]
                                                : reinterpret_cast<const uint2*>(rows[r])[it];
            half_decode<DT>(raw, x[r][q]);
          } else {
#pragma unroll
            for (int e = 0; e < HV; ++e) x[r][q][e] = -INFINITY;
          }
        } else {
          x[r][q][0] = in ? row_value<DT>(rows[r], it) : -INFINITY;
        }
      }
    float tm[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      tm[r] = -INFINITY;
#pragma unroll
      for (int q = 0; q < kStatUnits; ++q)
#pragma unroll
        for (int e = 0; e < HV; ++e)
          if (e < w) tm[r] = fmaxf(tm[r], x[r][q][e]);
      tm[r] = wave_max(tm[r]);
    }
    if ((threadIdx.x & 63) == 0) {
      wred[wv][0] = tm[0];
      wred[wv][1] = tm[1];
    }
    __syncthreads();
    double bm[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float m = wred[0][r];
#pragma unroll
      for (int q = 1; q < kWaves; ++q) m = fmaxf(m, static_cast<float>(wred[q][r]));
      bm[r] = fmax(M[r], static_cast<double>(m));   // the running maximum after this batch
    }
    double ts[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      ts[r] = 0.0;
      if (bm[r] != -INFINITY) {
#pragma unroll
        for (int q = 0; q < kStatUnits; ++q) {
          // only items of the slice: a wave with none at a batch position skips its exps
          if (r < nr && b0 + q * kBlock + static_cast<int>(threadIdx.x) < i1) {
            if (vec) {
              ts[r] += exp_nonpos_sum<HV, HV>(x[r][q], bm[r], tab);
            } else {
              ts[r] += exp_nonpos(static_cast<double>(x[r][q][0]) - bm[r], tab);
            }
          }
        }
      }
      ts[r] = wave_sum(ts[r]);
    }
    if ((threadIdx.x & 63) == 0) {   // (the sums go to entries 2 and 3, the maxima stay in 0 and 1)
      wred[wv][2] = ts[0];
      wred[wv][3] = ts[1];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      double bs = 0.0;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) bs += wred[q][2 + r];
      if (bm[r] != -INFINITY) {
        S[r] = (M[r] == -INFINITY ? 0.0 : S[r] * exp_nonpos(M[r] - bm[r], tab)) + bs;
        M[r] = bm[r];
      }
    }
    if (b0 + kBlock * kStatUnits < i1) __syncthreads();   // read before the next batch writes it
  }
  if (threadIdx.x == 0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      out[2 * r] = M[r];
      out[2 * r + 1] = S[r];
    }
  }
}

// Sum of the G <= 32 slice values vals[0 .. G), lane k % 32 holding value k, by a fixed
// reduction order: every wave of every workgroup adds them the same way, so all get the
// same bits.
__device__ __forceinline__ double group_sum(const double* vals, int G) {
  const int k = threadIdx.x & 31;
  double lo, hi;
  half_wave_reduce(k < G ? vals[k] : 0.0, [](double x, double y) { return x + y; }, lo, hi);
  return lo;
}

// log sum exp of the target (lanes 0..31) and draft (lanes 32..63) rows from the (max, sum)
// pairs of the G slices, vals[4 k .. 4 k + 3] = (target max, target sum, draft max, draft
// sum) of slice k: lane l merges slice l % 32 of its row, each half of the wave combines
// them. Every wave of every workgroup computes it the same way, so all see the same bits.
__device__ __forceinline__ void merged_lse2(const double* vals, int G, const double* tab, double& lt, double& ld) {
  const int lane = threadIdx.x & 63;
  const int k = lane & 31, r = lane >> 5;
  const double m = k < G ? vals[4 * k + 2 * r] : -INFINITY;
  const double sm = k < G ? vals[4 * k + 2 * r + 1] : 0.0;
  double Mt, Md;
  half_wave_reduce(m, [](double x, double y) { return y > x ? y : x; }, Mt, Md);
  const double M = r == 0 ? Mt : Md;
  double St, Sd;
  half_wave_reduce(m == -INFINITY ? 0.0 : sm * exp_nonpos(m - M, tab), [](double x, double y) { return x + y; },
                   St, Sd);
  const double l = log(r == 0 ? St : Sd);   // one log per lane: the target's in the first half
  lt = Mt + read_lane(l, 0);
  ld = Md + read_lane(l, 32);
}

// One rejection: out = max(p - q, 0) over this workgroup's units (entry j at j - d.base);
// returns the block-wide slice sum.
template <int DT>
__device__ double residual_slice(const WalkDist<DT>& d, double* out, const WalkGroup& g, SampleSmem& sm) {
  constexpr int VEC = WalkDist<DT>::VEC;
  const int w = d.width();
  double loc = 0.0;
#pragma unroll 2
  for (int a = g.u0 + static_cast<int>(threadIdx.x); a < g.u1; a += kBlock) {
    double pv[VEC], qv[VEC];
    d.p_unit(a, pv);
    d.q_unit(a, qv);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (e < w) {
        const double r = fmax(pv[e] - qv[e], 0.0);
        out[a * w + e - d.base] = r;
        loc += r;
      }
    }
  }
  return block_sum(loc, sm.rs.redd);
}

// Inverse CDF inside this workgroup's units, continuing a running sum `base` (the mass of
// all earlier units): the smallest entry k with base + sum_{j<=k} p(j) > target, or -1 if
// the slice does not reach it. Threads take contiguous runs of units in order, so one
// block scan of the per-thread sums orders them as the row.
template <int DT>
__device__ int slice_inverse_cdf(const WalkDist<DT>& d, const WalkGroup& g, double base, double target,
                                 SampleSmem& sm) {
  constexpr int VEC = WalkDist<DT>::VEC;
  const int w = d.width();
  const int n = g.u1 - g.u0;
  const int per = (n + kBlock - 1) / kBlock;
  const int a0 = g.u0 + static_cast<int>(threadIdx.x) * per, a1 = min(g.u1, a0 + per);
  double loc = 0.0;
#pragma unroll 2
  for (int a = a0; a < a1; ++a) {
    double pv[VEC];
    d.p_unit(a, pv);
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (e < w) loc += pv[e];
  }
  double total = 0.0;
  const double excl = base + block_exclusive_scan(loc, sm.wsum, &total);
  if (threadIdx.x == 0) {
    sm.first = kBlock;
    sm.pick = -1;
  }
  __syncthreads();
  if (a1 > a0 && excl + loc > target) atomicMin(&sm.first, static_cast<int>(threadIdx.x));
  __syncthreads();
  if (static_cast<int>(threadIdx.x) == sm.first) {
    double run = excl;
    int k = -1;
    for (int a = a0; a < a1 && k < 0; ++a) {
      double pv[VEC];
      d.p_unit(a, pv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        if (e < w) {
          run += pv[e];
          if (k < 0 && run > target) k = a * w + e;
        }
      }
    }
    sm.pick = k < 0 ? a1 * w - 1 : k;   // rounding between the two sums: end of the run
  }
  __syncthreads();
  return sm.pick;
}

// Shared-memory copies of a workgroup's units of a node's two rows: the node the walk is at
// and the child being tried, whose copies are loaded while the current node's tests and
// exchanges run (a slice of at most kStageUnits 16-byte units; larger slices read memory).
constexpr int kStageUnits = 512;

// Issues direct loads of units [g.u0, g.u1) of `row` into lds[0 .. g.u1 - g.u0). Waves 1..3
// issue them: a wave's loads finish in order with every later global load of that wave, and
// wave 0 polls the exchanges, which must not wait for these. Wave w covers the 64-unit
// blocks at 64 (w - 1) + 192 i (lane l of a direct load fills the 16 bytes at 16 l after
// the load's base); a block's units past u1 reload unit u1 - 1 into the buffer's tail, which
// nobody reads. Every block starts below u1 - u0 <= kStageUnits and kStageUnits is a
// multiple of 64, so every write stays inside the buffer. Every thread must call it; the
// data is there after drain() and a barrier. Shared-memory reads of the buffers wait for
// all of a wave's outstanding direct loads (the compiler cannot tell the two buffers
// apart), so the walk issues a prefetch only after the last read of the current copies.
__device__ __forceinline__ void stage_issue(const void* row, uint4* lds, const WalkGroup& g) {
  typedef __attribute__((address_space(3))) void lds_void_t;
  const int count = g.u1 - g.u0;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (w == 0) return;
  const uint4* src = reinterpret_cast<const uint4*>(row);
  for (int b0 = 64 * (w - 1); b0 < count; b0 += 64 * (kWaves - 1)) {
    const int u = g.u0 + min(b0 + lane, count - 1);
    __builtin_amdgcn_global_load_lds(src + u, (lds_void_t*)(lds + b0), 16, 0, 0);
  }
}

// The walk of sequence blockIdx.x / G, shared by its G workgroups (the exchanges need them
// all resident: the launch keeps the grid within what the device holds).
template <int DT>
__global__ __launch_bounds__(kBlock) void sample_walk_kernel(SampleArgs a) {
  __shared__ SampleSmem sm;
  __shared__ double gvals[kXchStride];
  __shared__ double slice_buf[3][kWalkSlice];   // residuals (two) and q of this slice
  __shared__ uint4 stage[2][2][kStageUnits];     // [node buffer][target, draft][unit]
  __shared__ int rowof[kSampleMaxNodes];         // every node's row
  using Rw = RowT<DT>;
  row_smem_init(sm.rs);
  const int s = blockIdx.x / a.G;
  const int cap = a.tree.n_cap;
  const int N = a.tree.n_nodes[s];
  if (N < 1 || N > cap) {   // every workgroup of the group leaves: no exchange is entered
    if (threadIdx.x == 0) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  const size_t tb = static_cast<size_t>(s) * cap;
  const size_t row_bytes = static_cast<size_t>(a.V) * Rw::ESIZE;
  if (threadIdx.x == 0) sm.flag = 0;
  __syncthreads();
  for (int v = threadIdx.x; v < N; v += kBlock) {
    sm.par[v] = static_cast<short>(a.tree.parent[tb + v]);
    sm.tok[v] = a.tree.token[tb + v];
    sm.uacc[v] = a.u_acc[tb + v];
    sm.ures[v] = a.u_res[tb + v];
    // rows are read at every node the walk may visit, tokens at every child tried: both
    // must lie inside the tables
    const int r = a.tree.row[tb + v];
    rowof[v] = r;
    if (r < 0 || r >= a.R || (v > 0 && (sm.tok[v] < 0 || sm.tok[v] >= a.V))) sm.flag = 1;
  }
  __syncthreads();   // also publishes the exp table
  if (sm.flag) {   // every workgroup of the group sees the same tree and leaves here
    if (blockIdx.x % a.G == 0 && threadIdx.x == 0) {
      atomicExch(&a.hdr->err, kErrBadRow);
      a.path_len[s] = 0;
      a.bonus[s] = -1;
      if (a.kvc.k != nullptr) a.kvc.P_new[s] = -1;
    }
    return;
  }
  const bool vec = a.vec != 0;   // decided by the host plan (rows aligned, V a multiple of VEC)
  WalkGroup grp;
  grp.gi = blockIdx.x % a.G;
  grp.G = a.G;
  {
    const int units = vec ? a.V / Rw::VEC : a.V;
    grp.u0 = static_cast<int>(static_cast<long>(units) * grp.gi / a.G);
    grp.u1 = static_cast<int>(static_cast<long>(units) * (grp.gi + 1) / a.G);
  }
  grp.max_pass = a.max_pass;
  grp.xch = reinterpret_cast<unsigned long long*>(a.xch) + static_cast<size_t>(s) * a.max_pass * kXchStride;
  grp.err = &a.hdr->err;
  grp.pass = 0;
  // residual buffers and q cache: this slice in shared memory when it fits, else the
  // sequence's rows of the workspace (indexed by entry)
  const int wdt = vec ? Rw::VEC : 1;
  const bool in_lds = (grp.u1 - grp.u0) * wdt <= kWalkSlice;
  const int base = in_lds ? grp.u0 * wdt : 0;
  double* P[2];
  double* Q;
  if (in_lds) {
    P[0] = slice_buf[0];
    P[1] = slice_buf[1];
    Q = slice_buf[2];
  } else {
    P[0] = a.pbuf + static_cast<size_t>(s) * 3 * a.V;
    P[1] = P[0] + a.V;
    Q = P[1] + a.V;
  }
  const double inv32 = 1.0 / 4294967296.0;
  const bool lead = grp.gi == 0;
  // shared-memory copies of the rows (this workgroup's units): the root's now
  const bool staged = vec && grp.u1 - grp.u0 <= kStageUnits && grp.u1 > grp.u0;
  int sbuf = 0;   // stage buffer holding the rows of the node the walk is at
  auto row_ptr = [&](const void* table, int r) {
    return static_cast<const char*>(table) + (static_cast<size_t>(s) * a.R + r) * row_bytes;
  };
  auto prefetch = [&](int node, int buf) {   // every thread; the rows were checked above
    stage_issue(row_ptr(a.target, rowof[node]), stage[buf][0], grp);
    stage_issue(row_ptr(a.draft, rowof[node]), stage[buf][1], grp);
  };
  if (staged) prefetch(0, 0);
  int v = 0, A = 0;
  if (lead && threadIdx.x == 0) a.path[tb] = 0;
  if (threadIdx.x == 0) sm.spath[0] = 0;
  for (;;) {
    // children of v in slot order: in each round of kBlock slots every wave ballots its 64,
    // and a child's place is the count in earlier waves and rounds plus its lane rank
    int nk = 0;
    for (int k0 = 0; k0 < N; k0 += kBlock) {
      const int k = k0 + static_cast<int>(threadIdx.x);
      const bool is = k >= 1 && k < N && sm.par[k] == v;
      const unsigned long long m = __ballot(is);
      if ((threadIdx.x & 63) == 0) sm.kmask[threadIdx.x >> 6] = m;
      __syncthreads();
      int before = nk, tot = nk;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        const int c = __popcll(sm.kmask[q]);
        before += q < static_cast<int>(threadIdx.x >> 6) ? c : 0;
        tot += c;
      }
      if (is) sm.kids[before + lanes_below(m)] = k;
      nk = tot;
      __syncthreads();   // the places are written and kmask is free for the next round
    }
    const int r = rowof[v];
    WalkDist<DT> d;
    d.trow = row_ptr(a.target, r);
    d.drow = row_ptr(a.draft, r);
    d.tst = staged ? stage[sbuf][0] : nullptr;
    d.dst = staged ? stage[sbuf][1] : nullptr;
    d.u0 = grp.u0;
    // this node's rows have landed once every wave's loads are done and a barrier has passed
    if (staged) {
      drain();
      __syncthreads();
    }
    // The node's normalisers: every workgroup reduces its slice of the target row (and of
    // the draft row when children are tried) and the group exchanges the four values.
    float t_first = 0.f, d_first = 0.f;
    uint32_t u_first = 0u;
    {
      double st[4];
      slice_stats<DT>(d.trow, d.drow, d.tst, d.dst, nk > 0 ? 2 : 1, grp, vec, sm.rs.exptab, sm.wpair, st);
      // the first child's rows load into the other buffer during the exchange and the test
      // (slice_stats ends with a barrier: every read of this node's copies is done)
      if (staged && nk > 0) prefetch(sm.kids[0], sbuf ^ 1);
      // thread 0 loads what the first acceptance test needs (the child's logits in both rows
      // and its uniform) during the exchange. Issued before the pass, these loads would hold
      // it up: a wave's reads of the staged copies wait for all of its outstanding loads.
      if (threadIdx.x == 0 && nk > 0) {
        const int x = sm.tok[sm.kids[0]];
        t_first = row_value<DT>(d.trow, x);
        d_first = row_value<DT>(d.drow, x);
        u_first = sm.uacc[sm.kids[0]];
      }
      if (!group_exchange(grp, st, 4, false, 0.0, 0.0, false, gvals, &sm.flag)) {
        drain();   // no stage load is left in flight
        return;
      }
      for (int k = threadIdx.x; k < 4 * grp.G; k += kBlock) sm.lsev[k] = gvals[k];
      merged_lse2(gvals, grp.G, sm.rs.exptab, d.lt, d.ld);
      if (nk == 0) d.ld = 0.0;
      __syncthreads();   // the copy is complete before gvals is reused
    }
    d.pc = nullptr;
    d.zc = 1.0;
    d.qc = Q;
    d.qvalid = false;
    d.base = base;
    d.tab = sm.rs.exptab;
    d.vec = vec;
    int cur = -1;
    int accepted = -1;
    double px_next = 0.0;   // p at the next child's token, as published by the last exchange
    double z_last = 0.0;    // sum of the last residual when it became p (its slice sums are in gvals)
    for (int q = 0; q < nk; ++q) {
      const int ch = sm.kids[q];
      if (threadIdx.x == 0) {
        // p and q at the child's token: the first try from the prefetched logits, a later
        // one from the value the last exchange published and the prefetched draft logit
        const double px = (q == 0) ? exp_nonpos(static_cast<double>(t_first) - d.lt, d.tab) : px_next;
        const double qx = exp_nonpos(static_cast<double>(d_first) - d.ld, d.tab);
        const double u = (static_cast<double>(u_first) + 0.5) * inv32;
        sm.accept = (qx > 0.0) ? (u < px / qx ? 1 : 0) : (px > 0.0 ? 1 : 0);
      }
      __syncthreads();
      if (sm.accept) {
        accepted = ch;
        __syncthreads();
        break;
      }
      // rejection: residual (p - q)+ into the other buffer; kept only if it sums to > 0.
      // The owner of the next child's token publishes, for that token, the new residual
      // and the current p (used if the residual sums to 0).
      const int nxt = (cur == 0) ? 1 : 0;
      const double part = residual_slice<DT>(d, P[nxt], grp, sm);
      d.qvalid = true;   // residual_slice ends with a block barrier: the cache is complete
      // the next child's rows load during this rejection's exchange (after the residual
      // pass, the last reader of this node's copies; the rejected child's copies, loaded
      // into the same buffer, have landed by now)
      if (staged && q + 1 < nk) {
        drain();
        prefetch(sm.kids[q + 1], sbuf ^ 1);
      }
      const int xn = (q + 1 < nk) ? sm.tok[sm.kids[q + 1]] : -1;
      const int xu = vec ? xn / Rw::VEC : xn;
      const bool owner = xn >= 0 && xu >= grp.u0 && xu < grp.u1;
      if (xn >= 0 && threadIdx.x == 0) {   // the next try's draft logit and uniform, during the exchange
        d_first = row_value<DT>(d.drow, xn);
        u_first = sm.uacc[sm.kids[q + 1]];
      }
      double e0 = 0.0, e1 = 0.0;
      if (owner && threadIdx.x == 0) {
        e1 = d.p(xn);
        e0 = fmax(e1 - d.q(xn), 0.0);   // the entry residual_slice stored for xn
      }
      if (!group_exchange(grp, &part, 1, owner, e0, e1, xn >= 0, gvals, &sm.flag)) {
        drain();   // no stage load is left in flight
        return;
      }
      const double z = group_sum(gvals, grp.G);
      if (z > 0.0) {
        cur = nxt;
        d.pc = P[cur];
        d.zc = z;
        px_next = gvals[grp.G] / z;
      } else {
        px_next = gvals[grp.G + 1];
      }
      z_last = z;
    }
    if (accepted >= 0) {
      v = accepted;
      sbuf ^= 1;   // the accepted child's rows are in the prefetch buffer
      ++A;
      if (lead && threadIdx.x == 0) a.path[tb + A] = v;
      if (threadIdx.x == 0) sm.spath[A] = v;
      continue;
    }
    // bonus: inverse CDF of the current p with u_res[v]; slice masses first. After a
    // rejection whose residual became p, they are that exchange's slice sums over z; while
    // p is still the target's softmax (a leaf, or residuals that summed to 0 every time),
    // they follow from the node's slice statistics, m_g and s_g: s_g exp(m_g - lt); else one
    // pass and an exchange find them.
    const double u = (static_cast<double>(sm.ures[v]) + 0.5) * inv32;
    if (z_last > 0.0) {
      __syncthreads();
      for (int k = threadIdx.x; k < grp.G; k += kBlock) gvals[k] /= z_last;
      __syncthreads();
    } else if (d.pc == nullptr) {
      __syncthreads();
      for (int k = threadIdx.x; k < grp.G; k += kBlock)
        gvals[k] = sm.lsev[4 * k] == -INFINITY ? 0.0 : sm.lsev[4 * k + 1] * exp_nonpos(sm.lsev[4 * k] - d.lt, d.tab);
      __syncthreads();
    } else {
      constexpr int VEC = Rw::VEC;
      const int w = d.width();
      double loc = 0.0;
#pragma unroll 2
      for (int a2 = grp.u0 + static_cast<int>(threadIdx.x); a2 < grp.u1; a2 += kBlock) {
        double pv[VEC];
        d.p_unit(a2, pv);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          if (e < w) loc += pv[e];
      }
      const double mass = block_sum(loc, sm.rs.redd);
      if (!group_exchange(grp, &mass, 1, false, 0.0, 0.0, false, gvals, &sm.flag)) {
        drain();   // no stage load is left in flight
        return;
      }
    }
    const double total = group_sum(gvals, grp.G);
    const double target = u * total;
    // the first workgroup whose slice takes the running sum past the target draws the
    // token; if rounding leaves the target at the end, the last slice with mass does. Lane
    // k of every wave holds slice k's mass and a prefix sum in registers gives the running
    // sums (the same order in every wave of every workgroup, hence the same bits).
    const int lk = threadIdx.x & 63;
    const double gk = lk < grp.G ? gvals[lk] : 0.0;
    const double incl = wave_inclusive_scan(gk);
    const double mybase = read_lane(wave_shift_up1(incl), grp.gi);   // the mass before this slice
    const unsigned long long passed = __ballot(lk < grp.G && gk > 0.0 && incl > target);
    const unsigned long long massive = __ballot(lk < grp.G && gk > 0.0);
    const int owner = passed != 0ull ? static_cast<int>(__builtin_ctzll(passed))
                                     : (massive != 0ull ? 63 - static_cast<int>(__builtin_clzll(massive)) : 0);
    if (grp.gi == owner) {
      int k = slice_inverse_cdf<DT>(d, grp, mybase, target, sm);
      if (threadIdx.x == 0) {
        const int hi = grp.u1 * d.width() - 1, lo = grp.u0 * d.width();
        if (k < 0) k = hi;
        while (k > lo && !(d.p(k) > 0.0)) --k;   // the drawn entry carries mass
        a.bonus[s] = k;
      }
    }
    break;
  }
  if (lead && threadIdx.x == 0) a.path_len[s] = A + 1;
  if (a.kvc.k != nullptr) {   // the group's workgroups share the (head, tensor) pairs
    __syncthreads();
    const bool done = walk_compact(a.kvc, s, cap, sm.spath, A + 1, grp.gi, grp.G);
    if (lead && threadIdx.x == 0) a.kvc.P_new[s] = done ? a.kvc.P[s] + A + 1 : -1;
  }
  // The last workgroup of the group to finish empties the exchange slots the walk used (every
  // workgroup arrives only after its last read of them), ready for the next call.
  if (last_arrival(&a.done[s], static_cast<unsigned>(grp.G), &sm.flag)) {
    const size_t used = static_cast<size_t>(grp.pass) * kXchStride;
    for (size_t k = threadIdx.x; k < used; k += kBlock) grp.xch[k] = 0ull;
  }
}

int launch_verify_sample(const SampleArgs& a, int S, int dtype, hipStream_t st) {
  // An ordinary launch on the caller's stream: the grid (S * G) is at most the number of
  // workgroups the device holds at once, so every group is resident together once the
  // stream reaches this kernel. (A cooperative launch is avoided: measured on MI355X it
  // let consecutive walks share the group barrier and time out now and then.)
  if (dtype == 1)
    DTV_LAUNCH(sample_walk_kernel<1>, dim3(S * a.G), dim3(kBlock), 0, st, a);
  else
    DTV_LAUNCH(sample_walk_kernel<0>, dim3(S * a.G), dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Workgroups of the walk kernel that can be resident at once (queried once per device).
int sample_walk_max_blocks(int dtype) {
  static int cached[64][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  int& c = cached[dev][dtype ? 1 : 0];
  if (c > 0) return c;
  int ncu = 0, per = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  const void* fn = dtype ? reinterpret_cast<const void*>(&sample_walk_kernel<1>)
                         : reinterpret_cast<const void*>(&sample_walk_kernel<0>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, kBlock, 0) != hipSuccess || per < 1) return -1;
  c = ncu * per;
  return c;
}

int launch_verify_greedy(const VerifyArgs& a, int S, int dtype, hipStream_t st) {
  if (dtype == 1) {   // parts of 32768 values; their slots fit the workspace's chunk slots
    const int np = parts_of(a.V);
    if (np > a.nch) return -1;
    DTV_LAUNCH(verify_greedy_bf16_kernel, dim3(S * a.tree.n_cap * np), dim3(kPartThreads), 0, st, a);
  } else {
    DTV_LAUNCH(verify_greedy_kernel<0>, dim3(S * a.tree.n_cap * a.nch), dim3(kBlock), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace dtv
