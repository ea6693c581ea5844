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
__device__ bool walk_compact(const KvCompactView& c, int s, int n_cap, const int* spath, int L, int pair0,
                             int pstep) {
  const int P = c.P[s];
  if (L < 1 || L > n_cap || P < 0 || P + n_cap > c.P_cap) return false;
  const int vpr = c.D * c.esize / 16;   // 16-byte vectors per row
  const size_t row_bytes = static_cast<size_t>(c.D) * c.esize;
  const int npairs = pair0 < 2 * c.Hkv ? (2 * c.Hkv - pair0 + pstep - 1) / pstep : 0;
  const int per_pair = L * vpr;
  const int total = npairs * per_pair;
  constexpr int kPer = 4;   // vectors per thread and batch, all loaded before any store
  for (int b0 = 0; b0 < total; b0 += kBlock * kPer) {
    uint4 val[kPer];
    char* dst[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int v = min(b0 + q * kBlock + static_cast<int>(threadIdx.x), total - 1);
      const int pi = v / per_pair, rem = v % per_pair;
      const int k = rem / vpr, ch = rem % vpr;
      const int pair = pair0 + pi * pstep;
      char* base = ((pair & 1) ? c.v : c.k) +
                   (static_cast<size_t>(s) * c.Hkv + (pair >> 1)) * c.P_cap * row_bytes;
      val[q] = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(P + spath[k]) * row_bytes + ch * 16);
      dst[q] = base + static_cast<size_t>(P + k) * row_bytes + ch * 16;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPer; ++q)
      if (b0 + q * kBlock + static_cast<int>(threadIdx.x) < total) *reinterpret_cast<uint4*>(dst[q]) = val[q];
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
  unsigned long long redu[kWaves];
  int flag;
};

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

  // ---- the walk, by the sequence's last workgroup. The tree is loaded first, so that its
  //      loads are in flight with the first polls; every thread then polls its share of
  //      the N * nch chunk slots (node-major), up to 8 at once, until all have reported,
  //      folds them into its node's maximum in shared memory and clears them for the next
  //      call.
  if (threadIdx.x == 0) sm.flag = 0;
  __syncthreads();
  for (int v = threadIdx.x; v < N; v += kBlock) {
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
  for (int j0 = 0; j0 < total; j0 += kBlock * 8) {
    unsigned long long b[8];
    long polls = 0;
    for (;;) {
      bool all = true;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q * kBlock + static_cast<int>(threadIdx.x);
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
      const int j = j0 + q * kBlock + static_cast<int>(threadIdx.x);
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
  for (int v = threadIdx.x; v < N; v += kBlock) {
    const int am = sort_key_index(sm.best[v]);
    sm.a[v] = am;
    if (a.argmax_out) a.argmax_out[tb + v] = am;
  }
  if (!ok) atomicExch(&a.hdr->err, kErrTimeout);
  __syncthreads();
  // a node is bad when its token is not the target argmax at its parent (or its parent
  // link is not an earlier slot, which also bounds every walk below)
  for (int v = threadIdx.x; v < N; v += kBlock) {
    const int p = sm.par[v];
    sm.bad[v] = (v > 0 && (p < 0 || p >= v || sm.tok[v] != sm.a[p])) ? 1 : 0;
  }
  __syncthreads();
  // deepest accepted node, lowest slot among equals: maximise (depth << 20) | (2^20 - 1 - slot);
  // node v is accepted when no node on its root path is bad (slots grow away from the root)
  unsigned long long pick = 0;
  for (int v = threadIdx.x; v < N; v += kBlock) {
    bool ok = true;
    for (int u = v; u > 0 && ok; u = sm.par[u]) ok = !sm.bad[u];
    if (ok) {
      const unsigned long long key2 = (static_cast<unsigned long long>(sm.dep[v]) << 20) |
                                      static_cast<unsigned long long>(0xFFFFF - v);
      pick = key2 > pick ? key2 : pick;
    }
  }
  pick = block_max(pick, sm.redu);
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
    const bool done = walk_compact(a.kvc, s, cap, sm.tok, A + 1, 0, 1);
    if (threadIdx.x == 0) a.kvc.P_new[s] = done ? a.kvc.P[s] + A + 1 : -1;
  }
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
// Work split: a grid of resident workgroups reduces every chunk of every node's target and
// draft rows to (max, float64 sum of exp), loading the next chunk while reducing the
// current one; the rows' log-sum-exps are merged from those (by a small kernel, or inside
// the walk for small trees). The walk of a sequence is shared by G workgroups, each owning
// a slice of the vocabulary: a first try needs only the two row values at the child's
// token; each rejection costs one residual pass over the slices (kept in shared memory
// when they fit) and one exchange of slice sums; the bonus draw is one prefix-sum pass.

struct SampleSmem {
  RowSmem rs;
  short par[kSampleMaxNodes];
  int tok[kSampleMaxNodes];
  double lset[kSampleMaxNodes];
  double lsed[kSampleMaxNodes];
  int kids[kSampleMaxNodes];
  int spath[kSampleMaxNodes];   // the accepted path so far (every workgroup of the group)
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
    row_vec<DT>(drow, a, x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      out[e] = exp_nonpos(static_cast<double>(x[e]) - ld, tab);
      qc[a * VEC + e - base] = out[e];
    }
  }
};

// The G workgroups of a sequence share every V-wide pass: workgroup gi owns units
// [u0, u1). Every exchange (one per pass) uses a slot of its own: entry gi receives
// workgroup gi's slice sum, entries G and G+1 two values from the owner of the next
// child's token (see the walk). The previous kernel fills every entry with an empty
// marker (a NaN no sum or probability takes), each entry is written once, and the readers
// poll the entries they need until none holds the marker, so an exchange costs one store
// and the polls, with no counter and no fence: the values are the signal. Every
// workgroup then adds the sums in workgroup order, so all of them see identical totals
// and take identical decisions.
constexpr unsigned long long kSlotEmpty = 0x7FF8DEAD00000000ull;
constexpr long kSpinLimit = 2000000;    // polls (each a memory round trip) before a timeout

struct WalkGroup {
  int gi, G;
  int u0, u1;                 // this workgroup's units
  double* xch;                // [max_pass][kXchStride] exchange slots
  int max_pass;
  int* err;
  int pass;                   // exchanges so far
};

// Publishes this workgroup's slice value (and, from the owner, e0 / e1 into slot entries G
// and G+1), waits until the group's G values (and the owner's two when `extra`) are in
// and copies them into sm_vals. Returns false on a timeout or when the slots are exhausted.
__device__ bool group_exchange(WalkGroup& g, double mine, bool owner, double e0, double e1, bool extra,
                               double* sm_vals, int* flag) {
  if (g.pass >= g.max_pass) {
    if (threadIdx.x == 0) atomicExch(g.err, kErrCapacity);
    return false;
  }
  double* slot = g.xch + static_cast<size_t>(g.pass) * kXchStride;
  if (threadIdx.x == 0) {
    st_cc(&slot[g.gi], mine);
    if (owner) {
      st_cc(&slot[g.G], e0);
      st_cc(&slot[g.G + 1], e1);
    }
  }
  ++g.pass;
  const int nv = g.G + (extra ? 2 : 0);
  if (threadIdx.x < 64) {   // wave 0: lane k waits for entry k
    const int k = threadIdx.x;
    int ok = 1;
    if (k < nv) {
      unsigned long long* e = reinterpret_cast<unsigned long long*>(&slot[k]);
      unsigned long long bits = ld_cc(e);
      long polls = 0;
      while (bits == kSlotEmpty) {
        __builtin_amdgcn_s_sleep(1);
        if (++polls > kSpinLimit) {
          ok = 0;
          break;
        }
        bits = ld_cc(e);
      }
      sm_vals[k] = __longlong_as_double(static_cast<long long>(bits));
    }
    if (!ok) atomicExch(g.err, kErrTimeout);
    const unsigned long long good = __ballot(ok);
    if (k == 0) *flag = (good == ~0ull) ? 1 : 0;
  }
  __syncthreads();
  return *flag != 0;
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

// log-sum-exp of a row from its chunk statistics (nch <= 64), by wave 0; the result is
// valid in lane 0.
__device__ __forceinline__ double chunk_lse(const ChunkStat* st, int nch, const double* tab) {
  const int c = threadIdx.x;
  const float mc = c < nch ? ld_cc(&st[c].maxv) : -INFINITY;
  const double sc = c < nch ? ld_cc(&st[c].sumexp) : 0.0;
  const float M = wave_max(mc);
  const double term = (c < nch && mc != -INFINITY)
                          ? sc * exp_nonpos(static_cast<double>(mc) - static_cast<double>(M), tab) : 0.0;
  const double sum = wave_sum(term);
  return static_cast<double>(M) + log(sum);
}

// Phase 1: (max, float64 sum of exp) of every chunk of every node's target and draft rows.
// Work item it = ((s * n_cap + i) * 2 + row kind) * nch + chunk, the index of its ChunkStat.
// A grid of resident workgroups walks the items with a stride of the grid size; each
// workgroup issues the loads of its next chunk (and the tree lookups of the one after)
// before reducing the current chunk, so loading overlaps the float64 exponentials. The
// statistics are plain stores read after the kernel boundary (by the merge kernel or the
// walk), so no workgroup waits on another here.
template <int DT>
__global__ __launch_bounds__(kBlock) void sample_lse_kernel(SampleArgs a) {
  __shared__ RowSmem rs;
  __shared__ float wmax[2][kWaves];    // per-wave results, double-buffered by item parity
  __shared__ double wse[2][kWaves];
  using Rw = RowT<DT>;
  row_smem_init(rs);
  {   // every exchange slot of the walk starts empty
    unsigned long long* x = reinterpret_cast<unsigned long long*>(a.xch);
    const size_t n = static_cast<size_t>(a.S) * a.max_pass * kXchStride;
    for (size_t q = static_cast<size_t>(blockIdx.x) * kBlock + threadIdx.x; q < n;
         q += static_cast<size_t>(gridDim.x) * kBlock)
      x[q] = kSlotEmpty;
  }
  __syncthreads();
  const int nch = a.nch;
  const int cap = a.tree.n_cap;
  const int items = a.S * cap * 2 * nch;
  const int step = static_cast<int>(gridDim.x);
  const size_t row_bytes = static_cast<size_t>(a.V) * Rw::ESIZE;
  const int w = threadIdx.x >> 6;

  // Reduces chunk values x of item `it` to its ChunkStat (wave results combined by thread 0).
  auto reduce = [&](const float (&x)[Rw::E], int it, bool real, int par) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < Rw::E; ++j) m = fmaxf(m, x[j]);
    const float mw = wave_max(m);
    double se = 0.0;
    if (mw != -INFINITY) se = exp_nonpos_sum<Rw::E>(x, static_cast<double>(mw), rs.exptab);
    se = wave_sum(se);
    if ((threadIdx.x & 63) == 0) {
      wmax[par][w] = mw;
      wse[par][w] = se;
    }
    __syncthreads();
    if (threadIdx.x == 0 && real) {
      float M = -INFINITY;
      for (int q = 0; q < kWaves; ++q) M = fmaxf(M, wmax[par][q]);
      double S = 0.0;
      for (int q = 0; q < kWaves; ++q)
        if (wmax[par][q] != -INFINITY)
          S += wse[par][q] * exp_nonpos(static_cast<double>(wmax[par][q]) - static_cast<double>(M), rs.exptab);
      a.st[it].maxv = M;
      a.st[it].sumexp = S;
    }
  };
  // Tree lookups (node count, row) of this workgroup's items, loaded once: lane j holds
  // those of its j-th item (the grid gives no workgroup more than 64 items), so the loop
  // reads them with a lane shuffle instead of waiting on a load per item.
  struct Meta {
    int n, r;
  };
  int bn, br;
  {
    const int itj = static_cast<int>(blockIdx.x) + (static_cast<int>(threadIdx.x) & 63) * step;
    const int node = min(itj, items - 1) / nch / 2;   // s * cap + i
    bn = a.tree.n_nodes[node / cap];
    br = a.tree.row[node];
  }
  auto meta = [&](int k) {   // k: the item's position in this workgroup's sequence
    Meta m;
    m.n = __shfl(bn, k, 64);
    m.r = __shfl(br, k, 64);
    return m;
  };
  // Row of item `it`; `real` is false for items past the end or past the sequence's node
  // count (those load row 0 of their sequence and store nothing).
  auto row_of = [&](int it, const Meta& m, bool& real) {
    const int b2 = min(it, items - 1) / nch;
    const int node = b2 >> 1, s = node / cap, i = node % cap;
    if (it < items && m.n > cap && threadIdx.x == 0) atomicExch(&a.hdr->err, kErrCapacity);
    const bool in_tree = it < items && i < m.n && m.n <= cap;
    real = in_tree && m.r >= 0 && m.r < a.R;
    // a row outside the table is never read; the walk refuses the tree
    if (in_tree && !real && threadIdx.x == 0) atomicExch(&a.hdr->err, kErrBadRow);
    return static_cast<const char*>((b2 & 1) ? a.draft : a.target) +
           (static_cast<size_t>(s) * a.R + (real ? m.r : 0)) * row_bytes;
  };

  const bool vec = a.V >= Rw::VEC && row_bytes % 16 == 0 &&
                   ((reinterpret_cast<uintptr_t>(a.target) | reinterpret_cast<uintptr_t>(a.draft)) & 15u) == 0;
  int par = 0;
  if (!vec) {   // unaligned rows: one synchronous chunk at a time
    for (int it = blockIdx.x, k = 0; it < items; it += step, ++k) {
      bool real;
      const char* row = row_of(it, meta(k), real);
      float x[Rw::E];
      uint32_t key[Rw::E];
      load_chunk<DT>(row, a.V, it % nch, x, key);
      reduce(x, it, real, par);
      par ^= 1;
    }
    return;
  }
  int it = blockIdx.x;
  bool real0;
  const char* row0 = row_of(it, meta(0), real0);
  RawChunk rc;
  raw_chunk_load<DT>(row0, a.V, min(it, items - 1) % nch, rc);
  for (int k = 1; it < items; it += step, ++k) {
    bool real1;
    const char* row1 = row_of(it + step, meta(k), real1);
    RawChunk rn;
    raw_chunk_load<DT>(row1, a.V, min(it + step, items - 1) % nch, rn);
    float x[Rw::E];
    raw_chunk_decode<DT>(row0, a.V, it % nch, rc, x);
    reduce(x, it, real0, par);
    par ^= 1;
    rc = rn;
    row0 = row1;
    real0 = real1;
  }
}

// log-sum-exp of one row from its nch chunk statistics, merged with a running maximum;
// the statistics are loaded 8 at a time (clamped indices, extra entries ignored) so that
// their loads are in flight together.
__device__ double row_lse_from_stats(const ChunkStat* st, int nch, const double* tab) {
  float M = -INFINITY;
  double S = 0.0;
  for (int c0 = 0; c0 < nch; c0 += 8) {
    float mc[8];
    double sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = min(c0 + j, nch - 1);
      mc[j] = st[c].maxv;
      sc[j] = st[c].sumexp;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (c0 + j >= nch || mc[j] == -INFINITY) continue;
      if (mc[j] > M) {
        S = S * exp_nonpos(static_cast<double>(M) - static_cast<double>(mc[j]), tab) + sc[j];
        M = mc[j];
      } else {
        S += sc[j] * exp_nonpos(static_cast<double>(mc[j]) - static_cast<double>(M), tab);
      }
    }
  }
  return static_cast<double>(M) + log(S);
}

// Phase 1b (trees of more than kBlock / 2 nodes): the log-sum-exp of every row, one thread
// per row. Smaller trees skip it: the walk merges its rows itself, one per thread.
__global__ __launch_bounds__(kBlock) void sample_lse_merge_kernel(SampleArgs a) {
  __shared__ double tab[64];
  exp_table_load(tab);
  __syncthreads();
  const int rows = a.S * a.tree.n_cap * 2;
  const int q = blockIdx.x * kBlock + threadIdx.x;
  if (q >= rows) return;
  a.lse[q] = row_lse_from_stats(a.st + static_cast<size_t>(q) * a.nch, a.nch, tab);
}

// Phase 2: the walk of sequence blockIdx.x / G, shared by its G workgroups (the group
// barrier needs them all resident: the launch keeps the grid within what the device holds).
template <int DT>
__global__ __launch_bounds__(kBlock) void sample_walk_kernel(SampleArgs a) {
  __shared__ SampleSmem sm;
  __shared__ double gvals[kXchStride];
  __shared__ double slice_buf[3][kWalkSlice];   // residuals (two) and q of this slice
  using Rw = RowT<DT>;
  row_smem_init(sm.rs);
  const int s = blockIdx.x / a.G;
  const int cap = a.tree.n_cap;
  const int N = a.tree.n_nodes[s];
  if (N < 1 || N > cap) {   // every workgroup of the group leaves: no barrier is entered
    if (threadIdx.x == 0) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  const size_t tb = static_cast<size_t>(s) * cap;
  const size_t row_bytes = static_cast<size_t>(a.V) * Rw::ESIZE;
  const bool merge_here = 2 * cap <= kBlock;   // else sample_lse_merge_kernel ran
  if (threadIdx.x == 0) sm.flag = 0;
  __syncthreads();
  for (int v = threadIdx.x; v < N; v += kBlock) {
    sm.par[v] = static_cast<short>(a.tree.parent[tb + v]);
    sm.tok[v] = a.tree.token[tb + v];
    if (!merge_here) {
      sm.lset[v] = a.lse[(tb + v) * 2 + 0];
      sm.lsed[v] = a.lse[(tb + v) * 2 + 1];
    }
    // rows are read at every node the walk may visit, tokens at every child tried: both
    // must lie inside the tables
    const int r = a.tree.row[tb + v];
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
  if (merge_here) {
    const int q = threadIdx.x;
    if (q < 2 * N) {
      const double l = row_lse_from_stats(a.st + ((tb + (q >> 1)) * 2 + (q & 1)) * a.nch, a.nch, sm.rs.exptab);
      ((q & 1) ? sm.lsed : sm.lset)[q >> 1] = l;
    }
    __syncthreads();
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
  grp.xch = a.xch + static_cast<size_t>(s) * a.max_pass * kXchStride;
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
  int v = 0, A = 0;
  if (lead && threadIdx.x == 0) a.path[tb] = 0;
  if (threadIdx.x == 0) sm.spath[0] = 0;
  for (;;) {
    // children of v in slot order
    const int seg = (N + kBlock - 1) / kBlock;
    const int n0 = threadIdx.x * seg, n1 = min(N, n0 + seg);
    int mine = 0;
    for (int k = max(n0, 1); k < n1; ++k) mine += (sm.par[k] == v) ? 1 : 0;
    int nk = 0;
    int pos = block_exclusive_scan(mine, sm.iwsum, &nk);
    for (int k = max(n0, 1); k < n1; ++k)
      if (sm.par[k] == v) sm.kids[pos++] = k;
    __syncthreads();
    const int r = a.tree.row[tb + v];
    WalkDist<DT> d;
    d.trow = static_cast<const char*>(a.target) + (static_cast<size_t>(s) * a.R + r) * row_bytes;
    d.drow = static_cast<const char*>(a.draft) + (static_cast<size_t>(s) * a.R + r) * row_bytes;
    d.lt = sm.lset[v];
    d.ld = sm.lsed[v];
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
        const int x = sm.tok[ch];
        const double px = (q == 0) ? d.p(x) : px_next;   // the first try reads the target row
        const double qx = d.q(x);
        const double u = (static_cast<double>(a.u_acc[tb + ch]) + 0.5) * inv32;
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
      const int xn = (q + 1 < nk) ? sm.tok[sm.kids[q + 1]] : -1;
      const int xu = vec ? xn / Rw::VEC : xn;
      const bool owner = xn >= 0 && xu >= grp.u0 && xu < grp.u1;
      double e0 = 0.0, e1 = 0.0;
      if (owner && threadIdx.x == 0) {
        e1 = d.p(xn);
        e0 = fmax(e1 - d.q(xn), 0.0);   // the entry residual_slice stored for xn
      }
      if (!group_exchange(grp, part, owner, e0, e1, xn >= 0, gvals, &sm.flag)) return;
      double z = 0.0;
      for (int k = 0; k < grp.G; ++k) z += gvals[k];
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
      ++A;
      if (lead && threadIdx.x == 0) a.path[tb + A] = v;
      if (threadIdx.x == 0) sm.spath[A] = v;
      continue;
    }
    // bonus: inverse CDF of the current p with u_res[v]; slice masses first. After a
    // rejection whose residual became p, they are that exchange's slice sums over z;
    // otherwise (a leaf, or p kept from before) one pass and an exchange find them.
    const double u = (static_cast<double>(a.u_res[tb + v]) + 0.5) * inv32;
    double mass = 0.0;
    if (z_last > 0.0) {
      __syncthreads();
      for (int k = threadIdx.x; k < grp.G; k += kBlock) gvals[k] /= z_last;
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
      mass = block_sum(loc, sm.rs.redd);
      if (!group_exchange(grp, mass, false, 0.0, 0.0, false, gvals, &sm.flag)) return;
    }
    double total = 0.0;
    for (int k = 0; k < grp.G; ++k) total += gvals[k];
    const double target = u * total;
    // the first workgroup whose slice takes the running sum past the target draws the
    // token; if rounding leaves the target at the end, the last slice with mass does
    double before = 0.0, mybase = 0.0;
    int owner = -1, last_pos = 0;
    for (int k = 0; k < grp.G; ++k) {
      if (k == grp.gi) mybase = before;
      if (owner < 0 && gvals[k] > 0.0 && before + gvals[k] > target) owner = k;
      if (gvals[k] > 0.0) last_pos = k;
      before += gvals[k];
    }
    if (owner < 0) owner = last_pos;
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
}

int launch_verify_sample(const SampleArgs& a, int S, int dtype, hipStream_t st) {
  const dim3 grid(a.lse_grid);
  if (dtype == 1)
    hipLaunchKernelGGL(sample_lse_kernel<1>, grid, dim3(kBlock), 0, st, a);
  else
    hipLaunchKernelGGL(sample_lse_kernel<0>, grid, dim3(kBlock), 0, st, a);
  if (hipGetLastError() != hipSuccess) return -1;
  if (2 * a.tree.n_cap > kBlock) {   // smaller trees merge their rows inside the walk
    hipLaunchKernelGGL(sample_lse_merge_kernel, dim3((S * a.tree.n_cap * 2 + kBlock - 1) / kBlock), dim3(kBlock),
                       0, st, a);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  // An ordinary launch on the caller's stream: the grid (S * G) is at most the number of
  // workgroups the device holds at once, so every group is resident together once the
  // stream reaches this kernel. (A cooperative launch is avoided: measured on MI355X it
  // let consecutive walks share the group barrier and time out now and then.)
  if (dtype == 1)
    hipLaunchKernelGGL(sample_walk_kernel<1>, dim3(S * a.G), dim3(kBlock), 0, st, a);
  else
    hipLaunchKernelGGL(sample_walk_kernel<0>, dim3(S * a.G), dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Workgroups of the chunk-statistics kernel that can be resident at once (queried once
// per device).
int sample_lse_max_blocks(int dtype) {
  static int cached[64][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  int& c = cached[dev][dtype ? 1 : 0];
  if (c > 0) return c;
  int ncu = 0, per = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  const void* fn = dtype ? reinterpret_cast<const void*>(&sample_lse_kernel<1>)
                         : reinterpret_cast<const void*>(&sample_lse_kernel<0>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, kBlock, 0) != hipSuccess || per < 1) return -1;
  c = ncu * per;
  return c;
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
  const dim3 grid(S * a.tree.n_cap * a.nch);
  if (dtype == 1)
    hipLaunchKernelGGL(verify_greedy_kernel<1>, grid, dim3(kBlock), 0, st, a);
  else
    hipLaunchKernelGGL(verify_greedy_kernel<0>, grid, dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace dtv
