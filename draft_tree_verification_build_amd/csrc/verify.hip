// Greedy verification on gfx950 (OPT-Tree summary, section 2; GOOSE page, section 2C).
//
// One workgroup per (sequence, node, chunk of the node's target row) finds the chunk's
// largest value and its lowest index and folds it into the node's 64-bit best key with
// one atomic max ((value key << 32) | ~index, so larger value wins, then lower index).
// The workgroup that completes a sequence last walks its tree: node c matches when its
// token equals the argmax at its parent; a node is accepted when every node on its root
// path matches (checked by following parent links in shared memory); the deepest accepted
// node, lowest slot first, ends the path.
#include "dtv_internal.h"
#include "rowstats.h"

namespace dtv {

constexpr int kVerifyMaxNodes = 1024;
constexpr int kVerifyMaxWords = 16;

struct VerifySmem {
  int a[kVerifyMaxNodes];       // target argmax at every node
  short par[kVerifyMaxNodes];   // parent slot
  short dep[kVerifyMaxNodes];   // depth
  int tok[kVerifyMaxNodes];     // drafted token
  unsigned char bad[kVerifyMaxNodes];   // 1: token differs from the argmax at the parent
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
  const int N = a.tree.n_nodes[s];
  if (i >= N) return;
  if (N > cap) {  // n_nodes is device data: refuse rather than read past the tree
    if (threadIdx.x == 0) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  const size_t tb = static_cast<size_t>(s) * cap;
  const int r = a.tree.row[tb + i];
  const char* row = static_cast<const char*>(a.target) +
                    (static_cast<size_t>(s) * a.R + r) * static_cast<size_t>(a.V) * Rw::ESIZE;
  float x[Rw::E];
  uint32_t key[Rw::E];
  load_chunk<DT>(row, a.V, c, x, key);
  unsigned long long best = 0;
#pragma unroll
  for (int ii = 0; ii < kLoads; ++ii)
#pragma unroll
    for (int e = 0; e < Rw::VEC; ++e) {
      const uint32_t k = key[ii * Rw::VEC + e];
      if (k == 0u) continue;
      const unsigned long long p = sort_key(x[ii * Rw::VEC + e], elem_index<DT>(c, ii, e));
      best = p > best ? p : best;
    }
  best = block_max(best, sm.redu);
  if (threadIdx.x == 0) atomicMax(&a.best[tb + i], best);
  if (!last_arrival(&a.tickets[s], static_cast<unsigned>(N * nch), &sm.flag)) return;

  // ---- the walk, by the last workgroup of sequence s. Everything it needs is loaded in
  //      one parallel pass; acceptance then follows parent links in shared memory.
  for (int v = threadIdx.x; v < N; v += kBlock) {
    const unsigned long long b = __hip_atomic_load(&a.best[tb + v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int p = a.tree.parent[tb + v];
    const int tok = a.tree.token[tb + v];
    const int d = a.tree.depth[tb + v];
    a.best[tb + v] = 0ull;  // ready for the next call
    const int am = sort_key_index(b);
    sm.a[v] = am;
    sm.tok[v] = tok;
    sm.par[v] = static_cast<short>(v == 0 ? -1 : p);
    sm.dep[v] = static_cast<short>(d);
    if (a.argmax_out) a.argmax_out[tb + v] = am;
  }
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
    for (int u = vstar; u >= 0; u = sm.par[u]) a.path[tb + sm.dep[u]] = u;
    a.path_len[s] = A + 1;
    a.bonus[s] = sm.a[vstar];
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
// Work split: one workgroup per (sequence, node, target-or-draft row, chunk) reduces its
// chunk to (max, float64 sum of exp); the last one of a row merges the row's log-sum-exp;
// the last one of a sequence walks. In the walk, a first try needs only the two row
// values at the child's token; each rejection costs one V-wide residual pass over
// float64 buffers in the workspace; the bonus draw is one V-wide prefix-sum pass.

constexpr int kSampleMaxNodes = 1024;

struct SampleSmem {
  RowSmem rs;
  short par[kSampleMaxNodes];
  int tok[kSampleMaxNodes];
  double lset[kSampleMaxNodes];
  double lsed[kSampleMaxNodes];
  int kids[kSampleMaxNodes];
  double wsum[kWaves];
  int iwsum[kWaves];
  int flag;
  int first;
  int pick;
  int nk;
  int accept;
};

template <int DT>
__device__ __forceinline__ float row_value(const void* row, int j) {
  return DT ? bf16_to_f32(static_cast<const uint16_t*>(row)[j]) : static_cast<const float*>(row)[j];
}

// Smallest k with sum_{j<=k} w_j > u * sum_j w_j (ascending float64 prefix sums), where
// w_j = weight(j). Threads take contiguous index segments in order.
template <typename W>
__device__ int inverse_cdf(int V, double u, W weight, SampleSmem& sm) {
  const int seg = (V + kBlock - 1) / kBlock;
  const int j0 = threadIdx.x * seg;
  const int j1 = min(V, j0 + seg);
  double loc = 0.0;
  for (int j = j0; j < j1; ++j) loc += weight(j);
  double total = 0.0;
  const double excl = block_exclusive_scan(loc, sm.wsum, &total);
  const double target = u * total;
  if (threadIdx.x == 0) sm.first = kBlock;
  __syncthreads();
  if (j1 > j0 && excl + loc > target) atomicMin(&sm.first, static_cast<int>(threadIdx.x));
  __syncthreads();
  if (threadIdx.x == 0) sm.pick = -1;
  __syncthreads();
  if (static_cast<int>(threadIdx.x) == sm.first) {
    double run = excl;
    int k = j1 - 1;
    for (int j = j0; j < j1; ++j) {
      run += weight(j);
      if (run > target) {
        k = j;
        break;
      }
    }
    sm.pick = k;
  }
  __syncthreads();
  if (sm.pick < 0 && threadIdx.x == 0) {  // rounding left the target at the very end
    int k = V - 1;
    while (k > 0 && !(weight(k) > 0.0)) --k;
    sm.pick = k;
  }
  __syncthreads();
  return sm.pick;
}

template <int DT>
__global__ __launch_bounds__(kBlock) void verify_sample_kernel(SampleArgs a) {
  __shared__ SampleSmem sm;
  using Rw = RowT<DT>;
  row_smem_init(sm.rs);
  __syncthreads();
  const int nch = a.nch;
  const int cap = a.tree.n_cap;
  int bid = blockIdx.x;
  const int c = bid % nch;
  bid /= nch;
  const int which = bid % 2;
  bid /= 2;
  const int i = bid % cap;
  const int s = bid / cap;
  const int N = a.tree.n_nodes[s];
  if (i >= N) return;
  if (N > cap) {
    if (threadIdx.x == 0) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  const size_t tb = static_cast<size_t>(s) * cap;
  const size_t row_bytes = static_cast<size_t>(a.V) * Rw::ESIZE;
  {
    const int r = a.tree.row[tb + i];
    const char* row = static_cast<const char*>(which ? a.draft : a.target) +
                      (static_cast<size_t>(s) * a.R + r) * row_bytes;
    float x[Rw::E];
    uint32_t key[Rw::E];
    load_chunk<DT>(row, a.V, c, x, key);
    const size_t rr = (tb + i) * 2 + which;
    chunk_reduce<DT>(x, key, c, a.V, 0, &a.st[rr * nch + c], nullptr, nullptr, nullptr, sm.rs);
    if (last_arrival(&a.rtick[rr], nch, &sm.flag)) {
      // log-sum-exp of the row from its chunks
      if (threadIdx.x == 0) {
        float M = -INFINITY;
        for (int q = 0; q < nch; ++q) M = fmaxf(M, ld_cc(&a.st[rr * nch + q].maxv));
        double sum = 0.0;
        for (int q = 0; q < nch; ++q)
          sum += ld_cc(&a.st[rr * nch + q].sumexp) *
                 exp(static_cast<double>(ld_cc(&a.st[rr * nch + q].maxv)) - static_cast<double>(M));
        st_cc(&a.lse[rr], static_cast<double>(M) + log(sum));
      }
    }
  }
  if (!last_arrival(&a.stick[s], static_cast<unsigned>(N * 2 * nch), &sm.flag)) return;

  // ---------------- the walk of sequence s
  for (int v = threadIdx.x; v < N; v += kBlock) {
    sm.par[v] = static_cast<short>(a.tree.parent[tb + v]);
    sm.tok[v] = a.tree.token[tb + v];
    sm.lset[v] = ld_cc(&a.lse[(tb + v) * 2 + 0]);
    sm.lsed[v] = ld_cc(&a.lse[(tb + v) * 2 + 1]);
  }
  __syncthreads();
  double* P[2] = {a.pbuf + static_cast<size_t>(s) * 2 * a.V, a.pbuf + (static_cast<size_t>(s) * 2 + 1) * a.V};
  const double inv32 = 1.0 / 4294967296.0;
  int v = 0, A = 0;
  int bonus = 0;
  if (threadIdx.x == 0) a.path[tb] = 0;
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
    const void* trow = static_cast<const char*>(a.target) + (static_cast<size_t>(s) * a.R + r) * row_bytes;
    const void* drow = static_cast<const char*>(a.draft) + (static_cast<size_t>(s) * a.R + r) * row_bytes;
    const double lt = sm.lset[v], ld = sm.lsed[v];
    int cur = -1;        // -1: p is softmax(target); else P[cur] / zc
    double zc = 1.0;
    int accepted = -1;
    for (int q = 0; q < nk; ++q) {
      const int ch = sm.kids[q];
      if (threadIdx.x == 0) {
        const int x = sm.tok[ch];
        const double px = (cur < 0) ? exp_nonpos(static_cast<double>(row_value<DT>(trow, x)) - lt, sm.rs.exptab)
                                    : P[cur][x] / zc;
        const double qx = exp_nonpos(static_cast<double>(row_value<DT>(drow, x)) - ld, sm.rs.exptab);
        const double u = (static_cast<double>(a.u_acc[tb + ch]) + 0.5) * inv32;
        sm.accept = (qx > 0.0) ? (u < px / qx ? 1 : 0) : (px > 0.0 ? 1 : 0);
      }
      __syncthreads();
      if (sm.accept) {
        accepted = ch;
        __syncthreads();
        break;
      }
      // rejection: residual (p - q)+ into the other buffer
      const int nxt = (cur == 0) ? 1 : 0;
      double loc = 0.0;
      for (int j = threadIdx.x; j < a.V; j += kBlock) {
        const double pj = (cur < 0) ? exp_nonpos(static_cast<double>(row_value<DT>(trow, j)) - lt, sm.rs.exptab)
                                    : P[cur][j] / zc;
        const double qj = exp_nonpos(static_cast<double>(row_value<DT>(drow, j)) - ld, sm.rs.exptab);
        const double rj = fmax(pj - qj, 0.0);
        P[nxt][j] = rj;
        loc += rj;
      }
      const double z = block_sum(loc, sm.rs.redd);
      if (z > 0.0) {  // otherwise p is kept
        cur = nxt;
        zc = z;
      }
      __syncthreads();
    }
    if (accepted >= 0) {
      v = accepted;
      ++A;
      if (threadIdx.x == 0) a.path[tb + A] = v;
      continue;
    }
    const double u = (static_cast<double>(a.u_res[tb + v]) + 0.5) * inv32;
    if (cur < 0) {
      bonus = inverse_cdf(a.V, u, [&](int j) {
        return exp_nonpos(static_cast<double>(row_value<DT>(trow, j)) - lt, sm.rs.exptab);
      }, sm);
    } else {
      const double* pc = P[cur];
      const double z = zc;
      bonus = inverse_cdf(a.V, u, [&](int j) { return pc[j] / z; }, sm);
    }
    break;
  }
  if (threadIdx.x == 0) {
    a.path_len[s] = A + 1;
    a.bonus[s] = bonus;
  }
}

int launch_verify_sample(const SampleArgs& a, int S, int dtype, hipStream_t st) {
  const dim3 grid(S * a.tree.n_cap * 2 * a.nch);
  if (dtype == 1)
    hipLaunchKernelGGL(verify_sample_kernel<1>, grid, dim3(kBlock), 0, st, a);
  else
    hipLaunchKernelGGL(verify_sample_kernel<0>, grid, dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
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
