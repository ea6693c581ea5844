// Greedy verification on gfx950 (OPT-Tree summary, section 2; GOOSE page, section 2C).
//
// One workgroup per (sequence, node, chunk of the node's target row) finds the chunk's
// largest value and its lowest index and folds it into the node's 64-bit best key with
// one atomic max ((value key << 32) | ~index, so larger value wins, then lower index).
// The workgroup that completes a sequence last walks its tree: node c matches when its
// token equals the argmax at its parent; a node is accepted when no node on its root path
// fails (one AND of its ancestor mask with the failure mask); the deepest accepted node,
// lowest slot first, ends the path.
#include "dtv_internal.h"
#include "rowstats.h"

namespace dtv {

constexpr int kVerifyMaxNodes = 1024;
constexpr int kVerifyMaxWords = 16;

struct VerifySmem {
  RowSmem rs;
  int a[kVerifyMaxNodes];
  unsigned long long fail[kVerifyMaxWords];
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

  // ---- the walk, by the last workgroup of sequence s
  const int words = a.tree.words;
  for (int v = threadIdx.x; v < N; v += kBlock) {
    const unsigned long long b = __hip_atomic_load(&a.best[tb + v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.a[v] = sort_key_index(b);
    a.best[tb + v] = 0ull;  // ready for the next call
    if (a.argmax_out) a.argmax_out[tb + v] = sm.a[v];
  }
  for (int w = threadIdx.x; w < kVerifyMaxWords; w += kBlock) sm.fail[w] = 0ull;
  __syncthreads();
  for (int v = 1 + threadIdx.x; v < N; v += kBlock) {
    const int p = a.tree.parent[tb + v];
    if (a.tree.token[tb + v] != sm.a[p]) atomicOr(&sm.fail[v >> 6], 1ull << (v & 63));
  }
  __syncthreads();
  // deepest accepted node, lowest slot among equals: maximise (depth << 20) | (2^20 - 1 - slot)
  unsigned long long pick = 0;
  for (int v = threadIdx.x; v < N; v += kBlock) {
    const uint64_t* an = a.tree.anc + (tb + v) * words;
    bool ok = true;
    for (int w = 0; w < words; ++w) ok = ok && ((an[w] & sm.fail[w]) == 0ull);
    if (ok) {
      const unsigned long long key2 = (static_cast<unsigned long long>(a.tree.depth[tb + v]) << 20) |
                                      static_cast<unsigned long long>(0xFFFFF - v);
      pick = key2 > pick ? key2 : pick;
    }
  }
  pick = block_max(pick, sm.redu);
  const int vstar = 0xFFFFF - static_cast<int>(pick & 0xFFFFFull);
  const int A = static_cast<int>(pick >> 20);
  const uint64_t* an = a.tree.anc + (tb + vstar) * words;
  for (int u = threadIdx.x; u < N; u += kBlock)
    if ((an[u >> 6] >> (u & 63)) & 1ull) a.path[tb + a.tree.depth[tb + u]] = u;
  if (threadIdx.x == 0) {
    a.path_len[s] = A + 1;
    a.bonus[s] = sm.a[vstar];
  }
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
