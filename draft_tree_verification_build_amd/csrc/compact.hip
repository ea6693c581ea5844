// KV compaction on gfx950 (concept page, "The protocol", step 4): the root and the
// accepted nodes move to the cache positions right behind the prefix, in path order.
//
// One workgroup per (sequence, KV head, k or v). Rows are processed in increasing path
// order in batches staged through LDS: each batch is read completely before any of it is
// written. That is safe in place because a node at depth k has slot >= k, so no later
// source row is ever an earlier destination, and within a batch every read precedes
// every write.
#include "dtv_internal.h"

namespace dtv {

constexpr int kCompactRows = 32;          // rows per batch
constexpr int kCompactRowBytes = 512;     // D * esize <= 512 (D <= 128 fp32)

__global__ __launch_bounds__(kBlock) void compact_kernel(CompactArgs a) {
  __shared__ uint4 stage[kCompactRows * kCompactRowBytes / 16];
  __shared__ int spath[kBlock];
  const int which = blockIdx.x & 1;
  const int kv = (blockIdx.x >> 1) % a.Hkv;
  const int s = (blockIdx.x >> 1) / a.Hkv;
  // the first kBlock path entries are read together with the path length and P (valid
  // memory whatever the length), so the row loads wait for one round trip, not two
  if (threadIdx.x < a.n_cap) spath[threadIdx.x] = a.path[static_cast<size_t>(s) * a.n_cap + threadIdx.x];
  const int L = a.path_len[s];
  const int P = a.P[s];
  __syncthreads();
  if (L < 1 || L > a.n_cap || P < 0 || P + a.n_cap > a.P_cap) {
    // inconsistent device inputs: leave the cache alone and mark the sequence
    if (which == 0 && kv == 0 && threadIdx.x == 0) a.P_new[s] = -1;
    return;
  }
  char* base = static_cast<char*>(which ? a.v : a.k) +
               (static_cast<size_t>(s) * a.Hkv + kv) * a.P_cap * static_cast<size_t>(a.D) * a.esize;
  const int vec_per_row = a.D * a.esize / 16;
  const size_t row_bytes = static_cast<size_t>(a.D) * a.esize;
  const int* path = a.path + static_cast<size_t>(s) * a.n_cap;
  for (int k0 = 0; k0 < L; k0 += kCompactRows) {
    const int nb = (L - k0) < kCompactRows ? (L - k0) : kCompactRows;
    for (int e = threadIdx.x; e < nb * vec_per_row; e += kBlock) {
      const int rr = e / vec_per_row, cc = e % vec_per_row;
      const int src = P + (k0 + rr < kBlock ? spath[k0 + rr] : path[k0 + rr]);
      stage[rr * (kCompactRowBytes / 16) + cc] =
          reinterpret_cast<const uint4*>(base + static_cast<size_t>(src) * row_bytes)[cc];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nb * vec_per_row; e += kBlock) {
      const int rr = e / vec_per_row, cc = e % vec_per_row;
      const int dst = P + k0 + rr;
      reinterpret_cast<uint4*>(base + static_cast<size_t>(dst) * row_bytes)[cc] =
          stage[rr * (kCompactRowBytes / 16) + cc];
    }
    __syncthreads();
  }
  // P_new may alias P: every workgroup of s must read P before it changes, so the
  // update is done by the (kv 0, k) workgroup only after reading, and readers of other
  // workgroups read P at their start. A separate P_new buffer avoids the question.
  if (which == 0 && kv == 0 && threadIdx.x == 0 && a.P_new != a.P) a.P_new[s] = P + L;
}

// P_new aliasing P: the new length is added after the copies. compact_kernel marks a
// sequence it refused with P[s] = -1 (a negative P is refused too), and that mark stays.
__global__ void compact_update_p(const int* path_len, int* P, int S) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < S && P[s] >= 0) P[s] += path_len[s];
}

int launch_compact(const CompactArgs& a, hipStream_t st) {
  DTV_LAUNCH(compact_kernel, dim3(a.S * a.Hkv * 2), dim3(kBlock), 0, st, a);
  if (hipGetLastError() != hipSuccess) return -1;
  if (a.P_new == a.P) {
    DTV_LAUNCH(compact_update_p, dim3((a.S + 255) / 256), dim3(256), 0, st, a.path_len,
                       a.P_new, a.S);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

}  // namespace dtv
