// Tree-masked attention on gfx950: the fp32 path and the dispatch.
//
// Each draft node attends to the whole KV prefix and to the tree keys of its own root
// path (OPT-Tree summary, section 2: one target pass over all tree tokens with a tree
// attention mask). The tree's keys and values sit at cache positions P + slot, so the
// key index space of a sequence is simply cache positions 0 .. P + n_nodes - 1; a key at
// position P + j is visible to node i when bit j of i's ancestor mask is set.
//
// bf16 runs on MFMA (attn_bf16.hip). fp32: one workgroup per (node, head), plain fp32
// arithmetic, for checking against the float64 oracle at 1e-4.
#include "dtv_internal.h"

namespace dtv {

__device__ __forceinline__ bool t_first() { return threadIdx.x == 0; }

// ------------------------------------------------------------------ fp32 path

constexpr int kF32MaxKeys = 16384;

__global__ __launch_bounds__(kBlock) void attn_f32_kernel(AttnArgs a) {
  __shared__ float p[kF32MaxKeys];
  __shared__ float qs[128];
  __shared__ float red[kWaves];
  __shared__ float part[kBlock];
  const int D = a.D;
  int bid = blockIdx.x;
  const int h = bid % a.Hq;
  bid /= a.Hq;
  const int i = bid % a.n_cap;
  const int s = bid / a.n_cap;
  const int N = a.n_nodes[s];
  if (i >= N) return;
  const int kv = h / a.g;
  const int P = a.P[s];
  if (N > a.n_cap || P < 0 || P + N > a.P_cap || P + N > kF32MaxKeys) {
    if (t_first()) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  const int T = P + N;
  const float* q = static_cast<const float*>(a.q) + ((static_cast<size_t>(s) * a.n_cap + i) * a.Hq + h) * D;
  const float* kb = static_cast<const float*>(a.k) + (static_cast<size_t>(s) * a.Hkv + kv) * a.P_cap * static_cast<size_t>(D);
  const float* vb = static_cast<const float*>(a.v) + (static_cast<size_t>(s) * a.Hkv + kv) * a.P_cap * static_cast<size_t>(D);
  const uint64_t* anc = a.anc + (static_cast<size_t>(s) * a.n_cap + i) * a.words;
  for (int d = threadIdx.x; d < D; d += kBlock) qs[d] = q[d];
  __syncthreads();
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < T; j += kBlock) {
    float v = -INFINITY;
    bool vis = j < P;
    if (!vis) {
      const int jj = j - P;
      vis = ((anc[jj >> 6] >> (jj & 63)) & 1ull) != 0ull;
    }
    if (vis) {
      float acc = 0.f;
      const float* kr = kb + static_cast<size_t>(j) * D;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[d], kr[d], acc);
      v = acc * a.scale;
    }
    p[j] = v;
    mx = fmaxf(mx, v);
  }
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int j = threadIdx.x; j < T; j += kBlock) {
    const float e = (p[j] == -INFINITY) ? 0.f : expf(p[j] - mx);
    p[j] = e;
    sum += e;
  }
  sum = block_sum(sum, red);
  // output: threads split as (d, key phase)
  const int phases = kBlock / D;
  const int d = threadIdx.x % D, ph = threadIdx.x / D;
  float acc = 0.f;
  if (ph < phases)
    for (int j = ph; j < T; j += phases) acc = fmaf(p[j], vb[static_cast<size_t>(j) * D + d], acc);
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < D) {
    float o = 0.f;
    for (int q2 = 0; q2 < phases; ++q2) o += part[q2 * D + threadIdx.x];
    static_cast<float*>(a.o)[((static_cast<size_t>(s) * a.n_cap + i) * a.Hq + h) * D + threadIdx.x] = o / sum;
  }
}

int launch_attn(const AttnArgs& a, int dtype, hipStream_t st) {
  if (dtype == 1) return launch_attn_bf16(a, st);
  DTV_LAUNCH(attn_f32_kernel, dim3(a.S * a.n_cap * a.Hq), dim3(kBlock), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace dtv
