// Tree-masked attention on gfx950.
//
// Each draft node attends to the whole KV prefix and to the tree keys of its own root
// path (OPT-Tree summary, section 2: one target pass over all tree tokens with a tree
// attention mask). The tree's keys and values sit at cache positions P + slot, so the
// key index space of a sequence is simply cache positions 0 .. P + n_nodes - 1; a key at
// position P + j is visible to node i when bit j of i's ancestor mask is set.
//
// bf16 path. Grouped-query heads are packed: for KV head kv the g = Hq / Hkv query heads
// of every node form M = g * n_nodes rows (row r = node r / g, head kv * g + r % g), so a
// K/V tile is read once for all of them. A workgroup owns a 128-row tile (4 waves x 32
// rows) and a contiguous key range (split); it walks the range in 64-key blocks staged
// through LDS (K row-major, V transposed), computes S^T = K Q^T and O += P V with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation) and keeps an online softmax per row.
// Computing S^T rather than S leaves every lane holding 16 keys of one query row, which
// is exactly the operand layout the P V product needs, so P never leaves registers.
// When a row's keys are split over several workgroups, each writes (m, l, O) partials
// and a second small kernel merges them (a kernel boundary is the cheapest way to make
// the partials of all XCDs visible to the merging workgroups).
//
// f32 path: one workgroup per (node, head), plain fp32 arithmetic.
#include "dtv_internal.h"

namespace dtv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kTileRows = 128;  // query rows per workgroup
constexpr int kKeyBlock = 64;   // keys per LDS block

__device__ __forceinline__ bool t_first() { return threadIdx.x == 0; }

union Frag8 {
  bf16x8 v;
  uint4 u;
  uint2 h[2];
  uint16_t s[8];
};

template <int D>
struct AttnSmem {
  static constexpr int KS = D + 8;           // K row stride (elements)
  static constexpr int VS = kKeyBlock + 4;   // V^T row stride (elements)
  uint16_t ks[kKeyBlock * KS];
  uint16_t vt[D * VS];
  float alpha[kWaves][32];
  float ml[kWaves][32][2];
};

template <int D>
__global__ __launch_bounds__(kBlock) void attn_bf16_kernel(AttnArgs a) {
  __shared__ AttnSmem<D> sm;
  constexpr int KS = AttnSmem<D>::KS;
  constexpr int VS = AttnSmem<D>::VS;
  constexpr int NKS = D / 16;   // MFMA k-steps over the head dim
  constexpr int NT = D / 32;    // 32-wide output column tiles

  int bid = blockIdx.x;
  const int mt = bid % a.n_mtiles;
  bid /= a.n_mtiles;
  const int sp = bid % a.n_split;
  bid /= a.n_split;
  const int kv = bid % a.Hkv;
  const int s = bid / a.Hkv;
  const int tile = (s * a.Hkv + kv) * a.n_mtiles + mt;

  const int N = a.n_nodes[s];
  const int g = a.g;
  const int M = g * N;
  if (mt * kTileRows >= M) return;
  const int P = a.P[s];
  if (N > a.n_cap || P < 0 || P + N > a.P_cap) {  // device-side sizes the host could not check
    if (t_first()) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  const int T = P + N;
  const int k_lo = sp * a.kps;
  const int k_hi = min(k_lo + a.kps, T);

  const int t = threadIdx.x;
  const int w = t >> 6;
  const int lane = t & 63;
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int r = mt * kTileRows + w * 32 + lr;
  const bool row_ok = r < M;
  const bool wave_active = (mt * kTileRows + w * 32) < M;
  const int node = row_ok ? r / g : 0;
  const int head = kv * g + (row_ok ? r % g : 0);

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) +
                          (static_cast<size_t>(s) * a.Hkv + kv) * a.P_cap * static_cast<size_t>(D);
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) +
                          (static_cast<size_t>(s) * a.Hkv + kv) * a.P_cap * static_cast<size_t>(D);
  const uint64_t* anc = a.anc + (static_cast<size_t>(s) * a.n_cap + node) * a.words;

  Frag8 qf[NKS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((static_cast<size_t>(s) * a.n_cap + node) * a.Hq + head) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (row_ok)
        qf[ks].u = *reinterpret_cast<const uint4*>(qrow + ks * 16 + 8 * h);
      else
        qf[ks].u = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  f32x16 oacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[nt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;

  for (int kb = k_lo; kb < k_hi; kb += kKeyBlock) {
    // ---- stage K (row-major) and V (transposed) of keys kb .. kb+63. All eight 16-byte
    //      loads are issued before any LDS store so their latencies overlap; each loads a
    //      clamped (valid) key unconditionally and is zeroed by a select past the range
    //      end, since a load under a branch gets a wait of its own.
    {
      constexpr int NV = kKeyBlock * D / 8 / kBlock;   // 16-byte vectors per thread (4 for D=128)
      uint4 kr[NV];
      Frag8 vv[NV];
      const int dcv = t % (D / 8), kg = t / (D / 8);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = t + kBlock * i;
        const int kk = kb + vi / (D / 8);
        kr[i] = *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(min(kk, k_hi - 1)) * D + (vi % (D / 8)) * 8);
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int kk = kb + kg * NV + u;
        vv[u].u = *reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(min(kk, k_hi - 1)) * D + dcv * 8);
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = t + kBlock * i;
        const int key = vi / (D / 8);
        if (kb + key >= k_hi) kr[i] = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(&sm.ks[key * KS + (vi % (D / 8)) * 8]) = kr[i];
      }
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (kb + kg * NV + u >= k_hi) vv[u].u = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint16_t* dst = &sm.vt[(dcv * 8 + e) * VS + kg * NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) dst[u] = vv[u].s[e];
      }
    }
    __syncthreads();

    if (wave_active) {
      // ---- S^T = K Q^T for two 32-key tiles
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          Frag8 kf;
          kf.u = *reinterpret_cast<const uint4*>(&sm.ks[(kt * 32 + lr) * KS + ks * 16 + 8 * h]);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v, qf[ks].v, sacc[kt], 0, 0, 0);
        }
      }
      // ---- mask and scale; lane holds keys kb + kt*32 + (i/4)*8 + 4h + i%4 of row lr
      uint64_t w0 = 0, w1 = 0;
      int wbase = 0;
      const bool has_tree = (kb + kKeyBlock > P);
      if (has_tree && row_ok) {
        wbase = (max(kb, P) - P) >> 6;
        w0 = anc[wbase];
        if (wbase + 1 < a.words) w1 = anc[wbase + 1];
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = kb + kt * 32 + (i >> 2) * 8 + 4 * h + (i & 3);
          float v = sacc[kt][i] * sl2;
          if (kk >= k_hi) {
            v = -INFINITY;
          } else if (kk >= P) {
            const int j = kk - P;
            const uint64_t word = ((j >> 6) == wbase) ? w0 : w1;
            if (((word >> (j & 63)) & 1ull) == 0ull) v = -INFINITY;
          }
          sacc[kt][i] = v;
          mloc = fmaxf(mloc, v);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float m_new = fmaxf(m_run, mloc);
      float alpha = 1.f;
      if (m_new != -INFINITY) alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = sacc[kt][i];
          const float p = (v == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(v - m_new);
          sacc[kt][i] = p;
          lsum += p;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      // ---- rescale O; O rows held by a lane are (i/4)*8 + 4h + i%4
      if (h == 0) sm.alpha[w][lr] = alpha;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 al = *reinterpret_cast<const float4*>(&sm.alpha[w][q4 * 8 + 4 * h]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          oacc[nt][q4 * 4 + 0] *= al.x;
          oacc[nt][q4 * 4 + 1] *= al.y;
          oacc[nt][q4 * 4 + 2] *= al.z;
          oacc[nt][q4 * 4 + 3] *= al.w;
        }
      }
      // ---- O += P V over four 16-key steps; the A operand of step k2 is p values
      //      8*(k2%2) .. +7 of key tile k2/2, i.e. keys 16*k2 + 8*(j/4) + 4h + j%4
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        Frag8 pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pf.s[j] = f32_to_bf16(sacc[k2 >> 1][8 * (k2 & 1) + j]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          Frag8 vf;
          const uint16_t* vr = &sm.vt[(nt * 32 + lr) * VS + 16 * k2 + 4 * h];
          vf.h[0] = *reinterpret_cast<const uint2*>(vr);
          vf.h[1] = *reinterpret_cast<const uint2*>(vr + 8);
          oacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf.v, vf.v, oacc[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // ---- row statistics to LDS in the O layout
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (h == 0) {
    sm.ml[w][lr][0] = m_run;
    sm.ml[w][lr][1] = l_tot;
  }
  __syncthreads();

  if (a.n_split == 1) {
    if (wave_active) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int rl = q4 * 8 + 4 * h + b;
          const int rr = mt * kTileRows + w * 32 + rl;
          if (rr >= M) continue;
          const float l = sm.ml[w][rl][1];
          const float inv = l > 0.f ? 1.f / l : 0.f;
          uint16_t* orow = static_cast<uint16_t*>(a.o) +
                           ((static_cast<size_t>(s) * a.n_cap + rr / g) * a.Hq + kv * g + rr % g) * D;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) orow[nt * 32 + lr] = f32_to_bf16(oacc[nt][q4 * 4 + b] * inv);
        }
    }
    return;
  }

  // ---- split: write (m, l, unnormalised O) partials; attn_combine_kernel merges them
  const size_t pbase = (static_cast<size_t>(tile) * a.n_split + sp) * kTileRows;
  if (wave_active) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int rl = q4 * 8 + 4 * h + b;
        float* prow = a.part_o + (pbase + w * 32 + rl) * D;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) prow[nt * 32 + lr] = oacc[nt][q4 * 4 + b];
      }
    if (h == 0) {
      a.part_ml[(pbase + w * 32 + lr) * 2 + 0] = m_run;
      a.part_ml[(pbase + w * 32 + lr) * 2 + 1] = l_tot;
    }
  }
}

// Merges the key splits of every query row: O = sum_q O_q 2^(m_q - M) / sum_q l_q 2^(m_q - M).
// One thread per 4 output values; D/4 threads per row.
template <int D>
__global__ __launch_bounds__(kBlock) void attn_combine_kernel(AttnArgs a) {
  constexpr int TPR = D / 4;                 // threads per row
  constexpr int RPB = kBlock / TPR;          // rows per workgroup
  constexpr int BPT = kTileRows / RPB;       // workgroups per tile
  const int tile = blockIdx.x / BPT;
  const int rl = (blockIdx.x % BPT) * RPB + threadIdx.x / TPR;
  const int c4 = threadIdx.x % TPR;
  const int mt = tile % a.n_mtiles;
  const int kv = (tile / a.n_mtiles) % a.Hkv;
  const int s = tile / (a.n_mtiles * a.Hkv);
  const int N = a.n_nodes[s];
  const int M = a.g * N;
  const int rr = mt * kTileRows + rl;
  if (N > a.n_cap || rr >= M) return;
  const size_t pb0 = static_cast<size_t>(tile) * a.n_split * kTileRows + rl;
  float mx = -INFINITY;
  for (int q = 0; q < a.n_split; ++q) {
    const float2 ml = *reinterpret_cast<const float2*>(&a.part_ml[(pb0 + static_cast<size_t>(q) * kTileRows) * 2]);
    if (ml.y > 0.f) mx = fmaxf(mx, ml.x);
  }
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q = 0; q < a.n_split; ++q) {
    const size_t pb = pb0 + static_cast<size_t>(q) * kTileRows;
    const float2 ml = *reinterpret_cast<const float2*>(&a.part_ml[pb * 2]);
    if (ml.y > 0.f) {
      const float sc = __builtin_amdgcn_exp2f(ml.x - mx);
      L += ml.y * sc;
      const float4 o = *reinterpret_cast<const float4*>(&a.part_o[pb * D + c4 * 4]);
      acc.x += o.x * sc;
      acc.y += o.y * sc;
      acc.z += o.z * sc;
      acc.w += o.w * sc;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.o) +
                   ((static_cast<size_t>(s) * a.n_cap + rr / a.g) * a.Hq + kv * a.g + rr % a.g) * D;
  uint2 packed;
  packed.x = static_cast<uint32_t>(f32_to_bf16(acc.x * inv)) | (static_cast<uint32_t>(f32_to_bf16(acc.y * inv)) << 16);
  packed.y = static_cast<uint32_t>(f32_to_bf16(acc.z * inv)) | (static_cast<uint32_t>(f32_to_bf16(acc.w * inv)) << 16);
  *reinterpret_cast<uint2*>(orow + c4 * 4) = packed;
}

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
  if (dtype == 1 && a.wide) return launch_attn_wide(a, st);
  if (dtype == 1) {
    const dim3 grid(a.S * a.Hkv * a.n_split * a.n_mtiles);
    if (a.D == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(kBlock), 0, st, a);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(kBlock), 0, st, a);
    if (a.n_split > 1) {
      if (hipGetLastError() != hipSuccess) return -1;
      const int tiles = a.S * a.Hkv * a.n_mtiles;
      const int bpt = kTileRows / (kBlock / (a.D / 4));
      if (a.D == 128)
        hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(tiles * bpt), dim3(kBlock), 0, st, a);
      else
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(tiles * bpt), dim3(kBlock), 0, st, a);
    }
  } else {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.S * a.n_cap * a.Hq), dim3(kBlock), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace dtv
