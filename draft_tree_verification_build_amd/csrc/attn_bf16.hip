// Tree-masked attention, bf16 on MFMA (gfx950).
//
// Each node attends to the prefix and to its ancestors (position P + j is visible to node
// i when bit j of i's ancestor mask is set). Grouped-query heads are packed: for KV head kv
// the g = Hq / Hkv query heads of every node form M = g * n_nodes rows (row r = node r / g,
// head kv * g + r % g), so a K/V tile is read once for all of them.
//
// * S^T = K Q^T and O += P V with v_mfma_f32_32x32x16_bf16 (fp32 accumulation). Computing
//   S^T rather than S leaves every lane holding 16 keys of one query row, exactly the
//   operand layout the P V product needs, so P never leaves registers.
// * A workgroup has 4 waves, each owning one 32-row group; two workgroups share a compute
//   unit so that one's softmax overlaps the other's MFMAs. The ceil(M/32) row groups of a
//   KV head are spread evenly over the tiles, so ragged row counts do not leave a tile
//   nearly empty.
// * K/V are double-buffered in LDS, both row-major as in HBM (V is transposed by the
//   fragment reads, not in memory): the global loads of block b+1 are issued before block
//   b is computed and land in the other buffer afterwards, one barrier per 64-key block. Every load is unconditional (clamped to
//   a valid key) so all of them are in flight together; every LDS access is a
//   conflict-free 16-byte access.
// * The tree mask and the key-range tail are applied only in blocks that need them, from
//   one 64-bit visibility word per row and block. The softmax runs in the exp2 domain with
//   the scale folded into one fma per score and a lazily moved reference maximum.
// * Workgroup numbering is XCD-aware: all tiles of one (sequence, KV head, key split)
//   share an XCD, hence its L2, since they stream the same keys and values.
//
// Key splits write (m, l, unnormalised O) partials per query row; attn_combine_rows merges
// them (a kernel boundary makes the partials of all XCDs visible).
#include "dtv_internal.h"

namespace dtv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kKeyBlock = 64;   // keys per LDS block
constexpr int kNumXcd = 8;    // XCDs of an MI355X; consecutive workgroups go to consecutive XCDs

union Frag8 {
  bf16x8 v;
  uint4 u;
  uint2 h[2];
  uint16_t s[8];
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ---- LDS layout of one 64-key block
// K and V sit row-major in LDS as in HBM (64 rows of D bf16 each), so the global loads
// write LDS directly: lane l of a global_load_lds_dwordx4 fills bytes 16 l .. 16 l + 15
// after the load's LDS base, with no registers and no stores on the way. The 16-byte
// chunks of a row are XOR-permuted by row, chunk c of row r at position c ^ fk(r) (K) or
// c ^ fv(r) (V), so that the fragment reads below are free of bank conflicts (LDS: 64 banks
// of 4 bytes); each load lane fetches the global chunk that belongs at its LDS position.
//  * K fragments (A operand of S^T = K Q^T) are 16-byte reads: 16 lanes read one chunk
//    index of 16 consecutive rows, which fk spreads over all 64 banks.
//  * V fragments (B operand of O += P V) come from ds_read_b64_tr_b16, which hands lane
//    16 g + i element i % 4 of the 8-byte words addressed by lanes 16 g + 4 j + i / 4,
//    j = 0..3: the transpose happens in the read. 32 lanes then address 4 consecutive rows
//    at 4 consecutive chunks, which fv spreads over all 64 banks.
template <int D>
struct KvLds {
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  static constexpr int kChunks = D / 8;                               // 16-byte chunks per row
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kRowShift = D == 128 ? 8 : 7;                  // log2(kRowBytes)
  static constexpr int kLoads = kKeyBlock * kChunks / 64 / kWaves;    // loads per wave per tensor
  __device__ static __forceinline__ int fk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static __forceinline__ int fv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// Issues direct-load pair i (one K and one V load) of keys kb .. kb+63 into (kd, vd)
// (requires kb < k_hi). A lane whose row is at or past k_hi reads the last 16 bytes of row
// k_hi - 1 instead: finite data of a key the softmax masks out, and a valid address.
// ofs[i] / ofs[L + i] hold the in-block byte offsets of this lane's K / V loads (multiples
// of 16); the LDS base of load i of wave w is byte 1024 (w L + i) of the block.
template <int D>
__device__ __forceinline__ void kv_issue_pair(int i, uint16_t* kd, uint16_t* vd, const uint16_t* kbase,
                                              const uint16_t* vbase, int kb, int k_hi,
                                              const int (&ofs)[2 * KvLds<D>::kLoads], int w) {
  using L = KvLds<D>;
  const char* kp = reinterpret_cast<const char*>(kbase + static_cast<size_t>(kb) * D);
  const char* vp = reinterpret_cast<const char*>(vbase + static_cast<size_t>(kb) * D);
  // One unsigned min per load against the offset of the last 16-byte chunk of row
  // k_hi - 1 - kb; the offset stays a 32-bit value over a wave-uniform base, which the load
  // can take as scalar base + vector offset.
  const uint32_t cap = static_cast<uint32_t>(k_hi - 1 - kb) * L::kRowBytes + (L::kRowBytes - 16);
  const uint32_t ko = min(static_cast<uint32_t>(ofs[i]), cap);
  const uint32_t vo = min(static_cast<uint32_t>(ofs[L::kLoads + i]), cap);
  const int lds_off = 1024 * (w * L::kLoads + i);
  __builtin_amdgcn_global_load_lds(kp + ko, (lds_void*)(reinterpret_cast<char*>(kd) + lds_off), 16, 0, 0);
  __builtin_amdgcn_global_load_lds(vp + vo, (lds_void*)(reinterpret_cast<char*>(vd) + lds_off), 16, 0, 0);
}

// Visibility of keys kb .. kb+63 to one query row as a 64-bit mask (bit o: key kb + o).
// Cache positions below P are the prefix, visible to every node; position P + j is tree
// node j, visible when bit j of the row's ancestor mask is set; keys at or past k_hi
// belong to another split or do not exist. Requires kb < k_hi <= P + n_nodes, so every
// ancestor word read is inside the row's mask. Padding rows (ok false) see the prefix only.
__device__ __forceinline__ uint64_t block_visibility(int kb, int P, int k_hi, const uint64_t* anc, bool ok) {
  const int nr = k_hi - kb;
  const uint64_t in_range = nr >= 64 ? ~0ull : ((1ull << nr) - 1ull);
  const int np = P - kb;
  const uint64_t prefix = np >= 64 ? ~0ull : (np <= 0 ? 0ull : ((1ull << np) - 1ull));
  uint64_t tree = 0ull;
  if (np < 64 && ok) {
    if (np > 0) {
      tree = anc[0] << np;
    } else {
      const int j0 = -np, wi = j0 >> 6, sh = j0 & 63;
      const uint64_t lo = anc[wi];
      tree = lo >> sh;
      if (sh != 0 && kb + (64 - sh) < k_hi) tree |= anc[wi + 1] << (64 - sh);
    }
  }
  return (prefix | tree) & in_range;
}

// Writes one 32-row group of O: normalised bf16 rows when the sequence's keys are not
// split (ns == 1), else the unnormalised fp32 rows and their (m, l) as partials. A lane
// holds O rows (i/4)*8 + 4h + i%4 of the group, column nt*32 + lr of tile nt.
template <int D>
__device__ __forceinline__ void o_store(const AttnArgs& a, const f32x16 (&oo)[D / 32], const float (*ml)[2],
                                           int s, int kv, int sp, int ns, int grp, int M, int h, int lr) {
  constexpr int NT = D / 32;
  const int g = a.g;
  const size_t prow0 = ((static_cast<size_t>(s) * a.Hkv + kv) * a.n_split + sp) * static_cast<size_t>(a.mcap);
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int rl = q4 * 8 + 4 * h + b;
      const int rr = grp * 32 + rl;
      if (rr >= M) continue;
      if (ns == 1) {
        const float l = ml[rl][1];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        __bf16* orow = static_cast<__bf16*>(a.o) +
                       ((static_cast<size_t>(s) * a.n_cap + rr / g) * a.Hq + kv * g + rr % g) * D;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) orow[nt * 32 + lr] = static_cast<__bf16>(oo[nt][q4 * 4 + b] * inv);
      } else {
        float* prow = a.part_o + (prow0 + rr) * D;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) prow[nt * 32 + lr] = oo[nt][q4 * 4 + b];
      }
    }
  if (ns > 1 && h == 0) {
    const int rr = grp * 32 + lr;
    if (rr < M) {
      a.part_ml[(prow0 + rr) * 2 + 0] = ml[lr][0];
      a.part_ml[(prow0 + rr) * 2 + 1] = ml[lr][1];
    }
  }
}

template <int D>
__global__ __launch_bounds__(kBlock, 2) void attn_bf16_kernel(AttnArgs a) {
  using L = KvLds<D>;
  // Two LDS buffers per tensor, as separate objects: the loop body is instantiated per
  // buffer, so the compiler can tell the block being read from the one being loaded.
  __shared__ alignas(16) uint16_t ks0[kKeyBlock * D];
  __shared__ alignas(16) uint16_t ks1[kKeyBlock * D];
  __shared__ alignas(16) uint16_t vs0[kKeyBlock * D];
  __shared__ alignas(16) uint16_t vs1[kKeyBlock * D];
  __shared__ alignas(16) float alpha_s[kWaves][32];
  __shared__ alignas(16) float ml_s[kWaves][32][2];
  constexpr int NKS = D / 16;
  constexpr int NT = D / 32;

  // ---- XCD-aware decode: the tiles of unit u = (s, kv, split) share XCD u % 8
  const int bid = blockIdx.x;
  const int xcd = bid % kNumXcd;
  const int local = bid / kNumXcd;
  const int tm = local % a.n_mtiles;
  const int u = (local / a.n_mtiles) * kNumXcd + xcd;
  if (u >= a.S * a.Hkv * a.n_split) return;
  const int sp = u % a.n_split;
  const int kv = (u / a.n_split) % a.Hkv;
  const int s = u / (a.n_split * a.Hkv);

  const int N = a.n_nodes[s];
  const int g = a.g;
  const int M = g * N;
  const int P = a.P[s];
  // Query rows come from the planned tiling (n_cap nodes), so their loads are issued with
  // the node count and prefix length rather than after them: a row past the sequence's
  // nodes reads a valid slot and is never stored.
  constexpr int NKS0 = D / 16;
  Frag8 qf[NKS0];
  const int Gp = (g * a.n_cap + 31) / 32;   // groups of the planned tiling
  {
    const int w0 = threadIdx.x >> 6, lane0 = threadIdx.x & 63;
    const int grp0 = tm * Gp / a.n_mtiles + w0;
    const int r0 = grp0 * 32 + (lane0 & 31);
    const int node0 = min(r0 / g, a.n_cap - 1);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((static_cast<size_t>(s) * a.n_cap + node0) * a.Hq + kv * g + r0 % g) * D;
#pragma unroll
    for (int ks = 0; ks < NKS0; ++ks) qf[ks].u = *reinterpret_cast<const uint4*>(qrow + ks * 16 + 8 * (lane0 >> 5));
  }
  if (N > a.n_cap || P < 0 || P + N > a.P_cap) {
    if (threadIdx.x == 0) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  // the sequence's own row groups over its own tiles (a smaller tree uses fewer tiles, each
  // with every wave busy, rather than spreading its groups over the planned tiles)
  const int G = (M + 31) / 32;
  const int mt = min(a.n_mtiles, (G + kWaves - 1) / kWaves);
  if (tm >= mt) return;
  const int gl = tm * G / mt, gh = (tm + 1) * G / mt;
  if (gl >= gh) return;
  const int T = P + N;
  // the sequence's own split count: a split past its keys does nothing (the merge reads
  // only this sequence's splits), and a sequence with one split writes its output directly
  const int ns = (T + a.kps - 1) / a.kps;
  if (ns > a.n_split) {   // a prefix longer than the plan's P_max: its keys have no split
    if (threadIdx.x == 0) atomicExch(&a.hdr->err, kErrCapacity);
    return;
  }
  if (sp >= ns) return;
  const int k_lo = sp * a.kps;
  const int k_hi = min(k_lo + a.kps, T);

  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform
  const int lane = t & 63;
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int grp = gl + w;          // this wave's 32-row group
  const bool act = grp < gh;
  const int r = grp * 32 + lr;     // this lane's query row (lanes lr and lr + 32 share it)
  const bool ok = act && r < M;
  const int node = ok ? r / g : 0;

  const size_t kvoff = (static_cast<size_t>(s) * a.Hkv + kv) * a.P_cap * static_cast<size_t>(D);
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + kvoff;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + kvoff;
  const uint64_t* anc = a.anc + (static_cast<size_t>(s) * a.n_cap + node) * a.words;

  if (G != Gp || mt != a.n_mtiles) {
    // fewer nodes than planned changes the tiling: this wave's rows are reloaded (a padding
    // row past M reads row 0's query, valid memory, and its output is never stored)
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((static_cast<size_t>(s) * a.n_cap + node) * a.Hq + kv * g + (ok ? r % g : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks].u = *reinterpret_cast<const uint4*>(qrow + ks * 16 + 8 * h);
  }

  // ---- per-lane LDS offsets, fixed for the whole kernel
  int lofs[2 * L::kLoads];   // in-block byte offsets of this lane's K and V loads
#pragma unroll
  for (int i = 0; i < L::kLoads; ++i) {
    const int pos = 64 * (w * L::kLoads + i) + lane;   // chunk position in the block
    const int row = pos / L::kChunks, c = pos % L::kChunks;
    lofs[i] = row * L::kRowBytes + ((c ^ L::fk(row)) << 4);
    lofs[L::kLoads + i] = row * L::kRowBytes + ((c ^ L::fv(row)) << 4);
  }
  int kread[NKS];            // K fragment of step ks: row lr, chunk 2 ks + h
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) kread[ks] = lr * L::kRowBytes + (((2 * ks + h) ^ L::fk(lr)) << 4);
  int vread[NT];             // V transpose read of tile nt (see KvLds)
  {
    const int gg = lane >> 4, jj = (lane >> 2) & 3, mm = lane & 3;
    const int row = 4 * (gg >> 1) + jj;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int c = 4 * nt + 2 * (gg & 1) + (mm >> 1);
      vread[nt] = row * L::kRowBytes + ((c ^ L::fv(row)) << 4) + 8 * (mm & 1);
    }
  }

  f32x16 oacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[nt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;   // reference max (log2 units) and row sum
  const float sl2 = a.scale * 1.4426950408889634f;

  const int nblk = (k_hi > k_lo) ? (k_hi - k_lo + kKeyBlock - 1) / kKeyBlock : 0;
  if (nblk > 0) {
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i) kv_issue_pair<D>(i, ks0, vs0, kbase, vbase, k_lo, k_hi, lofs, w);
  }
  // Nothing may be outstanding at the loop head: otherwise the wait inserted for the
  // query registers inside the loop also waits for the next block's loads.
  drain();
  __syncthreads();

  // One 64-key block from buffer (kc, vc) while the next one streams into (kn, vn).
  auto step = [&](int b, const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn) {
    const int kb = k_lo + b * kKeyBlock;
    const bool more = b + 1 < nblk;
    // Visibility of this block's keys (tree keys or the range tail only); the ancestor
    // words are read before the next block's loads are issued so that waiting for them
    // does not wait for those loads.
    const bool need_mask = (kb + kKeyBlock > P) || (kb + kKeyBlock > k_hi);
    uint64_t vis = ~0ull;
    if (need_mask) vis = block_visibility(kb, P, k_hi, anc, ok) >> (4 * h);
    // The next block's loads are spread over the S^T steps so that issuing them overlaps
    // the MFMAs. After the last block they reload this block into the idle buffer (valid
    // addresses, never read), which keeps every load unconditional.
    const int kb_next = more ? kb + kKeyBlock : kb;
    constexpr int QS = 2 * NKS;             // S^T steps (ks, kt), j = 2 ks + kt
    constexpr int QPL = QS / L::kLoads;     // steps per load pair
    constexpr int PS = 4 * NT;              // P V steps (k2, nt), j = NT k2 + nt
    constexpr int kAhead = 4;               // LDS fragment reads kept in flight
    const char* kcb = reinterpret_cast<const char*>(kc);
    const char* vcb = reinterpret_cast<const char*>(vc);
    auto kfrag = [&](int j) {
      Frag8 f;
      f.u = *reinterpret_cast<const uint4*>(kcb + (j & 1) * 32 * L::kRowBytes + kread[j >> 1]);
      return f;
    };
    auto vfrag = [&](int j) {
      Frag8 f;
      const char* vrow = vcb + 16 * (j / NT) * L::kRowBytes + vread[j % NT];
      f.h[0] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vrow)));
      f.h[1] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vrow + 8 * L::kRowBytes)));
      return f;
    };

    if (act) {
      // ---- S^T = K Q^T for two 32-key tiles; lane holds keys kb + kt*32 + (i/4)*8 + 4h + i%4.
      //      Software-pipelined: the K fragment of step j + kAhead is read while step j runs.
      f32x16 sc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kt][i] = 0.f;
      Frag8 kf[QS];
#pragma unroll
      for (int j = 0; j < kAhead; ++j) kf[j] = kfrag(j);
      // MFMA phases run at raised wave priority, so that the other workgroup's wave on this
      // SIMD fills the gaps with its softmax and loads rather than competing for issue
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < QS; ++j) {
        if (j + kAhead < QS) kf[j + kAhead] = kfrag(j + kAhead);
        if (j % QPL == 0) kv_issue_pair<D>(j / QPL, kn, vn, kbase, vbase, kb_next, k_hi, lofs, w);
        __builtin_amdgcn_sched_barrier(0);
        sc[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j].v, qf[j >> 1].v, sc[j & 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // the first V fragments are read while the softmax runs
      Frag8 vf[PS];
#pragma unroll
      for (int j = 0; j < kAhead; ++j) vf[j] = vfrag(j);
      // ---- masks (tree block, range tail) only where a block needs them
      if (need_mask) {
        const uint32_t v_lo = static_cast<uint32_t>(vis), v_hi = static_cast<uint32_t>(vis >> 32);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t bits = kt == 0 ? v_lo : v_hi;
            if (!((bits >> ((i >> 2) * 8 + (i & 3))) & 1u)) sc[kt][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
      // ---- lazy rescaling: the reference max only moves when the block's max exceeds it
      //      by more than 8 (log2 units), so p <= 2^8 and the O rescale is rare (the final
      //      division by l makes the result independent of the reference). The branch is
      //      wave-uniform.
      if (__ballot(mx > m_run + 8.f) != 0ull) {
        float alpha = 1.f;
        if (mx > m_run + 8.f) {
          alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
          l_run *= alpha;
          m_run = mx;
        }
        // a lane holds O rows (i/4)*8 + 4h + i%4 of the group
        if (h == 0) alpha_s[w][lr] = alpha;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 al = *reinterpret_cast<const float4*>(&alpha_s[w][q4 * 8 + 4 * h]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            oacc[nt][q4 * 4 + 0] *= al.x;
            oacc[nt][q4 * 4 + 1] *= al.y;
            oacc[nt][q4 * 4 + 2] *= al.z;
            oacc[nt][q4 * 4 + 3] *= al.w;
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
      const float mref = (m_run == -INFINITY) ? 0.f : m_run;
      float sum = 0.f;
      // the A operand of step k2 is p values 8*(k2%2) .. +7 of key tile k2/2, i.e. keys
      // 16 k2 + 8 (j/4) + 4h + j%4: the key order of the two transpose reads of a V fragment
      // (rows 16 k2 + 4h + j and 16 k2 + 8 + 4h + j)
      Frag8 pf8[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[kt][i], sl2, -mref));
          sum += p;
          pf8[2 * kt + (i >> 3)].v[i & 7] = static_cast<__bf16>(p);
        }
      l_run += sum;
      // ---- O += P V, software-pipelined like S^T
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < PS; ++j) {
        if (j + kAhead < PS) vf[j + kAhead] = vfrag(j + kAhead);
        __builtin_amdgcn_sched_barrier(0);
        oacc[j % NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf8[j / NT].v, vf[j].v, oacc[j % NT], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    } else {
#pragma unroll
      for (int i = 0; i < L::kLoads; ++i) kv_issue_pair<D>(i, kn, vn, kbase, vbase, kb_next, k_hi, lofs, w);
    }
    // the next block has landed (this wave's loads) and is visible (everyone's)
    drain();
    __syncthreads();
  };

  for (int b = 0; b < nblk; b += 2) {
    step(b, ks0, vs0, ks1, vs1);
    if (b + 1 < nblk) step(b + 1, ks1, vs1, ks0, vs0);
  }

  // ---- row statistics in the O layout
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (h == 0) {
    ml_s[w][lr][0] = m_run;
    ml_s[w][lr][1] = l_tot;
  }
  __syncthreads();
  if (act) o_store<D>(a, oacc, ml_s[w], s, kv, sp, ns, grp, M, h, lr);
}

// Merges the key splits of every query row (partials indexed by row): O = sum_q O_q w_q / sum_q l_q w_q
// with w_q = 2^(m_q - max m). One thread per 4 output values, D/4 threads per row.
template <int D, int NS>
__global__ __launch_bounds__(kBlock) void attn_combine_rows_kernel(AttnArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = kBlock / TPR;
  const int rows_per_head = a.mcap;
  const int blocks_per_head = (rows_per_head + RPB - 1) / RPB;
  const int head = blockIdx.x / blocks_per_head;   // (s, kv)
  const int rr = (blockIdx.x % blocks_per_head) * RPB + threadIdx.x / TPR;
  const int c4 = threadIdx.x % TPR;
  const int kv = head % a.Hkv;
  const int s = head / a.Hkv;
  const size_t pr0 = static_cast<size_t>(head) * a.n_split * rows_per_head + rr;
  // the sequence's own split count (a sequence with one split has its output written)
  const int N = a.n_nodes[s];
  const int ns = (a.P[s] + N + a.kps - 1) / a.kps;
  if (N > a.n_cap || rr >= a.g * N || ns <= 1 || ns > a.n_split) return;
  // every split's O row and every (m, l) are loaded together, one round trip (splits past
  // ns re-read split ns-1 and get weight 0)
  float4 o[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int qq = min(u, ns - 1);
    o[u] = *reinterpret_cast<const float4*>(&a.part_o[(pr0 + static_cast<size_t>(qq) * rows_per_head) * D + c4 * 4]);
  }
  float w[NS];
  const float L = attn_split_weights<NS>(a.part_ml + pr0 * 2, static_cast<size_t>(rows_per_head) * 2, ns, w);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const float sc = w[u];   // 0 past n_split
    acc.x += o[u].x * sc;
    acc.y += o[u].y * sc;
    acc.z += o[u].z * sc;
    acc.w += o[u].w * sc;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  __bf16* orow = static_cast<__bf16*>(a.o) +
                 ((static_cast<size_t>(s) * a.n_cap + rr / a.g) * a.Hq + kv * a.g + rr % a.g) * D + c4 * 4;
  const auto bits = [](float x) { return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x))); };
  // the four outputs in one 8-byte store
  *reinterpret_cast<uint2*>(orow) =
      make_uint2(bits(acc.x * inv) | (bits(acc.y * inv) << 16), bits(acc.z * inv) | (bits(acc.w * inv) << 16));
}

int launch_attn_bf16(const AttnArgs& a, hipStream_t st) {
  const int units = a.S * a.Hkv * a.n_split;
  const int grid = ((units + kNumXcd - 1) / kNumXcd) * kNumXcd * a.n_mtiles;
  if (a.D == 128)
    DTV_LAUNCH(attn_bf16_kernel<128>, dim3(grid), dim3(kBlock), 0, st, a);
  else
    DTV_LAUNCH(attn_bf16_kernel<64>, dim3(grid), dim3(kBlock), 0, st, a);
  if (hipGetLastError() != hipSuccess) return -1;
  if (a.n_split > 1) {
    const int rpb = kBlock / (a.D / 4);
    const dim3 blocks(a.S * a.Hkv * ((a.mcap + rpb - 1) / rpb));
    // one register per split of a row's partials, all loads in flight at once; the variant
    // with the fewest slots that hold n_split (a slot past a sequence's splits re-reads its
    // last split, a load that still takes issue slots)
    const int n = a.n_split;
    if (a.D == 128) {
      if (n <= 2)
        DTV_LAUNCH((attn_combine_rows_kernel<128, 2>), blocks, dim3(kBlock), 0, st, a);
      else if (n <= 4)
        DTV_LAUNCH((attn_combine_rows_kernel<128, 4>), blocks, dim3(kBlock), 0, st, a);
      else if (n <= 8)
        DTV_LAUNCH((attn_combine_rows_kernel<128, 8>), blocks, dim3(kBlock), 0, st, a);
      else if (n <= 12)
        DTV_LAUNCH((attn_combine_rows_kernel<128, 12>), blocks, dim3(kBlock), 0, st, a);
      else if (n <= 16)
        DTV_LAUNCH((attn_combine_rows_kernel<128, 16>), blocks, dim3(kBlock), 0, st, a);
      else if (n <= 24)
        DTV_LAUNCH((attn_combine_rows_kernel<128, 24>), blocks, dim3(kBlock), 0, st, a);
      else
        DTV_LAUNCH((attn_combine_rows_kernel<128, kAttnMaxSplit>), blocks, dim3(kBlock), 0, st, a);
    } else {
      if (n <= 4)
        DTV_LAUNCH((attn_combine_rows_kernel<64, 4>), blocks, dim3(kBlock), 0, st, a);
      else if (n <= 8)
        DTV_LAUNCH((attn_combine_rows_kernel<64, 8>), blocks, dim3(kBlock), 0, st, a);
      else if (n <= 16)
        DTV_LAUNCH((attn_combine_rows_kernel<64, 16>), blocks, dim3(kBlock), 0, st, a);
      else
        DTV_LAUNCH((attn_combine_rows_kernel<64, kAttnMaxSplit>), blocks, dim3(kBlock), 0, st, a);
    }
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

}  // namespace dtv
