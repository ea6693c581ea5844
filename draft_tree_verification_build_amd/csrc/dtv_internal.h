// Host/device argument blocks and launch wrappers shared between the kernel sources and
// the C entry points (api.cpp). Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dtv {

// Kernel timing (dtv_kernel_timing, timing.hip). While timing is on, a LaunchTimer brackets
// one launch with two HIP events recorded on the launch's stream; their elapsed time is
// folded into the kernel's totals when the caller reads them. While it is off, it does
// nothing.
class LaunchTimer {
 public:
  LaunchTimer(const char* kernel, hipStream_t stream);
  ~LaunchTimer();
  LaunchTimer(const LaunchTimer&) = delete;
  LaunchTimer& operator=(const LaunchTimer&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t begin_ = nullptr;
};

// Every kernel of the library is launched through this macro, so that timing sees it.
#define DTV_LAUNCH(kernel, grid, block, smem, stream, ...)                      \
  do {                                                                          \
    ::dtv::LaunchTimer dtv_launch_timer_(#kernel, stream);                      \
    hipLaunchKernelGGL(kernel, grid, block, smem, stream, __VA_ARGS__);         \
  } while (0)

struct ChunkStat;

struct TreeArgs {
  int n_cap, words;
  int* n_nodes;
  int* parent;
  int* token;
  int* depth;
  int* row;
  double* score;
  uint64_t* anc;
  int* layers;
};

// TALON. The whole-table build reduces rows 0..B-1 of `draft` (R rows per sequence, keyed
// by slot) and runs the layer loop in one launch. The layer-by-layer build reduces, per
// call, the first W[s] of the Wr rows per sequence of `draft` (the frontier's rows, in
// frontier order) and runs one layer, keeping the loop's state in the workspace.
struct TalonArgs {
  TreeArgs tree;
  const void* draft;
  int R, V, S, B, K, nch;
  int Wr;              // rows reduced per sequence: B (whole table) or the call's row capacity
  double log_alpha;
  WsHeader* hdr;
  ChunkStat* st;       // [S][Wr][nch]
  float* cval;         // [S][Wr][nch][K]
  int* cidx;           // [S][Wr][nch][K]
  unsigned* tickets;   // [S][Wr]
  double* rlse;        // [S][Wr]
  float* rv;           // [S][Wr][K]
  int* ri;             // [S][Wr][K]
  int* rcnt;           // [S][Wr]
  // layer-by-layer build only (null otherwise)
  int layer;           // 1 for the root layer
  int* state;          // [S][8]: nodes so far, first frontier slot, frontier width, layers, done
  int* w_out;          // [S] frontier width of the next layer (0 when done)
  int* done_out;       // [S] 1 when the tree is complete
};

constexpr int kSpineMaxForks = 128;

struct SpineArgs {
  TreeArgs tree;
  const int* spine;    // [S][n_spine]
  const void* draft;
  int R, V, S, n_spine, F, K, nch, n_nodes;
  int width[kSpineMaxForks];
  int offset[kSpineMaxForks];   // exclusive prefix of width
  WsHeader* hdr;
  ChunkStat* st;       // [S][F][nch]
  float* cval;         // [S][F][nch][K]
  int* cidx;
  unsigned* tickets;   // [S][F]
  double* rlse;        // [S][F]
  float* rv;           // [S][F][K]
  int* ri;
};

struct OptCand;

struct OptArgs {
  TreeArgs tree;
  const void* draft;
  int R, V, S, n, nch, max_layers;
  double delta;
  // per layer (set by the host before each layer's launches)
  int layer, W, Wcap, K, Kc;   // K: entries a row reports; Kc: per chunk (nch * Kc >= K)
  int Kw;                      // root layer in one launch: lane maxima per full wave (0: not used)
  WsHeader* hdr;
  ChunkStat* st;          // [S][Wcap][nch]
  float* cmax;            // [S][Wcap][nch] largest value of every chunk of the frontier rows
  float* cval;            // [S][Wcap][nch][Kmax]
  int* cidx;
  unsigned* tickets;      // [S][Wcap]
  double* rlse;           // [S][Wcap]
  float* rv;              // [S][Wcap][Kmax]
  int* ri;
  int* rcnt;              // [S][Wcap]
  double* lo;             // [S]
  unsigned* ccount;       // [S]
  int ccap;
  OptCand* cand;          // [S][ccap]
  double* lscore;         // [S][max_layers][n] per layer, frontier order
  int* lparent;           // parent's frontier position in the previous layer
  int* ltoken;
  double* bscore;         // [S][n] the best n so far by (score desc, layer asc, position asc), unordered
  int* blayer;
  int* bpos;
  int* bcount;            // [S]
  double* Eprev;          // [S]
  int* done;              // [S]
  int* nlayers;           // [S]
  // layer by layer: rows of `draft` are the call's frontier rows from row_base on (the
  // whole-table build has row_base -1 and reads row 1 + (l-2) n + f for layer l's row f)
  int row_base;
  int* fin;               // [S] tree written (null: the whole-table build finalizes once)
  int* w_out;             // [S] frontier width of the next layer (0 when done)
  int* done_out;          // [S]
  int w_next;             // frontier width of the next layer while not done
};

struct RowStatsArgs {
  const void* table;
  int R, V, K, nch;
  const int* row_idx;
  float* maxv;
  int* argmax;
  double* lse;
  int* topk;
  WsHeader* hdr;
  ChunkStat* st;       // [R][nch]
  float* cval;         // [R][nch][K]
  int* cidx;
  unsigned* tickets;   // [R]
  float* mval;         // [R][K] merged values (scratch)
};

constexpr int kAttnMaxSplit = 32;   // key splits per (sequence, KV head, query tile)

// Weights 2^(m_q - max) of the key splits of one query row, from its (m, l) partials at
// ml[q * stride] (q < n <= NS). All loads are issued before any is used (a split index
// past n re-reads split n-1 and gets weight 0). Returns the merged l.
template <int NS>
__device__ __forceinline__ float attn_split_weights(const float* ml, size_t stride, int n, float (&w)[NS]) {
  float m[NS], l[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    const int qq = q < n ? q : n - 1;
    const float2 v = *reinterpret_cast<const float2*>(ml + static_cast<size_t>(qq) * stride);
    m[q] = v.x;
    l[q] = (q < n) ? v.y : 0.f;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int q = 0; q < NS; ++q) mx = l[q] > 0.f ? fmaxf(mx, m[q]) : mx;
  float L = 0.f;
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    w[q] = l[q] > 0.f ? __builtin_amdgcn_exp2f(m[q] - mx) : 0.f;
    L += l[q] * w[q];
  }
  return L;
}

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int* P;
  int P_cap;
  const int* n_nodes;
  const uint64_t* anc;
  int n_cap, words;
  int S, Hq, Hkv, D, g;
  float scale;          // softmax scale (1/sqrt(D) by default)
  int n_mtiles, n_split, kps;  // query tiles per KV head, key splits, keys per split
  int mcap;             // partial rows per (sequence, KV head, split)
  float* part_o;        // [S*Hkv][n_split][mcap][D] unnormalised O of every key split
  float* part_ml;       // same rows, (m, l) pairs
  WsHeader* hdr;
};

// A KV cache that a verification compacts along its path in the same launch (k null: none).
struct KvCompactView {
  char* k;
  char* v;
  const int* P;
  int* P_new;
  int P_cap, Hkv, D, esize;
};

struct VerifyArgs {
  TreeArgs tree;
  const void* target;
  int R, V, nch;
  int* path;
  int* path_len;
  int* bonus;
  int* argmax_out;
  unsigned long long* cbest;  // [S][n_cap][nch] chunk argmax keys (0: not yet reported)
  WsHeader* hdr;
  KvCompactView kvc;
};

// Sizes of the rejection-sampling walk, shared by the host plan (api.hip) and the kernels.
constexpr int kSampleMaxNodes = 1024;   // tree slots the walk keeps in shared memory
constexpr int kSampleMaxGroup = 32;     // workgroups per sequence in the walk
constexpr int kXchStride = 4 * kSampleMaxGroup;   // entries per exchange slot (4 values per workgroup)
constexpr int kWalkSlice = 4096;        // slice entries kept in shared memory (else the workspace)
static_assert(kSampleMaxGroup + 2 <= kXchStride, "an exchange slot holds G sums and two values");

struct SampleArgs {
  TreeArgs tree;
  const void* target;
  const void* draft;
  int R, V, nch;
  const uint32_t* u_acc;     // [S][n_cap]
  const uint32_t* u_res;     // [S][n_cap]
  int* path;
  int* path_len;
  int* bonus;
  WsHeader* hdr;
  int S;
  int G;                     // workgroups per sequence in the walk
  int vec;                   // 1: rows are walked in 16-byte units (aligned, V a multiple of 8 / 4)
  int max_pass;              // exchange slots per sequence (visited nodes + rejections + 1)
  double* xch;               // [S][max_pass][kXchStride] exchange slots (all zero between calls)
  double* pbuf;              // [S][3][V] residual distributions and q (slices too large for LDS)
  unsigned* done;            // [S] workgroups that finished the walk (zero between calls)
  KvCompactView kvc;
};

struct CompactArgs {
  void* k;
  void* v;
  const int* P;
  int* P_new;
  int P_cap;
  const int* path;
  const int* path_len;
  int n_cap, S, Hkv, D, esize;
};

int launch_given(const TreeArgs& t, int S, WsHeader* hdr, hipStream_t st);
int launch_talon(const TalonArgs& a, int dtype, hipStream_t st);
int launch_talon_layer(const TalonArgs& a, int dtype, hipStream_t st);
int launch_spine(const SpineArgs& a, int dtype, hipStream_t st);
int launch_opt_init(const OptArgs& a, hipStream_t st);
int launch_opt_layer(OptArgs a, int dtype, hipStream_t st);
int launch_opt_root(const OptArgs& a, int dtype, hipStream_t st);
int opt_root_wave_quota(int V, int n, int dtype);
// The root layer in one 1024-thread workgroup per sequence (bf16, V <= 32768, ceil(V/8) >= n);
// that launch also sets the per-call state (no init launch needed before it).
bool opt_root_one_workgroup(int V, int n, int dtype);
int launch_opt_finalize(const OptArgs& a, hipStream_t st);
int launch_opt_report(const OptArgs& a, hipStream_t st);
int launch_row_stats(const RowStatsArgs& a, int dtype, hipStream_t st);
int launch_attn(const AttnArgs& a, int dtype, hipStream_t st);
int launch_attn_bf16(const AttnArgs& a, hipStream_t st);
int launch_verify_greedy(const VerifyArgs& a, int S, int dtype, hipStream_t st);
int launch_verify_sample(const SampleArgs& a, int S, int dtype, hipStream_t st);
int sample_walk_max_blocks(int dtype);
int launch_compact(const CompactArgs& a, hipStream_t st);

}  // namespace dtv
