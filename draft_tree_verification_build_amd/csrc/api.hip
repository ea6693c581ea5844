// C entry points of libdtv: argument checks on the host, workspace carving, launches.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "dtv.h"
#include "dtv_internal.h"
#include "rowstats.h"

namespace {

thread_local char g_msg[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Carves consecutive 256-byte aligned regions out of a workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += up(count * sizeof(T));
    return p;
  }
};

int esize_of(int dtype) { return dtype == DTV_BF16 ? 2 : 4; }
bool dtype_ok(int dtype) { return dtype == DTV_F32 || dtype == DTV_BF16; }
int nch_of(int V, int dtype) { return dtype == DTV_BF16 ? dtv::chunks_of<1>(V) : dtv::chunks_of<0>(V); }

int check_tree(const dtv_tree* t) {
  REQUIRE(t != nullptr, DTV_EINVAL, "tree is NULL");
  REQUIRE(t->n_cap >= 1 && t->n_cap <= 1024, DTV_EUNSUPPORTED, "n_cap %d outside 1..1024", t->n_cap);
  REQUIRE(t->words >= (t->n_cap + 63) / 64 && t->words <= 16, DTV_ECAPACITY,
          "words %d cannot hold %d slots", t->words, t->n_cap);
  REQUIRE(t->n_nodes && t->parent && t->token && t->depth && t->row && t->score && t->anc && t->layers,
          DTV_EINVAL, "a tree array is NULL");
  return DTV_OK;
}

dtv::TreeArgs tree_args(const dtv_tree* t) {
  dtv::TreeArgs a;
  a.n_cap = t->n_cap;
  a.words = t->words;
  a.n_nodes = t->n_nodes;
  a.parent = t->parent;
  a.token = t->token;
  a.depth = t->depth;
  a.row = t->row;
  a.score = t->score;
  a.anc = reinterpret_cast<uint64_t*>(t->anc);
  a.layers = t->layers;
  return a;
}

int launched(int rc) {
  if (rc != 0) return fail(DTV_EHIP, "kernel launch failed: %s", hipGetErrorString(hipGetLastError()));
  return DTV_OK;
}

// ------------------------------------------------------------------ layouts

struct RowStatsLayout {
  dtv::WsHeader* hdr;
  dtv::ChunkStat* st;
  float* cval;
  int* cidx;
  unsigned* tickets;
  float* mval;
  size_t bytes;
};
RowStatsLayout row_stats_layout(void* ws, int R, int V, int K, int dtype) {
  const int nch = nch_of(V, dtype);
  const size_t KK = K > 0 ? K : 1;
  Carver c(ws);
  RowStatsLayout L;
  L.hdr = c.take<dtv::WsHeader>(1);
  L.st = c.take<dtv::ChunkStat>(static_cast<size_t>(R) * nch);
  L.cval = c.take<float>(static_cast<size_t>(R) * nch * KK);
  L.cidx = c.take<int>(static_cast<size_t>(R) * nch * KK);
  L.tickets = c.take<unsigned>(R);
  L.mval = c.take<float>(static_cast<size_t>(R) * KK);
  L.bytes = c.off;
  return L;
}

struct TalonLayout {
  dtv::WsHeader* hdr;
  dtv::ChunkStat* st;
  float* cval;
  int* cidx;
  unsigned* tickets;
  double* rlse;
  float* rv;
  int* ri;
  int* rcnt;
  size_t bytes;
};
TalonLayout talon_layout(void* ws, int S, int B, int K, int V, int dtype) {
  const int nch = nch_of(V, dtype);
  const size_t rows = static_cast<size_t>(S) * B;
  Carver c(ws);
  TalonLayout L;
  L.hdr = c.take<dtv::WsHeader>(1);
  L.st = c.take<dtv::ChunkStat>(rows * nch);
  L.cval = c.take<float>(rows * nch * K);
  L.cidx = c.take<int>(rows * nch * K);
  L.tickets = c.take<unsigned>(rows);
  L.rlse = c.take<double>(rows);
  L.rv = c.take<float>(rows * K);
  L.ri = c.take<int>(rows * K);
  L.rcnt = c.take<int>(rows);
  L.bytes = c.off;
  return L;
}

struct SpineLayout {
  dtv::WsHeader* hdr;
  dtv::ChunkStat* st;
  float* cval;
  int* cidx;
  unsigned* tickets;
  double* rlse;
  float* rv;
  int* ri;
  size_t bytes;
};
SpineLayout spine_layout(void* ws, int S, int F, int K, int V, int dtype) {
  const int nch = nch_of(V, dtype);
  const size_t rows = static_cast<size_t>(S) * F;
  Carver c(ws);
  SpineLayout L;
  L.hdr = c.take<dtv::WsHeader>(1);
  L.st = c.take<dtv::ChunkStat>(rows * nch);
  L.cval = c.take<float>(rows * nch * K);
  L.cidx = c.take<int>(rows * nch * K);
  L.tickets = c.take<unsigned>(rows);
  L.rlse = c.take<double>(rows);
  L.rv = c.take<float>(rows * K);
  L.ri = c.take<int>(rows * K);
  L.bytes = c.off;
  return L;
}

struct OptLayout {
  dtv::WsHeader* hdr;
  dtv::ChunkStat* st;
  float* cmax;
  float* cval;
  int* cidx;
  unsigned* tickets;
  double* rlse;
  float* rv;
  int* ri;
  int* rcnt;
  double* lo;
  unsigned* ccount;
  void* cand;
  double* lscore;
  int* lparent;
  int* ltoken;
  double* bscore;
  int* blayer;
  int* bpos;
  int* bcount;
  double* Eprev;
  int* done;
  int* nlayers;
  int* fin;
  size_t bytes;
};
constexpr int kOptCandCap = 4096;
OptLayout opt_layout(void* ws, int S, int n, int V, int max_layers, int dtype) {
  const int nch = nch_of(V, dtype);
  const size_t Kmax = static_cast<size_t>(n < V ? n : V);
  const size_t rows = static_cast<size_t>(S) * n;
  Carver c(ws);
  OptLayout L;
  L.hdr = c.take<dtv::WsHeader>(1);
  L.st = c.take<dtv::ChunkStat>(rows * nch);
  L.cmax = c.take<float>(rows * nch);
  L.cval = c.take<float>(rows * nch * Kmax);
  L.cidx = c.take<int>(rows * nch * Kmax);
  L.tickets = c.take<unsigned>(rows);
  L.rlse = c.take<double>(rows);
  L.rv = c.take<float>(rows * Kmax);
  L.ri = c.take<int>(rows * Kmax);
  L.rcnt = c.take<int>(rows);
  L.lo = c.take<double>(S);
  L.ccount = c.take<unsigned>(S);
  L.cand = c.take<char>(static_cast<size_t>(S) * kOptCandCap * 16);
  L.lscore = c.take<double>(rows * max_layers);
  L.lparent = c.take<int>(rows * max_layers);
  L.ltoken = c.take<int>(rows * max_layers);
  L.bscore = c.take<double>(rows);
  L.blayer = c.take<int>(rows);
  L.bpos = c.take<int>(rows);
  L.bcount = c.take<int>(S);
  L.Eprev = c.take<double>(S);
  L.done = c.take<int>(S);
  L.nlayers = c.take<int>(S);
  L.fin = c.take<int>(S);
  L.bytes = c.off;
  return L;
}

// Compute units of the current device (queried once per device; 256 on an MI355X).
int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] > 0) return cached[dev];
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1) return 256;
  cached[dev] = ncu;
  return ncu;
}

struct AttnPlan {
  int n_mtiles, n_split, kps, mcap;
};
// Query rows of a KV head: M = g * n_cap (GQA heads packed), in ceil(M/32) groups of 32;
// a bf16 tile is 4 waves of one group each. The key range of every tile is split into
// n_split ranges (multiples of 64 keys, at least 128) chosen by a time model: workgroups run
// in rounds of the device's resident slots (two per compute unit), a round costs one
// 64-key block per block of its ranges, and every split adds an fp32 partial (m, l, O) per
// query row that is written and read back once; measured on MI355X, a 64-key block round
// takes about as long as moving 11 MB of partials.
AttnPlan attn_plan(int S, int n_cap, int Hq, int Hkv, int P_max, int D) {
  AttnPlan p;
  const int g = Hq / Hkv;
  const int M = g * n_cap;
  const int T = P_max + n_cap;
  const int G = (M + 31) / 32;
  p.n_mtiles = (G + dtv::kWaves - 1) / dtv::kWaves;
  p.mcap = G * 32;
  const int min_keys = 128;
  const long tiles = static_cast<long>(S) * Hkv * p.n_mtiles;
  const long slots = 2L * device_cus();
  const double partial_bytes = 2.0 * S * Hkv * static_cast<double>(p.mcap) * (D + 2) * 4.0;   // per split
  const double bytes_per_block = 11.0e6;
  int max_split = (T + min_keys - 1) / min_keys;
  if (max_split > dtv::kAttnMaxSplit) max_split = dtv::kAttnMaxSplit;
  // measured on MI355X: a workgroup streaming more than 48 blocks (3072 keys) loses more
  // than the extra round and partials cost (c5, 8257 keys: 2 splits 260 us, 3 splits 236 us)
  const int max_kps = 48 * 64;
  int best_kps = (T + 63) / 64 * 64;
  double best_cost = 1e300;
  for (int want = 1; want <= max_split; ++want) {
    int kps = (T + want - 1) / want;
    kps = (kps + 63) / 64 * 64;
    if (kps > max_kps && want < max_split) continue;
    const int ns = (T + kps - 1) / kps;
    const long rounds = (tiles * ns + slots - 1) / slots;
    const double cost = static_cast<double>(rounds) * (kps / 64) + (ns > 1 ? ns * partial_bytes / bytes_per_block : 0.0);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best_kps = kps;
    }
  }
  p.kps = best_kps;
  p.n_split = (T + best_kps - 1) / best_kps;
  return p;
}

struct AttnLayout {
  dtv::WsHeader* hdr;
  float* part_o;
  float* part_ml;
  size_t bytes;
};
AttnLayout attn_layout(void* ws, int S, int Hkv, int D, const AttnPlan& p) {
  const size_t np = p.n_split > 1 ? static_cast<size_t>(S) * Hkv * p.n_split * p.mcap : 0;
  Carver c(ws);
  AttnLayout L;
  L.hdr = c.take<dtv::WsHeader>(1);
  L.part_o = c.take<float>(np * D);
  L.part_ml = c.take<float>(np * 2);
  L.bytes = c.off;
  return L;
}

struct VerifyLayout {
  dtv::WsHeader* hdr;
  unsigned long long* cbest;
  size_t bytes;
};
VerifyLayout verify_layout(void* ws, int S, int n_cap, int nch) {
  Carver c(ws);
  VerifyLayout L;
  L.hdr = c.take<dtv::WsHeader>(1);
  L.cbest = c.take<unsigned long long>(static_cast<size_t>(S) * n_cap * nch);
  L.bytes = c.off;
  return L;
}

struct SampleLayout {
  dtv::WsHeader* hdr;
  double* xch;
  double* pbuf;
  unsigned* done;
  size_t bytes;
};
// Exchange slots of the walk per sequence: one per visited node (its normalisers), one per
// rejection, one for a bonus draw whose slice masses are not known from an earlier exchange.
int sample_max_pass(int n_cap) { return 2 * n_cap + 1; }

SampleLayout sample_layout(void* ws, int S, int n_cap, int V, int dtype) {
  (void)dtype;
  Carver c(ws);
  SampleLayout L;
  L.hdr = c.take<dtv::WsHeader>(1);
  L.xch = c.take<double>(static_cast<size_t>(S) * sample_max_pass(n_cap) * dtv::kXchStride);
  L.pbuf = c.take<double>(static_cast<size_t>(S) * 3 * V);   // two residuals and q per sequence
  L.done = c.take<unsigned>(S);
  L.bytes = c.off;
  return L;
}

// How the rejection-sampling walk divides its work, checked against every buffer it uses.
// `resident` = walk workgroups the device holds at once; `vec` = rows walked in 16-byte
// units. The walk of a sequence runs in G workgroups; workgroup gi owns units
// [units*gi/G, units*(gi+1)/G), so no slice exceeds ceil(units/G) units. A slice of at most
// kWalkSlice entries keeps its two residuals and q in shared memory (entries indexed from
// the slice's first), a larger one in the sequence's 3*V workspace entries (indexed by
// entry < V). Exchange slots: one per visited node (at most n_cap), one per rejection (at
// most n_cap - 1) and one for a bonus draw, each holding 4 values per workgroup.
struct WalkPlan {
  int G, units, slice_units, slice_entries, in_lds, xch_slots;
  long pbuf_entries;
};
int walk_plan(int S, int n_cap, int V, int dtype, int resident, int vec, WalkPlan* p) {
  REQUIRE(S >= 1 && n_cap >= 1 && V >= 1 && dtype_ok(dtype), DTV_EINVAL, "S=%d n_cap=%d V=%d dtype=%d", S,
          n_cap, V, dtype);
  REQUIRE(n_cap <= dtv::kSampleMaxNodes, DTV_EUNSUPPORTED, "n_cap=%d exceeds the walk's %d slots", n_cap,
          dtv::kSampleMaxNodes);
  REQUIRE(resident >= S, DTV_EUNSUPPORTED, "S=%d sequences exceed the %d co-resident walk workgroups", S,
          resident);
  const int VEC = dtype == DTV_BF16 ? 8 : 4;
  REQUIRE(!vec || V % VEC == 0, DTV_EINVAL, "16-byte units need V=%d to be a multiple of %d", V, VEC);
  int G = (resident < 256 ? resident : 256) / S;
  if (G > dtv::kSampleMaxGroup) G = dtv::kSampleMaxGroup;
  if (G < 1) G = 1;
  p->G = G;
  p->units = vec ? V / VEC : V;
  p->slice_units = (p->units + G - 1) / G;
  p->slice_entries = p->slice_units * (vec ? VEC : 1);
  p->in_lds = p->slice_entries <= dtv::kWalkSlice ? 1 : 0;
  p->xch_slots = sample_max_pass(n_cap);
  p->pbuf_entries = 3L * V;
  // the bounds the kernel relies on
  REQUIRE(4 * G <= dtv::kXchStride && G + 2 <= dtv::kXchStride, DTV_EUNSUPPORTED, "G=%d exceeds an exchange slot",
          G);
  REQUIRE(static_cast<long>(p->units) * (vec ? VEC : 1) <= V, DTV_EUNSUPPORTED, "units exceed the row");
  REQUIRE(p->in_lds || static_cast<long>(p->slice_entries) <= V, DTV_EUNSUPPORTED,
          "a slice of %d entries exceeds the %d-entry workspace rows", p->slice_entries, V);
  return DTV_OK;
}

}  // namespace

extern "C" {

int dtv_tree_verify_sample_plan(int32_t S, int32_t n_cap, int32_t V, int dtype, int32_t resident_blocks,
                                int32_t vec, int64_t* plan_h) {
  REQUIRE(plan_h != nullptr, DTV_EINVAL, "plan_h is NULL");
  WalkPlan p;
  const int rc = walk_plan(S, n_cap, V, dtype, resident_blocks, vec, &p);
  if (rc) return rc;
  plan_h[0] = p.G;
  plan_h[1] = p.units;
  plan_h[2] = p.slice_units;
  plan_h[3] = p.slice_entries;
  plan_h[4] = p.in_lds;
  plan_h[5] = p.xch_slots;
  plan_h[6] = p.pbuf_entries;
  return DTV_OK;
}

const char* dtv_status_str(int status) {
  switch (status) {
    case DTV_OK: return "ok";
    case DTV_EINVAL: return "invalid argument";
    case DTV_EUNSUPPORTED: return "unsupported";
    case DTV_ECAPACITY: return "capacity exceeded";
    case DTV_EWORKSPACE: return "workspace too small";
    case DTV_EHIP: return "HIP error";
    case DTV_EDEVICE: return "device-side error";
    default: return "unknown status";
  }
}

const char* dtv_last_error(void) { return g_msg; }

int dtv_ws_status(const void* ws, void* stream) {
  REQUIRE(ws != nullptr, DTV_EINVAL, "workspace is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess)
    return fail(DTV_EHIP, "stream synchronize failed: %s", hipGetErrorString(hipGetLastError()));
  int err = 0;
  if (hipMemcpy(&err, ws, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(DTV_EHIP, "reading the workspace status failed");
  if (err != 0) {
    int zero = 0;
    if (hipMemcpy(const_cast<void*>(ws), &zero, sizeof(int), hipMemcpyHostToDevice) != hipSuccess)
      return fail(DTV_EHIP, "clearing the workspace status failed");
  }
  switch (err) {
    case dtv::kErrNone: return DTV_OK;
    case dtv::kErrCapacity: return fail(DTV_ECAPACITY, "a kernel ran out of capacity");
    case dtv::kErrTimeout: return fail(DTV_EDEVICE, "a bounded grid-wide wait timed out");
    case dtv::kErrBadTree: return fail(DTV_EDEVICE, "a parent is not an earlier slot");
    case dtv::kErrBadRow:
      return fail(DTV_EDEVICE, "a node's row lies outside the logit table (0 <= row < R), its token outside "
                               "the vocabulary (0 <= token < V) or its depth outside the tree");
    default: return fail(DTV_EDEVICE, "device error %d", err);
  }
}

// ---------------------------------------------------------------- row statistics

size_t dtv_row_stats_ws_bytes(int32_t R, int32_t V, int32_t K, int dtype) {
  if (R < 1 || V < 1 || K < 0 || !dtype_ok(dtype)) return 0;
  return row_stats_layout(nullptr, R, V, K, dtype).bytes;
}

int dtv_row_stats(const void* table, int dtype, int32_t R, int32_t V, const int32_t* row_idx,
                  int32_t K, float* maxv, int32_t* argmax, double* lse, int32_t* topk,
                  void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(table != nullptr, DTV_EINVAL, "table is NULL");
  REQUIRE(dtype_ok(dtype), DTV_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(R >= 1 && V >= 1, DTV_EINVAL, "R=%d V=%d", R, V);
  REQUIRE(K >= 0 && K <= 1024 && K <= V, DTV_EUNSUPPORTED, "K=%d must be in 0..min(V,1024)", K);
  REQUIRE(K == 0 || topk != nullptr, DTV_EINVAL, "topk is NULL while K > 0");
  REQUIRE(nch_of(V, dtype) <= 64 && static_cast<long>(nch_of(V, dtype)) * K <= 8192, DTV_EUNSUPPORTED,
          "V=%d with K=%d exceeds the merge capacity (chunks * K <= 8192, chunks <= 64)", V, K);
  const RowStatsLayout L = row_stats_layout(ws, R, V, K, dtype);
  REQUIRE(ws != nullptr && ws_bytes >= L.bytes, DTV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, L.bytes);
  dtv::RowStatsArgs a;
  a.table = table;
  a.R = R;
  a.V = V;
  a.K = K;
  a.nch = nch_of(V, dtype);
  a.row_idx = row_idx;
  a.maxv = maxv;
  a.argmax = argmax;
  a.lse = lse;
  a.topk = topk;
  a.hdr = L.hdr;
  a.st = L.st;
  a.cval = L.cval;
  a.cidx = L.cidx;
  a.tickets = L.tickets;
  a.mval = L.mval;
  return launched(dtv::launch_row_stats(a, dtype, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- given trees

size_t dtv_tree_build_given_ws_bytes(int32_t S) { return S >= 1 ? up(sizeof(dtv::WsHeader)) : 0; }

int dtv_tree_build_given(const dtv_tree* tree, int32_t S, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_tree(tree);
  if (rc) return rc;
  REQUIRE(S >= 1, DTV_EINVAL, "S=%d", S);
  REQUIRE(ws != nullptr && ws_bytes >= dtv_tree_build_given_ws_bytes(S), DTV_EWORKSPACE, "workspace too small");
  return launched(dtv::launch_given(tree_args(tree), S, static_cast<dtv::WsHeader*>(ws),
                                    static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- TALON

size_t dtv_tree_build_talon_ws_bytes(int32_t S, int32_t B, int32_t K, int32_t V, int dtype) {
  if (S < 1 || B < 1 || K < 1 || V < 1 || !dtype_ok(dtype)) return 0;
  return talon_layout(nullptr, S, B, K, V, dtype).bytes;
}

int dtv_tree_build_talon(const dtv_tree* tree, int32_t S, const void* draft, int dtype, int32_t R,
                         int32_t V, int32_t B, int32_t K, double alpha, void* ws, size_t ws_bytes,
                         void* stream) {
  int rc = check_tree(tree);
  if (rc) return rc;
  REQUIRE(draft != nullptr, DTV_EINVAL, "draft is NULL");
  REQUIRE(dtype_ok(dtype), DTV_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(S >= 1, DTV_EINVAL, "S=%d", S);
  REQUIRE(V >= 1, DTV_EINVAL, "V=%d", V);
  REQUIRE(B >= 1, DTV_EINVAL, "B=%d", B);
  REQUIRE(B + 1 <= tree->n_cap, DTV_ECAPACITY, "B+1=%d exceeds n_cap=%d", B + 1, tree->n_cap);
  REQUIRE(R >= B + 1, DTV_EINVAL, "R=%d rows cannot key %d slots", R, B + 1);
  REQUIRE(K >= 1 && K <= 64, DTV_EUNSUPPORTED, "K=%d outside 1..64", K);
  REQUIRE(static_cast<long>(B) * K <= 4096, DTV_EUNSUPPORTED, "B*K=%ld exceeds 4096", static_cast<long>(B) * K);
  REQUIRE(nch_of(V, dtype) <= 32 && nch_of(V, dtype) * K <= 2048, DTV_EUNSUPPORTED,
          "V=%d with K=%d exceeds the merge capacity (chunks * K <= 2048, chunks <= 32)", V, K);
  REQUIRE(alpha >= 0.0 && alpha <= 1.0, DTV_EINVAL, "alpha=%g outside [0,1]", alpha);
  const TalonLayout L = talon_layout(ws, S, B, K, V, dtype);
  REQUIRE(ws != nullptr && ws_bytes >= L.bytes, DTV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, L.bytes);
  dtv::TalonArgs a;
  memset(&a, 0, sizeof(a));
  a.Wr = B;
  a.tree = tree_args(tree);
  a.draft = draft;
  a.R = R;
  a.V = V;
  a.S = S;
  a.B = B;
  a.K = K;
  a.nch = nch_of(V, dtype);
  a.log_alpha = alpha > 0.0 ? log(alpha) : -INFINITY;
  a.hdr = L.hdr;
  a.st = L.st;
  a.cval = L.cval;
  a.cidx = L.cidx;
  a.tickets = L.tickets;
  a.rlse = L.rlse;
  a.rv = L.rv;
  a.ri = L.ri;
  a.rcnt = L.rcnt;
  return launched(dtv::launch_talon(a, dtype == DTV_BF16 ? 1 : 0, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- GOOSE spine

size_t dtv_tree_build_spine_ws_bytes(int32_t S, int32_t F, int32_t max_width, int32_t V, int dtype) {
  if (S < 1 || F < 1 || max_width < 0 || V < 1 || !dtype_ok(dtype)) return 0;
  return spine_layout(nullptr, S, F, max_width + 1, V, dtype).bytes;
}

int dtv_tree_build_spine(const dtv_tree* tree, int32_t S, const int32_t* spine, int32_t n_spine,
                         const int32_t* widths_h, int32_t F, const void* draft, int dtype, int32_t R,
                         int32_t V, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_tree(tree);
  if (rc) return rc;
  REQUIRE(draft != nullptr && widths_h != nullptr, DTV_EINVAL, "draft or widths_h is NULL");
  REQUIRE(n_spine == 0 || spine != nullptr, DTV_EINVAL, "spine is NULL");
  REQUIRE(dtype_ok(dtype), DTV_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(S >= 1 && n_spine >= 0 && V >= 1, DTV_EINVAL, "S=%d n_spine=%d V=%d", S, n_spine, V);
  REQUIRE(F >= 1 && F <= dtv::kSpineMaxForks, DTV_EUNSUPPORTED, "F=%d outside 1..%d", F, dtv::kSpineMaxForks);
  REQUIRE(F <= n_spine + 1, DTV_EINVAL, "forks must be the root or spine nodes (F=%d, n_spine=%d)", F, n_spine);
  int total = 0, wmax = 0;
  for (int f = 0; f < F; ++f) {
    REQUIRE(widths_h[f] >= 0 && widths_h[f] <= 64, DTV_EUNSUPPORTED, "width[%d]=%d outside 0..64", f, widths_h[f]);
    REQUIRE(widths_h[f] + (f < n_spine ? 1 : 0) <= V, DTV_EINVAL, "width[%d]=%d needs a larger vocabulary", f,
            widths_h[f]);
    total += widths_h[f];
    wmax = widths_h[f] > wmax ? widths_h[f] : wmax;
  }
  const int N = 1 + n_spine + total;
  REQUIRE(N <= tree->n_cap, DTV_ECAPACITY, "tree of %d nodes exceeds n_cap=%d", N, tree->n_cap);
  REQUIRE(R >= F, DTV_EINVAL, "R=%d rows cannot key %d forks", R, F);
  const int K = wmax + 1;
  REQUIRE(nch_of(V, dtype) <= 32 && nch_of(V, dtype) * K <= 2048, DTV_EUNSUPPORTED,
          "V=%d with width %d exceeds the merge capacity", V, wmax);
  const SpineLayout L = spine_layout(ws, S, F, K, V, dtype);
  REQUIRE(ws != nullptr && ws_bytes >= L.bytes, DTV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, L.bytes);
  dtv::SpineArgs a;
  memset(&a, 0, sizeof(a));
  a.tree = tree_args(tree);
  a.spine = spine;
  a.draft = draft;
  a.R = R;
  a.V = V;
  a.S = S;
  a.n_spine = n_spine;
  a.F = F;
  a.K = K;
  a.nch = nch_of(V, dtype);
  a.n_nodes = N;
  int off = 0;
  for (int f = 0; f < F; ++f) {
    a.width[f] = widths_h[f];
    a.offset[f] = off;
    off += widths_h[f];
  }
  a.hdr = L.hdr;
  a.st = L.st;
  a.cval = L.cval;
  a.cidx = L.cidx;
  a.tickets = L.tickets;
  a.rlse = L.rlse;
  a.rv = L.rv;
  a.ri = L.ri;
  return launched(dtv::launch_spine(a, dtype == DTV_BF16 ? 1 : 0, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- OPT-Tree

}  // extern "C"

// The frontier width of OPT-Tree's layer l follows from n and V alone: layer 1 expands the
// root; layer l keeps min(n, W_l * min(n, V)) nodes, which are layer l+1's frontier.
static long opt_frontier_width(int layer, int n, int V) {
  long W = 1;
  const long per_row = n < V ? n : V;
  for (int l = 1; l < layer; ++l) {
    long kept = W * per_row;
    W = kept > n ? n : kept;
  }
  return W;
}

// Configures and launches OPT-Tree's layer `layer` on the rows `a` points at.
static int opt_launch_layer(dtv::OptArgs& a, int layer, int dtype, hipStream_t st) {
  const int n = a.n, V = a.V, nch = a.nch;
  const long W = opt_frontier_width(layer, n, V);
  const long per_row = n < V ? n : V;
  a.layer = layer;
  a.W = static_cast<int>(W);
  const long need = (n + W - 1) / W;                 // reported per row so that W*m >= n
  long K = need > 8 ? need : 8;
  if (K > per_row) K = per_row;
  a.K = static_cast<int>(K);
  long Kc = (K + nch - 1) / nch;
  if (Kc < 2) Kc = 2;
  if (Kc > K) Kc = K;
  a.Kc = static_cast<int>(Kc);
  const int dt = dtype == DTV_BF16 ? 1 : 0;
  a.Kw = layer == 1 ? dtv::opt_root_wave_quota(V, n, dt) : 0;
  if (layer == 1 && (a.Kw > 0 || dtv::opt_root_one_workgroup(V, n, dt)))
    return dtv::launch_opt_root(a, dt, st);   // the root layer in one launch
  return dtv::launch_opt_layer(a, dtype == DTV_BF16 ? 1 : 0, st);
}

extern "C" {

size_t dtv_tree_build_opt_ws_bytes(int32_t S, int32_t n, int32_t V, int32_t max_layers, int dtype) {
  if (S < 1 || n < 1 || V < 1 || max_layers < 1 || !dtype_ok(dtype)) return 0;
  return opt_layout(nullptr, S, n, V, max_layers, dtype).bytes;
}

int dtv_tree_build_opt(const dtv_tree* tree, int32_t S, const void* draft, int dtype, int32_t R, int32_t V,
                       int32_t n, double delta, int32_t max_layers, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_tree(tree);
  if (rc) return rc;
  REQUIRE(draft != nullptr, DTV_EINVAL, "draft is NULL");
  REQUIRE(dtype_ok(dtype), DTV_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(S >= 1 && V >= 1, DTV_EINVAL, "S=%d V=%d", S, V);
  REQUIRE(n >= 1 && n + 1 <= tree->n_cap, DTV_ECAPACITY, "n+1=%d exceeds n_cap=%d", n + 1, tree->n_cap);
  REQUIRE(n <= 1023, DTV_EUNSUPPORTED, "n=%d exceeds 1023", n);
  REQUIRE(V <= (1 << 22), DTV_EUNSUPPORTED, "V=%d exceeds 4194304", V);
  REQUIRE(max_layers >= 1 && max_layers <= 64, DTV_EUNSUPPORTED, "max_layers=%d outside 1..64", max_layers);
  REQUIRE(delta >= 0.0 && isfinite(delta), DTV_EINVAL, "delta=%g", delta);
  REQUIRE(static_cast<long>(R) >= 1 + static_cast<long>(max_layers - 1) * n, DTV_EINVAL,
          "R=%d rows cannot key %d layers of %d nodes", R, max_layers, n);
  const int nch = nch_of(V, dtype);
  const int Kmax = n < V ? n : V;
  REQUIRE(nch <= 64 && static_cast<long>(nch) * Kmax <= 8192, DTV_EUNSUPPORTED,
          "V=%d with n=%d exceeds the merge capacity", V, n);
  const OptLayout L = opt_layout(ws, S, n, V, max_layers, dtype);
  REQUIRE(ws != nullptr && ws_bytes >= L.bytes, DTV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, L.bytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  dtv::OptArgs a;
  memset(&a, 0, sizeof(a));
  a.tree = tree_args(tree);
  a.draft = draft;
  a.R = R;
  a.V = V;
  a.S = S;
  a.n = n;
  a.nch = nch;
  a.max_layers = max_layers;
  a.delta = delta;
  a.Wcap = n;
  a.hdr = L.hdr;
  a.st = L.st;
  a.cmax = L.cmax;
  a.cval = L.cval;
  a.cidx = L.cidx;
  a.tickets = L.tickets;
  a.rlse = L.rlse;
  a.rv = L.rv;
  a.ri = L.ri;
  a.rcnt = L.rcnt;
  a.lo = L.lo;
  a.ccount = L.ccount;
  a.ccap = kOptCandCap;
  a.cand = static_cast<dtv::OptCand*>(L.cand);
  a.lscore = L.lscore;
  a.lparent = L.lparent;
  a.ltoken = L.ltoken;
  a.bscore = L.bscore;
  a.blayer = L.blayer;
  a.bpos = L.bpos;
  a.bcount = L.bcount;
  a.Eprev = L.Eprev;
  a.done = L.done;
  a.nlayers = L.nlayers;
  a.row_base = -1;
  // the one-workgroup root launch sets the per-call state itself
  if (!dtv::opt_root_one_workgroup(V, n, dtype == DTV_BF16 ? 1 : 0) && dtv::launch_opt_init(a, st))
    return launched(-1);
  for (int layer = 1; layer <= max_layers; ++layer) {
    if (opt_launch_layer(a, layer, dtype, st)) return launched(-1);
  }
  return launched(dtv::launch_opt_finalize(a, st));
}

// ---------------------------------------------------------------- layer-by-layer builds

static int layered_check(const dtv_tree* tree, int32_t S, const dtv_build_params* p, int dtype, int32_t V,
                         const int32_t* W, const int32_t* done) {
  int rc = check_tree(tree);
  if (rc) return rc;
  REQUIRE(p != nullptr && W != nullptr && done != nullptr, DTV_EINVAL, "params, W or done is NULL");
  REQUIRE(dtype_ok(dtype), DTV_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(S >= 1 && V >= 1, DTV_EINVAL, "S=%d V=%d", S, V);
  if (p->mode == DTV_BUILD_TALON) {
    REQUIRE(p->B >= 1, DTV_EINVAL, "B=%d", p->B);
    REQUIRE(p->B + 1 <= tree->n_cap, DTV_ECAPACITY, "B+1=%d exceeds n_cap=%d", p->B + 1, tree->n_cap);
    REQUIRE(p->K >= 1 && p->K <= 64, DTV_EUNSUPPORTED, "K=%d outside 1..64", p->K);
    REQUIRE(static_cast<long>(p->B) * p->K <= 4096, DTV_EUNSUPPORTED, "B*K=%ld exceeds 4096",
            static_cast<long>(p->B) * p->K);
    REQUIRE(nch_of(V, dtype) <= 32 && nch_of(V, dtype) * p->K <= 2048, DTV_EUNSUPPORTED,
            "V=%d with K=%d exceeds the merge capacity (chunks * K <= 2048, chunks <= 32)", V, p->K);
    REQUIRE(p->alpha >= 0.0 && p->alpha <= 1.0, DTV_EINVAL, "alpha=%g outside [0,1]", p->alpha);
    return DTV_OK;
  }
  if (p->mode == DTV_BUILD_OPT) {
    const int n = p->n;
    REQUIRE(n >= 1 && n + 1 <= tree->n_cap, DTV_ECAPACITY, "n+1=%d exceeds n_cap=%d", n + 1, tree->n_cap);
    REQUIRE(n <= 1023, DTV_EUNSUPPORTED, "n=%d exceeds 1023", n);
    REQUIRE(V <= (1 << 22), DTV_EUNSUPPORTED, "V=%d exceeds 4194304", V);
    REQUIRE(p->max_layers >= 1 && p->max_layers <= 64, DTV_EUNSUPPORTED, "max_layers=%d outside 1..64",
            p->max_layers);
    REQUIRE(p->delta >= 0.0 && isfinite(p->delta), DTV_EINVAL, "delta=%g", p->delta);
    const int Kmax = n < V ? n : V;
    REQUIRE(nch_of(V, dtype) <= 64 && static_cast<long>(nch_of(V, dtype)) * Kmax <= 8192, DTV_EUNSUPPORTED,
            "V=%d with n=%d exceeds the merge capacity", V, n);
    return DTV_OK;
  }
  return fail(DTV_EINVAL, "build mode %d (DTV_BUILD_TALON or DTV_BUILD_OPT)", p->mode);
}

// TALON's layered workspace: the row lists of B rows, then the loop state [S][8].
static size_t talon_layered_bytes(int S, const dtv_build_params* p, int V, int dtype) {
  return talon_layout(nullptr, S, p->B, p->K, V, dtype).bytes + up(static_cast<size_t>(S) * 8 * sizeof(int));
}

size_t dtv_tree_build_layered_ws_bytes(const dtv_build_params* p, int32_t S, int32_t V, int dtype) {
  if (p == nullptr || S < 1 || V < 1 || !dtype_ok(dtype)) return 0;
  if (p->mode == DTV_BUILD_TALON && p->B >= 1 && p->K >= 1) return talon_layered_bytes(S, p, V, dtype);
  if (p->mode == DTV_BUILD_OPT && p->n >= 1 && p->max_layers >= 1)
    return opt_layout(nullptr, S, p->n, V, p->max_layers, dtype).bytes;
  return 0;
}

// One layer of a layered build: layer 1 from the root rows ([S][V]), layer l >= 2 from the
// frontier rows ([S][W_cap][V]).
static int layered_layer(const dtv_tree* tree, int32_t S, const dtv_build_params* p, int32_t layer,
                         const void* rows, int32_t W_cap, int dtype, int32_t V, int32_t* W, int32_t* done,
                         void* ws, size_t ws_bytes, void* stream) {
  int rc = layered_check(tree, S, p, dtype, V, W, done);
  if (rc) return rc;
  REQUIRE(rows != nullptr, DTV_EINVAL, "%s is NULL", layer == 1 ? "root_logits" : "frontier_logits");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = dtype == DTV_BF16 ? 1 : 0;
  if (p->mode == DTV_BUILD_TALON) {
    REQUIRE(layer == 1 || (W_cap >= 1 && W_cap <= p->B), DTV_EINVAL,
            "W_cap=%d: a frontier holds 1..B=%d nodes", W_cap, p->B);
    const size_t need = talon_layered_bytes(S, p, V, dtype);
    REQUIRE(ws != nullptr && ws_bytes >= need, DTV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, need);
    const TalonLayout L = talon_layout(ws, S, p->B, p->K, V, dtype);
    dtv::TalonArgs a;
    memset(&a, 0, sizeof(a));
    a.tree = tree_args(tree);
    a.draft = rows;
    a.R = layer == 1 ? 1 : W_cap;
    a.Wr = a.R;
    a.V = V;
    a.S = S;
    a.B = p->B;
    a.K = p->K;
    a.nch = nch_of(V, dtype);
    a.log_alpha = p->alpha > 0.0 ? log(p->alpha) : -INFINITY;
    a.hdr = L.hdr;
    a.st = L.st;
    a.cval = L.cval;
    a.cidx = L.cidx;
    a.tickets = L.tickets;
    a.rlse = L.rlse;
    a.rv = L.rv;
    a.ri = L.ri;
    a.rcnt = L.rcnt;
    a.layer = layer;
    a.state = reinterpret_cast<int*>(static_cast<char*>(ws) + L.bytes);
    a.w_out = W;
    a.done_out = done;
    return launched(dtv::launch_talon_layer(a, dt, st));
  }
  const int n = p->n;
  REQUIRE(layer <= p->max_layers, DTV_EINVAL, "layer %d beyond max_layers=%d", layer, p->max_layers);
  const long Wl = opt_frontier_width(layer, n, V);
  REQUIRE(layer == 1 || W_cap >= Wl, DTV_EINVAL, "layer %d's frontier has %ld nodes; frontier_logits holds %d rows",
          layer, Wl, W_cap);
  const OptLayout L = opt_layout(ws, S, n, V, p->max_layers, dtype);
  REQUIRE(ws != nullptr && ws_bytes >= L.bytes, DTV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, L.bytes);
  dtv::OptArgs a;
  memset(&a, 0, sizeof(a));
  a.tree = tree_args(tree);
  a.draft = rows;
  a.R = layer == 1 ? 1 : W_cap;
  a.V = V;
  a.S = S;
  a.n = n;
  a.nch = nch_of(V, dtype);
  a.max_layers = p->max_layers;
  a.delta = p->delta;
  a.Wcap = n;
  a.hdr = L.hdr;
  a.st = L.st;
  a.cmax = L.cmax;
  a.cval = L.cval;
  a.cidx = L.cidx;
  a.tickets = L.tickets;
  a.rlse = L.rlse;
  a.rv = L.rv;
  a.ri = L.ri;
  a.rcnt = L.rcnt;
  a.lo = L.lo;
  a.ccount = L.ccount;
  a.ccap = kOptCandCap;
  a.cand = static_cast<dtv::OptCand*>(L.cand);
  a.lscore = L.lscore;
  a.lparent = L.lparent;
  a.ltoken = L.ltoken;
  a.bscore = L.bscore;
  a.blayer = L.blayer;
  a.bpos = L.bpos;
  a.bcount = L.bcount;
  a.Eprev = L.Eprev;
  a.done = L.done;
  a.nlayers = L.nlayers;
  a.row_base = 0;
  a.fin = L.fin;
  a.w_out = W;
  a.done_out = done;
  a.w_next = static_cast<int>(opt_frontier_width(layer + 1, n, V));
  if (layer == 1 && dtv::launch_opt_init(a, st)) return launched(-1);
  if (opt_launch_layer(a, layer, dtype, st)) return launched(-1);
  if (dtv::launch_opt_report(a, st)) return launched(-1);
  return launched(dtv::launch_opt_finalize(a, st));
}

int dtv_tree_build_begin(const dtv_tree* tree, int32_t S, const dtv_build_params* params, const void* root_logits,
                         int dtype, int32_t V, int32_t* W, int32_t* done, void* ws, size_t ws_bytes, void* stream) {
  return layered_layer(tree, S, params, 1, root_logits, 1, dtype, V, W, done, ws, ws_bytes, stream);
}

int dtv_tree_build_step(const dtv_tree* tree, int32_t S, const dtv_build_params* params, int32_t layer,
                        const void* frontier_logits, int32_t W_cap, int dtype, int32_t V, int32_t* W, int32_t* done,
                        void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(layer >= 2, DTV_EINVAL, "layer %d: layer 1 is dtv_tree_build_begin's", layer);
  return layered_layer(tree, S, params, layer, frontier_logits, W_cap, dtype, V, W, done, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- attention

size_t dtv_tree_attn_ws_bytes(int32_t S, int32_t n_cap, int32_t Hq, int32_t Hkv, int32_t D,
                              int32_t P_max, int dtype) {
  if (S < 1 || n_cap < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || P_max < 0 || !dtype_ok(dtype)) return 0;
  if (dtype != DTV_BF16) return up(sizeof(dtv::WsHeader));
  return attn_layout(nullptr, S, Hkv, D, attn_plan(S, n_cap, Hq, Hkv, P_max, D)).bytes;
}

}  // extern "C"

// The checks, workspace layout and launches of tree attention, on a workspace `ws` of
// `ws_bytes` (a caller's buffer, or the no-allocation variant's static array). `ws_cap`
// (0: none) is the most any size may need from a fixed workspace; larger sizes are refused
// with DTV_ECAPACITY before launch. With `check_only` the call stops after the argument
// checks (ws may then be NULL) and launches nothing.
static int attn_impl(const void* q, const void* k, const void* v, const int32_t* P, int32_t P_cap,
                     int32_t P_max, const dtv_tree* tree, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                     int dtype, float scale, void* o, void* ws, size_t ws_bytes, size_t ws_cap,
                     bool check_only, void* stream) {
  int rc = check_tree(tree);
  if (rc) return rc;
  REQUIRE(q && k && v && P && o, DTV_EINVAL, "q, k, v, P or o is NULL");
  REQUIRE(dtype_ok(dtype), DTV_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(S >= 1 && Hq >= 1 && Hkv >= 1, DTV_EINVAL, "S=%d Hq=%d Hkv=%d", S, Hq, Hkv);
  REQUIRE(Hq % Hkv == 0, DTV_EINVAL, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  REQUIRE(P_max >= 0 && P_cap >= P_max + tree->n_cap, DTV_ECAPACITY,
          "P_cap=%d cannot hold P_max=%d plus %d tree slots", P_cap, P_max, tree->n_cap);
  REQUIRE(scale > 0.f && isfinite(scale), DTV_EINVAL, "scale=%g", scale);
  if (dtype == DTV_BF16) {
    REQUIRE(D == 64 || D == 128, DTV_EUNSUPPORTED, "bf16 attention supports D=64 or 128, got %d", D);
  } else {
    REQUIRE(D >= 4 && D <= 128 && D % 4 == 0, DTV_EUNSUPPORTED, "fp32 attention needs D%%4==0, D<=128, got %d", D);
    REQUIRE(P_max + tree->n_cap <= 16384, DTV_EUNSUPPORTED, "fp32 attention supports at most 16384 keys");
  }
  const AttnPlan plan = attn_plan(S, tree->n_cap, Hq, Hkv, P_max, D);
  size_t need = dtv_tree_attn_ws_bytes(S, tree->n_cap, Hq, Hkv, D, P_max, dtype);
  REQUIRE(ws_cap == 0 || need <= ws_cap, DTV_ECAPACITY,
          "these sizes need %zu bytes of key-split partials and status, more than the %zu-byte static scratch "
          "array; call dtv_tree_attn with a workspace",
          need, ws_cap);
  if (check_only) return DTV_OK;
  REQUIRE(ws != nullptr && ws_bytes >= need, DTV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  dtv::AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.P = P;
  a.P_cap = P_cap;
  a.n_nodes = tree->n_nodes;
  a.anc = reinterpret_cast<const uint64_t*>(tree->anc);
  a.n_cap = tree->n_cap;
  a.words = tree->words;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.g = Hq / Hkv;
  a.scale = scale;
  a.n_mtiles = plan.n_mtiles;
  a.n_split = plan.n_split;
  a.kps = plan.kps;
  a.mcap = plan.mcap;
  if (dtype == DTV_BF16) {
    const AttnLayout L = attn_layout(ws, S, Hkv, D, plan);
    a.part_o = L.part_o;
    a.part_ml = L.part_ml;
    a.hdr = L.hdr;
  } else {
    a.hdr = static_cast<dtv::WsHeader*>(ws);
  }
  return launched(dtv::launch_attn(a, dtype == DTV_BF16 ? 1 : 0, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- attention without a workspace
//
// The scratch of dtv_tree_attn_noalloc: the 256-byte status header and the key-split
// partials, in a static array that every GPU the library runs on holds until the process
// ends. Host code never passes the array's name to a kernel (on the host it is only a
// stand-in): the device address of each GPU's copy comes from hipGetSymbolAddress, called
// once per device with that device current, and is the only address used.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on its first use).
static int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DTV_EHIP, "no current device (or device index %d beyond %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(DTV_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DTV_OK;
}

extern "C" {

int dtv_tree_attn(const void* q, const void* k, const void* v, const int32_t* P, int32_t P_cap,
                  int32_t P_max, const dtv_tree* tree, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                  int dtype, float scale, void* o, void* ws, size_t ws_bytes, void* stream) {
  return attn_impl(q, k, v, P, P_cap, P_max, tree, S, Hq, Hkv, D, dtype, scale, o, ws, ws_bytes, 0, false, stream);
}

int dtv_tree_attn_noalloc(const void* q, const void* k, const void* v, const int32_t* P, int32_t P_cap,
                          int32_t P_max, const dtv_tree* tree, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                          int dtype, float scale, void* o, void* stream) {
  // every argument check, the array's capacity included, before any device call
  int rc = attn_impl(q, k, v, P, P_cap, P_max, tree, S, Hq, Hkv, D, dtype, scale, o, nullptr, 0,
                     kNoAllocScratchBytes, true, stream);
  if (rc) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return attn_impl(q, k, v, P, P_cap, P_max, tree, S, Hq, Hkv, D, dtype, scale, o, ws, kNoAllocScratchBytes,
                   kNoAllocScratchBytes, false, stream);
}

// ---------------------------------------------------------------- greedy verification

size_t dtv_tree_verify_greedy_ws_bytes(int32_t S, int32_t n_cap, int32_t V, int dtype) {
  if (S < 1 || n_cap < 1 || V < 1 || !dtype_ok(dtype)) return 0;
  return verify_layout(nullptr, S, n_cap, nch_of(V, dtype)).bytes;
}

// The compaction view of a fused verification (kv null: no compaction). A status code.
static int kv_view(const dtv_kv_cache* kv, int dtype, const dtv_tree* tree, dtv::KvCompactView* out) {
  memset(out, 0, sizeof(*out));
  if (kv == nullptr) return DTV_OK;
  REQUIRE(kv->k && kv->v && kv->P && kv->P_new, DTV_EINVAL, "kv: k, v, P or P_new is NULL");
  REQUIRE(static_cast<const void*>(kv->P) != static_cast<const void*>(kv->P_new), DTV_EINVAL,
          "kv: P_new must not alias P in a fused verification");
  REQUIRE(kv->Hkv >= 1 && kv->P_cap >= tree->n_cap, DTV_EINVAL, "kv: Hkv=%d P_cap=%d n_cap=%d", kv->Hkv,
          kv->P_cap, tree->n_cap);
  const int es = esize_of(dtype);
  REQUIRE(kv->D >= 1 && (kv->D * es) % 16 == 0 && kv->D * es <= 512, DTV_EUNSUPPORTED,
          "kv: row of D=%d elements must be a multiple of 16 bytes and at most 512", kv->D);
  out->k = static_cast<char*>(kv->k);
  out->v = static_cast<char*>(kv->v);
  out->P = kv->P;
  out->P_new = kv->P_new;
  out->P_cap = kv->P_cap;
  out->Hkv = kv->Hkv;
  out->D = kv->D;
  out->esize = es;
  return DTV_OK;
}

static int verify_greedy_impl(const dtv_tree* tree, int32_t S, const void* target, int dtype, int32_t R,
                              int32_t V, int32_t* path, int32_t* path_len, int32_t* bonus,
                              int32_t* argmax_out, const dtv_kv_cache* kv, void* ws, size_t ws_bytes,
                              void* stream) {
  int rc = check_tree(tree);
  if (rc) return rc;
  REQUIRE(target && path && path_len && bonus, DTV_EINVAL, "target, path, path_len or bonus is NULL");
  REQUIRE(dtype_ok(dtype), DTV_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(S >= 1 && R >= 1 && V >= 1, DTV_EINVAL, "S=%d R=%d V=%d", S, R, V);
  const VerifyLayout L = verify_layout(ws, S, tree->n_cap, nch_of(V, dtype));
  REQUIRE(ws != nullptr && ws_bytes >= L.bytes, DTV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, L.bytes);
  dtv::VerifyArgs a;
  a.tree = tree_args(tree);
  a.target = target;
  a.R = R;
  a.V = V;
  a.nch = nch_of(V, dtype);
  a.path = path;
  a.path_len = path_len;
  a.bonus = bonus;
  a.argmax_out = argmax_out;
  a.cbest = L.cbest;
  a.hdr = L.hdr;
  rc = kv_view(kv, dtype, tree, &a.kvc);
  if (rc) return rc;
  return launched(dtv::launch_verify_greedy(a, S, dtype == DTV_BF16 ? 1 : 0, static_cast<hipStream_t>(stream)));
}

int dtv_tree_verify_greedy(const dtv_tree* tree, int32_t S, const void* target, int dtype, int32_t R,
                           int32_t V, int32_t* path, int32_t* path_len, int32_t* bonus,
                           int32_t* argmax_out, void* ws, size_t ws_bytes, void* stream) {
  return verify_greedy_impl(tree, S, target, dtype, R, V, path, path_len, bonus, argmax_out, nullptr, ws,
                            ws_bytes, stream);
}

int dtv_tree_verify_greedy_compact(const dtv_tree* tree, int32_t S, const void* target, int dtype,
                                   int32_t R, int32_t V, int32_t* path, int32_t* path_len,
                                   int32_t* bonus, int32_t* argmax_out, const dtv_kv_cache* kv,
                                   void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(kv != nullptr, DTV_EINVAL, "kv is NULL");
  return verify_greedy_impl(tree, S, target, dtype, R, V, path, path_len, bonus, argmax_out, kv, ws,
                            ws_bytes, stream);
}

// ---------------------------------------------------------------- rejection sampling

size_t dtv_tree_verify_sample_ws_bytes(int32_t S, int32_t n_cap, int32_t V, int dtype) {
  if (S < 1 || n_cap < 1 || V < 1 || !dtype_ok(dtype)) return 0;
  return sample_layout(nullptr, S, n_cap, V, dtype).bytes;
}

static int verify_sample_impl(const dtv_tree* tree, int32_t S, const void* target, const void* draft,
                              int dtype, int32_t R, int32_t V, const uint32_t* u_acc, const uint32_t* u_res,
                              int32_t* path, int32_t* path_len, int32_t* bonus, const dtv_kv_cache* kv,
                              void* ws, size_t ws_bytes, void* stream) {
  int rc = check_tree(tree);
  if (rc) return rc;
  REQUIRE(target && draft && u_acc && u_res && path && path_len && bonus, DTV_EINVAL, "a pointer is NULL");
  REQUIRE(dtype_ok(dtype), DTV_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(S >= 1 && R >= 1 && V >= 1, DTV_EINVAL, "S=%d R=%d V=%d", S, R, V);
  const SampleLayout L = sample_layout(ws, S, tree->n_cap, V, dtype);
  REQUIRE(ws != nullptr && ws_bytes >= L.bytes, DTV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, L.bytes);
  dtv::SampleArgs a;
  a.tree = tree_args(tree);
  a.target = target;
  a.draft = draft;
  a.R = R;
  a.V = V;
  a.nch = nch_of(V, dtype);
  a.u_acc = u_acc;
  a.u_res = u_res;
  a.path = path;
  a.path_len = path_len;
  a.bonus = bonus;
  a.hdr = L.hdr;
  a.S = S;
  a.xch = L.xch;
  a.max_pass = sample_max_pass(tree->n_cap);
  a.pbuf = L.pbuf;
  a.done = L.done;
  // the walk's groups must all be resident at once: about one workgroup per compute unit
  // in total (far below what the device holds), at most kSampleMaxGroup per sequence
  const int max_blocks = dtv::sample_walk_max_blocks(dtype == DTV_BF16 ? 1 : 0);
  REQUIRE(max_blocks >= 1, DTV_EHIP, "occupancy query failed");
  const int VEC = dtype == DTV_BF16 ? 8 : 4;
  const int vec = (V % VEC == 0) &&
                  ((reinterpret_cast<uintptr_t>(target) | reinterpret_cast<uintptr_t>(draft)) & 15u) == 0;
  WalkPlan plan;
  rc = walk_plan(S, tree->n_cap, V, dtype, max_blocks, vec, &plan);
  if (rc) return rc;
  a.G = plan.G;
  a.vec = vec;
  rc = kv_view(kv, dtype, tree, &a.kvc);
  if (rc) return rc;
  return launched(dtv::launch_verify_sample(a, S, dtype == DTV_BF16 ? 1 : 0, static_cast<hipStream_t>(stream)));
}

int dtv_tree_verify_sample(const dtv_tree* tree, int32_t S, const void* target, const void* draft, int dtype,
                           int32_t R, int32_t V, const uint32_t* u_acc, const uint32_t* u_res, int32_t* path,
                           int32_t* path_len, int32_t* bonus, void* ws, size_t ws_bytes, void* stream) {
  return verify_sample_impl(tree, S, target, draft, dtype, R, V, u_acc, u_res, path, path_len, bonus, nullptr,
                            ws, ws_bytes, stream);
}

int dtv_tree_verify_sample_compact(const dtv_tree* tree, int32_t S, const void* target,
                                   const void* draft, int dtype, int32_t R, int32_t V,
                                   const uint32_t* u_acc, const uint32_t* u_res, int32_t* path,
                                   int32_t* path_len, int32_t* bonus, const dtv_kv_cache* kv,
                                   void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(kv != nullptr, DTV_EINVAL, "kv is NULL");
  return verify_sample_impl(tree, S, target, draft, dtype, R, V, u_acc, u_res, path, path_len, bonus, kv,
                            ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- compaction

int dtv_kv_compact(void* k, void* v, const int32_t* P, int32_t* P_new, int32_t P_cap, const int32_t* path,
                   const int32_t* path_len, int32_t n_cap, int32_t S, int32_t Hkv, int32_t D, int dtype,
                   void* stream) {
  REQUIRE(k && v && P && P_new && path && path_len, DTV_EINVAL, "a pointer is NULL");
  REQUIRE(dtype_ok(dtype), DTV_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(S >= 1 && Hkv >= 1 && n_cap >= 1 && P_cap >= n_cap, DTV_EINVAL, "S=%d Hkv=%d n_cap=%d P_cap=%d",
          S, Hkv, n_cap, P_cap);
  const int es = esize_of(dtype);
  REQUIRE(D >= 1 && (D * es) % 16 == 0 && D * es <= 512, DTV_EUNSUPPORTED,
          "row of D=%d elements must be a multiple of 16 bytes and at most 512", D);
  dtv::CompactArgs a;
  a.k = k;
  a.v = v;
  a.P = P;
  a.P_new = P_new;
  a.P_cap = P_cap;
  a.path = path;
  a.path_len = path_len;
  a.n_cap = n_cap;
  a.S = S;
  a.Hkv = Hkv;
  a.D = D;
  a.esize = es;
  return launched(dtv::launch_compact(a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- bookkeeping

int dtv_bookkeeping(const int32_t* accepted_h, int32_t n_passes, int64_t draft_steps, double gamma,
                    double* out_h) {
  REQUIRE(accepted_h && out_h, DTV_EINVAL, "accepted_h or out_h is NULL");
  REQUIRE(n_passes >= 1, DTV_EINVAL, "need at least one verification pass");
  REQUIRE(draft_steps >= 0 && gamma >= 0.0, DTV_EINVAL, "draft_steps and gamma must be >= 0");
  double L = 0.0;
  for (int32_t t = 0; t < n_passes; ++t) {
    REQUIRE(accepted_h[t] >= 0, DTV_EINVAL, "A_%d = %d < 0", t, accepted_h[t]);
    L += static_cast<double>(accepted_h[t]) + 1.0;
  }
  const double EA = L / n_passes;
  const double eta = static_cast<double>(draft_steps) / n_passes;
  out_h[0] = EA;
  out_h[1] = eta;
  out_h[2] = EA / (1.0 + gamma * eta);
  out_h[3] = L;
  return DTV_OK;
}

}  // extern "C"
