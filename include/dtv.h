/*
 * dtv.h - C ABI of one speculative-decoding draft-tree step on an MI355X (gfx950).
 *
 * The step has four parts: build a draft tree under a node budget, run tree-masked
 * attention over the KV prefix and each node's ancestors, verify the nodes against the
 * target, and move the accepted path's keys and values behind the prefix.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless the argument name ends in `_h` (host).
 * - Every call only enqueues work on `stream` (a hipStream_t; NULL = the default stream)
 *   and returns; nothing is synchronised.
 * - The caller owns every buffer. The library allocates nothing; calls that need scratch
 *   take a caller-provided workspace `ws` of `ws_bytes` bytes, sized by the matching
 *   `*_ws_bytes` query and zero-filled by the caller once after allocation. The library
 *   keeps it consistent from one call to the next as long as the calls' sizes (batch,
 *   capacity, rows, vocabulary, widths or budgets) stay the same: the layout of a call's
 *   per-call state follows its sizes, so a workspace reused by a call with other sizes
 *   must be zero-filled again first (dtv_tree_attn keeps no state and is exempt). One
 *   workspace must not be used by two calls that may run at the same time.
 * - Argument errors are detected on the host before any launch and returned as a
 *   negative dtv_status; a launch failure returns DTV_EHIP. Errors found by a kernel
 *   (capacity exceeded on the device, a bounded wait that ran out) are recorded in the
 *   workspace and read with dtv_ws_status(), which synchronises the stream. A
 *   workspace whose status is an error must be zero-filled again before its next use
 *   (an interrupted call can leave its per-call state set).
 *   dtv_last_error() returns a message for the last failing call of the thread.
 * - Logit tables are `[S][R][V]`, row-major, of the given dtype; a node's rows are
 *   addressed through the tree's `row` array. Stored values are compared exactly;
 *   ties go to the lowest index.
 * - No C++ exception crosses this interface.
 *
 * Tree layout (slot numbering)
 * ----------------------------
 * Slot 0 of every sequence is the root (the last committed token, whose key/value is not
 * cached yet); draft nodes follow in topological order (parent[i] < i). Every per-node
 * array is `[S][n_cap]`; `anc` is `[S][n_cap][words]` with bit (j % 64) of word (j / 64)
 * set when slot j is an ancestor-or-self of the node.
 */
#ifndef DTV_H
#define DTV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DTV_OK = 0,
  DTV_EINVAL = -1,        /* bad argument (null pointer, negative size, inconsistent shape) */
  DTV_EUNSUPPORTED = -2,  /* valid but not implemented (dtype, head dim, K or budget too large) */
  DTV_ECAPACITY = -3,     /* a tree would not fit its n_cap slots or words */
  DTV_EWORKSPACE = -4,    /* workspace missing or smaller than the *_ws_bytes query */
  DTV_EHIP = -5,          /* a HIP call or kernel launch failed */
  DTV_EDEVICE = -6        /* a kernel reported an error in the workspace (dtv_ws_status) */
} dtv_status;

typedef enum { DTV_F32 = 0, DTV_BF16 = 1 } dtv_dtype;

/* Device arrays of a batch of S trees (see "Tree layout" above). */
typedef struct dtv_tree {
  int32_t n_cap;      /* slots per sequence, root included */
  int32_t words;      /* 64-bit mask words per node, >= ceil(n_cap / 64) */
  int32_t* n_nodes;   /* [S] nodes in each tree, root included */
  int32_t* parent;    /* [S][n_cap] parent slot, -1 at the root */
  int32_t* token;     /* [S][n_cap] token id, -1 at the root */
  int32_t* depth;     /* [S][n_cap] root = 0 */
  int32_t* row;       /* [S][n_cap] row of the node in the draft and target tables */
  double* score;      /* [S][n_cap] log path score (sum of draft log-probabilities) */
  uint64_t* anc;      /* [S][n_cap][words] ancestor-or-self bitmask */
  int32_t* layers;    /* [S] draft passes (layers of draft rows) the build consumed */
} dtv_tree;

const char* dtv_status_str(int status);
const char* dtv_last_error(void);

/* Synchronise `stream` and return the device-side status recorded in a workspace
 * (DTV_OK, DTV_ECAPACITY, DTV_EDEVICE), clearing it. */
int dtv_ws_status(const void* ws, void* stream);

/* ---------------------------------------------------------------------------------
 * Row statistics (vocab-wide softmax normaliser, argmax and top-K).
 *
 * The TALON page (sections 5.2.1-5.2.2) scores candidates with products of draft
 * probabilities and initialises the root layer with TopK of the draft distribution;
 * the OPT-Tree summary (section 2) accepts the target's highest-probability token;
 * the concept page ("The protocol") compares p(x) with q(x). All need, per row:
 * maximum, index of the maximum, log-sum-exp and the K largest entries.
 *
 * For each of R rows `rows[r]` of a `[R][V]` table (or row `row_idx[r]` when row_idx is
 * not NULL): maxv[r] (float), argmax[r] (lowest index of the maximum), lse[r] (double,
 * log sum_j exp(x_j)), and, when K > 0, topk[r][0..K) = indices of the K largest values,
 * largest first, ties by lowest index. Any output pointer may be NULL. Requires
 * 1 <= K <= min(V, 1024) or K = 0.
 */
size_t dtv_row_stats_ws_bytes(int32_t R, int32_t V, int32_t K, int dtype);
int dtv_row_stats(const void* table, int dtype, int32_t R, int32_t V, const int32_t* row_idx,
                  int32_t K, float* maxv, int32_t* argmax, double* lse, int32_t* topk,
                  void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Tree build: given shape (random trees drafted elsewhere).
 *
 * The caller fills n_nodes, parent and token; the call writes depth, row (= slot),
 * score (= 0), layers (= 0) and the ancestor-or-self mask that tree attention needs
 * (OPT-Tree summary, section 2: all tree tokens verified in one pass with a tree mask).
 * A parent that is not an earlier slot is reported as DTV_EDEVICE by dtv_ws_status.
 */
size_t dtv_tree_build_given_ws_bytes(int32_t S);
int dtv_tree_build_given(const dtv_tree* tree, int32_t S, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Tree build: TALON budget-driven hybrid expansion (TALON page, sections 5.1-5.2).
 *
 * Layer 1 is the K most probable root children (no gate; at most B). Every later layer
 * pools the K most probable children of each node of the previous layer, scores them
 * with the log path score s(c) = s(parent) + log p_d(token | parent), keeps those with
 * s(c) >= log(alpha) + max s (the anchor), and, when more pass than budget remains,
 * the best by score (ties: lower parent slot, then lower rank). New nodes take slots in
 * (parent slot, rank) order. The build stops when B draft nodes exist (N = B + 1).
 * Draft rows are keyed by slot: node i expands with table row i, so `draft` holds
 * R >= B + 1 rows per sequence. Only slots 0..B-1 can be expanded, so the call reduces
 * rows 0..B-1 of every sequence in one data-parallel launch (Top-K and log-sum-exp per
 * row) and runs each sequence's layer loop in a second launch, one workgroup per sequence.
 * Limits: 1 <= B < n_cap <= 1024, 1 <= K <= 64, B * K <= 4096, 0 <= alpha <= 1,
 * chunks * K <= 2048 (chunks = ceil(V / 8192) for bf16, ceil(V / 4096) for fp32).
 */
size_t dtv_tree_build_talon_ws_bytes(int32_t S, int32_t B, int32_t K, int32_t V, int dtype);
int dtv_tree_build_talon(const dtv_tree* tree, int32_t S, const void* draft, int dtype,
                         int32_t R, int32_t V, int32_t B, int32_t K, double alpha,
                         void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Tree build: GOOSE anisotropic spine tree (GOOSE page, sections 2A and 2C).
 *
 * A deep chain of context-match tokens with shallow, wide branches at its nodes:
 * slots 1..n_spine hold spine[s][0..n_spine) as a chain (slot k has parent k-1); forks
 * are slots 0..F-1 (the root and the first spine nodes, F <= n_spine + 1), and fork f gets
 * widths_h[f] depth-1 branch nodes whose tokens are the most probable tokens of draft row
 * f that differ from the token of f's spine child (slot f+1), in slots
 * 1 + n_spine + sum(widths_h[0..f)) + j, j in rank order. The spine holds the lowest
 * slots, so a greedy walk that prefers low slots follows the spine first. Branch scores
 * are log p_d(token | fork); spine nodes score 0. spine is `[S][n_spine]` (device);
 * widths_h is a host array of F entries in 0..64; draft is `[S][R][V]` keyed by slot.
 */
size_t dtv_tree_build_spine_ws_bytes(int32_t S, int32_t F, int32_t max_width, int32_t V, int dtype);
int dtv_tree_build_spine(const dtv_tree* tree, int32_t S, const int32_t* spine, int32_t n_spine,
                         const int32_t* widths_h, int32_t F, const void* draft, int dtype, int32_t R,
                         int32_t V, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Tree build: OPT-Tree greedy expected-acceptance maximisation (OPT-Tree summary, sec. 3).
 *
 * Layer by layer, every frontier node proposes its children with score = its score +
 * log p_d(token | node) (a float64 sum of logs); the layer keeps the n best candidates
 * (ties: lower frontier position, then lower rank in the row), which become the next
 * frontier, ordered by (parent position, rank). After layer l, E_l = sum of exp(score)
 * over the best n nodes of all layers so far (ties: earlier layer, then position); the
 * drafting stops when E_l - E_{l-1} < delta (E_0 = 0) or after max_layers layers. The
 * tree is the best n nodes (root-closed, since a child never scores above its parent),
 * numbered by (layer, position). Row identity: the node at position p of layer l uses
 * row 1 + (l-1)*n + p of `draft` (`[S][R][V]`, R >= 1 + (max_layers-1)*n + ...); the root
 * uses row 0. tree.row receives these identities (the target rows of verification).
 * Limits: n <= 1023, n < n_cap, max_layers <= 64, V <= 4194304; more than 4096 candidates
 * within the selection bound of one layer, or more than 1024 tied at the layer's n-th best
 * score (extreme ties), is reported as DTV_ECAPACITY.
 */
size_t dtv_tree_build_opt_ws_bytes(int32_t S, int32_t n, int32_t V, int32_t max_layers, int dtype);
int dtv_tree_build_opt(const dtv_tree* tree, int32_t S, const void* draft, int dtype, int32_t R,
                       int32_t V, int32_t n, double delta, int32_t max_layers, void* ws,
                       size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Layer-by-layer builds (TALON page, sections 5.2.1 and 5.3; OPT-Tree summary, sec. 3).
 *
 * TALON's candidate pool for layer l is the expansion of layer l-1's nodes, and its cost
 * term counts one draft forward pass per layer; OPT-Tree likewise drafts one layer from
 * the previous one: a drafter produces the rows of a layer's frontier only once the layer
 * before is chosen. These calls take those rows layer by layer and give the same trees as
 * dtv_tree_build_talon / dtv_tree_build_opt on the same rows.
 *
 * dtv_tree_build_begin takes each sequence's root row (root_logits `[S][V]`) and builds
 * layer 1; dtv_tree_build_step builds layer `layer` (2, 3, ... in order) from the rows of
 * its frontier, the nodes of layer layer-1: frontier_logits `[S][W_cap][V]`, row f of
 * sequence s = the draft row of that sequence's frontier node f. The frontier of a TALON
 * tree is the nodes the previous call added, in slot order (slots cnt+1 .. cnt+W, where cnt
 * counts the draft nodes before that call); of an OPT-Tree tree, the previous layer's
 * nodes in frontier order (frontier position p of layer l has build identity, and tree
 * row, 1 + (l-1) n + p). Both calls write W[s] (device) = the next layer's frontier width,
 * 0 once the sequence is done, and done[s] (device) = 1 once its tree is complete; rows
 * past W[s], and later calls for a done sequence, are not read. A step needs W_cap >= the
 * frontier width (TALON: W_cap <= B; OPT-Tree: the width is min(n, W_{l-1} min(n, V)),
 * known in advance). When a sequence is done, its tree arrays, n_nodes, layers and masks
 * are complete; until then only its nodes so far are (TALON; OPT-Tree writes the tree when
 * it is done). Limits and tie rules are those of the whole-table calls. The workspace
 * (dtv_tree_build_layered_ws_bytes) carries the build's state from begin to the last step:
 * one workspace per build in flight.
 */
enum { DTV_BUILD_TALON = 1, DTV_BUILD_OPT = 2 };
typedef struct {
  int32_t mode;        /* DTV_BUILD_TALON or DTV_BUILD_OPT */
  int32_t B, K;        /* TALON: draft-node budget, children per expanded node */
  double alpha;        /* TALON: confidence gate */
  int32_t n;           /* OPT-Tree: nodes per layer and in the tree */
  double delta;        /* OPT-Tree: stop when E_l - E_{l-1} < delta */
  int32_t max_layers;  /* OPT-Tree: layer cap */
} dtv_build_params;

size_t dtv_tree_build_layered_ws_bytes(const dtv_build_params* params, int32_t S, int32_t V, int dtype);
int dtv_tree_build_begin(const dtv_tree* tree, int32_t S, const dtv_build_params* params, const void* root_logits,
                         int dtype, int32_t V, int32_t* W, int32_t* done, void* ws, size_t ws_bytes, void* stream);
int dtv_tree_build_step(const dtv_tree* tree, int32_t S, const dtv_build_params* params, int32_t layer,
                        const void* frontier_logits, int32_t W_cap, int dtype, int32_t V, int32_t* W,
                        int32_t* done, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Tree attention (OPT-Tree summary, section 2; concept page, "Why it is a win").
 *
 * For node i of sequence s and query head h (KV head kv = h / (Hq / Hkv)):
 *   o[s][i][h] = sum_j softmax_j(scale * q[s][i][h] . k[s][kv][j]) v[s][kv][j]
 * over the prefix j < P[s] and the tree keys j = P[s] + a for every ancestor-or-self a
 * of i (the tree's keys and values sit at cache positions P[s] + slot).
 * Layouts: q, o `[S][n_cap][Hq][D]`; k, v `[S][Hkv][P_cap][D]`; P `[S]` (device) with
 * P[s] + n_nodes[s] <= P_cap, and P_max >= every P[s] (host bound, sizes the grid; a
 * larger P[s] is reported as DTV_ECAPACITY by the workspace status).
 * Rows of o for slots >= n_nodes[s] are not written. bf16 runs on MFMA with fp32
 * accumulation; f32 runs in fp32. D must be 64 or 128; Hq % Hkv == 0.
 */
size_t dtv_tree_attn_ws_bytes(int32_t S, int32_t n_cap, int32_t Hq, int32_t Hkv, int32_t D,
                              int32_t P_max, int dtype);
int dtv_tree_attn(const void* q, const void* k, const void* v, const int32_t* P, int32_t P_cap,
                  int32_t P_max, const dtv_tree* tree, int32_t S, int32_t Hq, int32_t Hkv,
                  int32_t D, int dtype, float scale, void* o, void* ws, size_t ws_bytes,
                  void* stream);

/* Tree attention for callers that cannot allocate: code under HIP graph capture, serving
 * loops and harnesses that forbid allocation. The same computation and results as
 * dtv_tree_attn (the same launches and key-split plan, so bit-identical outputs), with no
 * workspace argument: the key-split partials and the status word live in a static device
 * array of 64 MiB (67108864 bytes) that each GPU the library runs on holds until the
 * process ends. Sizes whose partials would need more (dtv_tree_attn_ws_bytes > 64 MiB, for
 * example 16 sequences of 4096-key caches with 65-node trees and 32/8 heads) are refused
 * with DTV_ECAPACITY before any device call. The call allocates nothing: it calls no
 * hipMalloc or hipFree; its first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress) once. Every call on one GPU shares that GPU's array, which
 * keeps the last call's partials: nothing in it must start at zero (every partial a call
 * reads, that call writes first), but calls that may overlap on one GPU (concurrent streams
 * or threads) race on it and must be ordered by the caller. Device-side refusals
 * (n_nodes[s] > n_cap, P[s] + n_nodes[s] > P_cap, or P[s] > P_max) leave those rows of o
 * unwritten and are not reported (dtv_tree_attn reports them through its workspace).
 */
int dtv_tree_attn_noalloc(const void* q, const void* k, const void* v, const int32_t* P, int32_t P_cap,
                          int32_t P_max, const dtv_tree* tree, int32_t S, int32_t Hq, int32_t Hkv,
                          int32_t D, int dtype, float scale, void* o, void* stream);

/* ---------------------------------------------------------------------------------
 * Greedy verification (OPT-Tree summary, section 2; GOOSE page, section 2C).
 *
 * a[v] = argmax of target row row[v]; node c matches when token[c] == a[parent[c]];
 * the accepted node v* is the deepest node whose whole root path matches (lowest slot
 * among equals). Outputs per sequence: path[s][0..A] = slots root .. v* (by depth),
 * path_len[s] = A + 1, bonus[s] = a[v*]; optional argmax_out[s][n_cap] = a.
 * `target` is `[S][R][V]` with R > row[v] for every node (for an OPT-Tree tree, whose rows
 * reach max_layers * n, R >= 1 + max_layers * n). A node whose row lies outside [0, R), or
 * whose depth lies outside [0, n_nodes), is never read: the sequence gets path_len = 0 and
 * bonus = -1, and dtv_ws_status reports DTV_EDEVICE.
 */
size_t dtv_tree_verify_greedy_ws_bytes(int32_t S, int32_t n_cap, int32_t V, int dtype);
int dtv_tree_verify_greedy(const dtv_tree* tree, int32_t S, const void* target, int dtype,
                           int32_t R, int32_t V, int32_t* path, int32_t* path_len, int32_t* bonus,
                           int32_t* argmax_out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Rejection-sampling verification (concept page, "The protocol", steps 3-4).
 *
 * The chain rule of the page, applied to a tree: starting at the root, with
 * p = softmax(target row of v) and q = softmax(draft row of v) (rows row[v] of the
 * `[S][R][V]` tables; temperature 1), the children c of v are tried in slot order with
 * u = (u_acc[s][c] + 1/2) 2^-32: c is accepted when q(x_c) > 0 and u < p(x_c)/q(x_c), or
 * when q(x_c) = 0 < p(x_c); after each rejection p <- (p - q)+ / sum (p - q)+ (kept if the
 * sum is 0). The walk moves to the accepted child; when no child is accepted, or v is a
 * leaf, the bonus token is the smallest k with sum_{j<=k} p_j > u * sum p (ascending
 * float64 prefix sums, u from u_res[s][v]). Outputs as dtv_tree_verify_greedy. Decisions
 * are taken in float64; the result depends only on the inputs and the uniforms.
 * Both tables need R > row[v] for every node (OPT-Tree trees: R >= 1 + max_layers * n), and
 * every drafted token must lie in [0, V). A tree that breaks either is never read past
 * its tables: the sequence gets path_len = 0 and bonus = -1, and dtv_ws_status reports
 * DTV_EDEVICE. Sizes the walk cannot hold (more sequences than walk workgroups fit on the
 * device at once, more than 1024 slots) are refused with DTV_EUNSUPPORTED before launch.
 */
size_t dtv_tree_verify_sample_ws_bytes(int32_t S, int32_t n_cap, int32_t V, int dtype);
int dtv_tree_verify_sample(const dtv_tree* tree, int32_t S, const void* target, const void* draft,
                           int dtype, int32_t R, int32_t V, const uint32_t* u_acc, const uint32_t* u_res,
                           int32_t* path, int32_t* path_len, int32_t* bonus, void* ws, size_t ws_bytes,
                           void* stream);

/* How dtv_tree_verify_sample divides the walk of each sequence, for S sequences of n_cap
 * slots, vocabulary V and dtype, when the device holds `resident_blocks` walk workgroups at
 * once and rows are walked in 16-byte units (`vec` = 1: rows 16-byte aligned and V a
 * multiple of 8 bf16 / 4 fp32 values) or entry by entry (`vec` = 0). Host only, no device
 * call. Writes plan_h[0..7) = { G workgroups per sequence, units per row, units of the
 * largest slice, entries of the largest slice, 1 if a slice fits the workgroup's shared
 * memory (else it uses the workspace), exchange slots per sequence, workspace entries of
 * residuals and q per sequence }. Returns the status the verification would return for
 * these sizes (DTV_EUNSUPPORTED when S > resident_blocks or n_cap > 1024).
 */
int dtv_tree_verify_sample_plan(int32_t S, int32_t n_cap, int32_t V, int dtype, int32_t resident_blocks,
                                int32_t vec, int64_t* plan_h);

/* ---------------------------------------------------------------------------------
 * KV compaction (concept page, "The protocol", step 4: append the accepted tokens).
 *
 * For every sequence and KV head: cache[P + k] <- cache[P + path[k]] for k < path_len,
 * for both k and v (in place, all reads before any write), and P_new[s] = P[s] +
 * path_len[s]. P_new may alias P. Layout as in dtv_tree_attn; path `[S][n_cap]`. A
 * sequence whose path_len lies outside 1..n_cap, or whose P[s] is negative or leaves fewer
 * than n_cap rows of the cache, is left untouched and gets P_new[s] = -1 (also when P_new
 * aliases P).
 */
int dtv_kv_compact(void* k, void* v, const int32_t* P, int32_t* P_new, int32_t P_cap,
                   const int32_t* path, const int32_t* path_len, int32_t n_cap, int32_t S,
                   int32_t Hkv, int32_t D, int dtype, void* stream);

/* ---------------------------------------------------------------------------------
 * Verification and KV compaction in one launch (concept page, "The protocol", steps 3-4).
 *
 * The same results as dtv_tree_verify_greedy / dtv_tree_verify_sample followed by
 * dtv_kv_compact on their path: the workgroups that finish a sequence's walk copy the
 * accepted rows of every KV head in place (rows of one head and tensor in increasing
 * path order, every read of a batch before its writes), then set P_new[s] = P[s] +
 * path_len[s] (-1 when P[s] and the tree do not fit P_cap; the cache is then untouched).
 * `kv` describes the cache as in dtv_kv_compact: k, v `[S][Hkv][P_cap][D]` in the
 * verification's dtype, P `[S]`, P_new `[S]`, which must not alias P (other workgroups of
 * the sequence may still read P). Workspace: the size of the verification alone.
 * DTV_EINVAL for a NULL or inconsistent kv, otherwise the errors of the verification.
 */
typedef struct {
  void* k;
  void* v;
  const int32_t* P;
  int32_t* P_new;
  int32_t P_cap, Hkv, D;
} dtv_kv_cache;

int dtv_tree_verify_greedy_compact(const dtv_tree* tree, int32_t S, const void* target, int dtype,
                                   int32_t R, int32_t V, int32_t* path, int32_t* path_len,
                                   int32_t* bonus, int32_t* argmax_out, const dtv_kv_cache* kv,
                                   void* ws, size_t ws_bytes, void* stream);
int dtv_tree_verify_sample_compact(const dtv_tree* tree, int32_t S, const void* target,
                                   const void* draft, int dtype, int32_t R, int32_t V,
                                   const uint32_t* u_acc, const uint32_t* u_res, int32_t* path,
                                   int32_t* path_len, int32_t* bonus, const dtv_kv_cache* kv,
                                   void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Kernel timing, for measurement (not part of the pages' method).
 *
 * dtv_kernel_timing(enable, reset): with enable = 1, every later launch of the library
 * (any thread, any stream) is bracketed by two HIP events recorded on its stream, which
 * adds a few microseconds between kernels; with enable = 0 launches are not timed. With
 * reset = 1 the totals (and any launches not yet read) are dropped first. Host call;
 * returns DTV_OK or DTV_EHIP.
 * dtv_kernel_times(cap, names_h, name_bytes, total_ms_h, launches_h): waits for every timed
 * launch so far, then writes, for up to cap kernels, the kernel's name (without template
 * arguments, NUL-terminated in name_bytes bytes at names_h + i * name_bytes), the summed
 * event time in milliseconds and the number of timed launches. Any output may be NULL.
 * Returns the number of distinct kernels timed (which may exceed cap), or DTV_EHIP.
 */
int dtv_kernel_timing(int enable, int reset);
int dtv_kernel_times(int32_t cap, char* names_h, int32_t name_bytes, double* total_ms_h, int64_t* launches_h);

/* ---------------------------------------------------------------------------------
 * Draft-efficiency bookkeeping (TALON page, section 5.3). Host only.
 *
 * accepted_h[t] = A_t accepted draft tokens of verification pass t (t < n_passes),
 * draft_steps = N_d, gamma = draft-to-target cost ratio. Writes out_h[0..4] =
 * { E[A] = L / N_v with L = sum (A_t + 1), eta = N_d / N_v, Speedup = E[A] / (1 + gamma*eta),
 *   L }.
 */
int dtv_bookkeeping(const int32_t* accepted_h, int32_t n_passes, int64_t draft_steps,
                    double gamma, double* out_h);

#ifdef __cplusplus
}
#endif
#endif /* DTV_H */
