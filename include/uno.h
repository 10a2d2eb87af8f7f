/*
 * uno.h -- C ABI of the UNO decode-cycle sampling library for MI355X (gfx950).
 *
 * One UNO decode cycle runs two target-model forwards: a diffusion-pathway
 * forward that yields B draft marginals, and an autoregressive forward that
 * verifies them losslessly (SGLang PR #37667, "native SGLang serving support
 * for UNO", Motivation).  This library implements the sampling that sits
 * between and after those forwards, on logits already resident in HBM:
 *
 *   uno_filter         temperature / top-k / top-p filtering of logit rows
 *   uno_sample_linear  linear mode: proposals, rejection, residual / bonus
 *   uno_build_tree     tree mode: top-K candidates per position -> V-node tree
 *   uno_verify_tree    tree mode: target-sampled walk of the candidate tree
 *   uno_tree_attention tree mode: tree-suffix attention merged with the prefix state
 *
 * Conventions shared by every entry point
 *  - Pointers named logits / draft / target / out_* / node_* / request_ids /
 *    ws are DEVICE pointers owned by the caller; the library never allocates
 *    or frees memory and keeps no state between calls (apart from the last HIP
 *    error code, per host thread).
 *  - Logits are row-major and contiguous, one row of `vocab` elements per
 *    distribution, float32 (UNO_F32) or bfloat16 (UNO_BF16).
 *  - Sampling parameters follow the run_math_eval parameter rules (walk-through
 *    of SGLang benchmark/uno, "run_math_eval 全参数详解"): temperature >= 0,
 *    top_p in (0, 1].  temperature == 0 is greedy decoding; top_k <= 0 or
 *    top_k >= vocab disables top-k; top_p == 1 disables top-p.
 *  - Filter order (PR #37667 review thread on filter order): temperature, then
 *    top-k over the raw logits with ties to the smaller token id, then
 *    renormalise over the top-k set, then keep ids (in that order) while the
 *    exclusive cumulative probability is below top_p (the first id is always
 *    kept), then renormalise over the kept ids.  NaN logits count as -inf; a
 *    row holding +inf, or no finite logit, is invalid (empty support).
 *    With order == UNO_ORDER_JOINT (the regular sampler's joint filtering the
 *    same review thread describes) the top-p cut reads the softmax over the
 *    whole vocabulary instead, within the top-k set; the kept ids are then
 *    renormalised.  The orders differ only when top-k and top-p are both on.
 *  - Random numbers: Philox4x32-10 (Salmon et al., SC'11) with counter
 *    (request id, position, offset lo, offset hi) and key (seed lo, seed hi);
 *    word 0 draws proposals, word 1 the acceptance test, word 2 the residual /
 *    bonus / tree-walk sample; u = word * 2^-32.  `offset` is the decode-cycle
 *    index; request ids default to the batch index.
 *  - Sampling from a distribution is an inverse CDF in ascending token-id order.
 *  - Calls are asynchronous on `stream`.  Argument checks run on the host
 *    before anything is launched; on any error nothing is launched and no
 *    output is written.
 *  - Workspace: `ws` must hold at least the bytes uno_workspace_bytes reports
 *    for the same arguments and be 256-byte aligned.  Its contents need no
 *    initialisation; calls that share one workspace must be ordered (same
 *    stream or synchronised).
 */
#ifndef UNO_H
#define UNO_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    UNO_OK = 0,
    UNO_ERR_INVALID_ARG = -1,   /* a size, pointer or parameter is out of range      */
    UNO_ERR_UNSUPPORTED = -2,   /* valid request the library does not implement      */
    UNO_ERR_WORKSPACE = -3,     /* ws is NULL, too small or misaligned                 */
    UNO_ERR_HIP = -4,           /* a HIP launch failed (see uno_last_hip_error)        */
    UNO_ERR_SCRATCH_LIMIT = -5  /* the allocation-free entry point's fixed scratch is too small */
} uno_status_t;

typedef enum { UNO_F32 = 0, UNO_BF16 = 1 } uno_dtype_t;

typedef enum {
    UNO_OP_FILTER = 0,
    UNO_OP_SAMPLE_LINEAR = 1,
    UNO_OP_BUILD_TREE = 2,
    UNO_OP_VERIFY_TREE = 3
} uno_op_t;

typedef enum {
    UNO_ORDER_TOPK_FIRST = 0,   /* top-k, renormalise, then top-p (default)       */
    UNO_ORDER_JOINT = 1         /* top-p on the full softmax, within the top-k set */
} uno_order_t;

typedef struct uno_sampling {
    float temperature;   /* >= 0; 0 = greedy                                  */
    int32_t top_k;       /* <= 0 or >= vocab: off                              */
    float top_p;         /* (0, 1]; 1 = off                                    */
    int32_t order;       /* uno_order_t; anything else is UNO_ERR_INVALID_ARG   */
} uno_sampling_t;

/* Largest top_k the sparse (top-k) path accepts.  Larger finite top_k returns
 * UNO_ERR_UNSUPPORTED. */
#define UNO_MAX_TOP_K 256
/* Tree limits (walk-through of SGLang benchmark/uno, "启动期硬性约束"):
 * V >= B, V <= 128, V * K <= 2048. */
#define UNO_MAX_TREE_NODES 128
#define UNO_MAX_TREE_VK 2048

/* Workspace size for one call of `op`.
 * batch_or_rows: rows for UNO_OP_FILTER, requests otherwise.  B, K, V as in the
 * matching entry point (ignored where unused).  Writes *out_bytes; returns a
 * status (the same argument checks as the entry point, minus pointers). */
int uno_workspace_bytes(int32_t op, int64_t batch_or_rows, int32_t B, int32_t K, int32_t V,
                        int64_t vocab, int32_t dtype, const uno_sampling_t* sp,
                        size_t* out_bytes);

/* Filter `rows` logit rows.  (PR #37667 review thread on filter order.)
 * Sparse modes (temperature == 0, top-k on, or vocab <= UNO_MAX_TOP_K, where the
 *   whole vocabulary is the top-k set): out_ids / out_probs [rows][cap]
 *   receive the support in filter order (z desc, id asc); entries past the
 *   support hold -1 / 0.  out_count[rows] = support size, -1 for an invalid row.
 *   cap must be >= the effective top-k (1 when temperature == 0, vocab when
 *   top-k is off on a small vocabulary).
 * Dense modes (top-k off, temperature > 0, vocab > UNO_MAX_TOP_K): out_ids /
 *   out_probs are not written (may be NULL).
 *   - top_p == 1: the support is the whole vocabulary; out_count[r] = number
 *     of finite logits (-1: invalid row).
 *   - top_p < 1 (full-vocabulary nucleus): the support is the shortest prefix
 *     of the filter order whose softmax mass reaches top_p; out_count[r] = its
 *     size (-1: invalid row).
 * out_stats [rows][2] (nullable in sparse modes, required in dense modes):
 *   (m, S) such that the probability before any top-p renormalisation is
 *   exp((z - m) / T) / S; m is the row maximum. */
int uno_filter(const void* logits, int32_t dtype, int64_t rows, int64_t vocab,
               const uno_sampling_t* sp, int32_t cap,
               int32_t* out_ids, double* out_probs, int32_t* out_count, double* out_stats,
               void* ws, size_t ws_bytes, hipStream_t stream);

/* Linear UNO cycle for `batch` requests.  (PR #37667, Motivation: the linear
 * sampler draws each block token independently from its marginal;
 * Modifications: sparse and dense proposal and rejection sampling; walk-through
 * "启动期硬性约束": acceptance thresholds fixed at 1.0.)
 *   draft  [batch][B][vocab]   filtered draft marginals q_0 .. q_{B-1}
 *   target [batch][B+1][vocab] filtered target rows p_0 .. p_B (p_B = bonus row)
 * For j = 0..B-1: y_j ~ q_j; accept iff u1 * q_j(y_j) < p_j(y_j); j* = first
 * rejection (B if none).  j* < B: the last token ~ max(0, p_j* - q_j*)
 * renormalised (~ p_j* if that residual has no mass); j* = B: ~ p_B.
 *   out_tokens [batch][B+1]: y_0 .. y_{j*-1}, last token, then -1
 *   out_accept_len [batch]: j* + 1, in [1, B+1]
 *   out_proposals [batch][B] (nullable): every y_j (-1 if q_j is invalid)
 *   out_flags [batch] (nullable): bit 0 = an invalid row was met, bit 1 = the
 *     residual had no mass
 *   request_ids [batch] (nullable device pointer): Philox request ids, uint32
 *     (they fill the counter's first 32-bit word)
 * Sparse (top-k on, greedy, or vocab <= UNO_MAX_TOP_K) and dense (top-k off:
 * the whole vocabulary, or its nucleus when top_p < 1) filters are supported. */
int uno_sample_linear(const void* draft, const void* target, int32_t dtype, int32_t batch,
                      int32_t B, int64_t vocab, const uno_sampling_t* sp, uint64_t seed,
                      uint64_t offset, const uint32_t* request_ids,
                      int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_proposals,
                      uint32_t* out_flags, void* ws, size_t ws_bytes, hipStream_t stream);

/* Tree construction.  (PR #37667, Motivation: the tree sampler considers V
 * candidate sequences from the top K candidates of each marginal;
 * walk-through "B/K/V 参数映射".)
 * Candidates at depth d are the first K ids of the filtered draft row d in
 * filter order; a node's score is the product of the filtered draft
 * probabilities on its path (root = 1).  The tree is the V best non-root
 * nodes found best-first (ties: smaller depth, smaller parent index, smaller
 * candidate rank).  Node 0 is the root (token -1, parent -1, depth 0).
 *   node_token / node_parent / node_depth [batch][V+1] (unused slots: -1)
 *   node_score [batch][V+1] (nullable; unused slots 0)
 *   num_nodes [batch]: nodes including the root (< V+1 when candidates run out)
 * Requires 1 <= K, B <= V <= 128 and V * K <= 2048.  Without top-k
 * (temperature > 0) the candidates are the K most likely ids of the full
 * softmax -- of its nucleus when top_p < 1, renormalised over it -- and K must
 * be <= UNO_MAX_TOP_K (else UNO_ERR_UNSUPPORTED). */
int uno_build_tree(const void* draft, int32_t dtype, int32_t batch, int32_t B, int32_t K,
                   int32_t V, int64_t vocab, const uno_sampling_t* sp,
                   int32_t* node_token, int32_t* node_parent, int32_t* node_depth,
                   double* node_score, int32_t* num_nodes,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Tree verification by target-sampled walk.  (PR #37667, Modifications: tree
 * UNO reuses EAGLE tree verification with sparse target sampling;
 * walk-through "启动期硬性约束": acceptance thresholds 1.0.)
 *   target [batch][V+1][vocab]: row n is the target distribution following
 *     node n's prefix (row 0: the root); rows at or past num_nodes are not read.
 *   node_token / node_parent [batch][V+1], num_nodes [batch]: a tree as written
 *     by uno_build_tree (parents precede children).
 * At node n of depth d: t ~ p_n (word 2 of position d); emit t; move to the
 * child of n whose token is t, else stop.
 *   out_tokens [batch][B+1], out_path [batch][B+1] (visited nodes), -1 padded
 *   out_accept_len [batch] in [1, B+1]; out_flags as in uno_sample_linear.
 * Requires B <= V <= 128.  Without top-k (temperature > 0) each node's token
 * is drawn from the full softmax of its row (its nucleus when top_p < 1): the
 * fallback the PR names for tree verification when sparse target sampling does
 * not apply (PR #37667, Modifications). */
int uno_verify_tree(const void* target, int32_t dtype, int32_t batch, int32_t B, int32_t V,
                    int64_t vocab, const uno_sampling_t* sp, uint64_t seed, uint64_t offset,
                    const uint32_t* request_ids, const int32_t* node_token,
                    const int32_t* node_parent, const int32_t* num_nodes,
                    int32_t* out_tokens, int32_t* out_path, int32_t* out_accept_len,
                    uint32_t* out_flags, void* ws, size_t ws_bytes, hipStream_t stream);

/* Per-request sampling parameters.  Each *_ex entry point is its namesake with
 * `sp` an array of n_sp sets: n_sp == 1 is the namesake; n_sp == batch (rows
 * for uno_filter_ex) gives request b (row r) the set sp[b] (sp[r]), so requests
 * with their own temperature, top-k, top-p and order share one call (SGLang
 * PR #37667, Changes to shared SGLang infrastructure: verification takes each
 * request's sampling parameters; run_math_eval walk-through,
 * "run_math_eval 全参数详解").  Each set keeps its own path:
 *   - the top-k path (temperature == 0, top-k on with top_k <= UNO_MAX_TOP_K,
 *     or a vocabulary of at most UNO_MAX_TOP_K), in either filter order --
 *     a joint-order set at its own temperature;
 *   - the full-vocabulary path (top-k off, temperature > 0): the full softmax
 *     when top_p == 1, its nucleus when top_p < 1.
 * Top-k supports are sized for the largest k among the top-k sets (cap for
 * uno_filter_ex).  uno_filter_ex: the rows of full-vocabulary sets receive
 * out_count and out_stats only (their out_ids / out_probs rows hold -1 / 0),
 * and out_stats is required when any set is full-vocabulary.
 * uno_build_tree_ex: K <= UNO_MAX_TOP_K when any set is full-vocabulary.
 * `sp` is host memory, read during the call: the sets reach the workspace
 * through the arguments of small kernels launched on `stream` (64 sets per
 * launch), so the caller may reuse the array once the call returns.
 * Workspace sizes come from uno_workspace_bytes_ex with the same sets. */
int uno_workspace_bytes_ex(int32_t op, int64_t batch_or_rows, int32_t B, int32_t K, int32_t V,
                           int64_t vocab, int32_t dtype, const uno_sampling_t* sp, int32_t n_sp,
                           size_t* out_bytes);
int uno_filter_ex(const void* logits, int32_t dtype, int64_t rows, int64_t vocab,
                  const uno_sampling_t* sp, int32_t n_sp, int32_t cap,
                  int32_t* out_ids, double* out_probs, int32_t* out_count, double* out_stats,
                  void* ws, size_t ws_bytes, hipStream_t stream);
int uno_sample_linear_ex(const void* draft, const void* target, int32_t dtype, int32_t batch,
                         int32_t B, int64_t vocab, const uno_sampling_t* sp, int32_t n_sp,
                         uint64_t seed, uint64_t offset, const uint32_t* request_ids,
                         int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_proposals,
                         uint32_t* out_flags, void* ws, size_t ws_bytes, hipStream_t stream);
int uno_build_tree_ex(const void* draft, int32_t dtype, int32_t batch, int32_t B, int32_t K,
                      int32_t V, int64_t vocab, const uno_sampling_t* sp, int32_t n_sp,
                      int32_t* node_token, int32_t* node_parent, int32_t* node_depth,
                      double* node_score, int32_t* num_nodes,
                      void* ws, size_t ws_bytes, hipStream_t stream);
int uno_verify_tree_ex(const void* target, int32_t dtype, int32_t batch, int32_t B, int32_t V,
                       int64_t vocab, const uno_sampling_t* sp, int32_t n_sp, uint64_t seed,
                       uint64_t offset, const uint32_t* request_ids,
                       const int32_t* node_token, const int32_t* node_parent, const int32_t* num_nodes,
                       int32_t* out_tokens, int32_t* out_path, int32_t* out_accept_len,
                       uint32_t* out_flags, void* ws, size_t ws_bytes, hipStream_t stream);

/* Tree-suffix attention merged with the prefix attention state.  (PR #37667,
 * Modifications: an UNO-only fused kernel for tree-suffix attention and LSE
 * merge; Changes to shared SGLang infrastructure: it serves UNO tree
 * verification, where cascade attention takes the shared prefix once.)
 * The n verify tokens of request b (token t = b * n + i) are the nodes of its
 * tree (node 0 the root; node_parent as uno_build_tree writes it, parents
 * before children).  The query of node i, head h, attends to the suffix keys
 * of node i and its ancestors (key/value head h / (Hq / Hkv)) with scores
 * scale * q.k, giving (o_s, lse_s); with the same query's prefix state
 * (o_p, lse_p) -- its attention over the shared context, computed elsewhere --
 *   out_lse = log(exp(lse_p) + exp(lse_s)),
 *   out = exp(lse_p - out_lse) o_p + exp(lse_s - out_lse) o_s,
 * i.e. softmax attention over the prefix keys and the visible suffix keys.
 *   q, o_prefix, out [batch * n][Hq][D], k, v [batch * n][Hkv][D]: bf16
 *   lse_prefix, out_lse [batch * n][Hq]: fp32, natural log (-inf: no prefix)
 *   node_parent [batch][n]; num_nodes [batch] (nullable: n for every request)
 * Tokens at or past num_nodes[b] are neither read nor written.  Scores,
 * softmax and sums run in fp32.  No workspace.
 * Requires dtype UNO_BF16 and D == 128 (else UNO_ERR_UNSUPPORTED),
 * 1 <= n <= UNO_MAX_TREE_NODES + 1, Hq % Hkv == 0, scale > 0, and k, v
 * 16-byte aligned. */
int uno_tree_attention(const void* q, const void* k, const void* v, const void* o_prefix,
                       const float* lse_prefix, const int32_t* node_parent, const int32_t* num_nodes,
                       int32_t dtype, int32_t batch, int32_t n, int32_t Hq, int32_t Hkv, int32_t D,
                       float scale, void* out, float* out_lse, hipStream_t stream);

/* Allocation-free linear cycle, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  uno_sample_linear with the same arguments, but without a
 * workspace argument: the workspace is a fixed array of
 * UNO_NOALLOC_SCRATCH_BYTES in device memory that the library holds on each
 * GPU it runs on until the process ends (its address is looked up once per
 * device, on the first call there).  The call allocates nothing and calls no
 * allocating routine.  A call whose workspace (uno_workspace_bytes for
 * UNO_OP_SAMPLE_LINEAR with the same arguments) exceeds the array returns
 * UNO_ERR_SCRATCH_LIMIT and launches nothing; other errors as for
 * uno_sample_linear.  Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (different streams, or threads not ordered with each
 * other) race and must be serialised by the caller; the array keeps the last
 * call's contents, which no call reads before writing.  The GPU is the one
 * `stream` belongs to (the current device for the null stream). */
#define UNO_NOALLOC_SCRATCH_BYTES (32u << 20)
int uno_sample_linear_noalloc(const void* draft, const void* target, int32_t dtype, int32_t batch,
                              int32_t B, int64_t vocab, const uno_sampling_t* sp, uint64_t seed,
                              uint64_t offset, const uint32_t* request_ids,
                              int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_proposals,
                              uint32_t* out_flags, hipStream_t stream);

/* Measurement aid, not part of the sampling path: reads `bytes` of device
 * memory at `buf` once, in ranges of wg_bytes per workgroup, with the load
 * idiom of the top-k stream (16-byte non-temporal loads, the next iteration's
 * loads in flight), and writes one folded word per workgroup to
 * out[ceil(bytes / wg_bytes)].  Its duration is the achievable streaming rate
 * of that decomposition on the device (wg_bytes = one logit row: the top-k
 * stream's; small equal ranges: the chip's).  bytes and wg_bytes must be
 * multiples of 16 and buf 16-byte aligned (else UNO_ERR_INVALID_ARG). */
int uno_stream_read(const void* buf, int64_t bytes, int64_t wg_bytes, uint32_t* out, hipStream_t stream);

/* Static description of a status code. */
const char* uno_status_string(int status);

/* hipError_t of the last failed launch on this host thread (0 if none). */
int uno_last_hip_error(void);

/* Library version string. */
const char* uno_version(void);

#ifdef __cplusplus
}
#endif

#endif /* UNO_H */
