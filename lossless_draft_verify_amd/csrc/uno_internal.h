// uno_internal.h -- kernel launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace uno {

// Where logit row r lives.  Rows [0, rows0) are src0[r], rows [rows0, rows)
// are src1[r - rows0].  When num_nodes is set (tree verification), row r of
// src0 belongs to request r / rows_per_req and is skipped when its index in
// the request is >= num_nodes[request].
struct RowSource {
    const char* src0;
    int64_t rows0;
    const char* src1;
    const int32_t* num_nodes;
    int32_t rows_per_req;
};

// How a row is filtered (FilterParams::dense).
constexpr int32_t kRowTopK = 0;      // top-k path (greedy, top-k on, or a small vocabulary)
constexpr int32_t kRowFull = 1;      // full softmax (top-k off, top-p off)
constexpr int32_t kRowNucleus = 2;   // full-vocabulary nucleus (top-k off, top-p on)

struct FilterParams {
    float temperature;
    float top_p;
    int32_t k;        // effective top-k (1 when greedy)
    int32_t greedy;   // temperature == 0
    int32_t topp_on;  // top_p < 1
    float thr_init;   // -inf: initial admission threshold of the top-k stream
    // joint order: exact chunk statistics of the same rows, whose full-softmax
    // normaliser the top-p cut reads (null in the default order) ...
    const float* full_cmax;
    const double* full_csum;
    int32_t full_nc;
    // ... or, with joint set, the top-k stream sums the normaliser itself
    // (whole rows only, launched with joint_sums)
    int32_t joint;
    // kRowTopK / kRowFull / kRowNucleus: the dense kernels take the rows (and
    // the requests) that are not kRowTopK, the top-k samplers the others
    int32_t dense;
    // the top-k stream and merge leave this row alone (a full-vocabulary row of
    // a call that samples it with the dense kernels)
    int32_t skip_topk;
};

// Compact per-row supports in filter order.
struct SparseOut {
    int32_t* ids;      // [rows][cap]
    double* probs;     // [rows][cap]
    int32_t* count;    // [rows]; -1 invalid row
    double* stats;     // [rows][2] (m, S) or nullptr
    int32_t cap;
    // nullptr: ids/probs in filter order.  Otherwise [rows][cap]: the support
    // is stored in ascending id order, with its inclusive cumulative sums taken
    // in that order (the samplers' inverse CDF, computed once per row).
    double* cum;
};

// Per-chunk statistics of dense rows: m_c = chunk max, s_c = sum over the
// chunk of exp((z - m_c)/T), n_c = finite logits in the chunk.
struct DenseChunks {
    float* cmax;       // [rows][nchunks]
    double* csum;      // [rows][nchunks]
    int32_t* ccount;   // [rows][nchunks], or nullptr when no caller needs the counts
    // [rows][nchunks] bound on |csum - exact sum| for chunks summed with fp32
    // exponentials (0 for exact chunks), or nullptr when every row is exact
    float* cerr;
    // [3] counters of the linear samplers' lists (two of rows to make exact,
    // one of requests), set to 0 by the chunk pass (which runs before any
    // sampler appends), or nullptr
    uint32_t* xcount;
    int32_t nchunks;
    // [rows] keep thresholds of a full-vocabulary nucleus, or nullptr: logit i of
    // row r is in the support iff order_key(float_key(z_i), i) >= keep[r] (the
    // chunk sums are then sums over the support)
    uint64_t* keep;
};

// Request of row r: kind 0 one row per request, 1 linear (batch*B draft rows,
// then B+1 target rows per request), 2 rows_per_req consecutive rows each.
struct RowMap {
    int kind;
    int64_t batch;
    int32_t B;
    int32_t rows_per_req;
    __host__ __device__ int64_t req(int64_t r) const
    {
        if (kind == 0) return r;
        if (kind == 1) return r < batch * B ? r / B : (r - batch * B) / (B + 1);
        return r / rows_per_req;
    }
};

// Per-request filter parameters passed by value to launch_expand_params
// (64 sets: about 3 KB of kernel arguments).
constexpr int kParamSlots = 64;
struct ParamArgs {
    FilterParams p[kParamSlots];
};

constexpr int kDenseChunk = 2048;          // elements per dense chunk
constexpr int kMergeCap = 4096;            // candidates one merge workgroup holds
constexpr int kMaxSegments = 64;           // segments per row of the top-k stream

inline int32_t dense_nchunks(int64_t vocab) { return (int32_t)((vocab + kDenseChunk - 1) / kDenseChunk); }

// Segments per row for the top-k stream (rows * S workgroups).
int topk_segments(int64_t rows, int64_t vocab, int k);

size_t align_up(size_t x, size_t a);

// ---- launchers (return hipGetLastError() after the launch) ----------------
// Segment lists hold part_cap entries each; rowp (nullable): per-row
// parameters replacing fp (k at most part_cap, the k the segments were chosen
// for).  joint_sums (S == 1 only): the stream also sums each joint row's
// full-softmax normaliser.
hipError_t launch_topk_filter(const RowSource& src, int64_t rows, int64_t vocab, bool bf16,
                              const FilterParams& fp, const SparseOut& out, int S,
                              uint32_t* part_key, int32_t* part_id, int32_t* part_n, int part_cap,
                              const FilterParams* rowp, bool joint_sums, hipStream_t stream);

// out[r] = a.p[map.req(r) - first] for every row r whose request lies in
// [first, first + n), n <= kParamSlots (only those rows are written).
hipError_t launch_expand_params(const ParamArgs& a, int64_t first, int n, const RowMap& map, FilterParams* out,
                                hipStream_t stream);

// Which rows a chunk pass with per-row parameters takes.
constexpr int kChunkJointRows = 1;   // rows whose set is in the joint order (full_cmax set)
constexpr int kChunkDenseRows = 2;   // rows whose set is not kRowTopK

// Rows below exact_rows get exact (fp64 exp) chunk sums; the rest fast ones.
// rowp (nullable, device): per-row parameters; the pass then takes only the
// rows `select` names (nothing read or written for the others), each at its
// own temperature, and joint-order and nucleus rows always get exact sums.
// active_rows (when >= 0): how many rows the selection takes, which sets how
// many workgroups share each row.
hipError_t launch_dense_chunks(const RowSource& src, int64_t rows, int64_t vocab, bool bf16,
                               float temperature, const DenseChunks& dc, int64_t exact_rows, hipStream_t stream,
                               const FilterParams* rowp = nullptr, int select = 0, int64_t active_rows = -1);

// rowp (nullable): per-row temperatures; only the kRowFull rows are written.
hipError_t launch_dense_row_stats(int64_t rows, float temperature, const DenseChunks& dc,
                                  int32_t* out_count, double* out_stats, hipStream_t stream,
                                  const FilterParams* rowp = nullptr);

struct LinearOut {
    int32_t* tokens;
    int32_t* accept_len;
    int32_t* proposals;
    uint32_t* flags;
};

// rowp (nullable): per-row parameters; requests whose rows skip the top-k
// stream are left to the dense samplers.
hipError_t launch_linear_sparse(int32_t batch, int32_t B, const SparseOut& sup, uint64_t seed,
                                uint64_t offset, const uint32_t* request_ids, const LinearOut& o,
                                hipStream_t stream, const FilterParams* rowp = nullptr);

// Scratch of the dense linear path.
struct DenseScratch {
    float* row_m;      // [rows]
    double* row_S;     // [rows]
    double* row_E;     // [rows] bound on |row_S - exact S| (0: exact sums)
    int32_t* jstar;    // [batch]
    int32_t* y;        // [batch][B]
    int32_t* acc;      // [batch][B] acceptance results before they are settled
    uint32_t* flags;   // [batch]
    double* resid;     // [batch][nchunks]
    double* resid_err; // [batch][nchunks] bound on |resid - exact| of the fp32 residual totals
    int32_t* fin_redo; // [batch] the last draw was not certain: the exact kernels take it again
    int64_t* xrows;    // [2][batch * (2B + 1)] rows to make exact: after the draws, after the last draw
    int32_t* xreq;     // [batch] requests whose last draw the exact kernels take
};

// With exact_all every row's chunk sums are already exact (the nucleus needs
// them); otherwise every row has fast sums with error bounds, the proposal
// kernel certifies its draws and acceptance tests against them (redoing the
// uncertain ones from exact sums), and the rows each request draws its last
// token from are recomputed exactly.  rowp (nullable): per-row
// parameters; only the requests whose rows are not kRowTopK are sampled, each
// at its own temperature (a nucleus request's target rows are exact already).
hipError_t launch_linear_dense(const RowSource& src, int32_t batch, int32_t B, int64_t vocab,
                               bool bf16, float temperature, const DenseChunks& dc,
                               const DenseScratch& sc, uint64_t seed, uint64_t offset,
                               const uint32_t* request_ids, const LinearOut& o, bool exact_all,
                               hipStream_t stream, const FilterParams* rowp = nullptr);

// Full-vocabulary nucleus (top-p without top-k) of `rows` rows with exact chunk
// statistics in dc: writes dc.keep, rewrites dc.csum to sums over each row's
// support, and (when non-null) the support sizes and (m, S) statistics.
// rowp (nullable): per-row parameters; kRowNucleus rows are cut at their own
// temperature and top_p, kRowFull rows get keep = 0 (the whole vocabulary),
// kRowTopK rows are left alone.  active_rows (when >= 0): how many rows are
// nucleus rows, which sets the workgroup size.
hipError_t launch_nucleus(const RowSource& src, int64_t rows, int64_t vocab, bool bf16, float temperature,
                          float top_p, const DenseChunks& dc, int32_t* out_count, double* out_stats,
                          hipStream_t stream, const FilterParams* rowp = nullptr, int64_t active_rows = -1);

struct TreeOut {
    int32_t* node_token;
    int32_t* node_parent;
    int32_t* node_depth;
    double* node_score;
    int32_t* num_nodes;
};

hipError_t launch_tree_build(int32_t batch, int32_t B, int32_t K, int32_t V, const SparseOut& sup,
                             const TreeOut& o, hipStream_t stream);

struct WalkOut {
    int32_t* tokens;
    int32_t* path;
    int32_t* accept_len;
    uint32_t* flags;
};

// rowp (nullable): requests whose rows skip the top-k stream are left to the
// dense walk.
hipError_t launch_tree_walk(int32_t batch, int32_t B, int32_t V, const SparseOut& sup,
                            uint64_t seed, uint64_t offset, const uint32_t* request_ids,
                            const int32_t* node_token, const int32_t* node_parent,
                            const int32_t* num_nodes, const WalkOut& o, hipStream_t stream,
                            const FilterParams* rowp = nullptr);

// Dense tree mode (filters without top-k).  The build takes the top-K supports
// and rescales them to the full softmax, or to the nucleus when the chunk sums
// are over a nucleus (sup.stats holds the top-K normaliser on entry, the new
// one on exit); `limit` (nullable) caps each row's count at its nucleus size.
// The walk samples node rows from exact chunk statistics.
// rowp (nullable): only the rows that are not kRowTopK are rescaled (each at
// its own temperature), and `limit` applies to the kRowNucleus rows.
hipError_t launch_dense_support_scale(int64_t rows, float temperature, const DenseChunks& dc,
                                      const int32_t* limit, const SparseOut& sup, hipStream_t stream,
                                      const FilterParams* rowp = nullptr);

// rowp (nullable): only the requests whose rows are not kRowTopK walk here,
// each at its own temperature.  node_draw: batch * (V + 1) entries of
// workspace, every node row's draw, which the walk then follows.
hipError_t launch_tree_walk_dense(const RowSource& src, int32_t batch, int32_t B, int32_t V, int64_t vocab,
                                  bool bf16, float temperature, const DenseChunks& dc, uint64_t seed,
                                  uint64_t offset, const uint32_t* request_ids, const int32_t* node_token,
                                  const int32_t* node_parent, const int32_t* num_nodes, int32_t* node_draw,
                                  const WalkOut& o, hipStream_t stream, const FilterParams* rowp = nullptr);

// Tree-suffix attention merged with the prefix state (head dimension 128,
// bf16 tensors, fp32 log-sum-exps); one workgroup per (request, kv head).
hipError_t launch_tree_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o_prefix,
                                 const float* lse_prefix, const int32_t* node_parent, const int32_t* num_nodes,
                                 int32_t batch, int32_t n, int32_t Hq, int32_t Hkv, float scale, uint16_t* out,
                                 float* out_lse, hipStream_t stream);

// Read-only streaming reference: workgroup g reads bytes [g*wg_bytes,
// (g+1)*wg_bytes) of buf once and writes one folded word to out[g].
hipError_t launch_stream_read(const void* buf, int64_t bytes, int64_t wg_bytes, uint32_t* out, hipStream_t stream);

}  // namespace uno
