// uno_api.cpp -- C ABI of the UNO sampling library: argument checks, workspace
// layout and kernel launches.  Every check runs on the host before any launch.
#include "uno.h"
#include "uno_internal.h"

#include <math.h>
#include <string.h>

using namespace uno;

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;

// Sampling mode of a call: of its one parameter set, or of all its per-request
// sets together.
struct Mode {
    bool greedy;     // every set is greedy
    bool topk_on;
    bool topp_on;
    bool sparse;     // every row takes the top-k path (greedy: k = 1)
    bool joint;      // some set is in the joint order with top-k and top-p on (a top-k set)
    bool nucleus;    // one set: top-p without top-k over a full vocabulary
    bool per_request;// one parameter set per request (or per row for the filter)
    bool any_sparse; // some set takes the top-k path
    bool any_dense;  // some set takes a full-vocabulary path (full softmax or nucleus)
    bool any_full;   // some set is a full softmax (top-k and top-p off)
    bool any_nucleus;// some set is a nucleus
    int32_t k;       // largest effective k over the top-k sets (1 when there is none)
    float joint_T;   // one set in the joint order: its temperature
    int64_t n_sets;  // parameter sets of the call, and how many are in the joint order / full-vocabulary / nucleus
    int64_t n_joint_sets;
    int64_t n_dense_sets;
    int64_t n_nucleus_sets;
};

// Rows a per-request chunk pass takes (select: kChunkJointRows or
// kChunkDenseRows): every set covers the same number of rows.
int64_t chunk_rows(const Mode& m, int64_t rows, int select)
{
    if (!m.per_request || m.n_sets < 1) return rows;
    const int64_t n = select == kChunkJointRows ? m.n_joint_sets : m.n_dense_sets;
    return (rows * n + m.n_sets - 1) / m.n_sets;
}

// Rows a nucleus cut takes.
int64_t nucleus_rows(const Mode& m, int64_t rows)
{
    if (!m.per_request || m.n_sets < 1) return rows;
    return (rows * m.n_nucleus_sets + m.n_sets - 1) / m.n_sets;
}

int check_sampling(const uno_sampling_t* sp, int64_t vocab, Mode* m)
{
    if (sp == nullptr) return UNO_ERR_INVALID_ARG;
    const float T = sp->temperature, p = sp->top_p;
    if (!(T >= 0.0f) || !isfinite(T)) return UNO_ERR_INVALID_ARG;       // temperature >= 0
    if (!(p > 0.0f && p <= 1.0f)) return UNO_ERR_INVALID_ARG;           // top_p in (0, 1]
    if (sp->order != UNO_ORDER_TOPK_FIRST && sp->order != UNO_ORDER_JOINT) return UNO_ERR_INVALID_ARG;
    m->greedy = (T == 0.0f);
    m->topk_on = sp->top_k > 0 && (int64_t)sp->top_k < vocab;
    m->topp_on = p < 1.0f;
    // a vocabulary of at most UNO_MAX_TOP_K ids is filtered whole by the top-k path
    m->sparse = m->greedy || m->topk_on || vocab <= UNO_MAX_TOP_K;
    m->k = m->greedy ? 1 : (m->topk_on ? sp->top_k : (int32_t)vocab);
    // the orders differ only when top-k and top-p both act on a sampled row
    m->joint = sp->order == UNO_ORDER_JOINT && !m->greedy && m->topk_on && m->topp_on;
    if (m->sparse && m->k > UNO_MAX_TOP_K) return UNO_ERR_UNSUPPORTED;
    m->nucleus = !m->sparse && m->topp_on;
    m->per_request = false;
    m->any_sparse = m->sparse;
    m->any_dense = !m->sparse;
    m->any_nucleus = m->nucleus;
    m->any_full = !m->sparse && !m->nucleus;
    m->joint_T = T;
    m->n_sets = 1;
    m->n_joint_sets = m->joint ? 1 : 0;
    m->n_dense_sets = m->sparse ? 0 : 1;
    m->n_nucleus_sets = m->nucleus ? 1 : 0;
    if (!m->sparse && vocab > (int64_t)65535 * 4 * kDenseChunk) return UNO_ERR_UNSUPPORTED;
    return UNO_OK;
}

// Sampling parameters of a call: one set for every row, or one per request.
struct SpSet {
    const uno_sampling_t* sp;
    int64_t n;
};

// One set: its mode.  One per request (n == requests): each set is checked
// alone and keeps its own path -- top-k, full softmax or nucleus -- and its
// own temperature; the combined mode says which paths the call runs, and its
// k is the largest k of the top-k sets (the stride of their supports).
int check_set(const SpSet& s, int64_t requests, int64_t vocab, Mode* m)
{
    if (s.sp == nullptr) return UNO_ERR_INVALID_ARG;
    if (s.n == 1) return check_sampling(s.sp, vocab, m);
    if (s.n != requests || s.n < 1) return UNO_ERR_INVALID_ARG;
    Mode all{};
    all.sparse = true;
    all.per_request = true;
    all.greedy = true;
    all.k = 1;
    for (int64_t i = 0; i < s.n; ++i) {
        Mode mi;
        const int st = check_sampling(&s.sp[i], vocab, &mi);
        if (st) return st;
        all.n_sets += 1;
        all.n_joint_sets += mi.joint ? 1 : 0;
        all.n_dense_sets += mi.sparse ? 0 : 1;
        all.n_nucleus_sets += mi.nucleus ? 1 : 0;
        all.greedy = all.greedy && mi.greedy;
        all.topk_on = all.topk_on || mi.topk_on;
        all.topp_on = all.topp_on || mi.topp_on;
        all.joint = all.joint || mi.joint;
        if (mi.sparse) {
            all.any_sparse = true;
            all.k = mi.k > all.k ? mi.k : all.k;
        } else {
            all.sparse = false;
            all.any_dense = true;
            all.any_nucleus = all.any_nucleus || mi.nucleus;
            all.any_full = all.any_full || !mi.nucleus;
        }
    }
    *m = all;
    return UNO_OK;
}

int check_common(int32_t dtype, int64_t vocab)
{
    if (dtype != UNO_F32 && dtype != UNO_BF16) return UNO_ERR_UNSUPPORTED;
    if (vocab < 1 || vocab > 0x7FFFFFFFLL) return UNO_ERR_INVALID_ARG;
    return UNO_OK;
}

size_t elem_size(int32_t dtype) { return dtype == UNO_BF16 ? 2 : 4; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Bump allocator over the caller's workspace (or a size-only dry run).
struct Carve {
    char* base;
    size_t used = 0;
    template <typename T>
    T* take(size_t n)
    {
        const size_t off = used;
        used = align_up(used + n * sizeof(T), kAlign);
        return base ? reinterpret_cast<T*>(base + off) : nullptr;
    }
};

struct SparseWs {
    SparseOut sup;
    int S;
    uint32_t* part_key;
    int32_t* part_id;
    int32_t* part_n;
    DenseChunks full;    // joint order: exact chunk statistics of the rows
    int32_t* nucleus_n;  // tree build with nucleus rows: support sizes
    int32_t* node_draw;  // dense tree walk: every node row's draw
    FilterParams* rowp;  // per-request parameters: one set per row
    int part_cap;        // entries per segment list (the largest k)
};

DenseChunks carve_chunks(Carve& cv, int64_t rows, int64_t vocab, bool counts, bool keep, bool err = false);

// Supports (when own_supports; in id order with cumulative sums when id_order)
// and segment partials for `rows` top-k rows with supports of m.k entries;
// with one set in the joint order, that order's chunk statistics too (per
// request, the joint rows share the call's chunk statistics instead).
void carve_sparse(Carve& cv, int64_t rows, int64_t vocab, const Mode& m, bool own_supports, bool id_order,
                  SparseWs* w)
{
    w->S = topk_segments(rows, vocab, m.k);
    w->part_cap = m.k;
    if (own_supports) {
        w->sup.cap = m.k;
        w->sup.ids = cv.take<int32_t>((size_t)rows * m.k);
        w->sup.probs = cv.take<double>((size_t)rows * m.k);
        w->sup.count = cv.take<int32_t>((size_t)rows);
        w->sup.stats = nullptr;
        w->sup.cum = id_order ? cv.take<double>((size_t)rows * m.k) : nullptr;
    }
    w->part_key = nullptr;
    w->part_id = nullptr;
    w->part_n = nullptr;
    if (w->S > 1) {
        w->part_key = cv.take<uint32_t>((size_t)rows * w->S * m.k);
        w->part_id = cv.take<int32_t>((size_t)rows * w->S * m.k);
        w->part_n = cv.take<int32_t>((size_t)rows * w->S);
    }
    w->nucleus_n = nullptr;
    if (!m.per_request) {
        w->full = DenseChunks{};
        if (m.joint) w->full = carve_chunks(cv, rows, vocab, false, false);
    }
}

// Chunk statistics; the finite counts only for uno_filter, whose dense mode
// reports each row's support size (the samplers never read them); error
// bounds for the linear samplers, which certify draws made from fast sums.
DenseChunks carve_chunks(Carve& cv, int64_t rows, int64_t vocab, bool counts, bool keep, bool err)
{
    DenseChunks dc;
    dc.nchunks = dense_nchunks(vocab);
    dc.cmax = cv.take<float>((size_t)rows * dc.nchunks);
    dc.csum = cv.take<double>((size_t)rows * dc.nchunks);
    dc.ccount = counts ? cv.take<int32_t>((size_t)rows * dc.nchunks) : nullptr;
    dc.cerr = err ? cv.take<float>((size_t)rows * dc.nchunks) : nullptr;
    dc.xcount = err ? cv.take<uint32_t>(3) : nullptr;
    dc.keep = keep ? cv.take<uint64_t>((size_t)rows) : nullptr;
    return dc;
}

DenseScratch carve_dense_scratch(Carve& cv, int64_t rows, int32_t batch, int32_t B, int32_t nchunks)
{
    DenseScratch s;
    s.row_m = cv.take<float>((size_t)rows);
    s.row_S = cv.take<double>((size_t)rows);
    s.row_E = cv.take<double>((size_t)rows);
    s.jstar = cv.take<int32_t>((size_t)batch);
    s.y = cv.take<int32_t>((size_t)batch * B);
    s.acc = cv.take<int32_t>((size_t)batch * B);
    s.flags = cv.take<uint32_t>((size_t)batch);
    s.resid = cv.take<double>((size_t)batch * nchunks);
    s.resid_err = cv.take<double>((size_t)batch * nchunks);
    s.fin_redo = cv.take<int32_t>((size_t)batch);
    s.xrows = cv.take<int64_t>((size_t)2 * rows);
    s.xreq = cv.take<int32_t>((size_t)batch);
    return s;
}

// Per-request sets: the row table, and one chunk-statistics array that the
// joint-order rows and the full-vocabulary rows share (a row is one or the
// other).
void carve_per_request(Carve& cv, int64_t rows, int64_t vocab, const Mode& m, bool counts, SparseWs* sw,
                       DenseChunks* dc, bool err = false)
{
    sw->rowp = cv.take<FilterParams>((size_t)rows);
    if (m.any_dense || m.joint) {
        *dc = carve_chunks(cv, rows, vocab, counts, m.any_nucleus, err);
        if (m.joint) sw->full = *dc;
    }
}

int check_ws(void* ws, size_t ws_bytes, size_t need)
{
    if (need == 0) return UNO_OK;
    if (ws == nullptr || ws_bytes < need || !aligned(ws, kAlign)) return UNO_ERR_WORKSPACE;
    return UNO_OK;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return UNO_OK;
    g_last_hip_error = (int)e;
    return UNO_ERR_HIP;
}

FilterParams filter_params(const uno_sampling_t* sp, const Mode& m)
{
    FilterParams fp;
    fp.temperature = sp->temperature;
    fp.top_p = sp->top_p;
    fp.k = m.k;
    fp.greedy = m.greedy ? 1 : 0;
    fp.topp_on = m.topp_on ? 1 : 0;
    fp.thr_init = -INFINITY;
    fp.full_cmax = nullptr;
    fp.full_csum = nullptr;
    fp.full_nc = 0;
    fp.joint = 0;
    fp.dense = m.sparse ? kRowTopK : (m.nucleus ? kRowNucleus : kRowFull);
    fp.skip_topk = m.sparse ? 0 : 1;
    return fp;
}

// Per-request sets to the row table (sw.rowp), on the stream: each set rides
// in the arguments of a small kernel that writes it to its request's rows
// (kParamSlots sets per launch), so the host array is not read after the call
// returns.  Joint-order rows point at the call's chunk statistics; with
// build_K > 0 (tree build) the full-vocabulary rows take the top-k stream with
// k = build_K and no top-p (their candidates are the K most likely ids, the
// probabilities rescaled to the full softmax or the nucleus afterwards).
hipError_t expand_row_params(const SpSet& sps, int64_t vocab, const RowMap& map, const SparseWs& sw,
                             int32_t build_K, hipStream_t stream)
{
    for (int64_t first = 0; first < sps.n; first += kParamSlots) {
        ParamArgs a;
        const int n = (int)(sps.n - first < kParamSlots ? sps.n - first : kParamSlots);
        for (int i = 0; i < n; ++i) {
            const uno_sampling_t* s = &sps.sp[first + i];
            Mode mi;
            check_sampling(s, vocab, &mi);
            a.p[i] = filter_params(s, mi);
            if (mi.joint) {
                a.p[i].full_cmax = sw.full.cmax;
                a.p[i].full_csum = sw.full.csum;
                a.p[i].full_nc = sw.full.nchunks;
            }
            if (build_K > 0 && !mi.sparse) {
                a.p[i].k = build_K;
                a.p[i].topp_on = 0;
                a.p[i].skip_topk = 0;
            }
        }
        const hipError_t e = launch_expand_params(a, first, n, map, sw.rowp, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The top-k filter of `rows` rows into `out` (rows of full-vocabulary sets
// skipped when per-request).  The joint order needs each row's full-softmax
// normaliser: with one set for whole rows (one segment each) the top-k stream
// sums it while it streams; otherwise exact chunk statistics of the joint rows
// come first (per request: each at its own temperature).
hipError_t launch_sparse_filter(const RowSource& src, int64_t rows, int64_t vocab, bool bf16,
                                const SpSet& sps, const Mode& m, const SparseWs& sw,
                                const SparseOut& out, hipStream_t stream)
{
    FilterParams fp = filter_params(sps.sp, m);
    // (per-request sets keep the chunk pass, over their joint rows only: the
    // summing stream runs at lower occupancy for every row of its launch)
    const bool joint_sums = m.joint && sw.S == 1 && !m.per_request;
    if (joint_sums) {
        fp.joint = 1;
    } else if (m.joint) {
        const hipError_t e = launch_dense_chunks(src, rows, vocab, bf16, m.joint_T, sw.full, rows, stream,
                                                 m.per_request ? sw.rowp : nullptr, kChunkJointRows,
                                                 chunk_rows(m, rows, kChunkJointRows));
        if (e != hipSuccess) return e;
        fp.full_cmax = sw.full.cmax;
        fp.full_csum = sw.full.csum;
        fp.full_nc = sw.full.nchunks;
    }
    return launch_topk_filter(src, rows, vocab, bf16, fp, out, sw.S, sw.part_key, sw.part_id, sw.part_n,
                              sw.part_cap, sw.rowp, joint_sums, stream);
}

int check_tree_shape(int32_t B, int32_t K, int32_t V, bool need_k)
{
    if (B < 1 || V < B || V > UNO_MAX_TREE_NODES) return UNO_ERR_INVALID_ARG;
    if (need_k && (K < 1 || (int64_t)V * K > UNO_MAX_TREE_VK)) return UNO_ERR_INVALID_ARG;
    return UNO_OK;
}

// ---- per-op layout (shared by the size query and the calls) ---------------------
int layout_filter(int64_t rows, int64_t vocab, int32_t dtype, const SpSet& sps, Carve& cv,
                  Mode* m, SparseWs* sw, DenseChunks* dc)
{
    int st = check_common(dtype, vocab);
    if (st) return st;
    if (rows < 0 || rows > 0x7FFFFFFF) return UNO_ERR_INVALID_ARG;
    st = check_set(sps, rows, vocab, m);
    if (st) return st;
    if (rows == 0) return UNO_OK;
    if (m->per_request) {
        // counts: a full-softmax row reports its number of finite logits
        carve_per_request(cv, rows, vocab, *m, m->any_full, sw, dc);
        if (m->any_sparse) carve_sparse(cv, rows, vocab, *m, false, false, sw);
    } else if (m->sparse) {
        carve_sparse(cv, rows, vocab, *m, false, false, sw);
    } else if (m->nucleus) {
        *dc = carve_chunks(cv, rows, vocab, false, true);   // counts come from the nucleus
    } else {
        *dc = carve_chunks(cv, rows, vocab, true, false);
    }
    return UNO_OK;
}

int layout_linear(int64_t batch, int32_t B, int64_t vocab, int32_t dtype, const SpSet& sps,
                  Carve& cv, Mode* m, SparseWs* sw, DenseChunks* dc, DenseScratch* ds)
{
    int st = check_common(dtype, vocab);
    if (st) return st;
    if (batch < 0 || B < 1 || B > 128 || batch * (2 * (int64_t)B + 1) > 0x7FFFFFFF) return UNO_ERR_INVALID_ARG;
    st = check_set(sps, batch, vocab, m);
    if (st) return st;
    if (batch == 0) return UNO_OK;
    const int64_t rows = batch * (2 * (int64_t)B + 1);
    if (m->per_request) carve_per_request(cv, rows, vocab, *m, false, sw, dc, true);
    if (m->any_sparse) carve_sparse(cv, rows, vocab, *m, true, true, sw);
    if (m->any_dense) {
        if (!m->per_request) *dc = carve_chunks(cv, rows, vocab, false, m->nucleus, true);
        *ds = carve_dense_scratch(cv, rows, (int32_t)batch, B, dc->nchunks);
    }
    return UNO_OK;
}

int layout_tree(int32_t op, int64_t batch, int32_t B, int32_t K, int32_t V, int64_t vocab, int32_t dtype,
                const SpSet& sps, Carve& cv, Mode* m, SparseWs* sw, DenseChunks* dc)
{
    int st = check_common(dtype, vocab);
    if (st) return st;
    if (batch < 0 || batch * ((int64_t)V + 1) > 0x7FFFFFFF) return UNO_ERR_INVALID_ARG;
    const bool build = op == UNO_OP_BUILD_TREE;
    st = check_tree_shape(B, K, V, build);
    if (st) return st;
    st = check_set(sps, batch, vocab, m);
    if (st) return st;
    // a full-vocabulary build selects its K candidates with the top-k path
    if (m->any_dense && build && K > UNO_MAX_TOP_K) return UNO_ERR_UNSUPPORTED;
    if (batch == 0) return UNO_OK;
    const int64_t rows = batch * (build ? (int64_t)B : (int64_t)V + 1);
    if (m->per_request) carve_per_request(cv, rows, vocab, *m, false, sw, dc);
    if (build) {
        // every row's candidates in filter order: the top-k rows with their own
        // k, the full-vocabulary rows with k = K (rescaled afterwards)
        Mode mk = *m;
        if (m->any_dense) mk.k = (m->any_sparse && m->k > K) ? m->k : K;
        carve_sparse(cv, rows, vocab, mk, true, false, sw);
        if (m->any_dense) {
            sw->sup.stats = cv.take<double>((size_t)rows * 2);
            if (!m->per_request) *dc = carve_chunks(cv, rows, vocab, false, m->nucleus);
            sw->nucleus_n = m->any_nucleus ? cv.take<int32_t>((size_t)rows) : nullptr;
        }
    } else {
        // the walk samples top-k rows in id order
        if (m->any_sparse) carve_sparse(cv, rows, vocab, *m, true, true, sw);
        if (m->any_dense && !m->per_request) *dc = carve_chunks(cv, rows, vocab, false, m->nucleus);
        sw->node_draw = m->any_dense ? cv.take<int32_t>((size_t)rows) : nullptr;
    }
    return UNO_OK;
}

}  // namespace

extern "C" {

int uno_workspace_bytes_ex(int32_t op, int64_t batch_or_rows, int32_t B, int32_t K, int32_t V, int64_t vocab,
                           int32_t dtype, const uno_sampling_t* sp, int32_t n_sp, size_t* out_bytes)
{
    const SpSet sps{ sp, n_sp };
    if (out_bytes == nullptr) return UNO_ERR_INVALID_ARG;
    Carve cv{ nullptr };
    Mode m;
    SparseWs sw{};
    DenseChunks dc{};
    DenseScratch ds{};
    int st;
    switch (op) {
    case UNO_OP_FILTER: st = layout_filter(batch_or_rows, vocab, dtype, sps, cv, &m, &sw, &dc); break;
    case UNO_OP_SAMPLE_LINEAR: st = layout_linear(batch_or_rows, B, vocab, dtype, sps, cv, &m, &sw, &dc, &ds); break;
    case UNO_OP_BUILD_TREE:
    case UNO_OP_VERIFY_TREE: st = layout_tree(op, batch_or_rows, B, K, V, vocab, dtype, sps, cv, &m, &sw, &dc); break;
    default: return UNO_ERR_INVALID_ARG;
    }
    if (st) return st;
    *out_bytes = cv.used;
    return UNO_OK;
}

int uno_filter_ex(const void* logits, int32_t dtype, int64_t rows, int64_t vocab, const uno_sampling_t* sp,
                  int32_t n_sp, int32_t cap, int32_t* out_ids, double* out_probs, int32_t* out_count,
                  double* out_stats, void* ws, size_t ws_bytes, hipStream_t stream)
{
    const SpSet sps{ sp, n_sp };
    const RowMap map{ 0, rows, 0, 1 };
    Carve sizing{ nullptr };
    Mode m;
    SparseWs sw{};
    DenseChunks dc{};
    int st = layout_filter(rows, vocab, dtype, sps, sizing, &m, &sw, &dc);
    if (st) return st;
    if (rows == 0) return UNO_OK;
    if (logits == nullptr || out_count == nullptr || !aligned(logits, elem_size(dtype))) return UNO_ERR_INVALID_ARG;
    if (m.any_sparse && (out_ids == nullptr || out_probs == nullptr || cap < m.k)) return UNO_ERR_INVALID_ARG;
    if (m.any_dense && out_stats == nullptr) return UNO_ERR_INVALID_ARG;
    st = check_ws(ws, ws_bytes, sizing.used);
    if (st) return st;
    Carve cv{ static_cast<char*>(ws) };
    layout_filter(rows, vocab, dtype, sps, cv, &m, &sw, &dc);

    RowSource src{ static_cast<const char*>(logits), rows, nullptr, nullptr, 1 };
    const bool bf16 = dtype == UNO_BF16;
    const FilterParams* rowp = m.per_request ? sw.rowp : nullptr;
    hipError_t e = hipSuccess;
    if (m.per_request) e = expand_row_params(sps, vocab, map, sw, 0, stream);
    if (e == hipSuccess && m.any_sparse) {
        SparseOut out{ out_ids, out_probs, out_count, out_stats, cap, nullptr };
        e = launch_sparse_filter(src, rows, vocab, bf16, sps, m, sw, out, stream);
    }
    if (e == hipSuccess && m.any_dense) {
        e = launch_dense_chunks(src, rows, vocab, bf16, sp->temperature, dc, rows, stream, rowp, kChunkDenseRows,
                                chunk_rows(m, rows, kChunkDenseRows));
        if (e == hipSuccess && m.any_nucleus)
            e = launch_nucleus(src, rows, vocab, bf16, sp->temperature, sp->top_p, dc, out_count, out_stats, stream,
                               rowp, nucleus_rows(m, rows));
        if (e == hipSuccess && m.any_full)
            e = launch_dense_row_stats(rows, sp->temperature, dc, out_count, out_stats, stream, rowp);
    }
    return hip_status(e);
}

int uno_sample_linear_ex(const void* draft, const void* target, int32_t dtype, int32_t batch, int32_t B,
                         int64_t vocab, const uno_sampling_t* sp, int32_t n_sp, uint64_t seed, uint64_t offset,
                         const uint32_t* request_ids, int32_t* out_tokens, int32_t* out_accept_len,
                         int32_t* out_proposals, uint32_t* out_flags, void* ws, size_t ws_bytes,
                         hipStream_t stream)
{
    const SpSet sps{ sp, n_sp };
    const RowMap map{ 1, batch, B, 1 };
    Carve sizing{ nullptr };
    Mode m;
    SparseWs sw{};
    DenseChunks dc{};
    DenseScratch ds{};
    int st = layout_linear(batch, B, vocab, dtype, sps, sizing, &m, &sw, &dc, &ds);
    if (st) return st;
    if (batch == 0) return UNO_OK;
    const size_t es = elem_size(dtype);
    if (draft == nullptr || target == nullptr || out_tokens == nullptr || out_accept_len == nullptr ||
        !aligned(draft, es) || !aligned(target, es))
        return UNO_ERR_INVALID_ARG;
    st = check_ws(ws, ws_bytes, sizing.used);
    if (st) return st;
    Carve cv{ static_cast<char*>(ws) };
    layout_linear(batch, B, vocab, dtype, sps, cv, &m, &sw, &dc, &ds);

    const int64_t rows = (int64_t)batch * (2 * B + 1);
    RowSource src{ static_cast<const char*>(draft), (int64_t)batch * B, static_cast<const char*>(target),
                   nullptr, 1 };
    const bool bf16 = dtype == UNO_BF16;
    const FilterParams* rowp = m.per_request ? sw.rowp : nullptr;
    LinearOut o{ out_tokens, out_accept_len, out_proposals, out_flags };
    hipError_t e = hipSuccess;
    if (m.per_request) e = expand_row_params(sps, vocab, map, sw, 0, stream);
    if (e == hipSuccess && m.any_sparse) {
        e = launch_sparse_filter(src, rows, vocab, bf16, sps, m, sw, sw.sup, stream);
        if (e == hipSuccess) e = launch_linear_sparse(batch, B, sw.sup, seed, offset, request_ids, o, stream, rowp);
    }
    if (e == hipSuccess && m.any_dense) {
        // fast sums with error bounds on every row: the samplers certify each
        // draw and acceptance against the bounds and redo the rare uncertain
        // ones from exact sums; the rows each request draws its last token
        // from are recomputed exactly (a nucleus needs exact sums on every
        // row: one set, all rows; per request, the chunk pass makes the
        // nucleus rows exact itself)
        const bool exact_all = !m.per_request && m.nucleus;
        e = launch_dense_chunks(src, rows, vocab, bf16, sp->temperature, dc, exact_all ? rows : 0, stream, rowp,
                                kChunkDenseRows, chunk_rows(m, rows, kChunkDenseRows));
        if (e == hipSuccess && m.any_nucleus)
            e = launch_nucleus(src, rows, vocab, bf16, sp->temperature, sp->top_p, dc, nullptr, nullptr, stream, rowp,
                               nucleus_rows(m, rows));
        if (e == hipSuccess)
            e = launch_linear_dense(src, batch, B, vocab, bf16, sp->temperature, dc, ds, seed, offset,
                                    request_ids, o, exact_all, stream, rowp);
    }
    return hip_status(e);
}

int uno_build_tree_ex(const void* draft, int32_t dtype, int32_t batch, int32_t B, int32_t K, int32_t V,
                      int64_t vocab, const uno_sampling_t* sp, int32_t n_sp, int32_t* node_token,
                      int32_t* node_parent, int32_t* node_depth, double* node_score, int32_t* num_nodes, void* ws,
                      size_t ws_bytes, hipStream_t stream)
{
    const SpSet sps{ sp, n_sp };
    const RowMap map{ 2, batch, B, B };
    Carve sizing{ nullptr };
    Mode m;
    SparseWs sw{};
    DenseChunks dc{};
    int st = layout_tree(UNO_OP_BUILD_TREE, batch, B, K, V, vocab, dtype, sps, sizing, &m, &sw, &dc);
    if (st) return st;
    if (batch == 0) return UNO_OK;
    if (draft == nullptr || node_token == nullptr || node_parent == nullptr || node_depth == nullptr ||
        num_nodes == nullptr || !aligned(draft, elem_size(dtype)))
        return UNO_ERR_INVALID_ARG;
    st = check_ws(ws, ws_bytes, sizing.used);
    if (st) return st;
    Carve cv{ static_cast<char*>(ws) };
    layout_tree(UNO_OP_BUILD_TREE, batch, B, K, V, vocab, dtype, sps, cv, &m, &sw, &dc);

    const int64_t rows = (int64_t)batch * B;
    const bool bf16 = dtype == UNO_BF16;
    RowSource src{ static_cast<const char*>(draft), rows, nullptr, nullptr, 1 };
    hipError_t e = hipSuccess;
    if (m.per_request) {
        // each row with its own set; the full-vocabulary rows: exact row
        // normalisers (over the nucleus when top-p is on) first, then the K
        // best ids by the same stream as the top-k rows, then their
        // probabilities under the full softmax (renormalised over the nucleus)
        e = expand_row_params(sps, vocab, map, sw, K, stream);
        if (e == hipSuccess && m.any_dense)
            e = launch_dense_chunks(src, rows, vocab, bf16, sp->temperature, dc, rows, stream, sw.rowp,
                                    kChunkDenseRows, chunk_rows(m, rows, kChunkDenseRows));
        if (e == hipSuccess && m.any_nucleus)
            e = launch_nucleus(src, rows, vocab, bf16, sp->temperature, sp->top_p, dc, sw.nucleus_n, nullptr, stream,
                               sw.rowp, nucleus_rows(m, rows));
        if (e == hipSuccess) e = launch_sparse_filter(src, rows, vocab, bf16, sps, m, sw, sw.sup, stream);
        if (e == hipSuccess && m.any_dense)
            e = launch_dense_support_scale(rows, sp->temperature, dc, sw.nucleus_n, sw.sup, stream, sw.rowp);
    } else if (m.sparse) {
        e = launch_sparse_filter(src, rows, vocab, bf16, sps, m, sw, sw.sup, stream);
    } else {
        // full-vocabulary filter: exact row normalisers (over the nucleus when
        // top-p is on), the K best ids, then their probabilities under the
        // full softmax (renormalised over the nucleus)
        Mode mk = m;
        mk.k = K;
        mk.topp_on = false;
        mk.sparse = true;     // the K best ids come from the top-k stream
        e = launch_dense_chunks(src, rows, vocab, bf16, sp->temperature, dc, rows, stream);
        if (e == hipSuccess && m.nucleus)
            e = launch_nucleus(src, rows, vocab, bf16, sp->temperature, sp->top_p, dc, sw.nucleus_n, nullptr, stream);
        if (e == hipSuccess)
            e = launch_topk_filter(src, rows, vocab, bf16, filter_params(sp, mk), sw.sup, sw.S, sw.part_key,
                                   sw.part_id, sw.part_n, sw.part_cap, nullptr, false, stream);
        if (e == hipSuccess)
            e = launch_dense_support_scale(rows, sp->temperature, dc, sw.nucleus_n, sw.sup, stream);
    }
    if (e == hipSuccess) {
        TreeOut o{ node_token, node_parent, node_depth, node_score, num_nodes };
        e = launch_tree_build(batch, B, K, V, sw.sup, o, stream);
    }
    return hip_status(e);
}

int uno_verify_tree_ex(const void* target, int32_t dtype, int32_t batch, int32_t B, int32_t V, int64_t vocab,
                       const uno_sampling_t* sp, int32_t n_sp, uint64_t seed, uint64_t offset,
                       const uint32_t* request_ids, const int32_t* node_token, const int32_t* node_parent,
                       const int32_t* num_nodes, int32_t* out_tokens, int32_t* out_path, int32_t* out_accept_len,
                       uint32_t* out_flags, void* ws, size_t ws_bytes, hipStream_t stream)
{
    const SpSet sps{ sp, n_sp };
    const RowMap map{ 2, batch, B, V + 1 };
    Carve sizing{ nullptr };
    Mode m;
    SparseWs sw{};
    DenseChunks dc{};
    int st = layout_tree(UNO_OP_VERIFY_TREE, batch, B, 1, V, vocab, dtype, sps, sizing, &m, &sw, &dc);
    if (st) return st;
    if (batch == 0) return UNO_OK;
    if (target == nullptr || node_token == nullptr || node_parent == nullptr || num_nodes == nullptr ||
        out_tokens == nullptr || out_path == nullptr || out_accept_len == nullptr ||
        !aligned(target, elem_size(dtype)))
        return UNO_ERR_INVALID_ARG;
    st = check_ws(ws, ws_bytes, sizing.used);
    if (st) return st;
    Carve cv{ static_cast<char*>(ws) };
    layout_tree(UNO_OP_VERIFY_TREE, batch, B, 1, V, vocab, dtype, sps, cv, &m, &sw, &dc);

    const int64_t rows = (int64_t)batch * (V + 1);
    const bool bf16 = dtype == UNO_BF16;
    RowSource src{ static_cast<const char*>(target), rows, nullptr, num_nodes, V + 1 };
    const FilterParams* rowp = m.per_request ? sw.rowp : nullptr;
    WalkOut o{ out_tokens, out_path, out_accept_len, out_flags };
    hipError_t e = hipSuccess;
    if (m.per_request) e = expand_row_params(sps, vocab, map, sw, 0, stream);
    if (e == hipSuccess && m.any_sparse) {
        e = launch_sparse_filter(src, rows, vocab, bf16, sps, m, sw, sw.sup, stream);
        if (e == hipSuccess)
            e = launch_tree_walk(batch, B, V, sw.sup, seed, offset, request_ids, node_token, node_parent,
                                 num_nodes, o, stream, rowp);
    }
    if (e == hipSuccess && m.any_dense) {
        // every node row a walk may sample gets exact chunk statistics (and
        // its nucleus when top-p is on)
        e = launch_dense_chunks(src, rows, vocab, bf16, sp->temperature, dc, rows, stream, rowp, kChunkDenseRows,
                                chunk_rows(m, rows, kChunkDenseRows));
        if (e == hipSuccess && m.any_nucleus)
            e = launch_nucleus(src, rows, vocab, bf16, sp->temperature, sp->top_p, dc, nullptr, nullptr, stream, rowp,
                               nucleus_rows(m, rows));
        if (e == hipSuccess)
            e = launch_tree_walk_dense(src, batch, B, V, vocab, bf16, sp->temperature, dc, seed, offset,
                                       request_ids, node_token, node_parent, num_nodes, sw.node_draw, o, stream,
                                       rowp);
    }
    return hip_status(e);
}

// ---- one parameter set for every row -------------------------------------------
int uno_workspace_bytes(int32_t op, int64_t batch_or_rows, int32_t B, int32_t K, int32_t V, int64_t vocab,
                        int32_t dtype, const uno_sampling_t* sp, size_t* out_bytes)
{
    return uno_workspace_bytes_ex(op, batch_or_rows, B, K, V, vocab, dtype, sp, 1, out_bytes);
}

int uno_filter(const void* logits, int32_t dtype, int64_t rows, int64_t vocab, const uno_sampling_t* sp,
               int32_t cap, int32_t* out_ids, double* out_probs, int32_t* out_count, double* out_stats,
               void* ws, size_t ws_bytes, hipStream_t stream)
{
    return uno_filter_ex(logits, dtype, rows, vocab, sp, 1, cap, out_ids, out_probs, out_count, out_stats, ws,
                         ws_bytes, stream);
}

int uno_sample_linear(const void* draft, const void* target, int32_t dtype, int32_t batch, int32_t B,
                      int64_t vocab, const uno_sampling_t* sp, uint64_t seed, uint64_t offset,
                      const uint32_t* request_ids, int32_t* out_tokens, int32_t* out_accept_len,
                      int32_t* out_proposals, uint32_t* out_flags, void* ws, size_t ws_bytes,
                      hipStream_t stream)
{
    return uno_sample_linear_ex(draft, target, dtype, batch, B, vocab, sp, 1, seed, offset, request_ids, out_tokens,
                                out_accept_len, out_proposals, out_flags, ws, ws_bytes, stream);
}

int uno_build_tree(const void* draft, int32_t dtype, int32_t batch, int32_t B, int32_t K, int32_t V,
                   int64_t vocab, const uno_sampling_t* sp, int32_t* node_token, int32_t* node_parent,
                   int32_t* node_depth, double* node_score, int32_t* num_nodes, void* ws, size_t ws_bytes,
                   hipStream_t stream)
{
    return uno_build_tree_ex(draft, dtype, batch, B, K, V, vocab, sp, 1, node_token, node_parent, node_depth,
                             node_score, num_nodes, ws, ws_bytes, stream);
}

int uno_verify_tree(const void* target, int32_t dtype, int32_t batch, int32_t B, int32_t V, int64_t vocab,
                    const uno_sampling_t* sp, uint64_t seed, uint64_t offset, const uint32_t* request_ids,
                    const int32_t* node_token, const int32_t* node_parent, const int32_t* num_nodes,
                    int32_t* out_tokens, int32_t* out_path, int32_t* out_accept_len, uint32_t* out_flags,
                    void* ws, size_t ws_bytes, hipStream_t stream)
{
    return uno_verify_tree_ex(target, dtype, batch, B, V, vocab, sp, 1, seed, offset, request_ids, node_token,
                              node_parent, num_nodes, out_tokens, out_path, out_accept_len, out_flags, ws, ws_bytes,
                              stream);
}

int uno_tree_attention(const void* q, const void* k, const void* v, const void* o_prefix, const float* lse_prefix,
                       const int32_t* node_parent, const int32_t* num_nodes, int32_t dtype, int32_t batch,
                       int32_t n, int32_t Hq, int32_t Hkv, int32_t D, float scale, void* out, float* out_lse,
                       hipStream_t stream)
{
    if (dtype != UNO_BF16 || D != 128) return UNO_ERR_UNSUPPORTED;
    if (batch < 0 || n < 1 || n > UNO_MAX_TREE_NODES + 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
        Hkv > 65535 || !(scale > 0.0f) || !isfinite(scale))
        return UNO_ERR_INVALID_ARG;
    if (batch == 0) return UNO_OK;
    if (q == nullptr || k == nullptr || v == nullptr || o_prefix == nullptr || lse_prefix == nullptr ||
        node_parent == nullptr || out == nullptr || out_lse == nullptr)
        return UNO_ERR_INVALID_ARG;
    if (!aligned(k, 16) || !aligned(v, 16))          // staged 16 bytes at a time
        return UNO_ERR_INVALID_ARG;
    return hip_status(launch_tree_attention(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                            static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o_prefix),
                                            lse_prefix, node_parent, num_nodes, batch, n, Hq, Hkv, scale,
                                            static_cast<uint16_t*>(out), out_lse, stream));
}

int uno_stream_read(const void* buf, int64_t bytes, int64_t wg_bytes, uint32_t* out, hipStream_t stream)
{
    if (bytes < 0 || wg_bytes <= 0 || bytes % 16 != 0 || wg_bytes % 16 != 0) return UNO_ERR_INVALID_ARG;
    if (bytes == 0) return UNO_OK;
    if ((bytes + wg_bytes - 1) / wg_bytes > 0x7FFFFFFF) return UNO_ERR_INVALID_ARG;
    if (buf == nullptr || out == nullptr || !aligned(buf, 16)) return UNO_ERR_INVALID_ARG;
    return hip_status(launch_stream_read(buf, bytes, wg_bytes, out, stream));
}

const char* uno_status_string(int status)
{
    switch (status) {
    case UNO_OK: return "ok";
    case UNO_ERR_INVALID_ARG: return "invalid argument";
    case UNO_ERR_UNSUPPORTED: return "unsupported configuration";
    case UNO_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case UNO_ERR_HIP: return "HIP launch failure";
    case UNO_ERR_SCRATCH_LIMIT: return "workspace exceeds the allocation-free entry point's fixed scratch";
    default: return "unknown status";
    }
}

int uno_last_hip_error(void) { return g_last_hip_error; }

const char* uno_version(void) { return "uno-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
