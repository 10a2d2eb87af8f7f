/*
 * uno_oracle.c -- plain fp64 CPU reference for the UNO decode-cycle sampling path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * cpu_baseline leg may load this library.  The GPU library shares no code,
 * header, table or constant with it; the two meet only in the seeded inputs.
 *
 * Sources (the method's pages):
 *   [PR]   SGLang pull request #37667, "native SGLang serving support for UNO":
 *          "Motivation" (linear and tree samplers, two forwards per cycle),
 *          "Modifications" (proposal + rejection sampling; tree sampling with the
 *          EAGLE tree-verification path; sparse target sampling),
 *          review thread on filter order (top-k first, then renormalise, then top-p).
 *   [Blog] run_math_eval walk-through (SGLang benchmark/uno), sections
 *          "B/K/V 参数映射" (B, K, V meaning), "启动期硬性约束" (tree limits,
 *          acceptance thresholds fixed at 1.0), "run_math_eval 全参数详解"
 *          (temperature >= 0, top_k > 0, top_p in (0, 1]), "TPF 统计口径".
 *   Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
 *          as 1, 2, 3", SC'11 (the counter-based generator both sides implement
 *          from its published definition).
 *
 * The pages name the operations but print no formula; the readings taken where
 * they are silent are listed in the design notes and restated at each function.
 * Everything is computed in double precision, one request at a time, in the
 * order the definitions state (sequential sums in the stated order).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (SC'11, Sec. 5): 10 rounds of the Philox S-box on a 4x32-bit
 * counter with a 2x32-bit key; the key is bumped by the Weyl constants between
 * rounds.  Round: (L0,R0,L1,R1) -> (hi(M1*L1)^R0^k0, lo(M1*L1), hi(M0*L0)^R1^k1,
 * lo(M0*L0)) with L0 = c0, R0 = c1, L1 = c2, R1 = c3.                         */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint64_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t p0 = M0 * (uint64_t)c0;
        uint64_t p1 = M1 * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The four uniforms of one draw.  Counter = (request, position, offset lo,
 * offset hi), key = (seed lo, seed hi).  Word 0 drives the proposal, word 1 the
 * acceptance test, word 2 the residual / bonus / tree-walk sample, word 3 is
 * unused.  u = w * 2^-32, exact in double, in [0, 1).                         */
static void draw4(uint64_t seed, uint32_t req, uint32_t pos, uint64_t offset, double u[4])
{
    uint32_t ctr[4] = { req, pos, (uint32_t)offset, (uint32_t)(offset >> 32) };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    for (int i = 0; i < 4; ++i) u[i] = (double)w[i] * 0x1p-32;
}

double oracle_uniform(uint64_t seed, uint32_t req, uint32_t pos, uint64_t offset, int lane)
{
    double u[4];
    draw4(seed, req, pos, offset, u);
    return u[lane & 3];
}

/* ------------------------------------------------------------------------ */
/* Row filter.  [PR] review thread on filter order: temperature, then top-k,
 * then renormalise over the top-k set, then top-p on that renormalised
 * distribution, then renormalise over the kept set.
 * Readings: the top-k set is the first k ids under (z desc, id asc) on the raw
 * logits; T = 0 is greedy (one-hot at the smallest id among the maxima);
 * top_k <= 0 or >= vocab disables top-k; top_p >= 1 disables top-p; the top-p
 * rule keeps an id while the exclusive cumulative sum (in filter order) is
 * below top_p, and always keeps the first; NaN logits count as -inf; a row
 * holding +inf, or no finite logit, is invalid (empty support).              */
/* Joint order ([PR] review thread: the regular sampler's joint filtering takes
 * top-p from the full softmax): keep an id when it is in the top-k set and the
 * exclusive cumulative full-vocabulary probability before it (filter order)
 * is below top_p (the first id always), then renormalise over the kept ids.
 * It differs from the default order only when both top-k and top-p are on.   */
#define ORACLE_ORDER_TOPK_FIRST 0
#define ORACLE_ORDER_JOINT 1

typedef struct { double v; int32_t id; } vid_t;

static int cmp_filter_order(const void* a, const void* b)
{
    const vid_t* x = (const vid_t*)a;
    const vid_t* y = (const vid_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->id < y->id) ? -1 : (x->id > y->id);
}

typedef struct {
    int32_t n;       /* support size; -1 = invalid row                        */
    double* p;       /* [N] filtered probabilities, zero outside the support  */
    int32_t* ids;    /* [N] support ids in filter order (z desc, id asc)      */
    double* sp;      /* [N] support probabilities in filter order             */
    vid_t* pairs;    /* [N] scratch for the sort                               */
    double m, S;     /* p_i = exp((z_i - m)/T) / S before any top-p renorm    */
    double margin;   /* |exclusive cumsum - top_p| nearest the cut (inf: none) */
} row_t;

static int row_alloc(row_t* r, int64_t N)
{
    r->p = (double*)malloc(sizeof(double) * (size_t)N);
    r->ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    r->sp = (double*)malloc(sizeof(double) * (size_t)N);
    r->pairs = (vid_t*)malloc(sizeof(vid_t) * (size_t)N);
    return r->p && r->ids && r->sp && r->pairs;
}

static void row_free(row_t* r)
{
    free(r->p); free(r->ids); free(r->sp); free(r->pairs);
}

static void filter_row(const float* z, int64_t N, double T, int32_t top_k, double top_p, int32_t order,
                       row_t* r)
{
    memset(r->p, 0, sizeof(double) * (size_t)N);
    r->n = 0; r->m = NAN; r->S = NAN; r->margin = INFINITY;

    int64_t n_use = 0;
    for (int64_t i = 0; i < N; ++i) {
        if (isnan(z[i])) continue;
        if (z[i] == INFINITY) { r->n = -1; return; }
        if (z[i] > -INFINITY) r->pairs[n_use++] = (vid_t){ (double)z[i], (int32_t)i };
    }
    if (n_use == 0) { r->n = -1; return; }

    if (T == 0.0) {                       /* greedy: one-hot at the argmax    */
        int64_t a = 0;
        for (int64_t j = 1; j < n_use; ++j)
            if (r->pairs[j].v > r->pairs[a].v) a = j;   /* first maximum wins */
        int32_t id = r->pairs[a].id;
        r->p[id] = 1.0; r->ids[0] = id; r->sp[0] = 1.0; r->n = 1;
        r->m = r->pairs[a].v; r->S = 1.0;
        return;
    }

    const int topk_on = top_k > 0 && (int64_t)top_k < N;
    const int topp_on = top_p < 1.0;

    /* the filter order over every usable id */
    qsort(r->pairs, (size_t)n_use, sizeof(vid_t), cmp_filter_order);
    const double m = r->pairs[0].v;
    r->m = m;

    if (!topk_on && !topp_on) {
        /* full softmax at temperature T; normaliser summed in id order */
        double S = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            if (isnan(z[i]) || !(z[i] > -INFINITY)) continue;
            double e = exp(((double)z[i] - m) / T);
            r->p[i] = e;
            S += e;
        }
        for (int64_t i = 0; i < N; ++i) r->p[i] = r->p[i] / S;
        r->S = S;
        int32_t n = 0;
        for (int64_t j = 0; j < n_use; ++j) {
            int32_t id = r->pairs[j].id;
            if (r->p[id] > 0.0) { r->ids[n] = id; r->sp[n] = r->p[id]; ++n; }
        }
        r->n = n;
        return;
    }

    const int64_t k_eff = topk_on ? (n_use < top_k ? n_use : top_k) : n_use;
    double S = 0.0;
    if (order == ORACLE_ORDER_JOINT && topk_on && topp_on) {
        /* joint order: the top-p cut reads the softmax over the whole
         * vocabulary (normaliser summed in id order), restricted to the
         * top-k set */
        for (int64_t i = 0; i < N; ++i) {
            if (isnan(z[i]) || !(z[i] > -INFINITY)) continue;
            S += exp(((double)z[i] - m) / T);
        }
        for (int64_t j = 0; j < k_eff; ++j) r->sp[j] = exp((r->pairs[j].v - m) / T);
    } else {
        /* softmax over the top-k set; normaliser summed in filter order */
        for (int64_t j = 0; j < k_eff; ++j) {
            r->sp[j] = exp((r->pairs[j].v - m) / T);
            S += r->sp[j];
        }
    }
    r->S = S;
    for (int64_t j = 0; j < k_eff; ++j) r->sp[j] = r->sp[j] / S;      /* pi_j */

    int64_t n_keep = k_eff;
    if (topp_on) {
        double c = 0.0;
        n_keep = 0;
        for (int64_t j = 0; j < k_eff; ++j) {
            if (j > 0) {
                double gap = fabs(c - top_p);
                if (gap < r->margin) r->margin = gap;
                if (c >= top_p) break;
            }
            c += r->sp[j];
            ++n_keep;
        }
        for (int64_t j = 0; j < n_keep; ++j) r->sp[j] = r->sp[j] / c;
    }
    int32_t n = 0;
    for (int64_t j = 0; j < n_keep; ++j) {
        if (!(r->sp[j] > 0.0)) break;          /* underflowed tail (filter order) */
        r->ids[n] = r->pairs[j].id;
        r->sp[n] = r->sp[j];
        r->p[r->pairs[j].id] = r->sp[j];
        ++n;
    }
    r->n = n;
}

/* ------------------------------------------------------------------------ */
/* Sampling primitive (reading: inverse CDF in ascending token-id order).
 * W = sum of the weights in id order, t = u * W, and the pick is the smallest
 * id whose inclusive cumulative weight exceeds t.  Weights need not be
 * normalised.  Returns -1 when W is 0.  *margin = distance of u from the nearest
 * boundary of the picked interval, in units of u.                            */
static int32_t sample_weights(const double* w, int64_t N, double u, double* margin)
{
    double W = 0.0;
    for (int64_t i = 0; i < N; ++i) W += w[i];
    if (!(W > 0.0)) { *margin = INFINITY; return -1; }
    const double t = u * W;
    double c = 0.0;
    for (int64_t i = 0; i < N; ++i) {
        const double prev = c;
        c += w[i];
        if (c > t) {
            const double a = t - prev, b = c - t;
            *margin = (a < b ? a : b) / W;
            return (int32_t)i;
        }
    }
    for (int64_t i = N - 1; i >= 0; --i)
        if (w[i] > 0.0) { *margin = 0.0; return (int32_t)i; }
    *margin = INFINITY;
    return -1;
}

static inline void fmin_into(double* acc, double v) { if (v < *acc) *acc = v; }

/* ------------------------------------------------------------------------ */
/* Filter many rows (test aid).  Support written in filter order.             */
int oracle_filter(const float* z, int64_t rows, int64_t N, double T, int32_t top_k, double top_p,
                  int32_t order, double* dense, int32_t* sup_ids, double* sup_p, int32_t* sup_n, int32_t cap,
                  double* stats, double* margin)
{
    int err = 0;
    #pragma omp parallel
    {
        row_t r;
        int ok = row_alloc(&r, N);
        if (!ok) {
            #pragma omp atomic write
            err = 1;
        }
        #pragma omp for schedule(dynamic)
        for (int64_t i = 0; i < rows; ++i) {
            if (!ok) continue;
            filter_row(z + i * N, N, T, top_k, top_p, order, &r);
            if (dense) memcpy(dense + i * N, r.p, sizeof(double) * (size_t)N);
            if (sup_n) sup_n[i] = r.n;
            for (int32_t j = 0; j < r.n && j < cap; ++j) {
                if (sup_ids) sup_ids[i * cap + j] = r.ids[j];
                if (sup_p) sup_p[i * cap + j] = r.sp[j];
            }
            if (stats) { stats[2 * i] = r.m; stats[2 * i + 1] = r.S; }
            if (margin) margin[i] = r.margin;
        }
        row_free(&r);
    }
    return err ? -1 : 0;
}

/* Sampling primitive exposed for the distribution tests. */
int32_t oracle_sample(const double* w, int64_t N, double u, double* margin)
{
    double mg;
    int32_t s = sample_weights(w, N, u, &mg);
    if (margin) *margin = mg;
    return s;
}

/* ------------------------------------------------------------------------ */
/* Linear UNO cycle.  [PR] "Motivation": the linear sampler draws each of the
 * B block tokens independently from its marginal; "Modifications": proposal
 * and rejection sampling; [Blog] "启动期硬性约束": acceptance thresholds are 1.0,
 * i.e. plain speculative rejection sampling:
 *   y_j ~ q_j (word 0), accept iff u1 * q_j(y_j) < p_j(y_j) (word 1),
 *   j* = first rejected position (B if none),
 *   j* < B: final ~ max(0, p_j* - q_j*) renormalised (word 2 of position j*),
 *           or ~ p_j* when that residual has zero mass;
 *   j* = B: final ~ p_B (word 2 of position B).
 * Draft row j is judged by target row j; target row B is the bonus row.
 * tokens = y_0 .. y_{j*-1}, final, then -1; accept_len = j* + 1.
 * All B proposals are reported (positions past j* included), so the margin
 * covers every proposal's draw as well as the decisions up to j*.
 * Layout: draft + b*draft_req_stride + j*N, target + b*target_req_stride + j*N;
 * a zero stride shares one block of rows between all requests.
 * offsets (nullable): request b takes the decode-cycle index offsets[b]
 * instead of `offset` (independent cycles side by side in one call).       */
void oracle_linear(const float* draft, const float* target, int32_t batch, int32_t B, int64_t N,
                   int64_t draft_req_stride, int64_t target_req_stride,
                   double T, int32_t top_k, double top_p, int32_t order, uint64_t seed, uint64_t offset,
                   const uint32_t* request_ids, const uint64_t* offsets,
                   int32_t* tokens, int32_t* accept_len, int32_t* proposals, double* min_margin)
{
    #pragma omp parallel
    {
        row_t* q = (row_t*)calloc((size_t)B, sizeof(row_t));
        row_t* p = (row_t*)calloc((size_t)B + 1, sizeof(row_t));
        double* res = (double*)malloc(sizeof(double) * (size_t)N);
        for (int32_t j = 0; j < B; ++j) row_alloc(&q[j], N);
        for (int32_t j = 0; j <= B; ++j) row_alloc(&p[j], N);
        int64_t shared_done = 0;   /* zero strides: filter once per thread */

        #pragma omp for schedule(dynamic)
        for (int32_t b = 0; b < batch; ++b) {
            const uint32_t req = request_ids ? request_ids[b] : (uint32_t)b;
            const uint64_t cyc = offsets ? offsets[b] : offset;
            double mg = INFINITY, m1;
            if (!(shared_done && draft_req_stride == 0 && target_req_stride == 0)) {
                for (int32_t j = 0; j < B; ++j)
                    filter_row(draft + (int64_t)b * draft_req_stride + (int64_t)j * N, N, T, top_k, top_p, order, &q[j]);
                for (int32_t j = 0; j <= B; ++j)
                    filter_row(target + (int64_t)b * target_req_stride + (int64_t)j * N, N, T, top_k, top_p, order, &p[j]);
                shared_done = 1;
            }
            for (int32_t j = 0; j < B; ++j) fmin_into(&mg, q[j].margin);
            for (int32_t j = 0; j <= B; ++j) fmin_into(&mg, p[j].margin);

            int32_t* tok = tokens + (int64_t)b * (B + 1);
            for (int32_t j = 0; j <= B; ++j) tok[j] = -1;

            int32_t y[B > 0 ? B : 1];
            double ym[B > 0 ? B : 1];
            for (int32_t j = 0; j < B; ++j) {
                double u[4];
                draw4(seed, req, (uint32_t)j, cyc, u);
                ym[j] = INFINITY;
                y[j] = (q[j].n > 0) ? sample_weights(q[j].p, N, u[0], &ym[j]) : -1;
                if (proposals) proposals[(int64_t)b * B + j] = y[j];
                fmin_into(&mg, ym[j]);
            }

            int32_t jstar = B;
            for (int32_t j = 0; j < B; ++j) {
                double u[4];
                draw4(seed, req, (uint32_t)j, cyc, u);
                int accept = 0;
                if (y[j] >= 0) {
                    const double qy = q[j].p[y[j]];
                    const double py = (p[j].n > 0) ? p[j].p[y[j]] : 0.0;
                    accept = u[1] * qy < py;
                    if (py < qy) fmin_into(&mg, fabs(u[1] - py / qy));
                }
                if (!accept) { jstar = j; break; }
                tok[j] = y[j];
            }

            double u[4];
            draw4(seed, req, (uint32_t)jstar, cyc, u);
            int32_t final_tok = -1;
            if (jstar < B) {
                for (int64_t i = 0; i < N; ++i) {
                    const double pi = (p[jstar].n > 0) ? p[jstar].p[i] : 0.0;
                    const double qi = (q[jstar].n > 0) ? q[jstar].p[i] : 0.0;
                    const double d = pi - qi;
                    res[i] = d > 0.0 ? d : 0.0;
                }
                final_tok = sample_weights(res, N, u[2], &m1);
                if (final_tok < 0 && p[jstar].n > 0) final_tok = sample_weights(p[jstar].p, N, u[2], &m1);
            } else if (p[B].n > 0) {
                final_tok = sample_weights(p[B].p, N, u[2], &m1);
            }
            if (final_tok >= 0) fmin_into(&mg, m1);
            tok[jstar] = final_tok;
            accept_len[b] = jstar + 1;
            if (min_margin) min_margin[b] = mg;
        }
        for (int32_t j = 0; j < B; ++j) row_free(&q[j]);
        for (int32_t j = 0; j <= B; ++j) row_free(&p[j]);
        free(q); free(p); free(res);
    }
}

/* ------------------------------------------------------------------------ */
/* Tree construction.  [PR] "Motivation": the tree sampler considers V candidate
 * sequences built from the top K candidates of each marginal; [Blog] "B/K/V 参数
 * 映射": B = draft width, K = candidates kept per expansion, V = verify width.
 * Readings: candidates of depth d are the first K support ids of the filtered
 * draft row d in filter order; a node's score is the product of the filtered
 * draft probabilities along its path (root score 1, multiplied root to leaf);
 * the tree is the V best non-root nodes, found best-first: pop the frontier
 * entry with the highest score (ties: smaller depth, then smaller parent node
 * index, then smaller candidate rank) and push all of its children.
 * Node 0 is the root (token -1, parent -1, depth 0); node n >= 1 holds the
 * token chosen at depth node_depth[n] - 1; num_nodes counts the root.
 * *min_gap = smallest relative gap between the popped score and any distinct
 * competing frontier score (a near-tie measure; exact ties are excluded).    */
typedef struct { double score; int32_t depth, parent, rank; } fr_t;

static int fr_better(const fr_t* a, const fr_t* b)
{
    if (a->score != b->score) return a->score > b->score;
    if (a->depth != b->depth) return a->depth < b->depth;
    if (a->parent != b->parent) return a->parent < b->parent;
    return a->rank < b->rank;
}

void oracle_build_tree(const float* draft, int32_t batch, int32_t B, int32_t K, int32_t V, int64_t N,
                       int64_t req_stride, double T, int32_t top_k, double top_p, int32_t order,
                       int32_t* node_token, int32_t* node_parent, int32_t* node_depth,
                       double* node_score, int32_t* num_nodes, double* min_gap)
{
    #pragma omp parallel
    {
        row_t* q = (row_t*)calloc((size_t)B, sizeof(row_t));
        for (int32_t j = 0; j < B; ++j) row_alloc(&q[j], N);
        const int64_t fcap = (int64_t)V * K + K + 1;
        fr_t* fr = (fr_t*)malloc(sizeof(fr_t) * (size_t)fcap);

        #pragma omp for schedule(dynamic)
        for (int32_t b = 0; b < batch; ++b) {
            for (int32_t d = 0; d < B; ++d)
                filter_row(draft + (int64_t)b * req_stride + (int64_t)d * N, N, T, top_k, top_p, order, &q[d]);
            int32_t cn[B > 0 ? B : 1];
            for (int32_t d = 0; d < B; ++d) cn[d] = q[d].n > 0 ? (q[d].n < K ? q[d].n : K) : 0;

            int32_t* tk = node_token + (int64_t)b * (V + 1);
            int32_t* pa = node_parent + (int64_t)b * (V + 1);
            int32_t* dp = node_depth + (int64_t)b * (V + 1);
            double* sc = node_score ? node_score + (int64_t)b * (V + 1) : NULL;
            for (int32_t n = 0; n <= V; ++n) { tk[n] = -1; pa[n] = -1; dp[n] = -1; if (sc) sc[n] = 0.0; }
            tk[0] = -1; pa[0] = -1; dp[0] = 0; if (sc) sc[0] = 1.0;

            double gap = INFINITY;
            int64_t nf = 0;
            for (int32_t r = 0; r < cn[0]; ++r)
                fr[nf++] = (fr_t){ 1.0 * q[0].sp[r], 1, 0, r };
            int32_t num = 1;
            while (num < V + 1 && nf > 0) {
                int64_t best = 0;
                for (int64_t i = 1; i < nf; ++i)
                    if (fr_better(&fr[i], &fr[best])) best = i;
                const fr_t e = fr[best];
                for (int64_t i = 0; i < nf; ++i)
                    if (i != best && fr[i].score != e.score) {
                        double g = fabs(e.score - fr[i].score) / e.score;
                        if (g < gap) gap = g;
                    }
                fr[best] = fr[--nf];
                tk[num] = q[e.depth - 1].ids[e.rank];
                pa[num] = e.parent;
                dp[num] = e.depth;
                if (sc) sc[num] = e.score;
                if (e.depth < B)
                    for (int32_t r = 0; r < cn[e.depth]; ++r)
                        fr[nf++] = (fr_t){ e.score * q[e.depth].sp[r], e.depth + 1, num, r };
                ++num;
            }
            num_nodes[b] = num;
            if (min_gap) min_gap[b] = gap;
        }
        for (int32_t j = 0; j < B; ++j) row_free(&q[j]);
        free(q); free(fr);
    }
}

/* ------------------------------------------------------------------------ */
/* Tree verification.  [PR] "Modifications": tree UNO reuses EAGLE tree
 * verification; [Blog] "启动期硬性约束": both acceptance thresholds are 1.0.
 * Reading: with deterministic (top-K) drafts this is the target-sampled walk:
 * at node n of depth d draw t ~ p_n (word 2 of position d), emit t, move to
 * the child of n whose token is t if there is one (and d < B), else stop.
 * Target row n of a request is the distribution that follows node n's prefix
 * (row 0: the root).  Rows past num_nodes are never read.
 * tokens/path = emitted tokens / visited nodes, then -1; accept_len = #emitted.
 * offsets (nullable): request b takes the cycle index offsets[b].            */
void oracle_verify_tree(const float* target, int32_t batch, int32_t B, int32_t V, int64_t N,
                        int64_t req_stride, double T, int32_t top_k, double top_p, int32_t order,
                        uint64_t seed, uint64_t offset, const uint32_t* request_ids, const uint64_t* offsets,
                        const int32_t* node_token, const int32_t* node_parent, const int32_t* num_nodes,
                        int32_t* tokens, int32_t* path, int32_t* accept_len, double* min_margin)
{
    #pragma omp parallel
    {
        row_t r;
        row_alloc(&r, N);
        #pragma omp for schedule(dynamic)
        for (int32_t b = 0; b < batch; ++b) {
            const uint32_t req = request_ids ? request_ids[b] : (uint32_t)b;
            const uint64_t cyc = offsets ? offsets[b] : offset;
            const int32_t* tk = node_token + (int64_t)b * (V + 1);
            const int32_t* pa = node_parent + (int64_t)b * (V + 1);
            const int32_t nn = num_nodes[b];
            int32_t* tok = tokens + (int64_t)b * (B + 1);
            int32_t* pth = path + (int64_t)b * (B + 1);
            for (int32_t j = 0; j <= B; ++j) { tok[j] = -1; pth[j] = -1; }
            double mg = INFINITY, m1;
            int32_t n = 0, d = 0;
            for (;;) {
                filter_row(target + (int64_t)b * req_stride + (int64_t)n * N, N, T, top_k, top_p, order, &r);
                fmin_into(&mg, r.margin);
                double u[4];
                draw4(seed, req, (uint32_t)d, cyc, u);
                int32_t t = -1;
                if (r.n > 0) { t = sample_weights(r.p, N, u[2], &m1); fmin_into(&mg, m1); }
                tok[d] = t;
                pth[d] = n;
                int32_t child = -1;
                if (t >= 0 && d < B)
                    for (int32_t c = 1; c < nn; ++c)
                        if (pa[c] == n && tk[c] == t) { child = c; break; }
                if (child < 0) break;
                n = child;
                ++d;
            }
            accept_len[b] = d + 1;
            if (min_margin) min_margin[b] = mg;
        }
        row_free(&r);
    }
}

/* ------------------------------------------------------------------------ */
/* Tree-suffix attention merged with the prefix attention.  [PR]
 * "Modifications": an UNO-only fused kernel for tree-suffix attention and LSE
 * merge, with the FlashAttention + state-merge path as fallback; "Changes to
 * shared SGLang infrastructure": the fused merge serves UNO tree verification
 * (cascade attention: the shared prefix once, the V-node tree suffix apart).
 * Reading: each request's n = V + 1 verify tokens are the tree's nodes (node 0
 * the root); the query of node i attends, among the suffix keys, to node i and
 * its ancestors.  With scores s_j = scale * q_i . k_j over those nodes,
 *   lse_s = log sum_j exp(s_j),  o_s = sum_j exp(s_j - lse_s) v_j,
 * and the prefix state (o_p, lse_p) of the same query (its attention over the
 * shared context, computed elsewhere):
 *   lse = log(exp(lse_p) + exp(lse_s)),
 *   o   = exp(lse_p - lse) o_p + exp(lse_s - lse) o_s,
 * i.e. softmax attention over the prefix keys and the visible suffix keys
 * together.  lse_p = -inf means an empty prefix.  Query head h reads key/value
 * head h / (Hq / Hkv).  Layout: token t = b * n + i; q, o_p, o [t][Hq][D],
 * k, v [t][Hkv][D], lse_p, lse [t][Hq].  Nodes at or past num_nodes[b] are not
 * read or written.                                                            */
void oracle_tree_attention(const float* q, const float* k, const float* v, const float* o_p,
                           const float* lse_p, const int32_t* node_parent, const int32_t* num_nodes,
                           int32_t batch, int32_t n, int32_t Hq, int32_t Hkv, int32_t D, double scale,
                           double* o, double* lse)
{
    const int32_t G = Hq / Hkv;
    #pragma omp parallel for schedule(dynamic)
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t nn = num_nodes[b] < n ? num_nodes[b] : n;
        const int32_t* par = node_parent + (int64_t)b * n;
        double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        char* vis = (char*)malloc((size_t)(n > 0 ? n : 1));
        for (int32_t i = 0; i < nn; ++i) {
            /* node i and its ancestors */
            memset(vis, 0, (size_t)n);
            for (int32_t a = i, steps = 0; a >= 0 && a < nn && steps <= n; a = par[a], ++steps) vis[a] = 1;
            const int64_t t = (int64_t)b * n + i;
            for (int32_t h = 0; h < Hq; ++h) {
                const int32_t hk = h / G;
                const float* qi = q + (t * Hq + h) * D;
                double mx = -INFINITY;
                for (int32_t j = 0; j < nn; ++j) {
                    if (!vis[j]) continue;
                    const float* kj = k + (((int64_t)b * n + j) * Hkv + hk) * D;
                    double d = 0.0;
                    for (int32_t e = 0; e < D; ++e) d += (double)qi[e] * (double)kj[e];
                    s[j] = scale * d;
                    if (s[j] > mx) mx = s[j];
                }
                double sum = 0.0;
                for (int32_t j = 0; j < nn; ++j)
                    if (vis[j]) sum += exp(s[j] - mx);
                const double ls = mx + log(sum);
                const double lp = (double)lse_p[t * Hq + h];
                const double l = (lp == -INFINITY) ? ls : (lp > ls ? lp + log1p(exp(ls - lp))
                                                                   : ls + log1p(exp(lp - ls)));
                const double wp = (lp == -INFINITY) ? 0.0 : exp(lp - l);
                const double ws = exp(ls - l);
                double* oi = o + (t * Hq + h) * D;
                const float* pi = o_p + (t * Hq + h) * D;
                for (int32_t e = 0; e < D; ++e) {
                    double acc = 0.0;
                    for (int32_t j = 0; j < nn; ++j)
                        if (vis[j]) acc += exp(s[j] - ls) * (double)v[(((int64_t)b * n + j) * Hkv + hk) * D + e];
                    oi[e] = wp * (double)pi[e] + ws * acc;
                }
                lse[t * Hq + h] = l;
            }
        }
        free(s);
        free(vis);
    }
}

/* ------------------------------------------------------------------------ */
/* Tokens per forward.  [Blog] "TPF 统计口径" and [PR] "Validation": each UNO
 * cycle runs two target forwards, so TPF = emitted tokens / (2 * cycles).   */
double oracle_tpf(const int32_t* accept_len, int64_t n_request_cycles)
{
    double tokens = 0.0;
    for (int64_t i = 0; i < n_request_cycles; ++i) tokens += accept_len[i];
    return tokens / (2.0 * (double)n_request_cycles);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
