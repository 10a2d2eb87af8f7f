// sample_kernels.hip -- proposal / rejection / residual sampling, tree build and
// tree walk for the UNO decode cycle on gfx950.
//
// Method: SGLang PR #37667 ("native SGLang serving support for UNO"),
// Motivation (linear and tree samplers) and Modifications (sparse and dense
// proposal + rejection sampling; tree sampling with EAGLE tree verification and
// sparse target sampling); the run_math_eval walk-through's startup
// constraints fix both acceptance thresholds at 1.0.
//
// Sampling from a distribution is an inverse CDF in ascending token-id order.
// A sparse support (<= 256 ids) arrives in id order with its cumulative sums,
// taken in that order in double precision by the filter (the same additions,
// in the same order, as a sequential scan over the dense vector, whose zeros
// add nothing); one wave holds it in registers and picks by ballot.  Dense
// rows are located chunk by chunk from per-chunk statistics and finished
// inside one 2048-logit chunk; a full-vocabulary nucleus restricts every
// weight to the logits at or above the row's keep threshold.
#include "uno_device.h"
#include "uno_internal.h"

#include <math.h>

namespace uno {

namespace {

constexpr int kMaxK = 256;
constexpr int kMaxLinearB = 128;
constexpr int kMaxNodes = 129;          // V + 1 with V <= 128
constexpr int kMaxTreeVK = 2048;        // V * K limit the C ABI enforces

// ---- sparse helpers ------------------------------------------------------------
constexpr int kQ = kMaxK / kWave;      // support entries per lane

// A support held by one wave: entry q*64 + lane in id[q] / w[q].
struct WaveRow {
    int32_t id[kQ];
    double w[kQ];
    double c[kQ];      // inclusive cumulative sums in id order (supports that carry them)
};

// Load the n <= cap <= 256 entries of a support (unordered); slots past n hold
// id INT32_MAX, weight 0.
__device__ __forceinline__ void wave_load_support(const int32_t* ids, const double* p, const double* cum, int n,
                                                  int cap, WaveRow& R, int lane)
{
    // every slot below cap is read (the filter pads supports to cap), so the
    // loads do not wait for the count
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const int i = q * kWave + lane;
        int32_t id = 0x7FFFFFFF;
        double w = 0.0, c = 0.0;
        if (q * kWave < cap && i < cap) {
            id = ids[i];
            w = p[i];
            if (cum) c = cum[i];
        }
        R.id[q] = (i < n) ? id : 0x7FFFFFFF;
        R.w[q] = (i < n) ? w : 0.0;
        R.c[q] = (i < n) ? c : 0.0;
    }
}

// Inverse CDF over the n id-ordered entries of R with uniform u: the first
// entry whose inclusive cumulative weight exceeds u * W (W the total); when
// rounding leaves none, the last entry with positive weight.  Returns its id
// (-1 when W is not positive) and its weight in *wpick.  The cumulative sums
// are taken in id order by one lane over cum (LDS, n doubles), one add per
// step; the pick is a ballot.
__device__ __forceinline__ int32_t wave_sample_sorted(const WaveRow& R, int n, double u, double* wpick, int lane,
                                                      double* cum)
{
    *wpick = 0.0;
    if (n <= 0) return -1;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const int i = q * kWave + lane;
        if (q * kWave < n && i < n) cum[i] = R.w[q];
    }
    wave_sync();
    if (lane == 0) {
        double acc = 0.0;
#pragma unroll 8
        for (int i = 0; i < n; ++i) {
            acc += cum[i];
            cum[i] = acc;
        }
    }
    wave_sync();
    const double W = cum[n - 1];
    int32_t pick = -1;
    if (W > 0.0) {
        const double t = u * W;
        bool found = false;
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            if (q * kWave >= n || found) break;
            const uint64_t m = __ballot(q * kWave + lane < n && cum[q * kWave + lane] > t);
            if (m) {
                const int src = wave_first_lane(m);
                *wpick = readlane_f64(R.w[q], src);
                pick = __builtin_amdgcn_readlane(R.id[q], src);
                found = true;
            }
        }
#pragma unroll
        for (int q = kQ - 1; q >= 0; --q) {
            if (found) break;
            const uint64_t m = __ballot(q * kWave + lane < n && R.w[q] > 0.0);
            if (m) {
                const int src = 63 - __clzll((long long)m);
                *wpick = readlane_f64(R.w[q], src);
                pick = __builtin_amdgcn_readlane(R.id[q], src);
                found = true;
            }
        }
    }
    wave_sync();             // cum is reused by the caller
    return pick;
}

// Inverse CDF over the n id-ordered entries of R whose inclusive cumulative
// sums R.c came with the support (the filter takes them in id order, one add
// per step, exactly as wave_sample_sorted would): the same rule, with the
// pick a ballot and W the last sum.
__device__ __forceinline__ int32_t wave_sample_cum(const WaveRow& R, int n, double u, double* wpick, int lane)
{
    *wpick = 0.0;
    if (n <= 0) return -1;
    double W = 0.0;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
        if (((n - 1) >> 6) == q) W = readlane_f64(R.c[q], (n - 1) & (kWave - 1));
    int32_t pick = -1;
    if (W > 0.0) {
        const double t = u * W;
        bool found = false;
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            if (q * kWave >= n || found) break;
            const uint64_t m = __ballot(q * kWave + lane < n && R.c[q] > t);
            if (m) {
                const int src = wave_first_lane(m);
                *wpick = readlane_f64(R.w[q], src);
                pick = __builtin_amdgcn_readlane(R.id[q], src);
                found = true;
            }
        }
#pragma unroll
        for (int q = kQ - 1; q >= 0; --q) {
            if (found) break;
            const uint64_t m = __ballot(q * kWave + lane < n && R.w[q] > 0.0);
            if (m) {
                const int src = 63 - __clzll((long long)m);
                *wpick = readlane_f64(R.w[q], src);
                pick = __builtin_amdgcn_readlane(R.id[q], src);
                found = true;
            }
        }
    }
    return pick;
}

// Weight of token y in a wave's register support (0 when absent).
__device__ __forceinline__ double reg_lookup(const WaveRow& R, int n, int32_t y, int lane)
{
    double v = 0.0;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if (q * kWave >= n) break;
        const uint64_t m = __ballot(q * kWave + lane < n && R.id[q] == y);
        if (m) v = readlane_f64(R.w[q], wave_first_lane(m));
    }
    return v;
}

// Per-wave LDS copy of one id-ordered support (ids, weights, cumulative sums).
struct SupportScratch {
    int32_t id[kMaxK];
    double w[kMaxK];
    double cum[kMaxK];
};

// ---- linear, sparse supports -----------------------------------------------------
// One workgroup per request.  Each wave takes block positions j (and the
// bonus position B): it proposes y_j ~ q_j, tests it against p_j and, when the
// proposal is rejected, already draws the last token that a first rejection
// at j would emit -- from the residual max(0, p_j - q_j), or from p_j when the
// residual has no mass; at position B it draws the bonus token from p_B.  The
// first rejection j* then only selects among these draws.
constexpr int kLinWaves = 9;     // B = 8 positions and the bonus in one round
constexpr int kLinThreads = kLinWaves * kWave;

// Weight of token `id` in an id-sorted list in LDS (0 when absent).
__device__ __forceinline__ double sorted_lookup(const int32_t* ids, const double* w, int n, int32_t id)
{
    int lo = 0, hi = n;                 // first index with ids[index] >= id
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (ids[mid] < id) lo = mid + 1; else hi = mid;
    }
    return (lo < n && ids[lo] == id) ? w[lo] : 0.0;
}

__global__ __launch_bounds__(kLinThreads) void linear_sparse_kernel(
    int32_t batch, int32_t B, SparseOut sup, uint64_t seed, uint64_t offset,
    const uint32_t* req_ids, LinearOut o)
{
    __shared__ SupportScratch s_q[kLinWaves];     // q_j in id order for the residual's lookups; its cumulative sums
    __shared__ int32_t s_y[kMaxLinearB];
    __shared__ int32_t s_acc[kMaxLinearB];
    __shared__ int32_t s_fin[kMaxLinearB + 1];
    __shared__ uint32_t s_ffl[kMaxLinearB + 1];
    __shared__ uint32_t s_flags;

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x;
    const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
    const int64_t qbase = (int64_t)b * B;
    const int64_t pbase = (int64_t)batch * B + (int64_t)b * (B + 1);
    const int cap = sup.cap;
    if (threadIdx.x == 0) s_flags = 0;
    __syncthreads();

    uint32_t flags = 0;
    for (int j = w; j <= B; j += kLinWaves) {
        const Draw d = uno_draw(seed, req, (uint32_t)j, offset);
        const int64_t pr = pbase + j;
        const int np = sup.count[pr];
        WaveRow P;                       // p_j (id order, with its cumulative sums), loaded up front
        wave_load_support(sup.ids + pr * cap, sup.probs + pr * cap, sup.cum + pr * cap, np, cap, P, lane);
        int32_t fin = -1;
        uint32_t ffl = 0;
        if (j == B) {                    // bonus draw
            double dummy;
            if (np > 0) fin = wave_sample_cum(P, np, d.u[2], &dummy, lane);
            else ffl = 1u;
            if (lane == 0) { s_fin[j] = fin; s_ffl[j] = ffl; }
            continue;
        }
        const int64_t qr = qbase + j;
        const int nq = sup.count[qr];
        int32_t y = -1;
        double qy = 0.0;
        WaveRow Q;
        wave_load_support(sup.ids + qr * cap, sup.probs + qr * cap, sup.cum + qr * cap, nq, cap, Q, lane);
        if (nq > 0) y = wave_sample_cum(Q, nq, d.u[0], &qy, lane);
        else flags |= 1u;
        int acc = 0;
        if (y >= 0) {
            double py = 0.0;
            if (np > 0) py = reg_lookup(P, np, y, lane);
            else flags |= 1u;
            acc = (d.u[1] * qy < py) ? 1 : 0;
        }
        if (!acc) {
            // the last token if j is the first rejection: residual max(0, p - q)
            // over p's support (ids outside it have zero residual)
            double dummy;
            if (np > 0) {
                // q's entries in LDS (already in id order) for the lookups
                const int nqq = nq > 0 ? nq : 0;
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    const int i = q * kWave + lane;
                    if (q * kWave < nqq && i < nqq) { s_q[w].id[i] = Q.id[q]; s_q[w].w[i] = Q.w[q]; }
                }
                wave_sync();
                WaveRow Rz = P;
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    if (q * kWave >= np) break;
                    const double qv = (q * kWave + lane < np) ? sorted_lookup(s_q[w].id, s_q[w].w, nqq, P.id[q]) : 0.0;
                    const double dlt = P.w[q] - qv;
                    Rz.w[q] = dlt > 0.0 ? dlt : 0.0;
                }
                fin = wave_sample_sorted(Rz, np, d.u[2], &dummy, lane, s_q[w].cum);
                if (fin < 0) {
                    ffl = 2u;
                    fin = wave_sample_cum(P, np, d.u[2], &dummy, lane);
                }
            } else {
                ffl = 1u;
            }
        }
        if (lane == 0) {
            s_y[j] = y;
            s_acc[j] = acc;
            s_fin[j] = fin;
            s_ffl[j] = ffl;
            if (o.proposals) o.proposals[(int64_t)b * B + j] = y;
        }
    }
    if (flags && lane == 0) atomicOr(&s_flags, flags);
    __syncthreads();
    if (w != 0) return;

    int jstar = B;
    for (int base = 0; base < B; base += kWave) {
        const int j = base + lane;
        const uint64_t m = __ballot(j < B && s_acc[j] == 0);
        if (m) { jstar = base + wave_first_lane(m); break; }
    }
    const int32_t fin = s_fin[jstar];
    int32_t* tok = o.tokens + (int64_t)b * (B + 1);
    for (int j = lane; j <= B; j += kWave) tok[j] = (j < jstar) ? s_y[j] : (j == jstar ? fin : -1);
    if (lane == 0) {
        o.accept_len[b] = jstar + 1;
        if (o.flags) o.flags[b] = s_flags | s_ffl[jstar];
    }
}

// ---- tree build (one wave per request) ------------------------------------------
// Best-first expansion with lazily pushed siblings: a popped node pushes its
// next sibling and its first child.  Siblings come in non-increasing score
// (candidate order), so the frontier always holds the best unexpanded entry.
// Order of frontier entries: larger score first, then smaller depth, parent,
// candidate rank.  Scores are non-negative doubles, so their bit patterns
// order as integers; (depth, parent, rank) pack into one word, smaller first.
//
// Everything a pop touches lives in registers, spread over the lanes: entry
// (or node, or depth) i sits in lane i % 64 of slot i / 64.  The frontier is
// an unordered set; each pop is a wave maximum of the score's high word, and
// only lanes that tie on it go on to the low word and then the tie word.  The
// only memory access of a pop is the next sibling's probability, from the
// candidate table (first K ids and probabilities of each depth's filtered
// row) staged in LDS.

__device__ __forceinline__ uint32_t tree_tie(int depth, int parent, int rank)
{
    return ((uint32_t)depth << 20) | ((uint32_t)parent << 12) | (uint32_t)rank;
}

// Lane (i % 64) of slot (i / 64), i uniform.
template <int N>
__device__ __forceinline__ int slot_get_i32(const int (&a)[N], int i)
{
    int r = 0;
#pragma unroll
    for (int q = 0; q < N; ++q)
        if ((i >> 6) == q) r = __builtin_amdgcn_readlane(a[q], i & (kWave - 1));
    return r;
}

template <int N>
__device__ __forceinline__ double slot_get_f64(const double (&a)[N], int i)
{
    double r = 0.0;
#pragma unroll
    for (int q = 0; q < N; ++q)
        if ((i >> 6) == q) r = readlane_f64(a[q], i & (kWave - 1));
    return r;
}

// FS register slots per lane for the frontier and for the node records: at
// most 1 + V entries are ever live, since a popped entry's slot takes its next
// sibling and only first children need new slots (FS = ceil((V + 1) / 64)).
template <int FS>
__global__ __launch_bounds__(kWave) void tree_build_kernel(int32_t batch, int32_t B, int32_t K, int32_t V,
                                                           SparseOut sup, TreeOut o)
{
    __shared__ int32_t c_id[kMaxTreeVK];       // depth d, rank r at d*K + r (B*K <= V*K <= 2048)
    __shared__ double c_p[kMaxTreeVK];

    const int lane = lane_id();
    const int b = blockIdx.x;
    const int cap = sup.cap;
    const int64_t rbase = (int64_t)b * B;
    // per depth (B <= 128): candidate count (at most K) and first probability
    int cn[2];
    double p0[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int d = s * kWave + lane;
        int n = 0;
        double f = 0.0;
        if (d < B) {
            n = sup.count[rbase + d];
            f = sup.probs[(rbase + d) * cap];
        }
        cn[s] = n > 0 ? (n < K ? n : K) : 0;
        p0[s] = f;
    }
    // the candidate table is read whole (supports are padded to cap); entries
    // past a count are never used
    const int kk = K < cap ? K : cap;
    for (int i = lane; i < B * K; i += kWave) {
        const int d = i / K, r = i - d * K;
        if (r < kk) {
            c_id[i] = sup.ids[(rbase + d) * cap + r];
            c_p[i] = sup.probs[(rbase + d) * cap + r];
        }
    }
    wave_sync();

    uint64_t fs[FS];                                   // frontier: score bits (0 = empty)
    uint32_t ft[FS];                                   // frontier: tie word (~0 = empty)
    double ns[FS];                                     // node records: score
    uint32_t nt[FS];                                   // node records: tie word of the entry
#pragma unroll
    for (int q = 0; q < FS; ++q) { fs[q] = 0ull; ft[q] = ~0u; ns[q] = 0.0; nt[q] = 0u; }
    if (lane == 0) ns[0] = 1.0;
    auto put = [&](int slot, double sc, uint32_t tie) __attribute__((always_inline)) {
        const int qs = slot >> 6, ls = slot & (kWave - 1);
#pragma unroll
        for (int q = 0; q < FS; ++q)
            if (q == qs && lane == ls) { fs[q] = (uint64_t)__double_as_longlong(sc); ft[q] = tie; }
    };

    int nf = 0;                                        // slots handed out (uniform)
    int live = 0;
    if (__builtin_amdgcn_readlane(cn[0], 0) > 0) { put(nf++, 1.0 * readlane_f64(p0[0], 0), tree_tie(1, 0, 0)); ++live; }
    int num = 1;
    while (num <= V && live > 0) {
        // this lane's best slot
        uint64_t bs = fs[0];
        uint32_t bt = ft[0];
        int bq = 0;
#pragma unroll
        for (int q = 1; q < FS; ++q)
            if (fs[q] > bs || (fs[q] == bs && ft[q] < bt)) { bs = fs[q]; bt = ft[q]; bq = q; }
        // the wave's best: high score word, then (on ties) low word, tie word
        const uint32_t bh = (uint32_t)(bs >> 32), bl = (uint32_t)bs;
        const uint32_t hm = wave_ext_u32<true>(bh);
        uint64_t hit = __ballot(bh == hm);
        if (__popcll(hit) > 1) {
            const uint32_t lm = wave_ext_u32<true>(bh == hm ? bl : 0u);
            const bool c = bh == hm && bl == lm;
            hit = __ballot(c);
            if (__popcll(hit) > 1) {
                const uint32_t tm = wave_ext_u32<false>(c ? bt : ~0u);
                hit = __ballot(c && bt == tm);
            }
        }
        const int wl = wave_first_lane(hit);
        const uint32_t tie = (uint32_t)__builtin_amdgcn_readlane((int)bt, wl);
        const int wq = __builtin_amdgcn_readlane(bq, wl);
        const double score = __longlong_as_double(
            (long long)(((uint64_t)hm << 32) | (uint32_t)__builtin_amdgcn_readlane((int)bl, wl)));
        // the owner of the winning entry frees its slot, which the sibling reuses
#pragma unroll
        for (int q = 0; q < FS; ++q)
            if (lane == wl && q == wq) { fs[q] = 0ull; ft[q] = ~0u; }
        --live;
        const int depth = (int)(tie >> 20), parent = (int)((tie >> 12) & 0xFFu), rank = (int)(tie & 0xFFFu);
        int si = (depth - 1) * K + rank + 1;
        si = si < kMaxTreeVK ? si : kMaxTreeVK - 1;
        const double sp = c_p[si];
#pragma unroll
        for (int q = 0; q < FS; ++q)
            if (q == (num >> 6) && lane == (num & (kWave - 1))) { ns[q] = score; nt[q] = tie; }
        if (rank + 1 < slot_get_i32(cn, depth - 1)) {
            put(wq * kWave + wl, slot_get_f64(ns, parent) * sp, tree_tie(depth, parent, rank + 1));
            ++live;
        }
        if (depth < B && slot_get_i32(cn, depth) > 0) {
            put(nf++, score * slot_get_f64(p0, depth), tree_tie(depth + 1, num, 0));
            ++live;
        }
        ++num;
    }
    const int64_t ob = (int64_t)b * (V + 1);
#pragma unroll
    for (int q = 0; q < FS; ++q) {
        const int n = q * kWave + lane;
        const bool used = n < num;
        const uint32_t t = nt[q];
        const int depth = (int)(t >> 20), parent = (int)((t >> 12) & 0xFFu), rank = (int)(t & 0xFFFu);
        int tok = -1, par = -1, dep = -1;
        if (n == 0) { dep = 0; }
        else if (used) { tok = c_id[(depth - 1) * K + rank]; par = parent; dep = depth; }
        if (n <= V) {
            o.node_token[ob + n] = tok;
            o.node_parent[ob + n] = par;
            o.node_depth[ob + n] = dep;
            if (o.node_score) o.node_score[ob + n] = used ? ns[q] : 0.0;
        }
    }
    if (lane == 0) o.num_nodes[b] = num;
}

// ---- tree walk (one workgroup per request) ---------------------------------------
constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / kWave;

// LDS copy of one request's tree and every node's depth.  Node arrays are read
// at once (all V + 1 slots); depths come from pointer jumping: (anc, dist)
// climbs towards the root in doubling steps; -1 marks the root reached, -2 a
// broken parent link (depth -1).  Called by all kWalkThreads threads.
struct TreeLds {
    int32_t dep[kMaxNodes], tok[kMaxNodes], par[kMaxNodes];
    int32_t anc[2][kMaxNodes], dist[2][kMaxNodes];
};

__device__ __forceinline__ void tree_depths(const int32_t* node_token, const int32_t* node_parent, int64_t ob,
                                            int nn, int V, TreeLds& L)
{
    const int t = (int)threadIdx.x;
    int anc = -2, dist = 0;
    if (t <= V) {
        const int p = node_parent[ob + t];
        const int tk = node_token[ob + t];
        if (t == 0) { anc = -1; L.par[0] = -1; L.tok[0] = -1; }
        else if (t < nn) { anc = (p >= 0 && p < t) ? p : -2; dist = 1; L.par[t] = p; L.tok[t] = tk; }
        L.anc[0][t] = anc;
        L.dist[0][t] = dist;
    }
    __syncthreads();
    for (int it = 0; it < 8; ++it) {
        const int cur = it & 1;
        if (t < nn && anc >= 0) {
            const int a = L.anc[cur][anc];
            dist += L.dist[cur][anc];
            anc = a;
        }
        if (t < nn) { L.anc[cur ^ 1][t] = anc; L.dist[cur ^ 1][t] = dist; }
        __syncthreads();
    }
    if (t < nn) L.dep[t] = (anc == -1) ? dist : -1;
    __syncthreads();
}

// The walk itself from every node's sample s_t (one wave): emit the node's
// sample, then move to the child carrying that token, found by ballot.
__device__ __forceinline__ void follow_path(int b, int B, int nn, const int32_t* s_t, const TreeLds& L,
                                            const WalkOut& o, int lane)
{
    int32_t* tok = o.tokens + (int64_t)b * (B + 1);
    int32_t* pth = o.path + (int64_t)b * (B + 1);
    int n = 0, d = 0;
    uint32_t fl = 0;
    for (;;) {
        const int32_t t = s_t[n];
        if (lane == 0) { tok[d] = t; pth[d] = n; }
        if (t < 0) fl |= 1u;
        int child = -1;
        if (t >= 0 && d < B)
            for (int base = 1; base < nn && child < 0; base += kWave) {
                const int c = base + lane;
                const uint64_t m = __ballot(c < nn && L.par[c] == n && L.tok[c] == t);
                if (m) child = base + wave_first_lane(m);
            }
        if (child < 0) break;
        n = child;
        ++d;
    }
    for (int j = d + 1 + lane; j <= B; j += kWave) { tok[j] = -1; pth[j] = -1; }
    if (lane == 0) {
        o.accept_len[b] = d + 1;
        if (o.flags) o.flags[b] = fl;
    }
}

__global__ __launch_bounds__(kWalkThreads) void tree_walk_kernel(
    int32_t batch, int32_t B, int32_t V, SparseOut sup, uint64_t seed, uint64_t offset,
    const uint32_t* req_ids, const int32_t* node_token, const int32_t* node_parent,
    const int32_t* num_nodes, WalkOut o)
{
    __shared__ TreeLds L;
    __shared__ int32_t s_t[kMaxNodes];

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x;
    const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
    const int cap = sup.cap;
    int nn = num_nodes[b];
    nn = nn < 1 ? 1 : (nn > V + 1 ? V + 1 : nn);
    const int64_t ob = (int64_t)b * (V + 1);
    tree_depths(node_token, node_parent, ob, nn, V, L);
    // every node's sample, drawn with the uniform of its depth
    // the next node's support is loaded while this one is sampled
    auto node_live = [&](int n, int* cnt) __attribute__((always_inline)) {
        const int dep = L.dep[n];
        *cnt = sup.count[ob + n];
        return dep >= 0 && dep <= B && *cnt > 0;
    };
    WaveRow R;
    int cnt = 0;
    bool live = false;
    if (w < nn) {
        live = node_live(w, &cnt);
        wave_load_support(sup.ids + (ob + w) * cap, sup.probs + (ob + w) * cap, sup.cum + (ob + w) * cap,
                          live ? cnt : 0, cap, R, lane);
    }
    for (int n = w; n < nn; n += kWalkWaves) {
        const int nx = n + kWalkWaves;
        WaveRow Rn;
        int cntn = 0;
        bool liven = false;
        if (nx < nn) {
            liven = node_live(nx, &cntn);
            wave_load_support(sup.ids + (ob + nx) * cap, sup.probs + (ob + nx) * cap, sup.cum + (ob + nx) * cap,
                              liven ? cntn : 0, cap, Rn, lane);
        }
        int32_t t = -1;
        if (live) {
            const Draw d = uno_draw(seed, req, (uint32_t)L.dep[n], offset);
            double dummy;
            t = wave_sample_cum(R, cnt, d.u[2], &dummy, lane);
        }
        if (lane == 0) s_t[n] = t;
        R = Rn;
        cnt = cntn;
        live = liven;
    }
    __syncthreads();
    if (w == 0) follow_path(b, B, nn, s_t, L, o, lane);
}

// ---- dense linear ------------------------------------------------------------------
constexpr int kDenseThreads = 256;
constexpr int kProposeMaxThreads = 1024;   // dense_propose_kernel: up to one wave per proposal
constexpr int kDenseWaves = kDenseThreads / kWave;
constexpr int kPerLane = kDenseChunk / kWave;   // 32 logits per lane per chunk

// Chunk c of a row into registers: element (j*64 + lane)*EPV + e at x[j*EPV + e];
// -inf past the end of the row.
template <bool BF16>
__device__ __forceinline__ void load_chunk(const char* row, int64_t N, int64_t c, float* x, int lane)
{
    using V = Vec<BF16>;
    constexpr int EPV = V::EPV, ESZ = V::ESZ, NV = kPerLane / EPV;
    const int64_t beg = c * kDenseChunk;
    const int64_t n = (N - beg < kDenseChunk) ? (N - beg) : kDenseChunk;
    const bool vec_ok = (n == kDenseChunk) && ((((uintptr_t)(row + beg * ESZ)) & 15u) == 0);
    if (vec_ok) {
        const typename V::T* p = reinterpret_cast<const typename V::T*>(row + beg * ESZ);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const typename V::T v = V::load_stream(p + j * kWave + lane);
#pragma unroll
            for (int e = 0; e < EPV; ++e) x[j * EPV + e] = V::get(v, e);
        }
    } else {
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int64_t i = (int64_t)(j * kWave + lane) * EPV + e;
                x[j * EPV + e] = (i < n) ? load_scalar<BF16>(row, beg + i) : -INFINITY;
            }
    }
}

// Chunk-stat term of chunk c relative to the row max m.
__device__ __forceinline__ double chunk_term(const float* cm, const double* cs, int c, float m, const DenseExp& ex)
{
    return (cm[c] > -INFINITY) ? cs[c] * ex((double)cm[c] - (double)m) : 0.0;
}

// Row max m and normaliser S from chunk statistics; S accumulates 64-chunk
// blocks of an inclusive wave scan, the same sums dense_locate walks.
__device__ bool dense_row_stat(const float* cm, const double* cs, int nc, const DenseExp& ex, int lane,
                               float* m_out, double* S_out)
{
    float m = -INFINITY;
    bool bad = false;
    for (int c = lane; c < nc; c += kWave) {
        m = fmaxf(m, cm[c]);
        bad |= (cm[c] == INFINITY);
    }
    m = wave_max_f32(m);
    bad = __ballot(bad) != 0ull;
    if (bad || !(m > -INFINITY)) { *m_out = NAN; *S_out = NAN; return false; }
    double S = 0.0;
    for (int base = 0; base < nc; base += kWave) {
        const int c = base + lane;
        const double term = (c < nc) ? chunk_term(cm, cs, c, m, ex) : 0.0;
        const double incl = wave_incl_scan_f64(term, lane);
        S += __shfl(incl, kWave - 1, kWave);
    }
    *m_out = m;
    *S_out = S;
    return S > 0.0;
}

// First chunk whose cumulative term exceeds t; *before = cumulative before it.
// -1 if none (t at or past the total).
template <typename TermF>
__device__ int dense_locate(int nc, double t, TermF term_of, int lane, double* before)
{
    double C = 0.0;
    for (int base = 0; base < nc; base += kWave) {
        const int c = base + lane;
        const double term = (c < nc) ? term_of(c) : 0.0;
        const double incl = wave_incl_scan_f64(term, lane);
        const uint64_t hit = __ballot(c < nc && term > 0.0 && C + incl > t);
        if (hit) {
            const int l = wave_first_lane(hit);
            *before = C + __shfl(incl - term, l, kWave);
            return base + l;
        }
        C += __shfl(incl, kWave - 1, kWave);
    }
    *before = C;
    return -1;
}

// Last chunk with a positive term (-1 if none).
template <typename TermF>
__device__ int dense_last_positive_chunk(int nc, TermF term_of, int lane)
{
    int best = -1;
    for (int c = lane; c < nc; c += kWave)
        if (term_of(c) > 0.0) best = c;
    for (int d = kWave / 2; d >= 1; d >>= 1) best = max(best, __shfl_xor(best, d, kWave));
    return best;
}

// Smallest element of a chunk (weights from wf, element layout of load_chunk)
// whose cumulative weight exceeds tau; the last positive element if none does.
template <int EPV, typename WeightF>
__device__ int pick_in_chunk(WeightF wf, double tau, int lane)
{
    constexpr int NV = kPerLane / EPV;
    double run = 0.0;
    int last_pos = -1;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        double wl[EPV];
        double lsum = 0.0;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            wl[e] = wf(j * EPV + e);
            lsum += wl[e];
            if (wl[e] > 0.0) last_pos = (j * kWave + lane) * EPV + e;
        }
        const double incl = wave_incl_scan_f64(lsum, lane);
        const uint64_t hit = __ballot(run + incl > tau);
        if (hit) {
            const int l = wave_first_lane(hit);
            int ep = -1;
            if (lane == l) {
                double cc = run + (incl - lsum);
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    cc += wl[e];
                    if (ep < 0 && cc > tau) ep = e;
                }
                if (ep < 0) {
#pragma unroll
                    for (int e = EPV - 1; e >= 0; --e)
                        if (ep < 0 && wl[e] > 0.0) ep = e;
                }
            }
            ep = __shfl(ep, l, kWave);
            return (j * kWave + l) * EPV + ep;
        }
        run += __shfl(incl, kWave - 1, kWave);
    }
    for (int d = kWave / 2; d >= 1; d >>= 1) last_pos = max(last_pos, __shfl_xor(last_pos, d, kWave));
    return last_pos;
}

// Chunk total with the accumulation order of pick_in_chunk.
template <int EPV, typename WeightF>
__device__ double chunk_total(WeightF wf, int lane)
{
    constexpr int NV = kPerLane / EPV;
    double run = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        double lsum = 0.0;
#pragma unroll
        for (int e = 0; e < EPV; ++e) lsum += wf(j * EPV + e);
        const double incl = wave_incl_scan_f64(lsum, lane);
        run += __shfl(incl, kWave - 1, kWave);
    }
    return run;
}

// Support test of a dense row: finite, and at or above the row's keep
// threshold (0 keeps every finite logit).
__device__ __forceinline__ bool dense_keeps(uint64_t thr, float x, int64_t id)
{
    return finite_f32(x) && order_key(float_key(x), (int32_t)id) >= thr;
}

// Id of entry i of chunk c as load_chunk lays it out in this lane.
template <int EPV>
__device__ __forceinline__ int64_t chunk_elem_id(int64_t c, int i, int lane)
{
    return c * kDenseChunk + (int64_t)((i / EPV) * kWave + lane) * EPV + i % EPV;
}

__device__ __forceinline__ uint64_t row_keep(const DenseChunks& dc, int64_t r)
{
    return dc.keep ? dc.keep[r] : 0ull;
}

// Sample a dense filtered row p = exp((z - m)/T) / S (over the logits the keep
// threshold admits) with uniform u.
template <bool BF16>
__device__ int32_t dense_sample_row(const char* row, int64_t N, const float* cm, const double* cs, int nc,
                                    float m, double S, double u, const DenseExp& ex, int lane, uint64_t thr)
{
    auto term = [&](int c) { return chunk_term(cm, cs, c, m, ex); };
    const double t = u * S;
    double before;
    int c = dense_locate(nc, t, term, lane, &before);
    double tau;
    if (c < 0) {
        c = dense_last_positive_chunk(nc, term, lane);
        if (c < 0) return -1;
        tau = INFINITY;
    } else {
        tau = (t - before) / ex((double)cm[c] - (double)m);
    }
    float x[kPerLane];
    load_chunk<BF16>(row, N, c, x, lane);
    const double mc = (double)cm[c];
    constexpr int EPV = Vec<BF16>::EPV;
    auto wf = [&](int i) { return dense_keeps(thr, x[i], chunk_elem_id<EPV>(c, i, lane)) ? ex((double)x[i] - mc) : 0.0; };
    const int l = pick_in_chunk<Vec<BF16>::EPV>(wf, tau, lane);
    return l < 0 ? -1 : (int32_t)(c * (int64_t)kDenseChunk + l);
}

// Global row index of local row i of request b (draft rows 0..B-1, then target 0..B).
__device__ __forceinline__ int64_t linear_row(int32_t batch, int32_t B, int b, int i)
{
    return i < B ? (int64_t)b * B + i : (int64_t)batch * B + (int64_t)b * (B + 1) + (i - B);
}

template <bool BF16>
__device__ __forceinline__ float load_one(const char* row, int64_t i)
{
    if constexpr (BF16) {
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[i] << 16);
    } else {
        return reinterpret_cast<const float*>(row)[i];
    }
}

// Row stats of every row, proposals, acceptance and the first rejection.
template <bool BF16>
__global__ __launch_bounds__(kProposeMaxThreads) void dense_propose_kernel(
    RowSource src, int32_t batch, int32_t B, int64_t N, double log2e_over_T, DenseChunks dc,
    uint64_t seed, uint64_t offset, const uint32_t* req_ids, float* row_m, double* row_S,
    int32_t* jstar_out, int32_t* y_out, uint32_t* flag_out, LinearOut o)
{
    __shared__ double s_exp2[kExp2Entries];
    __shared__ int32_t s_acc[kMaxLinearB];
    __shared__ uint32_t s_flags;
    load_exp2_table(s_exp2);
    __syncthreads();
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x;
    const DenseExp ex{ log2e_over_T, s_exp2 };
    const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
    const int nc = dc.nchunks;
    const int64_t row_bytes = N * Vec<BF16>::ESZ;
    if (threadIdx.x == 0) s_flags = 0;

    const int nw = (int)(blockDim.x / kWave);   // one wave per proposal, up to 16
    for (int i = w; i < 2 * B + 1; i += nw) {
        const int64_t r = linear_row(batch, B, b, i);
        float m;
        double S;
        dense_row_stat(dc.cmax + r * nc, dc.csum + r * nc, nc, ex, lane, &m, &S);
        if (lane == 0) { row_m[r] = m; row_S[r] = S; }
    }
    __syncthreads();

    uint32_t flags = 0;
    for (int j = w; j < B; j += nw) {
        const Draw d = uno_draw(seed, req, (uint32_t)j, offset);
        const int64_t qr = linear_row(batch, B, b, j), pr = linear_row(batch, B, b, B + j);
        const float mq = row_m[qr], mp = row_m[pr];
        const double Sq = row_S[qr], Sp = row_S[pr];
        const char* qrow = row_pointer(src, qr, row_bytes);
        const char* prow = row_pointer(src, pr, row_bytes);
        int32_t y = -1;
        int acc = 0;
        if (Sq > 0.0) {
            y = dense_sample_row<BF16>(qrow, N, dc.cmax + qr * nc, dc.csum + qr * nc, nc, mq, Sq, d.u[0], ex, lane,
                                       row_keep(dc, qr));
        } else {
            flags |= 1u;
        }
        if (y >= 0) {
            const double qy = ex((double)load_one<BF16>(qrow, y) - (double)mq) / Sq;
            double py = 0.0;
            if (Sp > 0.0) {
                const float zp = load_one<BF16>(prow, y);
                if (dense_keeps(row_keep(dc, pr), zp, y)) py = ex((double)zp - (double)mp) / Sp;
            } else {
                flags |= 1u;
            }
            acc = (d.u[1] * qy < py) ? 1 : 0;
        }
        if (lane == 0) {
            s_acc[j] = acc;
            y_out[(int64_t)b * B + j] = y;
            if (o.proposals) o.proposals[(int64_t)b * B + j] = y;
        }
    }
    if (flags && lane == 0) atomicOr(&s_flags, flags);
    __syncthreads();
    if (threadIdx.x == 0) {
        int js = B;
        for (int j = 0; j < B; ++j)
            if (!s_acc[j]) { js = j; break; }
        jstar_out[b] = js;
        flag_out[b] = s_flags;
    }
}

// Exact chunk statistics of the target row each request draws its last token
// from (p_j* after a rejection, the bonus row p_B otherwise).  The chunk pass
// gave target rows fast sums, which only enter acceptance ratios.
template <bool BF16>
__global__ __launch_bounds__(kDenseThreads) void dense_exact_row_kernel(
    RowSource src, int32_t batch, int32_t B, int64_t N, double log2e_over_T, DenseChunks dc,
    const int32_t* jstar_in)
{
    __shared__ double s_exp2[kExp2Entries];
    load_exp2_table(s_exp2);
    __syncthreads();
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x;
    const int nc = dc.nchunks;
    const int js = jstar_in[b];
    const int64_t pr = linear_row(batch, B, b, B + (js < B ? js : B));
    const DenseExp ex{ log2e_over_T, s_exp2 };
    // the row's chunks dealt over gridDim.y workgroups, round robin over their waves
    for (int c = blockIdx.y * kDenseWaves + w; c < nc; c += gridDim.y * kDenseWaves) {
        float x[kPerLane];
        load_chunk<BF16>(row_pointer(src, pr, N * Vec<BF16>::ESZ), N, c, x, lane);
        float mx;
        double sum;
        uint32_t cntf;
        chunk_stats_exact<true>(x, ex, &mx, &sum, &cntf);
        if (lane == 0) {
            const int64_t slot = pr * nc + c;
            dc.cmax[slot] = mx;
            dc.csum[slot] = (mx < INFINITY) ? sum : NAN;
            if (dc.ccount) dc.ccount[slot] = (int32_t)cntf;
        }
    }
}

// Residual mass per chunk for requests that rejected a proposal.
template <bool BF16>
__global__ __launch_bounds__(kDenseThreads) void dense_residual_kernel(
    RowSource src, int32_t batch, int32_t B, int64_t N, double log2e_over_T, DenseChunks dc,
    const float* row_m, const double* row_S, const int32_t* jstar_in, double* resid)
{
    const int nc = dc.nchunks;
    __shared__ double s_exp2[kExp2Entries];
    load_exp2_table(s_exp2);
    __syncthreads();
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x;
    const int c0 = blockIdx.y * kDenseWaves + w;
    const int js = jstar_in[b];
    if (js >= B || c0 >= nc) return;
    const DenseExp ex{ log2e_over_T, s_exp2 };
    const int64_t qr = linear_row(batch, B, b, js), pr = linear_row(batch, B, b, B + js);
    float mpf;
    double Sp;
    dense_row_stat(dc.cmax + pr * nc, dc.csum + pr * nc, nc, ex, lane, &mpf, &Sp);   // exact chunks
    const double Sq = row_S[qr];
    // the request's chunks dealt over gridDim.y workgroups, round robin over their waves
    for (int c = c0; c < nc; c += gridDim.y * kDenseWaves) {
        double total = 0.0;
        if (Sp > 0.0) {
            const int64_t row_bytes = N * Vec<BF16>::ESZ;
            const bool q_ok = Sq > 0.0;
            float xp[kPerLane], xq[kPerLane];
            load_chunk<BF16>(row_pointer(src, pr, row_bytes), N, c, xp, lane);
            if (q_ok) load_chunk<BF16>(row_pointer(src, qr, row_bytes), N, c, xq, lane);
            const double mp = (double)mpf, mq = (double)row_m[qr];
            const double iSp = 1.0 / Sp, iSq = q_ok ? 1.0 / Sq : 0.0;
            const uint64_t tp = row_keep(dc, pr), tq = row_keep(dc, qr);
            constexpr int EPV = Vec<BF16>::EPV;
            auto wf = [&](int i) {
                const int64_t id = chunk_elem_id<EPV>(c, i, lane);
                const double pv = dense_keeps(tp, xp[i], id) ? ex((double)xp[i] - mp) * iSp : 0.0;
                const double qv = (q_ok && dense_keeps(tq, xq[i], id)) ? ex((double)xq[i] - mq) * iSq : 0.0;
                const double dl = pv - qv;
                return dl > 0.0 ? dl : 0.0;
            };
            total = chunk_total<EPV>(wf, lane);
        }
        if (lane == 0) resid[(int64_t)b * nc + c] = total;
    }
}

// Residual (or bonus) sample and the cycle's outputs.
template <bool BF16>
__global__ __launch_bounds__(kWave) void dense_finish_kernel(
    RowSource src, int32_t batch, int32_t B, int64_t N, double log2e_over_T, DenseChunks dc,
    uint64_t seed, uint64_t offset, const uint32_t* req_ids, const float* row_m, const double* row_S,
    const int32_t* jstar_in, const int32_t* y_in, const uint32_t* flag_in, const double* resid,
    LinearOut o)
{
    __shared__ double s_exp2[kExp2Entries];
    load_exp2_table(s_exp2);
    __syncthreads();
    const int lane = lane_id();
    const int b = blockIdx.x;
    const DenseExp ex{ log2e_over_T, s_exp2 };
    const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
    const int nc = dc.nchunks;
    const int64_t row_bytes = N * Vec<BF16>::ESZ;
    const int js = jstar_in[b];
    const Draw d = uno_draw(seed, req, (uint32_t)js, offset);
    uint32_t fl = flag_in[b];
    int32_t fin = -1;
    const int64_t pr = linear_row(batch, B, b, B + js);
    const char* prow = row_pointer(src, pr, row_bytes);
    float mp;
    double Sp;
    dense_row_stat(dc.cmax + pr * nc, dc.csum + pr * nc, nc, ex, lane, &mp, &Sp);   // exact chunks
    if (!(Sp > 0.0)) {
        fl |= 1u;
    } else if (js < B) {
        const int64_t qr = linear_row(batch, B, b, js);
        const double Sq = row_S[qr];
        const bool q_ok = Sq > 0.0;
        const double* R = resid + (int64_t)b * nc;
        auto rterm = [&](int c) { return R[c]; };
        double Rtot = 0.0;
        for (int base = 0; base < nc; base += kWave) {
            const int c = base + lane;
            const double incl = wave_incl_scan_f64(c < nc ? R[c] : 0.0, lane);
            Rtot += __shfl(incl, kWave - 1, kWave);
        }
        if (Rtot > 0.0) {
            const double t = d.u[2] * Rtot;
            double before;
            int c = dense_locate(nc, t, rterm, lane, &before);
            double tau = t - before;
            if (c < 0) { c = dense_last_positive_chunk(nc, rterm, lane); tau = INFINITY; }
            float xp[kPerLane], xq[kPerLane];
            load_chunk<BF16>(prow, N, c, xp, lane);
            if (q_ok) load_chunk<BF16>(row_pointer(src, qr, row_bytes), N, c, xq, lane);
            const double mpd = (double)mp, mq = (double)row_m[qr];
            const double iSp = 1.0 / Sp, iSq = q_ok ? 1.0 / Sq : 0.0;
            const uint64_t tp = row_keep(dc, pr), tq = row_keep(dc, qr);
            constexpr int EPV = Vec<BF16>::EPV;
            auto wf = [&](int i) {
                const int64_t id = chunk_elem_id<EPV>(c, i, lane);
                const double pv = dense_keeps(tp, xp[i], id) ? ex((double)xp[i] - mpd) * iSp : 0.0;
                const double qv = (q_ok && dense_keeps(tq, xq[i], id)) ? ex((double)xq[i] - mq) * iSq : 0.0;
                const double dl = pv - qv;
                return dl > 0.0 ? dl : 0.0;
            };
            const int l = pick_in_chunk<EPV>(wf, tau, lane);
            fin = l < 0 ? -1 : (int32_t)(c * (int64_t)kDenseChunk + l);
        } else {
            fl |= 2u;
        }
        if (fin < 0)
            fin = dense_sample_row<BF16>(prow, N, dc.cmax + pr * nc, dc.csum + pr * nc, nc, mp, Sp, d.u[2], ex, lane,
                                         row_keep(dc, pr));
    } else {
        fin = dense_sample_row<BF16>(prow, N, dc.cmax + pr * nc, dc.csum + pr * nc, nc, mp, Sp, d.u[2], ex, lane,
                                     row_keep(dc, pr));
    }
    int32_t* tok = o.tokens + (int64_t)b * (B + 1);
    for (int j = lane; j <= B; j += kWave) tok[j] = (j < js) ? y_in[(int64_t)b * B + j] : (j == js ? fin : -1);
    if (lane == 0) {
        o.accept_len[b] = js + 1;
        if (o.flags) o.flags[b] = fl;
    }
}

// ---- full-vocabulary nucleus (top-p without top-k) -------------------------------
// The support is the shortest prefix of the filter order (z desc, id asc) whose
// mass reaches top_p (the first logit always kept).  One workgroup per row
// finds the cut by a mass-weighted select over the 32-bit order keys of the
// logits: a key range known to hold the cut is split into up to 2048 equal
// bins, one pass over the row accumulates each bin's logit count and exact
// fp64 mass exp((z - m)/T), and the bin where the mass counted from the top
// reaches top_p * S becomes the next range, until one key is left.  The
// first range starts at the value below which all logits together hold less
// than (1 - top_p) / 2 of the mass.  The number of tied logits kept at the cut
// follows from the mass left; which ties (smaller ids first) from an ordered
// count over ids.  The row's keep threshold is the order key of its last kept
// logit; the chunk sums are then rewritten over the support.
// When the first level's chosen bin holds few logits, one more pass instead
// collects them (as order keys) together with the chunk sums above the bin;
// the collected logits are ranked in LDS and the cut is the first whose
// inclusive mass, counted from the top in the filter order, reaches the target.
constexpr int kNucThreads = 256;
constexpr int kNucWaves = kNucThreads / kWave;
constexpr int kNucBins = 2048;
constexpr int kNucCand = kNucBins / 2 / kNucWaves;   // collected logits per wave (in s_cnt)

// Three workgroups per CU (168 VGPRs; a few spills, outside the streaming
// loops' loads); the LDS of four would not fit.
template <bool BF16>
__global__ __launch_bounds__(kNucThreads, 3) void nucleus_kernel(RowSource src, int64_t N, double log2e_over_T,
                                                              double top_p, DenseChunks dc, int32_t* out_count,
                                                              double* out_stats)
{
    __shared__ double s_exp2[kExp2Entries];
    __shared__ double s_mass[kNucBins];
    __shared__ uint32_t s_cnt[kNucBins];
    __shared__ double s_row[2];              // S, mass above the cut's bin
    __shared__ float s_m;
    __shared__ int64_t s_cab;                // logits above the cut's bin
    __shared__ int s_bin;
    __shared__ int64_t s_wc[kNucWaves];
    __shared__ int64_t s_nab[kNucWaves];
    __shared__ int32_t s_idlim;
    constexpr int EPV = Vec<BF16>::EPV;
    load_exp2_table(s_exp2);
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t r = blockIdx.x;
    const int nc = dc.nchunks;
    const float* cm = dc.cmax + r * nc;
    double* cs = dc.csum + r * nc;
    const char* row = row_pointer(src, r, N * Vec<BF16>::ESZ);
    const DenseExp ex{ log2e_over_T, s_exp2 };
    __syncthreads();
    if (w == 0) {
        float m = NAN;
        double S = -1.0;
        const bool ok = row != nullptr && dense_row_stat(cm, cs, nc, ex, lane, &m, &S);
        if (lane == 0) { s_row[0] = ok ? S : -1.0; s_m = m; }
    }
    __syncthreads();
    const double S = s_row[0];
    const float m = s_m;
    if (!(S > 0.0)) {                        // invalid or absent row: an empty support
        if (threadIdx.x == 0) {
            dc.keep[r] = ~0ull;
            if (out_count) out_count[r] = -1;
            if (out_stats) { out_stats[2 * r] = NAN; out_stats[2 * r + 1] = NAN; }
        }
        return;
    }
    const double target = top_p * S;
    // chunks c = w, w + kNucWaves, ... handed to body(c, x).  No prefetch of
    // the next chunk: its 32 registers would hold the kernel to two waves per
    // SIMD, and three waves hide more latency (measured 614 -> about 480 us on
    // 1088 rows of 151936 logits).
    auto each_chunk = [&](auto body) __attribute__((always_inline)) {
        for (int c = w; c < nc; c += kNucWaves) {
            float xc[kPerLane];
            load_chunk<BF16>(row, N, c, xc, lane);
            body(c, xc);
        }
    };
    // logits below z_lo weigh less than (1 - p) S / (2N) each, (1 - p) S / 2 in all
    const double T = 1.0 / (log2e_over_T * 0.69314718055994530942);
    const double z_lo = (double)m + T * log((1.0 - top_p) * S / (2.0 * (double)N));
    // First level: equal value bins over [vlo, m], so the logits near the cut
    // spread over the bins (equal key bins would stack whole octaves into a
    // few); later levels: equal key bins within the chosen value bin.
    const float vlo_f = (float)(z_lo > -3.0e38 ? (z_lo < (double)m ? z_lo : (double)m) : -3.0e38);
    const double vlo = (double)vlo_f;
    const double vscale = (vlo < (double)m) ? (double)kNucBins / ((double)m - vlo) : 0.0;
    const float vscale_f = (float)(vscale < 3.0e38 ? vscale : 3.0e38);
    // The value bin of a logit z >= vlo, in fp32: monotone in z (a difference
    // with a constant, a positive scale, a clamp and a truncation of a
    // non-negative number), which is all the levels rely on.
    auto vbin = [&](float z) __attribute__((always_inline)) {
        return (int)fminf((z - vlo_f) * vscale_f, (float)(kNucBins - 1));
    };
    // Smallest key in [ka, kb] whose logit's value bin reaches tb (kb + 1 when
    // none does): the keys of bin tb are [first_key(tb), first_key(tb + 1)).
    const uint32_t kvlo = float_key(vlo_f), kvm = float_key(m);
    auto first_key = [&](int tb) __attribute__((always_inline)) {
        uint32_t a = kvlo, b = kvm + 1u;
        while (a < b) {
            const uint32_t mid = a + (b - a) / 2u;
            if (vbin(key_float(mid)) >= tb) b = mid;
            else a = mid + 1u;
        }
        return a;
    };
    int b0 = -1;                             // the chosen value bin
    uint32_t lo = 0, hi = 0;                 // later levels: keys in [lo, hi)
    double A = 0.0;                          // mass above the current range
    int64_t cab = 0;                         // logits above the current range
    // With the one-pass finish available, the first level keeps masses only:
    // the finish counts the logits above the chosen bin itself (a non-empty
    // bin is one of positive mass, every finite logit weighing at least 2^-1000).
    const bool one_pass = nc <= kNucWaves * kWave;
    auto level = [&]() __attribute__((always_inline)) {
        const bool first = b0 < 0;
        const bool counts = !(first && one_pass);
        const uint32_t width = hi - lo;
        const int nb = first ? kNucBins : (width < (uint32_t)kNucBins ? (int)width : kNucBins);
        for (int b = (int)threadIdx.x; b < nb; b += kNucThreads) { s_mass[b] = 0.0; s_cnt[b] = 0u; }
        __syncthreads();
        each_chunk([&](int, const float (&x)[kPerLane]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) {
                if (!finite_f32(x[i]) || !(x[i] >= vlo_f)) continue;
                int bin;
                if (first) {
                    bin = vbin(x[i]);
                } else {
                    const uint32_t key = float_key(x[i]);
                    if (key < lo || key >= hi) continue;
                    bin = (int)((uint64_t)(key - lo) * (uint64_t)nb / width);
                }
                atomicAdd(&s_mass[bin], ex((double)x[i] - (double)m));
                if (counts) atomicAdd(&s_cnt[bin], 1u);
            }
        });
        __syncthreads();
        if (w == 0) {
            // bins from the top down: the first non-empty bin whose inclusive
            // mass reaches the target holds the last kept logit
            double run = A, crun = (double)cab;
            int found = -1, last = -1;
            double fa = 0.0, fc = 0.0, la = 0.0, lc = 0.0;
            for (int top = nb - 1; top >= 0 && found < 0; top -= kWave) {
                const int b = top - lane;
                const double mb = b >= 0 ? s_mass[b] : 0.0;
                const double cb = (b >= 0 && counts) ? (double)s_cnt[b] : 0.0;
                const bool filled = counts ? cb > 0.0 : mb > 0.0;
                const double incl = wave_incl_scan_f64(mb, lane);
                const double cincl = wave_incl_scan_f64(cb, lane);
                const uint64_t hit = __ballot(filled && run + incl >= target);
                if (hit) {
                    const int l = wave_first_lane(hit);
                    found = top - l;
                    fa = run + __shfl(incl - mb, l, kWave);
                    fc = crun + __shfl(cincl - cb, l, kWave);
                } else {
                    const uint64_t nz = __ballot(filled);
                    if (nz) {
                        const int l = 63 - __clzll((long long)nz);
                        last = top - l;
                        la = run + __shfl(incl - mb, l, kWave);
                        lc = crun + __shfl(cincl - cb, l, kWave);
                    }
                    run += __shfl(incl, kWave - 1, kWave);
                    crun += __shfl(cincl, kWave - 1, kWave);
                }
            }
            if (found < 0) { found = last; fa = la; fc = lc; }   // target past the summed mass: keep all
            if (lane == 0) { s_bin = found; s_row[1] = fa; s_cab = (int64_t)fc; }
        }
        __syncthreads();
        if (first) {
            // exactly the keys of the value bin's logits
            b0 = s_bin;
            lo = first_key(b0);
            hi = first_key(b0 + 1);
        } else {
            // bin b holds the keys k with floor((k - lo) * nb / width) == b
            const uint64_t fb = (uint64_t)s_bin;
            const uint32_t nlo = lo + (uint32_t)((fb * width + (uint64_t)nb - 1) / (uint64_t)nb);
            const uint32_t nhi = lo + (uint32_t)(((fb + 1) * width + (uint64_t)nb - 1) / (uint64_t)nb);
            lo = nlo;
            hi = nhi;
        }
        A = s_row[1];
        cab = s_cab;
    };
    level();
    // ---- one-pass finish when the chosen value bin holds few logits ----------
    if (one_pass) {
        // Candidates: this wave's logits of bin b0 as order keys (hi, lo words
        // in s_cnt), appended chunk by chunk, so each chunk's run is
        // contiguous; lane q holds the run bounds and the sum above the bin
        // of the wave's q-th chunk (chunks w, w + kNucWaves, ...).
        uint32_t* cl = s_cnt + 2 * kNucCand * w;
        int ncl = 0;
        int64_t nab = 0;                      // this wave's logits above the bin
        int run_b = 0, run_e = 0;
        double above = 0.0;
        each_chunk([&](int c, const float (&x)[kPerLane]) __attribute__((always_inline)) {
            const int q = (c - w) / kNucWaves;
            const int start = ncl;
            double sum = 0.0;
            const float mcf = cm[c];
            if (mcf > -INFINITY) {
                const double mc = (double)mcf;
#pragma unroll
                for (int i = 0; i < kPerLane; ++i) {
                    const float z = x[i];
                    const int vb = (finite_f32(z) && z >= vlo_f) ? vbin(z) : -1;
                    if (vb > b0) sum += ex((double)z - mc);
                    nab += __popcll(__ballot(vb > b0));
                    const bool cand = vb == b0;
                    const uint64_t mk = __ballot(cand);
                    if (mk) {
                        const int pos = ncl + __popcll(mk & lanes_below(lane));
                        if (cand && pos < kNucCand) {
                            const uint64_t ok = order_key(float_key(z), (int32_t)chunk_elem_id<EPV>(c, i, lane));
                            cl[2 * pos] = (uint32_t)(ok >> 32);
                            cl[2 * pos + 1] = (uint32_t)ok;
                        }
                        ncl += __popcll(mk);
                    }
                }
            }
            sum = wave_sum_f64(sum);
            if (lane == q) { run_b = start; run_e = ncl; above = sum; }
        });
        if (lane == 0) { s_wc[w] = ncl; s_nab[w] = nab; }
        __syncthreads();
        int64_t ntot = 0;
        bool fits = true;
        cab = 0;
#pragma unroll
        for (int o = 0; o < kNucWaves; ++o) {
            ntot += s_wc[o];
            fits = fits && s_wc[o] <= kNucCand;
            cab += s_nab[o];
        }
        if (fits && ntot > 0) {
            // rank every candidate over the four lists; sorted masses go to
            // s_mass[0, half), sorted keys (bit patterns) to s_mass[half, ...)
            constexpr int half = kNucBins / 2;
            for (int g = (int)threadIdx.x; g < (int)ntot; g += kNucThreads) {
                int o = 0, i = g;
                while (i >= s_wc[o]) { i -= (int)s_wc[o]; ++o; }
                const uint32_t* lo_list = s_cnt + 2 * kNucCand * o;
                const uint64_t pk = ((uint64_t)lo_list[2 * i] << 32) | lo_list[2 * i + 1];
                int rank = 0;
                for (int o2 = 0; o2 < kNucWaves; ++o2) {
                    const uint32_t* l2 = s_cnt + 2 * kNucCand * o2;
                    const int n2 = (int)s_wc[o2];
                    for (int j = 0; j < n2; ++j) rank += ((((uint64_t)l2[2 * j] << 32) | l2[2 * j + 1]) > pk) ? 1 : 0;
                }
                s_mass[rank] = ex((double)key_float((uint32_t)(pk >> 32)) - (double)m);
                s_mass[half + rank] = __longlong_as_double((long long)pk);
            }
            __syncthreads();
            if (w == 0) {
                // first sorted candidate whose inclusive mass from the top
                // reaches the target (all of them when rounding leaves the
                // target unreached)
                double run = A;
                int jcut = -1;
                for (int top = 0; top < (int)ntot && jcut < 0; top += kWave) {
                    const int j = top + lane;
                    const double e = j < (int)ntot ? s_mass[j] : 0.0;
                    const double incl = wave_incl_scan_f64(e, lane);
                    const uint64_t hit = __ballot(j < (int)ntot && run + incl >= target);
                    if (hit) jcut = top + wave_first_lane(hit);
                    run += __shfl(incl, kWave - 1, kWave);
                }
                if (jcut < 0) jcut = (int)ntot - 1;
                if (lane == 0) s_bin = jcut;
            }
            __syncthreads();
            const int jcut = s_bin;
            const uint64_t thr = (uint64_t)__double_as_longlong(s_mass[half + jcut]);
            // chunk sums over the support: the sum above the bin plus the
            // run's kept candidates
            for (int c = w; c < nc; c += kNucWaves) {
                const int q = (c - w) / kNucWaves;
                const int b = __shfl(run_b, q, kWave), e = __shfl(run_e, q, kWave);
                const double ab = __shfl(above, q, kWave);
                const float mcf = cm[c];
                double add = 0.0;
                if (mcf > -INFINITY)
                    for (int i = b + lane; i < e; i += kWave) {
                        const uint64_t pk = ((uint64_t)cl[2 * i] << 32) | cl[2 * i + 1];
                        if (pk >= thr) add += ex((double)key_float((uint32_t)(pk >> 32)) - (double)mcf);
                    }
                add = wave_sum_f64(add);
                if (lane == 0) cs[c] = ab + add;
            }
            if (threadIdx.x == 0) {
                dc.keep[r] = thr;
                if (out_count) out_count[r] = (int32_t)(cab + jcut + 1);
                if (out_stats) { out_stats[2 * r] = (double)m; out_stats[2 * r + 1] = S; }
            }
            return;
        }
        __syncthreads();                      // the later levels reset s_mass and s_cnt
    }
    while (hi - lo > 1u) level();
    // ties at the cut: keep the j-th (by id) while the mass before it is below
    // the target
    const uint32_t tau = lo;
    const int64_t ctau = (int64_t)s_cnt[s_bin];
    const double etau = ex((double)key_float(tau) - (double)m);
    int64_t t = ctau;
    if (etau > 0.0) {
        const double x = ceil((target - A) / etau);
        t = x < 1.0 ? 1 : (x < (double)ctau ? (int64_t)x : ctau);
    }
    // the t-th tie in id order: each wave counts the ties in its run of whole
    // chunks, then the wave holding the t-th finds it chunk by chunk, and in
    // its chunk vector by vector (ids rise with the vector, the lane, then the
    // element)
    const int c0 = (int)((int64_t)nc * w / kNucWaves), c1 = (int)((int64_t)nc * (w + 1) / kNucWaves);
    auto chunk_ties = [&](int c, float (&x)[kPerLane]) __attribute__((always_inline)) {
        int n = 0;
        if (cm[c] > -INFINITY && float_key(cm[c]) >= tau) {
            load_chunk<BF16>(row, N, c, x, lane);
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) n += (finite_f32(x[i]) && float_key(x[i]) == tau) ? 1 : 0;
        } else {
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) x[i] = -INFINITY;
        }
        return (int64_t)wave_sum_f64((double)n);
    };
    // (all ties kept -- always so without ties -- needs no search: the
    // largest id keeps every logit of key tau)
    const bool search = t < ctau;
    if (threadIdx.x == 0) s_idlim = 0x7FFFFFFF;
    int64_t cw = 0;
    if (search)
        for (int c = c0; c < c1; ++c) {
            float x[kPerLane];
            cw += chunk_ties(c, x);
        }
    if (lane == 0) s_wc[w] = cw;
    __syncthreads();
    int64_t before = 0;
    for (int o = 0; o < w; ++o) before += s_wc[o];
    if (search && t > before && t <= before + cw) {
        int64_t need = t - before;
        for (int c = c0; c < c1; ++c) {
            float x[kPerLane];
            const int64_t n = chunk_ties(c, x);
            if (need > n) { need -= n; continue; }
            constexpr int NVEC = kPerLane / EPV;
#pragma unroll
            for (int j = 0; j < NVEC; ++j) {
                int nl = 0;
#pragma unroll
                for (int e = 0; e < EPV; ++e) nl += (finite_f32(x[j * EPV + e]) && float_key(x[j * EPV + e]) == tau) ? 1 : 0;
                const double incl = wave_incl_scan_f64((double)nl, lane);
                const double tot = __shfl(incl, kWave - 1, kWave);
                if ((double)need <= tot) {
                    const uint64_t at = __ballot((double)need <= incl && (double)need > incl - (double)nl);
                    const int l = wave_first_lane(at);
                    if (lane == l) {
                        int64_t k = need - (int64_t)(incl - (double)nl);      // k-th tie of this lane's vector
                        for (int e = 0; e < EPV; ++e) {
                            if (finite_f32(x[j * EPV + e]) && float_key(x[j * EPV + e]) == tau && --k == 0) {
                                s_idlim = (int32_t)(c * (int64_t)kDenseChunk + (int64_t)(j * kWave + lane) * EPV + e);
                                break;
                            }
                        }
                    }
                    break;
                }
                need -= (int64_t)tot;
            }
            break;
        }
    }
    __syncthreads();
    const uint64_t thr = order_key(tau, s_idlim);
    // chunk sums over the support, relative to each chunk's (unchanged) maximum
    each_chunk([&](int c, const float (&x)[kPerLane]) __attribute__((always_inline)) {
        double sum = 0.0;
        const float mcf = cm[c];
        if (mcf > -INFINITY) {
            const double mc = (double)mcf;
#pragma unroll
            for (int i = 0; i < kPerLane; ++i)
                if (dense_keeps(thr, x[i], chunk_elem_id<EPV>(c, i, lane))) sum += ex((double)x[i] - mc);
        }
        sum = wave_sum_f64(sum);
        if (lane == 0) cs[c] = sum;
    });
    if (threadIdx.x == 0) {
        dc.keep[r] = thr;
        if (out_count) out_count[r] = (int32_t)(cab + t);
        if (out_stats) { out_stats[2 * r] = (double)m; out_stats[2 * r + 1] = S; }
    }
}

// ---- dense tree (full-vocabulary filters) ------------------------------------------
// Target-sampled walk over node rows whose filter keeps the whole vocabulary:
// each live node's token is drawn from its row's exact chunk statistics (one
// wave per node, the uniform of the node's depth), then wave 0 follows the
// path as in the sparse walk.
template <bool BF16>
__global__ __launch_bounds__(kWalkThreads) void dense_walk_kernel(
    RowSource src, int32_t batch, int32_t B, int32_t V, int64_t N, double log2e_over_T, DenseChunks dc,
    uint64_t seed, uint64_t offset, const uint32_t* req_ids, const int32_t* node_token,
    const int32_t* node_parent, const int32_t* num_nodes, WalkOut o)
{
    __shared__ double s_exp2[kExp2Entries];
    __shared__ TreeLds L;
    __shared__ int32_t s_t[kMaxNodes];
    load_exp2_table(s_exp2);
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x;
    const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
    int nn = num_nodes[b];
    nn = nn < 1 ? 1 : (nn > V + 1 ? V + 1 : nn);
    const int64_t ob = (int64_t)b * (V + 1);
    tree_depths(node_token, node_parent, ob, nn, V, L);      // its barriers also publish the table
    const DenseExp ex{ log2e_over_T, s_exp2 };
    const int nc = dc.nchunks;
    const int64_t row_bytes = N * Vec<BF16>::ESZ;
    for (int n = w; n < nn; n += kWalkWaves) {
        const int dep = L.dep[n];
        int32_t t = -1;
        if (dep >= 0 && dep <= B) {
            const int64_t r = ob + n;
            const float* cm = dc.cmax + r * nc;
            const double* cs = dc.csum + r * nc;
            float m;
            double S;
            if (dense_row_stat(cm, cs, nc, ex, lane, &m, &S)) {
                const Draw d = uno_draw(seed, req, (uint32_t)dep, offset);
                t = dense_sample_row<BF16>(row_pointer(src, r, row_bytes), N, cm, cs, nc, m, S, d.u[2], ex, lane,
                                           row_keep(dc, r));
            }
        }
        if (lane == 0) s_t[n] = t;
    }
    __syncthreads();
    if (w == 0) follow_path(b, B, nn, s_t, L, o, lane);
}

// Tree build over full-vocabulary filters: the top-K supports come normalised
// over their K ids; this rescales them to the full softmax, whose normaliser
// the exact chunk statistics give (one wave per row).
__global__ __launch_bounds__(kDenseThreads) void dense_support_scale_kernel(int64_t rows, double inv_T,
                                                                           DenseChunks dc, const int32_t* limit,
                                                                           SparseOut sup)
{
    const int lane = lane_id();
    const int64_t r = (int64_t)blockIdx.x * kDenseWaves + threadIdx.x / kWave;
    if (r >= rows) return;
    int n = sup.count[r];
    if (n <= 0) return;
    if (limit && limit[r] < n) {
        // the nucleus ends inside the top K: both are prefixes of the filter order
        n = limit[r];
        if (lane == 0) sup.count[r] = n;
    }
    const int nc = dc.nchunks;
    const float* cm = dc.cmax + r * nc;
    const double* cs = dc.csum + r * nc;
    float m = -INFINITY;
    for (int c = lane; c < nc; c += kWave) m = fmaxf(m, cm[c]);
    m = wave_max_f32(m);
    double S = 0.0;
    for (int c = lane; c < nc; c += kWave)
        if (cm[c] > -INFINITY) S += cs[c] * exp(((double)cm[c] - (double)m) * inv_T);
    S = wave_sum_f64(S);
    const double scale = sup.stats[2 * r + 1] / S;
    double* p = sup.probs + r * sup.cap;
    for (int i = lane; i < n; i += kWave) p[i] *= scale;
    if (lane == 0) sup.stats[2 * r + 1] = S;
}

}  // namespace

hipError_t launch_linear_sparse(int32_t batch, int32_t B, const SparseOut& sup, uint64_t seed,
                                uint64_t offset, const uint32_t* request_ids, const LinearOut& o,
                                hipStream_t stream)
{
    if (sup.cum == nullptr) return hipErrorInvalidValue;     // needs id-ordered supports
    linear_sparse_kernel<<<dim3((unsigned)batch), kLinThreads, 0, stream>>>(batch, B, sup, seed, offset,
                                                                           request_ids, o);
    return hipGetLastError();
}

hipError_t launch_linear_dense(const RowSource& src, int32_t batch, int32_t B, int64_t vocab,
                               bool bf16, float temperature, const DenseChunks& dc,
                               const DenseScratch& sc, uint64_t seed, uint64_t offset,
                               const uint32_t* request_ids, const LinearOut& o, bool exact_all,
                               hipStream_t stream)
{
    const double c = 1.4426950408889634074 / (double)temperature;
    // about 2048 workgroups: with many requests each wave takes several chunks,
    // so fewer workgroups load the exponential table
    const int per_req = (dc.nchunks + kDenseWaves - 1) / kDenseWaves;
    const int want = (2048 + batch - 1) / batch;
    const int gy = per_req < want ? per_req : want;
    const dim3 rgrid((unsigned)batch, (unsigned)gy);
    // the proposals of a request run side by side: one wave each (4 to 16 waves)
    const int pw = B < kDenseWaves ? kDenseWaves : (B > kProposeMaxThreads / kWave ? kProposeMaxThreads / kWave : B);
    const unsigned pthreads = (unsigned)(pw * kWave);
    if (bf16) {
        dense_propose_kernel<true><<<dim3((unsigned)batch), pthreads, 0, stream>>>(
            src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.row_m, sc.row_S, sc.jstar, sc.y,
            sc.flags, o);
        if (!exact_all)
            dense_exact_row_kernel<true><<<rgrid, kDenseThreads, 0, stream>>>(src, batch, B, vocab, c, dc, sc.jstar);
        dense_residual_kernel<true><<<rgrid, kDenseThreads, 0, stream>>>(
            src, batch, B, vocab, c, dc, sc.row_m, sc.row_S, sc.jstar, sc.resid);
        dense_finish_kernel<true><<<dim3((unsigned)batch), kWave, 0, stream>>>(
            src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.row_m, sc.row_S, sc.jstar, sc.y,
            sc.flags, sc.resid, o);
    } else {
        dense_propose_kernel<false><<<dim3((unsigned)batch), pthreads, 0, stream>>>(
            src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.row_m, sc.row_S, sc.jstar, sc.y,
            sc.flags, o);
        if (!exact_all)
            dense_exact_row_kernel<false><<<rgrid, kDenseThreads, 0, stream>>>(src, batch, B, vocab, c, dc, sc.jstar);
        dense_residual_kernel<false><<<rgrid, kDenseThreads, 0, stream>>>(
            src, batch, B, vocab, c, dc, sc.row_m, sc.row_S, sc.jstar, sc.resid);
        dense_finish_kernel<false><<<dim3((unsigned)batch), kWave, 0, stream>>>(
            src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.row_m, sc.row_S, sc.jstar, sc.y,
            sc.flags, sc.resid, o);
    }
    return hipGetLastError();
}

hipError_t launch_tree_build(int32_t batch, int32_t B, int32_t K, int32_t V, const SparseOut& sup,
                             const TreeOut& o, hipStream_t stream)
{
    // live frontier entries <= 1 + V
    if (V + 1 <= kWave)
        tree_build_kernel<1><<<dim3((unsigned)batch), kWave, 0, stream>>>(batch, B, K, V, sup, o);
    else if (V + 1 <= 2 * kWave)
        tree_build_kernel<2><<<dim3((unsigned)batch), kWave, 0, stream>>>(batch, B, K, V, sup, o);
    else
        tree_build_kernel<3><<<dim3((unsigned)batch), kWave, 0, stream>>>(batch, B, K, V, sup, o);
    return hipGetLastError();
}

hipError_t launch_tree_walk(int32_t batch, int32_t B, int32_t V, const SparseOut& sup, uint64_t seed,
                            uint64_t offset, const uint32_t* request_ids, const int32_t* node_token,
                            const int32_t* node_parent, const int32_t* num_nodes, const WalkOut& o,
                            hipStream_t stream)
{
    if (sup.cum == nullptr) return hipErrorInvalidValue;     // needs id-ordered supports
    tree_walk_kernel<<<dim3((unsigned)batch), kWalkThreads, 0, stream>>>(
        batch, B, V, sup, seed, offset, request_ids, node_token, node_parent, num_nodes, o);
    return hipGetLastError();
}

hipError_t launch_tree_walk_dense(const RowSource& src, int32_t batch, int32_t B, int32_t V, int64_t vocab,
                                  bool bf16, float temperature, const DenseChunks& dc, uint64_t seed,
                                  uint64_t offset, const uint32_t* request_ids, const int32_t* node_token,
                                  const int32_t* node_parent, const int32_t* num_nodes, const WalkOut& o,
                                  hipStream_t stream)
{
    const double c = 1.4426950408889634074 / (double)temperature;
    if (bf16)
        dense_walk_kernel<true><<<dim3((unsigned)batch), kWalkThreads, 0, stream>>>(
            src, batch, B, V, vocab, c, dc, seed, offset, request_ids, node_token, node_parent, num_nodes, o);
    else
        dense_walk_kernel<false><<<dim3((unsigned)batch), kWalkThreads, 0, stream>>>(
            src, batch, B, V, vocab, c, dc, seed, offset, request_ids, node_token, node_parent, num_nodes, o);
    return hipGetLastError();
}

hipError_t launch_dense_support_scale(int64_t rows, float temperature, const DenseChunks& dc,
                                      const int32_t* limit, const SparseOut& sup, hipStream_t stream)
{
    if (sup.stats == nullptr) return hipErrorInvalidValue;
    dense_support_scale_kernel<<<dim3((unsigned)((rows + kDenseWaves - 1) / kDenseWaves)), kDenseThreads, 0,
                                 stream>>>(rows, 1.0 / (double)temperature, dc, limit, sup);
    return hipGetLastError();
}

hipError_t launch_nucleus(const RowSource& src, int64_t rows, int64_t vocab, bool bf16, float temperature,
                          float top_p, const DenseChunks& dc, int32_t* out_count, double* out_stats,
                          hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    if (dc.keep == nullptr) return hipErrorInvalidValue;
    const double c = 1.4426950408889634074 / (double)temperature;
    if (bf16)
        nucleus_kernel<true><<<dim3((unsigned)rows), kNucThreads, 0, stream>>>(src, vocab, c, (double)top_p, dc,
                                                                             out_count, out_stats);
    else
        nucleus_kernel<false><<<dim3((unsigned)rows), kNucThreads, 0, stream>>>(src, vocab, c, (double)top_p, dc,
                                                                              out_count, out_stats);
    return hipGetLastError();
}

}  // namespace uno
