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

// The first cap slots of a support as stored (no count applied: slots past
// cap hold id INT32_MAX, weight 0), so no loaded value is read here.
__device__ __forceinline__ void wave_load_support_raw(const int32_t* ids, const double* p, const double* cum,
                                                      int cap, WaveRow& R, int lane)
{
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const int i = q * kWave + lane;
        R.id[q] = 0x7FFFFFFF;
        R.w[q] = 0.0;
        R.c[q] = 0.0;
        if (q * kWave < cap && i < cap) {
            R.id[q] = ids[i];
            R.w[q] = p[i];
            if (cum) R.c[q] = cum[i];
        }
    }
}

// Entries n and above of R become padding (id INT32_MAX, weight 0).
__device__ __forceinline__ void wave_mask_support(WaveRow& R, int n, int lane)
{
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const bool in = q * kWave + lane < n;
        R.id[q] = in ? R.id[q] : 0x7FFFFFFF;
        R.w[q] = in ? R.w[q] : 0.0;
        R.c[q] = in ? R.c[q] : 0.0;
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
    const uint32_t* req_ids, LinearOut o, const FilterParams* rowp)
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
    if (rowp && rowp[(int64_t)b * B].skip_topk) return;      // a request of the dense samplers
    const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
    const int64_t qbase = (int64_t)b * B;
    const int64_t pbase = (int64_t)batch * B + (int64_t)b * (B + 1);
    const int cap = sup.cap;
    if (threadIdx.x == 0) s_flags = 0;
    __syncthreads();

    uint32_t flags = 0;
    for (int j = w; j <= B; j += kLinWaves) {
        const Draw d = uno_draw(seed, req, (uint32_t)j, offset);
        // every read of this position first, one round trip: both counts in
        // one lane-indexed load (lane 0: p_j, lane 1: q_j), both supports
        // unmasked; nothing reads a loaded value until all are issued
        const int64_t pr = pbase + j;
        const int64_t qr = qbase + j;
        const int cpair = sup.count[((lane & 1) && j < B) ? qr : pr];
        WaveRow P;                       // p_j (id order, with its cumulative sums)
        wave_load_support_raw(sup.ids + pr * cap, sup.probs + pr * cap, sup.cum + pr * cap, cap, P, lane);
        WaveRow Q;                       // q_j (j < B)
        if (j < B) wave_load_support_raw(sup.ids + qr * cap, sup.probs + qr * cap, sup.cum + qr * cap, cap, Q, lane);
        const int np = __builtin_amdgcn_readlane(cpair, 0);
        const int nq = j < B ? __builtin_amdgcn_readlane(cpair, 1) : 0;
        wave_mask_support(P, np, lane);
        int32_t fin = -1;
        uint32_t ffl = 0;
        if (j == B) {                    // bonus draw
            double dummy;
            if (np > 0) fin = wave_sample_cum(P, np, d.u[2], &dummy, lane);
            else ffl = 1u;
            if (lane == 0) { s_fin[j] = fin; s_ffl[j] = ffl; }
            continue;
        }
        wave_mask_support(Q, nq, lane);
        int32_t y = -1;
        double qy = 0.0;
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
// only lanes that tie on it go on to the low word and then the tie word.
// An entry is its score and tie word only: the pop that takes it reads the
// parent's score from the node records (by lane) and the next sibling's
// probability from the candidate table (first K ids and probabilities of each
// depth's filtered row, staged in LDS; the read is issued as soon as the entry
// is known and used last), and writes that sibling (parent score times
// probability, the product the oracle forms) into the entry's slot.  Per-depth
// counts and first probabilities sit in registers, read by uniform lane index.

__device__ __forceinline__ uint32_t tree_tie(int depth, int parent, int rank)
{
    return ((uint32_t)depth << 20) | ((uint32_t)parent << 12) | (uint32_t)rank;
}

// FS register slots per lane for the frontier and for the node records: at
// most 1 + V entries are ever live, since a popped entry's slot takes its next
// sibling and only first children need new slots (FS = ceil((V + 1) / 64)).
// Four waves stage the candidate table, every load in flight at once; wave 0
// alone then expands the tree.
constexpr int kBuildThreads = 256;
constexpr int kBuildPer = kMaxTreeVK / kBuildThreads;     // table entries per thread

// Slot i / 64 of lane i % 64 of a per-lane array (i uniform), without branches.
template <int N>
__device__ __forceinline__ int sel_i32(const int (&a)[N], int i)
{
    int r = __builtin_amdgcn_readlane(a[0], i & (kWave - 1));
#pragma unroll
    for (int q = 1; q < N; ++q) {
        const int v = __builtin_amdgcn_readlane(a[q], i & (kWave - 1));
        r = (i >> 6) == q ? v : r;
    }
    return r;
}

template <int N>
__device__ __forceinline__ double sel_f64(const double (&a)[N], int i)
{
    double r = readlane_f64(a[0], i & (kWave - 1));
#pragma unroll
    for (int q = 1; q < N; ++q) {
        const double v = readlane_f64(a[q], i & (kWave - 1));
        r = (i >> 6) == q ? v : r;
    }
    return r;
}

// Wave maximum: within rows of 16 lanes by DPP, then across the four rows'
// results by lane reads and scalar maxima (no row broadcasts and their waits).
__device__ __forceinline__ uint32_t wave_max_u32_rows(uint32_t v)
{
    auto mx = [](uint32_t a, uint32_t b) __attribute__((always_inline)) { return a > b ? a : b; };
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
    return mx(mx(r0, r1), mx(r2, r3));
}

template <int FS>
__global__ __launch_bounds__(kBuildThreads) void tree_build_kernel(int32_t batch, int32_t B, int32_t K, int32_t V,
                                                                   SparseOut sup, TreeOut o)
{
    __shared__ int32_t c_id[kMaxTreeVK];       // depth d, rank r at d*K + r (B*K <= V*K <= 2048)
    __shared__ double c_p[kMaxTreeVK];

    const int lane = lane_id();
    const int b = blockIdx.x;
    const int cap = sup.cap;
    const int64_t rbase = (int64_t)b * B;
    const int kk = K < cap ? K : cap;
    // per depth (B <= 128; B <= V < 64 when FS == 1): candidate count (at
    // most K) and first probability
    constexpr int DS = FS == 1 ? 1 : 2;
    int cn[DS];
    double p0[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
        const int d = s * kWave + lane;
        int n = 0;
        double f0 = 0.0;
        if (d < B && threadIdx.x < kWave) {
            n = sup.count[rbase + d];
            f0 = sup.probs[(rbase + d) * cap];
        }
        cn[s] = n > 0 ? (n < K ? n : K) : 0;
        p0[s] = f0;
    }
    // the candidate table is read whole (supports are padded to cap); entries
    // past a count are never used
    {
        int32_t tid[kBuildPer];
        double tpr[kBuildPer];
#pragma unroll
        for (int j = 0; j < kBuildPer; ++j) {
            const int i = j * kBuildThreads + (int)threadIdx.x;
            const int d = i / K, r = i - d * K;
            tid[j] = 0;
            tpr[j] = 0.0;
            if (i < B * K && r < kk) {
                tid[j] = sup.ids[(rbase + d) * cap + r];
                tpr[j] = sup.probs[(rbase + d) * cap + r];
            }
        }
#pragma unroll
        for (int j = 0; j < kBuildPer; ++j) {
            const int i = j * kBuildThreads + (int)threadIdx.x;
            const int d = i / K, r = i - d * K;
            if (i < B * K && r < kk) {
                c_id[i] = tid[j];
                c_p[i] = tpr[j];
            }
        }
    }
    __syncthreads();
    if (threadIdx.x >= kWave) return;

    uint64_t fs[FS];                                   // frontier: score bits (0 = empty)
    uint32_t ft[FS];                                   // frontier: tie word (~0 = empty)
    double ns[FS];                                     // node records: score
    uint32_t nt[FS];                                   // node records: tie word of the entry
#pragma unroll
    for (int q = 0; q < FS; ++q) { fs[q] = 0ull; ft[q] = ~0u; ns[q] = 0.0; nt[q] = 0u; }
    if (lane == 0) ns[0] = 1.0;
    // the lane that holds slot i of a per-lane array, and its register slot
    // (every slot is below 64 when FS == 1)
    auto at = [&](int i, int q) __attribute__((always_inline)) {
        return FS == 1 ? lane == i : (lane == (i & (kWave - 1)) && q == (i >> 6));
    };
    auto put = [&](int slot, double sc, uint32_t tie) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < FS; ++q) {
            const bool m = at(slot, q);
            fs[q] = m ? (uint64_t)__double_as_longlong(sc) : fs[q];
            ft[q] = m ? tie : ft[q];
        }
    };

    int nf = 0;                                        // slots handed out (uniform)
    int live = 0;
    if (sel_i32(cn, 0) > 0) {
        put(nf++, 1.0 * sel_f64(p0, 0), tree_tie(1, 0, 0));
        ++live;
    }
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
        const uint32_t hm = wave_max_u32_rows(bh);
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
        const int wl = __builtin_ctzll(hit);            // some lane holds the maximum
        const uint32_t tie = (uint32_t)__builtin_amdgcn_readlane((int)bt, wl);
        const int wq = __builtin_amdgcn_readlane(bq, wl);
        const double score = __longlong_as_double(
            (long long)(((uint64_t)hm << 32) | (uint32_t)__builtin_amdgcn_readlane((int)bl, wl)));
        const int depth = (int)(tie >> 20), parent = (int)((tie >> 12) & 0xFFu), rank = (int)(tie & 0xFFFu);
        // the next sibling's probability, from LDS (used last)
        int si = (depth - 1) * K + rank + 1;
        si = si < kMaxTreeVK ? si : kMaxTreeVK - 1;
        const double sp1 = c_p[si];
        const bool sib = rank + 1 < sel_i32(cn, depth - 1);
        // the parent's score, from the node records
        const double psc = sel_f64(ns, parent);
        // the node
#pragma unroll
        for (int q = 0; q < FS; ++q) {
            const bool m = at(num, q);
            ns[q] = m ? score : ns[q];
            nt[q] = m ? tie : nt[q];
        }
        // its first child in a new slot
        const bool child = depth < B && sel_i32(cn, depth) > 0;
        if (child) {
            put(nf++, score * sel_f64(p0, depth), tree_tie(depth + 1, num, 0));
            ++live;
        }
        // its next sibling in the slot it leaves (or the slot emptied)
        put(wq * kWave + wl, sib ? psc * sp1 : 0.0, sib ? tree_tie(depth, parent, rank + 1) : ~0u);
        live -= sib ? 0 : 1;
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
constexpr int kWalkAhead = 3;     // nodes per wave whose supports are read up front

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
    const int32_t* num_nodes, WalkOut o, const FilterParams* rowp)
{
    __shared__ TreeLds L;
    __shared__ int32_t s_t[kMaxNodes];

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x;
    if (rowp && rowp[(int64_t)b * (V + 1)].skip_topk) return;   // a request of the dense walk
    const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
    const int cap = sup.cap;
    int nn = num_nodes[b];
    nn = nn < 1 ? 1 : (nn > V + 1 ? V + 1 : nn);
    const int64_t ob = (int64_t)b * (V + 1);
    // The wave's first kWalkAhead nodes (n = w + a * 16): their supports are
    // read at once, before the depths are known, so every round trip overlaps
    // (a row past num_nodes is read, in bounds, and ignored).  Further nodes
    // (more than 48 in a tree) are read one at a time afterwards.
    // (the counts in one lane-indexed load, lane a: node w + 16 a, read only
    // after every load is issued)
    WaveRow R[kWalkAhead];
    const int na = w + (lane < kWalkAhead ? lane : 0) * kWalkWaves;
    const int cnt_l = na <= V ? sup.count[ob + na] : 0;
#pragma unroll
    for (int a = 0; a < kWalkAhead; ++a) {
        const int n = w + a * kWalkWaves;
        if (n <= V)
            wave_load_support_raw(sup.ids + (ob + n) * cap, sup.probs + (ob + n) * cap, sup.cum + (ob + n) * cap, cap,
                                  R[a], lane);
    }
    tree_depths(node_token, node_parent, ob, nn, V, L);
    int cnt[kWalkAhead];
#pragma unroll
    for (int a = 0; a < kWalkAhead; ++a) cnt[a] = __builtin_amdgcn_readlane(cnt_l, a);
    // every node's sample, drawn with the uniform of its depth
    auto sample_node = [&](int n, WaveRow& Rw, int c) __attribute__((always_inline)) {
        const int dep = L.dep[n];
        int32_t t = -1;
        if (dep >= 0 && dep <= B && c > 0) {
            wave_mask_support(Rw, c, lane);
            const Draw d = uno_draw(seed, req, (uint32_t)dep, offset);
            double dummy;
            t = wave_sample_cum(Rw, c, d.u[2], &dummy, lane);
        }
        if (lane == 0) s_t[n] = t;
    };
#pragma unroll
    for (int a = 0; a < kWalkAhead; ++a) {
        const int n = w + a * kWalkWaves;
        if (n < nn) sample_node(n, R[a], cnt[a]);
    }
    for (int n = w + kWalkAhead * kWalkWaves; n < nn; n += kWalkWaves) {
        WaveRow Rn;
        wave_load_support_raw(sup.ids + (ob + n) * cap, sup.probs + (ob + n) * cap, sup.cum + (ob + n) * cap, cap, Rn,
                              lane);
        sample_node(n, Rn, sup.count[ob + n]);
    }
    __syncthreads();
    if (w == 0) follow_path(b, B, nn, s_t, L, o, lane);
}

// ---- dense linear ------------------------------------------------------------------
constexpr int kDenseThreads = 256;
constexpr int kProposeMaxThreads = 512;    // dense_propose_kernel: up to eight waves, one proposal each at a time
constexpr int kDenseWaves = kDenseThreads / kWave;
constexpr int kPerLane = kDenseChunk / kWave;   // 32 logits per lane per chunk
constexpr int kListGroups = 768;               // workgroups of dense_exact_list_kernel (one round)
constexpr int kExactJobs = 24;                 // grid rows of the exact fallback kernels over listed requests

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

// Chunk c of a row as the raw vectors load_chunk reads (same element layout:
// entry i is element (i/EPV*64 + lane)*EPV + i%EPV); -inf past the end of the
// row.  Half the registers of the unpacked floats for 2-byte rows.
template <bool BF16>
struct RawChunk {
    using V = Vec<BF16>;
    static constexpr int EPV = V::EPV, NV = kPerLane / EPV;
    typename V::T v[NV];

    __device__ __forceinline__ void load(const char* row, int64_t N, int64_t c, int lane)
    {
        const int64_t beg = c * kDenseChunk;
        const int64_t n = (N - beg < kDenseChunk) ? (N - beg) : kDenseChunk;
        if (n == kDenseChunk && (((uintptr_t)(row + beg * V::ESZ)) & 15u) == 0) {
            const typename V::T* p = reinterpret_cast<const typename V::T*>(row + beg * V::ESZ);
#pragma unroll
            for (int j = 0; j < NV; ++j) v[j] = V::load_stream(p + j * kWave + lane);
            return;
        }
        // offsets from one per-lane base and compile-time constants, so that
        // nothing here is worth hoisting out of a caller's loop
        const int lim = (int)n - lane * EPV;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int k0 = j * kWave * EPV;
            if constexpr (BF16) {
                const uint16_t* h = reinterpret_cast<const uint16_t*>(row) + beg + lane * EPV;
                uint32_t wd[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = (k0 + 2 * e < lim) ? h[k0 + 2 * e] : 0xFF80u;
                    const uint32_t hi = (k0 + 2 * e + 1 < lim) ? h[k0 + 2 * e + 1] : 0xFF80u;
                    wd[e] = lo | (hi << 16);
                }
                v[j] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
            } else {
                const float* f = reinterpret_cast<const float*>(row) + beg + lane * EPV;
                v[j] = make_float4(k0 < lim ? f[k0] : -INFINITY, k0 + 1 < lim ? f[k0 + 1] : -INFINITY,
                                   k0 + 2 < lim ? f[k0 + 2] : -INFINITY, k0 + 3 < lim ? f[k0 + 3] : -INFINITY);
            }
        }
    }
    __device__ __forceinline__ float get(int i) const { return V::get(v[i / EPV], i % EPV); }
};

// Chunk-stat term of chunk c relative to the row max m.
__device__ __forceinline__ double chunk_term(const float* cm, const double* cs, int c, float m, const DenseExp& ex)
{
    return (cm[c] > -INFINITY) ? cs[c] * ex((double)cm[c] - (double)m) : 0.0;
}

// Row max m and normaliser S from chunk statistics; S accumulates 64-chunk
// blocks of an inclusive wave scan, the same sums dense_locate walks.  With
// chunk error bounds ce, *E_out bounds |S - exact S| (0 when every chunk is
// exact).
__device__ bool dense_row_stat(const float* cm, const double* cs, int nc, const DenseExp& ex, int lane,
                               float* m_out, double* S_out, const float* ce = nullptr, double* E_out = nullptr)
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
    double S = 0.0, E = 0.0;
    for (int base = 0; base < nc; base += kWave) {
        const int c = base + lane;
        const double term = (c < nc) ? chunk_term(cm, cs, c, m, ex) : 0.0;
        const double incl = wave_incl_scan_f64(term, lane);
        S += lane_value(incl, kWave - 1);
        if (ce != nullptr && c < nc && cm[c] > -INFINITY) E += (double)ce[c] * ex((double)cm[c] - (double)m);
    }
    if (E_out) *E_out = (ce != nullptr) ? wave_sum_f64(E) * (1.0 + 1e-6) : 0.0;
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
            *before = C + lane_value(incl - term, l);
            return base + l;
        }
        C += lane_value(incl, kWave - 1);
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
    best = wave_max_i32(best);
    return best;
}

// Smallest element of a chunk (weights from wf, element layout of load_chunk)
// whose cumulative weight exceeds tau; the last positive element if none does.
// *margin (when given): the distance from tau to the nearer end of the picked
// element's cumulative interval, -1 when tau lies in no interval.
template <int EPV, typename WeightF>
__device__ int pick_in_chunk(WeightF wf, double tau, int lane, double* margin = nullptr)
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
            double mg = -1.0;
            if (lane == l) {
                double cc = run + (incl - lsum);
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const double prev = cc;
                    cc += wl[e];
                    if (ep < 0 && cc > tau) {
                        ep = e;
                        mg = fmin(tau - prev, cc - tau);
                    }
                }
                if (ep < 0) {
#pragma unroll
                    for (int e = EPV - 1; e >= 0; --e)
                        if (ep < 0 && wl[e] > 0.0) ep = e;
                }
            }
            ep = lane_value(ep, l);
            if (margin) *margin = lane_value(mg, l);
            return (j * kWave + l) * EPV + ep;
        }
        run += lane_value(incl, kWave - 1);
    }
    last_pos = wave_max_i32(last_pos);
    if (margin) *margin = -1.0;
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
        run += lane_value(incl, kWave - 1);
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
// threshold admits) with uniform u: the chunk from the chunk sums, then the
// element from the chunk's exact terms.  With chunk error bounds ce and the
// row's bound E (> 0: fast sums), *certain tells whether the pick is the one
// exact sums give: the target's offset inside the chunk can be off by at most
// (u E + the bound of the chunks before it) / the chunk's scale, so the pick
// stands when its cumulative interval holds the offset with more than that
// to spare.  With exact sums (E == 0) the pick is certain.
template <bool BF16>
__device__ int32_t dense_sample_row(const char* row, int64_t N, const float* cm, const double* cs, int nc,
                                    float m, double S, double u, const DenseExp& ex, int lane, uint64_t thr,
                                    const float* ce = nullptr, double E = 0.0, bool* certain = nullptr)
{
    const bool fast = ce != nullptr && E > 0.0;
    const double t = u * S;
    double before;
    int c;
    double tau, scale = 1.0, ebefore = 0.0, mc;
    if (nc <= 2 * kWave) {
        // At most two chunks per lane: every statistic the draw reads is read
        // before any is used, and the terms, scans and sums below are formed
        // from the registers in the same order as from memory.
        float m0 = -INFINITY, m1 = -INFINITY, e0 = 0.0f, e1 = 0.0f;
        double s0 = 0.0, s1 = 0.0;
        if (lane < nc) {
            m0 = cm[lane];
            s0 = cs[lane];
            if (fast) e0 = ce[lane];
        }
        if (lane + kWave < nc) {
            m1 = cm[lane + kWave];
            s1 = cs[lane + kWave];
            if (fast) e1 = ce[lane + kWave];
        }
        const double x0 = (m0 > -INFINITY) ? ex((double)m0 - (double)m) : 0.0;
        const double x1 = (m1 > -INFINITY) ? ex((double)m1 - (double)m) : 0.0;
        const double t0 = (m0 > -INFINITY) ? s0 * x0 : 0.0, t1 = (m1 > -INFINITY) ? s1 * x1 : 0.0;
        auto term = [&](int k) { return k < kWave ? t0 : t1; };     // k = lane or lane + 64
        c = dense_locate(nc, t, term, lane, &before);
        if (c < 0) {
            c = dense_last_positive_chunk(nc, term, lane);
            if (certain) *certain = !fast;
            if (c < 0) return -1;
            tau = INFINITY;
        } else {
            scale = lane_value(c < kWave ? x0 : x1, c & (kWave - 1));
            tau = (t - before) / scale;
            if (fast) {
                double eb = 0.0;
                if (lane < c && m0 > -INFINITY) eb += (double)e0 * x0;
                if (lane + kWave < c && m1 > -INFINITY) eb += (double)e1 * x1;
                ebefore = wave_sum_f64(eb);
            }
        }
        mc = (double)__int_as_float(lane_value(__float_as_int(c < kWave ? m0 : m1), c & (kWave - 1)));
    } else {
        auto term = [&](int k) { return chunk_term(cm, cs, k, m, ex); };
        c = dense_locate(nc, t, term, lane, &before);
        if (c < 0) {
            c = dense_last_positive_chunk(nc, term, lane);
            if (certain) *certain = !fast;
            if (c < 0) return -1;
            tau = INFINITY;
        } else {
            scale = ex((double)cm[c] - (double)m);
            tau = (t - before) / scale;
            if (fast) {
                // error bound of the chunks before c, relative to the row max
                double eb = 0.0;
                for (int k = lane; k < c; k += kWave)
                    if (cm[k] > -INFINITY) eb += (double)ce[k] * ex((double)cm[k] - (double)m);
                ebefore = wave_sum_f64(eb);
            }
        }
        mc = (double)cm[c];
    }
    float x[kPerLane];
    load_chunk<BF16>(row, N, c, x, lane);
    constexpr int EPV = Vec<BF16>::EPV;
    auto wf = [&](int i) { return dense_keeps(thr, x[i], chunk_elem_id<EPV>(c, i, lane)) ? ex((double)x[i] - mc) : 0.0; };
    double margin = -1.0;
    const int l = pick_in_chunk<Vec<BF16>::EPV>(wf, tau, lane, &margin);
    if (certain && tau < INFINITY) {
        // the fp64 sums themselves round at the 1e-12 level, far inside the bound
        const double bound = ((u * E + ebefore) * (1.0 + 1e-6) + 1e-12 * S) / scale;
        *certain = !fast || margin > bound;
    }
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

// Proposals and acceptance in four kernels.  Rows may carry fast chunk sums
// with error bounds (dc.cerr): every draw and every acceptance test is
// certified against them.
//  - dense_row_stat_kernel (chip-wide, one wave per row): every row's
//    maximum, normaliser and bound.
//  - dense_propose_kernel: the draws, and the acceptance test of every
//    proposal whose draw is certain.  acc[j]: 1 accepted, 0 rejected, 2 test
//    not certain, 3 draw not certain.
//  - dense_exact_list_kernel (chip-wide): exact chunk sums for the rows those
//    uncertain results read (the first exact-row list, which the proposal
//    kernel fills): q_j of an uncertain draw; q_j and p_j of an uncertain
//    test before the first certain rejection.
//  - dense_settle_kernel: the uncertain draws and tests again from the exact
//    rows, the rare test that is still uncertain (a redrawn proposal's test
//    on a fast target row) after the block has made its rows exact, and the
//    first rejection.

// Row statistics of row r (one wave) into row_m / row_S / row_E.
__device__ __forceinline__ void row_stat_to(const DenseChunks& dc, int64_t r, const DenseExp& ex, int lane,
                                            float* row_m, double* row_S, double* row_E)
{
    const int nc = dc.nchunks;
    float m;
    double S, E;
    dense_row_stat(dc.cmax + r * nc, dc.csum + r * nc, nc, ex, lane, &m, &S, dc.cerr ? dc.cerr + r * nc : nullptr,
                   &E);
    if (lane == 0) { row_m[r] = m; row_S[r] = S; row_E[r] = E; }
}

// Draw of proposal j of request b (uniform 0 of draw (request, j)) from draft
// row q_j with the row's current statistics; *certain as dense_sample_row.
template <bool BF16>
__device__ __forceinline__ int32_t propose_draw(const RowSource& src, int32_t batch, int32_t B, int64_t N,
                                                const DenseChunks& dc, const DenseExp& ex, uint64_t seed,
                                                uint64_t offset, uint32_t req, int b, int j, const float* row_m,
                                                const double* row_S, const double* row_E, int lane, bool* certain,
                                                uint32_t* flags)
{
    const Draw d = uno_draw(seed, req, (uint32_t)j, offset);
    const int nc = dc.nchunks;
    const int64_t qr = linear_row(batch, B, b, j);
    const double Sq = row_S[qr];
    *certain = true;
    if (!(Sq > 0.0)) { *flags |= 1u; return -1; }
    return dense_sample_row<BF16>(row_pointer(src, qr, N * Vec<BF16>::ESZ), N, dc.cmax + qr * nc, dc.csum + qr * nc,
                                  nc, row_m[qr], Sq, d.u[0], ex, lane, row_keep(dc, qr),
                                  dc.cerr ? dc.cerr + qr * nc : nullptr, row_E[qr], certain);
}

// Acceptance test u1 q(y) < p(y) of proposal j: 1 accepted, 0 rejected, 2
// when the two sides differ by no more than their sums' error bounds allow.
template <bool BF16>
__device__ __forceinline__ int propose_test(const RowSource& src, int32_t batch, int32_t B, int64_t N,
                                            const DenseChunks& dc, const DenseExp& ex, uint64_t seed, uint64_t offset,
                                            uint32_t req, int b, int j, int32_t y, const float* row_m,
                                            const double* row_S, const double* row_E, uint32_t* flags)
{
    if (y < 0) return 0;
    const Draw d = uno_draw(seed, req, (uint32_t)j, offset);
    const int64_t row_bytes = N * Vec<BF16>::ESZ;
    const int64_t qr = linear_row(batch, B, b, j), pr = linear_row(batch, B, b, B + j);
    // every read of the test goes out before any is used (both rows of a
    // linear cycle are always present, and y is inside them)
    const float zq = load_one<BF16>(row_pointer(src, qr, row_bytes), y);
    const float zp = load_one<BF16>(row_pointer(src, pr, row_bytes), y);
    const double Sq = row_S[qr], Sp = row_S[pr];
    const float mq = row_m[qr], mp = row_m[pr];
    const double Eq = row_E[qr], Ep = row_E[pr];
    const uint64_t thr = row_keep(dc, pr);
    const double qy = ex((double)zq - (double)mq) / Sq;
    double py = 0.0;
    if (Sp > 0.0) {
        if (dense_keeps(thr, zp, y)) py = ex((double)zp - (double)mp) / Sp;
    } else {
        *flags |= 1u;
    }
    const double lhs = d.u[1] * qy;
    if (Eq > 0.0 || Ep > 0.0) {
        const double rq = Eq / Sq, rp = (Sp > 0.0) ? Ep / Sp : 0.0;
        const double bound = (lhs * rq + py * rp) * (1.0 + 1e-3) + 1e-12 * (lhs + py);
        if (!(fabs(lhs - py) > bound)) return 2;
    }
    return (lhs < py) ? 1 : 0;
}

// Every row's maximum, normaliser and bound from its chunk statistics, two
// rows per wave (rows of the linear layout; with per-request sets each at its
// own temperature, top-k rows skipped).  For rows of at most 128 chunks every
// load of both rows is issued before any is used; the sums are dense_row_stat's
// (the same terms, scans and order), so the statistics are the same.
constexpr int kRowStatThreads = 1024;
constexpr int kRowStatWaves = kRowStatThreads / kWave;

__global__ __launch_bounds__(kRowStatThreads) void dense_row_stat_kernel(int64_t rows, double log2e_over_T,
                                                                         DenseChunks dc, float* row_m, double* row_S,
                                                                         double* row_E, const FilterParams* rowp)
{
    __shared__ double s_exp2[kExp2Entries];
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t r0 = 2 * ((int64_t)blockIdx.x * kRowStatWaves + w);
    const int nc = dc.nchunks;
    // rows of at most 128 chunks: both rows' chunk statistics are read first
    // (unconditionally within the rows; the per-row parameters applied
    // afterwards), so they travel with the table's loads
    float cm[2][2], ce[2][2];
    double cs[2][2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = q * kWave + lane;
            const bool in = nc <= 2 * kWave && r0 + k < rows && c < nc;
            const int64_t slot = (r0 + k) * nc + c;
            cm[k][q] = in ? dc.cmax[slot] : -INFINITY;
            cs[k][q] = in ? dc.csum[slot] : 0.0;
            ce[k][q] = (in && dc.cerr) ? dc.cerr[slot] : 0.0f;
        }
    load_exp2_table(s_exp2);
    __syncthreads();
    if (r0 >= rows) return;
    bool on[2];
    double c2[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int64_t r = r0 + k;
        on[k] = r < rows;
        c2[k] = log2e_over_T;
        if (on[k] && rowp) {
            const FilterParams& f = rowp[r];
            on[k] = f.dense != kRowTopK;
            c2[k] = 1.4426950408889634074 / (double)f.temperature;
        }
    }
    if (nc > 2 * kWave) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
            if (on[k]) row_stat_to(dc, r0 + k, DenseExp{ c2[k], s_exp2 }, lane, row_m, row_S, row_E);
        return;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (!on[k]) continue;
        const DenseExp ex{ c2[k], s_exp2 };
        float m = fmaxf(cm[k][0], cm[k][1]);
        const bool bad = __ballot(cm[k][0] == INFINITY || cm[k][1] == INFINITY) != 0ull;
        m = wave_max_f32(m);
        double S = NAN, E = 0.0;
        if (!bad && m > -INFINITY) {
            S = 0.0;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (q * kWave >= nc) break;
                const double sc = (cm[k][q] > -INFINITY) ? ex((double)cm[k][q] - (double)m) : 0.0;
                const double term = cm[k][q] > -INFINITY ? cs[k][q] * sc : 0.0;
                const double incl = wave_incl_scan_f64(term, lane);
                S += lane_value(incl, kWave - 1);
                E += (double)ce[k][q] * sc;
            }
            E = dc.cerr ? wave_sum_f64(E) * (1.0 + 1e-6) : 0.0;
        } else {
            m = NAN;
        }
        if (lane == 0) { row_m[r0 + k] = m; row_S[r0 + k] = S; row_E[r0 + k] = E; }
    }
}

template <bool BF16>
__global__ __launch_bounds__(kProposeMaxThreads) void dense_propose_kernel(
    RowSource src, int32_t batch, int32_t B, int64_t N, double log2e_over_T, DenseChunks dc,
    uint64_t seed, uint64_t offset, const uint32_t* req_ids, float* row_m, double* row_S, double* row_E,
    int32_t* y_scr, int32_t* acc, uint32_t* flag_out, int64_t* xrows, const FilterParams* rowp)
{
    __shared__ double s_exp2[kExp2Entries];
    __shared__ int32_t s_acc[kMaxLinearB];
    __shared__ uint32_t s_flags;
    if (rowp) {                              // per-request parameters: the request's own temperature
        const FilterParams& f = rowp[(int64_t)blockIdx.x * B];
        if (f.dense == kRowTopK) return;
        log2e_over_T = 1.4426950408889634074 / (double)f.temperature;
    }
    load_exp2_table(s_exp2);
    if (threadIdx.x == 0) s_flags = 0;
    __syncthreads();
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nw = (int)(blockDim.x / kWave);
    const int b = blockIdx.x;
    const DenseExp ex{ log2e_over_T, s_exp2 };
    const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
    uint32_t flags = 0;
    for (int j = w; j < B; j += nw) {
        bool certain;
        const int32_t y = propose_draw<BF16>(src, batch, B, N, dc, ex, seed, offset, req, b, j, row_m, row_S, row_E,
                                             lane, &certain, &flags);
        const int a = certain ? propose_test<BF16>(src, batch, B, N, dc, ex, seed, offset, req, b, j, y, row_m,
                                                   row_S, row_E, &flags)
                              : 3;
        if (lane == 0) { y_scr[(int64_t)b * B + j] = y; acc[(int64_t)b * B + j] = a; s_acc[j] = a; }
    }
    if (flags && lane == 0) atomicOr(&s_flags, flags);
    __syncthreads();
    if (threadIdx.x == 0) {
        flag_out[b] = s_flags;
        // the rows whose uncertain results need exact sums go to the first
        // exact-row list: q_j of an uncertain draw; q_j and p_j of an
        // uncertain test before the first certain rejection
        if (dc.xcount != nullptr) {
            // two passes over the results: count, reserve, write
            int64_t* out = nullptr;
            for (int pass = 0; pass < 2; ++pass) {
                int n = 0;
                bool counts = true;
                auto put = [&](int64_t r) { if (out) out[n] = r; ++n; };
                for (int j = 0; j < B; ++j) {
                    const int a = s_acc[j];
                    if (a == 3) put(linear_row(batch, B, b, j));
                    if (a == 0) counts = false;
                    if (a == 2 && counts) {
                        const int64_t qr = linear_row(batch, B, b, j), pr = linear_row(batch, B, b, B + j);
                        if (row_E[qr] > 0.0) put(qr);
                        if (row_E[pr] > 0.0) put(pr);
                    }
                }
                if (pass == 0) {
                    if (n == 0) break;
                    out = xrows + atomicAdd(&dc.xcount[0], (uint32_t)n);
                }
            }
        }
    }
}

// Exact chunk statistics of chunk c of row r (one wave), bound 0.
template <bool BF16>
__device__ __forceinline__ void exact_chunk_to(const char* row, int64_t N, int64_t r, int c, const DenseChunks& dc,
                                               const DenseExp& ex, int lane)
{
    float x[kPerLane];
    load_chunk<BF16>(row, N, c, x, lane);
    float mx;
    double sum;
    uint32_t cntf;
    chunk_stats_exact<true>(x, ex, &mx, &sum, &cntf);
    if (lane == 0) {
        const int64_t slot = r * dc.nchunks + c;
        dc.cmax[slot] = mx;
        dc.csum[slot] = (mx < INFINITY) ? sum : NAN;
        if (dc.ccount) dc.ccount[slot] = (int32_t)cntf;
        if (dc.cerr) dc.cerr[slot] = 0.0f;
    }
}

// Exact chunk statistics for the rows of an exact-row list (count rows at
// rows[0 ..]): chunk t % nchunks of row rows[t / nchunks] for every task t,
// dealt one per wave over a fixed grid, so a few rows still spread over the
// whole chip.  Each row keeps its own temperature (per-request sets).
template <bool BF16>
__global__ __launch_bounds__(kDenseThreads) void dense_exact_list_kernel(
    RowSource src, int64_t N, double log2e_over_T, DenseChunks dc, const int64_t* rows, const uint32_t* count,
    const FilterParams* rowp)
{
    __shared__ double s_exp2[kExp2Entries];
    const int nc = dc.nchunks;
    const int64_t tasks = (int64_t)(*count) * nc;
    if ((int64_t)blockIdx.x * kDenseWaves >= tasks) return;
    load_exp2_table(s_exp2);
    __syncthreads();
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row_bytes = N * Vec<BF16>::ESZ;
    for (int64_t t = (int64_t)blockIdx.x * kDenseWaves + w; t < tasks; t += (int64_t)gridDim.x * kDenseWaves) {
        const int64_t r = rows[t / nc];
        const int c = (int)(t - (t / nc) * nc);
        const double c2 = rowp ? 1.4426950408889634074 / (double)rowp[r].temperature : log2e_over_T;
        const DenseExp ex{ c2, s_exp2 };
        exact_chunk_to<BF16>(row_pointer(src, r, row_bytes), N, r, c, dc, ex, lane);
    }
}

template <bool BF16>
__global__ __launch_bounds__(kProposeMaxThreads) void dense_settle_kernel(
    RowSource src, int32_t batch, int32_t B, int64_t N, double log2e_over_T, DenseChunks dc,
    uint64_t seed, uint64_t offset, const uint32_t* req_ids, float* row_m, double* row_S, double* row_E,
    const int32_t* y_scr, const int32_t* acc, int32_t* jstar_out, int32_t* y_out, uint32_t* flag_out,
    LinearOut o, const FilterParams* rowp)
{
    __shared__ double s_exp2[kExp2Entries];
    __shared__ int32_t s_acc[kMaxLinearB];
    __shared__ int32_t s_y[kMaxLinearB];
    __shared__ uint32_t s_flags;
    __shared__ int s_any;
    if (rowp) {
        const FilterParams& f = rowp[(int64_t)blockIdx.x * B];
        if (f.dense == kRowTopK) return;
        log2e_over_T = 1.4426950408889634074 / (double)f.temperature;
    }
    const int b = blockIdx.x;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nw = (int)(blockDim.x / kWave);
    if (threadIdx.x == 0) { s_flags = 0; s_any = 0; }
    __syncthreads();
    for (int j = threadIdx.x; j < B; j += blockDim.x) {
        const int a = acc[(int64_t)b * B + j];
        s_acc[j] = a;
        s_y[j] = y_scr[(int64_t)b * B + j];
        if (a >= 2) atomicOr(&s_any, 1);
    }
    __syncthreads();
    uint32_t flags = 0;
    const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
    if (s_any) {
        load_exp2_table(s_exp2);
        __syncthreads();
        const DenseExp ex{ log2e_over_T, s_exp2 };
        // the redone rows' statistics, then the draws and tests again
        for (int j = w; j < B; j += nw) {
            const int a = s_acc[j];
            if (a < 2) continue;
            const int64_t qr = linear_row(batch, B, b, j), pr = linear_row(batch, B, b, B + j);
            row_stat_to(dc, qr, ex, lane, row_m, row_S, row_E);
            row_stat_to(dc, pr, ex, lane, row_m, row_S, row_E);
        }
        __syncthreads();
        for (int j = w; j < B; j += nw) {
            const int a = s_acc[j];
            if (a < 2) continue;
            int32_t y = s_y[j];
            if (a == 3) {
                bool certain;
                y = propose_draw<BF16>(src, batch, B, N, dc, ex, seed, offset, req, b, j, row_m, row_S, row_E, lane,
                                       &certain, &flags);
            }
            const int a2 = propose_test<BF16>(src, batch, B, N, dc, ex, seed, offset, req, b, j, y, row_m, row_S,
                                              row_E, &flags);
            if (lane == 0) { s_y[j] = y; s_acc[j] = a2; }
        }
        __syncthreads();
        // a test still uncertain before the first rejection: exact rows here
        for (int j = 0; j < B; ++j) {        // uniform: s_acc is in LDS
            const int a = s_acc[j];
            if (a == 0) break;
            if (a != 2) continue;
            const int64_t qr = linear_row(batch, B, b, j), pr = linear_row(batch, B, b, B + j);
            const int64_t row_bytes = N * Vec<BF16>::ESZ;
            for (int k = 0; k < 2; ++k) {
                const int64_t r = k == 0 ? qr : pr;
                if (!(row_E[r] > 0.0)) continue;
                for (int c = w; c < dc.nchunks; c += nw)
                    exact_chunk_to<BF16>(row_pointer(src, r, row_bytes), N, r, c, dc, ex, lane);
                __syncthreads();
                if (w == 0) row_stat_to(dc, r, ex, lane, row_m, row_S, row_E);
                __syncthreads();
            }
            if (w == 0) {
                const int a2 = propose_test<BF16>(src, batch, B, N, dc, ex, seed, offset, req, b, j, s_y[j], row_m,
                                                  row_S, row_E, &flags);
                if (lane == 0) s_acc[j] = a2 == 1 ? 1 : 0;
            }
            __syncthreads();
            if (s_acc[j] == 0) break;
        }
    }
    if (flags && lane == 0) atomicOr(&s_flags, flags);
    for (int j = threadIdx.x; j < B; j += blockDim.x) {
        y_out[(int64_t)b * B + j] = s_y[j];
        if (o.proposals) o.proposals[(int64_t)b * B + j] = s_y[j];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int js = B;
        for (int j = 0; j < B; ++j)
            if (s_acc[j] == 0) { js = j; break; }
        jstar_out[b] = js;
        flag_out[b] |= s_flags;
    }
}

// Residual mass per chunk from exact terms and exact sums, for requests that
// rejected a proposal: every request (one per blockIdx.x) or, with a list,
// the listed requests (those whose certified draw was not certain), dealt
// over the grid's rows.
template <bool BF16>
__global__ __launch_bounds__(kDenseThreads) void dense_residual_exact_kernel(
    RowSource src, int32_t batch, int32_t B, int64_t N, double log2e_over_T0, DenseChunks dc,
    const int32_t* jstar_in, const int32_t* list, const uint32_t* list_n, double* resid, const FilterParams* rowp)
{
    const int njobs = list ? (int)*list_n : (int)gridDim.x;
    if ((int)blockIdx.x >= njobs) return;
    const int nc = dc.nchunks;
    __shared__ double s_exp2[kExp2Entries];
    load_exp2_table(s_exp2);
    __syncthreads();
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    for (int job = blockIdx.x; job < njobs; job += gridDim.x) {
    const int b = list ? list[job] : job;
    double log2e_over_T = log2e_over_T0;
    if (rowp) {
        const FilterParams& f = rowp[(int64_t)b * B];
        if (f.dense == kRowTopK) continue;
        log2e_over_T = 1.4426950408889634074 / (double)f.temperature;
    }
    const int c0 = blockIdx.y * kDenseWaves + w;
    const int js = jstar_in[b];
    if (js >= B || c0 >= nc) continue;
    const DenseExp ex{ log2e_over_T, s_exp2 };
    const int64_t qr = linear_row(batch, B, b, js), pr = linear_row(batch, B, b, B + js);
    float mpf;
    double Sp;
    dense_row_stat(dc.cmax + pr * nc, dc.csum + pr * nc, nc, ex, lane, &mpf, &Sp);   // exact chunks
    float mqf;
    double Sq;
    dense_row_stat(dc.cmax + qr * nc, dc.csum + qr * nc, nc, ex, lane, &mqf, &Sq);   // exact chunks
    // the request's chunks dealt over gridDim.y workgroups, round robin over their waves
    for (int c = c0; c < nc; c += gridDim.y * kDenseWaves) {
        double total = 0.0;
        if (Sp > 0.0) {
            const int64_t row_bytes = N * Vec<BF16>::ESZ;
            const bool q_ok = Sq > 0.0;
            float xp[kPerLane], xq[kPerLane];
            load_chunk<BF16>(row_pointer(src, pr, row_bytes), N, c, xp, lane);
            if (q_ok) load_chunk<BF16>(row_pointer(src, qr, row_bytes), N, c, xq, lane);
            const double mp = (double)mpf, mq = (double)mqf;
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
}

// Vectors j0 .. j0 + NJ - 1 of chunk c of a row (the layout of load_chunk:
// element (j*64 + lane)*EPV + e at x[(j - j0)*EPV + e]); -inf past the end.
template <bool BF16, int NJ>
__device__ __forceinline__ void load_chunk_part(const char* row, int64_t N, int64_t c, int j0, float* x, int lane)
{
    using V = Vec<BF16>;
    constexpr int EPV = V::EPV, ESZ = V::ESZ;
    const int64_t beg = c * kDenseChunk;
    const int64_t n = (N - beg < kDenseChunk) ? (N - beg) : kDenseChunk;
    if (n == kDenseChunk && ((((uintptr_t)(row + beg * ESZ)) & 15u) == 0)) {
        const typename V::T* p = reinterpret_cast<const typename V::T*>(row + beg * ESZ);
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
            const typename V::T v = V::load_stream(p + (j0 + jj) * kWave + lane);
#pragma unroll
            for (int e = 0; e < EPV; ++e) x[jj * EPV + e] = V::get(v, e);
        }
    } else {
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int64_t i = (int64_t)((j0 + jj) * kWave + lane) * EPV + e;
                x[jj * EPV + e] = (i < n) ? load_scalar<BF16>(row, beg + i) : -INFINITY;
            }
    }
}

// Residual (or bonus) sample from exact sums and the cycle's outputs: every
// request (one per workgroup) or, with a list, the listed requests (those
// whose certified draw was not certain), dealt over the workgroups.  Four
// waves per request: the two rows' statistics and the residual total side by
// side, then the picked chunk's residual weights a quarter of its vectors per
// wave.  The cumulative sums are those of one wave stepping through the chunk
// (each 64-lane block's total added in block order), so the pick is the same.
constexpr int kFinishWaves = 4;
constexpr int kFinishThreads = kFinishWaves * kWave;

template <bool BF16>
__global__ __launch_bounds__(kFinishThreads) void dense_finish_exact_kernel(
    RowSource src, int32_t batch, int32_t B, int64_t N, double log2e_over_T0, DenseChunks dc,
    uint64_t seed, uint64_t offset, const uint32_t* req_ids, const int32_t* jstar_in, const int32_t* y_in,
    const uint32_t* flag_in, const int32_t* list, const uint32_t* list_n, const double* resid, LinearOut o,
    const FilterParams* rowp)
{
    constexpr int EPV = Vec<BF16>::EPV;
    constexpr int NV = kPerLane / EPV;                 // 64-lane blocks of a chunk
    constexpr int NVW = NV / kFinishWaves;             // blocks per wave
    static_assert(NV % kFinishWaves == 0, "a chunk's blocks split evenly over the waves");
    const int njobs = list ? (int)*list_n : (int)gridDim.x;
    if ((int)blockIdx.x >= njobs) return;
    __shared__ double s_exp2[kExp2Entries];
    __shared__ double s_S[3];            // Sp, Sq, residual total
    __shared__ float s_m[2];             // row maxima of p and q
    __shared__ double s_bt[NV];          // block totals of the picked chunk
    __shared__ int s_hit[kFinishWaves], s_last[kFinishWaves];
    __shared__ int s_fin;
    load_exp2_table(s_exp2);
    __syncthreads();
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    for (int job = blockIdx.x; job < njobs; job += gridDim.x) {
        const int b = list ? list[job] : job;
        double log2e_over_T = log2e_over_T0;
        if (rowp) {
            const FilterParams& f = rowp[(int64_t)b * B];
            if (f.dense == kRowTopK) continue;
            log2e_over_T = 1.4426950408889634074 / (double)f.temperature;
        }
        const DenseExp ex{ log2e_over_T, s_exp2 };
        const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
        const int nc = dc.nchunks;
        const int64_t row_bytes = N * Vec<BF16>::ESZ;
        const int js = jstar_in[b];
        const Draw d = uno_draw(seed, req, (uint32_t)js, offset);
        const int64_t pr = linear_row(batch, B, b, B + js);
        const int64_t qr = linear_row(batch, B, b, js < B ? js : 0);
        const char* prow = row_pointer(src, pr, row_bytes);
        const double* R = resid + (int64_t)b * nc;
        auto rterm = [&](int c) { return R[c]; };
        // the rows' statistics (exact chunks) and the residual total, side by side
        if (w == 0 || (w == 1 && js < B)) {
            const int64_t r = w == 0 ? pr : qr;
            float m;
            double S;
            dense_row_stat(dc.cmax + r * nc, dc.csum + r * nc, nc, ex, lane, &m, &S);
            if (lane == 0) { s_m[w] = m; s_S[w] = S; }
        } else if (w == 2 && js < B) {
            double Rtot = 0.0;
            for (int base = 0; base < nc; base += kWave) {
                const int c = base + lane;
                const double incl = wave_incl_scan_f64(c < nc ? R[c] : 0.0, lane);
                Rtot += lane_value(incl, kWave - 1);
            }
            if (lane == 0) s_S[2] = Rtot;
        }
        __syncthreads();
        const float mp = s_m[0];
        const double Sp = s_S[0];
        uint32_t fl = flag_in[b];
        int32_t fin = -1;
        bool fallback = false;
        if (!(Sp > 0.0)) {
            fl |= 1u;
        } else if (js < B) {
            const float mqf = s_m[1];
            const double Sq = s_S[1], Rtot = s_S[2];
            const bool q_ok = Sq > 0.0;
            if (Rtot > 0.0) {
                const double t = d.u[2] * Rtot;
                double before;
                int c = dense_locate(nc, t, rterm, lane, &before);
                double tau = t - before;
                if (c < 0) { c = dense_last_positive_chunk(nc, rterm, lane); tau = INFINITY; }
                // this wave's blocks of chunk c: weights, block totals
                float xp[NVW * EPV], xq[NVW * EPV];
                load_chunk_part<BF16, NVW>(prow, N, c, w * NVW, xp, lane);
                if (q_ok) load_chunk_part<BF16, NVW>(row_pointer(src, qr, row_bytes), N, c, w * NVW, xq, lane);
                const double mpd = (double)mp, mq = (double)mqf;
                const double iSp = 1.0 / Sp, iSq = q_ok ? 1.0 / Sq : 0.0;
                const uint64_t tp = row_keep(dc, pr), tq = row_keep(dc, qr);
                double wl[NVW * EPV], lsum[NVW], incl[NVW];
                int last_pos = -1;
#pragma unroll
                for (int jj = 0; jj < NVW; ++jj) {
                    const int j = w * NVW + jj;
                    lsum[jj] = 0.0;
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const int i = jj * EPV + e;
                        const int64_t id = chunk_elem_id<EPV>(c, j * EPV + e, lane);
                        const double pv = dense_keeps(tp, xp[i], id) ? ex((double)xp[i] - mpd) * iSp : 0.0;
                        const double qv = (q_ok && dense_keeps(tq, xq[i], id)) ? ex((double)xq[i] - mq) * iSq : 0.0;
                        const double dl = pv - qv;
                        wl[i] = dl > 0.0 ? dl : 0.0;
                        lsum[jj] += wl[i];
                        if (wl[i] > 0.0) last_pos = (j * kWave + lane) * EPV + e;
                    }
                    incl[jj] = wave_incl_scan_f64(lsum[jj], lane);
                    if (lane == kWave - 1) s_bt[j] = incl[jj];
                }
                last_pos = wave_max_i32(last_pos);
                __syncthreads();
                // the running sum before this wave's first block, in block order
                double run = 0.0;
                for (int j = 0; j < w * NVW; ++j) run += s_bt[j];
                int hit_at = -1;
#pragma unroll
                for (int jj = 0; jj < NVW; ++jj) {
                    if (hit_at >= 0) break;
                    const uint64_t hit = __ballot(run + incl[jj] > tau);
                    if (hit) {
                        const int l = wave_first_lane(hit);
                        int ep = -1;
                        if (lane == l) {
                            double cc = run + (incl[jj] - lsum[jj]);
#pragma unroll
                            for (int e = 0; e < EPV; ++e) {
                                cc += wl[jj * EPV + e];
                                if (ep < 0 && cc > tau) ep = e;
                            }
                            if (ep < 0) {
#pragma unroll
                                for (int e = EPV - 1; e >= 0; --e)
                                    if (ep < 0 && wl[jj * EPV + e] > 0.0) ep = e;
                            }
                        }
                        ep = lane_value(ep, l);
                        hit_at = ((w * NVW + jj) * kWave + l) * EPV + ep;
                    }
                    run += lane_value(incl[jj], kWave - 1);
                }
                if (lane == 0) { s_hit[w] = hit_at; s_last[w] = last_pos; }
                __syncthreads();
                int l = -1, lp = -1;
                for (int q = 0; q < kFinishWaves; ++q) {
                    if (l < 0 && s_hit[q] >= 0) l = s_hit[q];
                    lp = s_last[q] > lp ? s_last[q] : lp;
                }
                if (l < 0) l = lp;
                fin = l < 0 ? -1 : (int32_t)(c * (int64_t)kDenseChunk + l);
            } else {
                fl |= 2u;
            }
            fallback = fin < 0;
        } else {
            fallback = true;
        }
        if (fallback) {
            // the bonus draw, or a residual without mass: from p (one wave)
            if (w == 0) {
                const int32_t f = dense_sample_row<BF16>(prow, N, dc.cmax + pr * nc, dc.csum + pr * nc, nc, mp, Sp,
                                                         d.u[2], ex, lane, row_keep(dc, pr));
                if (lane == 0) s_fin = f;
            }
            __syncthreads();
            fin = s_fin;
        }
        if (w == 0) {
            int32_t* tok = o.tokens + (int64_t)b * (B + 1);
            for (int j = lane; j <= B; j += kWave) tok[j] = (j < js) ? y_in[(int64_t)b * B + j] : (j == js ? fin : -1);
            if (lane == 0) {
                o.accept_len[b] = js + 1;
                if (o.flags) o.flags[b] = fl;
            }
        }
        __syncthreads();       // the LDS above is reused by the next job
    }
}

// Residual weights of chunk c from fp32 terms: r(x) = max(0, p(x) - q(x)) with
// p(x) = t_p(x) * Ap, t_p = 2^y (y as in the chunk pass, relative to the
// chunk's maximum) and Ap = (the chunk's scale to the row maximum) / Sp, the
// same for q.  ResidualTerms holds one chunk of both rows in registers.
struct ResidualChunk {
    float mpc, mqc;         // chunk maxima of p and q
    double Ap, Aq;          // chunk scale / row normaliser
    float Ap32, Aq32;
};

__device__ __forceinline__ ResidualChunk residual_chunk(const DenseChunks& dc, int64_t pr, int64_t qr, int c,
                                                        double mp, double Sp, double mq, double Sq, bool q_ok,
                                                        double log2e_over_T)
{
    ResidualChunk k;
    const int nc = dc.nchunks;
    k.mpc = dc.cmax[pr * nc + c];
    k.mqc = q_ok ? dc.cmax[qr * nc + c] : 0.0f;
    k.Ap = (k.mpc > -INFINITY) ? exp2(((double)k.mpc - mp) * log2e_over_T) / Sp : 0.0;
    k.Aq = (q_ok && k.mqc > -INFINITY) ? exp2(((double)k.mqc - mq) * log2e_over_T) / Sq : 0.0;
    k.Ap32 = (float)k.Ap;
    k.Aq32 = (float)k.Aq;
    return k;
}

// One element's fp32 terms and residual weight.
__device__ __forceinline__ float residual_weight(const ResidualChunk& k, float xp, float xq, bool kp, bool kq,
                                                 float c32, float* tp, float* yp, float* tq, float* yq)
{
    *yp = fmaxf((xp - k.mpc) * c32, -200.0f);
    *tp = kp ? __builtin_amdgcn_exp2f(*yp) : 0.0f;
    *yq = fmaxf((xq - k.mqc) * c32, -200.0f);
    *tq = kq ? __builtin_amdgcn_exp2f(*yq) : 0.0f;
    return fmaxf(fmaf(*tp, k.Ap32, -(*tq * k.Aq32)), 0.0f);
}

// Residual mass per chunk for requests that rejected a proposal, from fp32
// terms, and a bound on each chunk total's error: the terms' own error, the
// row normalisers' bounds, and 2^-22 of the chunk's p and q mass for the fp32
// products and difference (max(0, .) moves nothing by more than its argument
// does).  The bound holds for every partial sum of the chunk's weights too.
// The terms are the chunk pass's own (same maximum, same fp32 arithmetic), so
// for rows whose chunk sums are still the fast ones (row bound > 0) and
// without keep thresholds, the chunk pass's error and sum bound them; rows
// made exact since then have lost those, and their term errors are summed
// here from the terms.
template <bool BF16, bool KEEP>
__global__ __launch_bounds__(kDenseThreads) void dense_residual_kernel(
    RowSource src, int32_t batch, int32_t B, int64_t N, double log2e_over_T, DenseChunks dc,
    const float* row_m, const double* row_S, const double* row_E, const int32_t* jstar_in, double* resid,
    double* resid_err, const FilterParams* rowp)
{
    const int nc = dc.nchunks;
    if (rowp) {
        const FilterParams& f = rowp[(int64_t)blockIdx.x * B];
        if (f.dense == kRowTopK) return;
        log2e_over_T = 1.4426950408889634074 / (double)f.temperature;
    }
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x;
    const int c0 = blockIdx.y * kDenseWaves + w;
    const int js = jstar_in[b];
    if (js >= B || c0 >= nc) return;
    const int64_t qr = linear_row(batch, B, b, js), pr = linear_row(batch, B, b, B + js);
    const int64_t row_bytes = N * Vec<BF16>::ESZ;
    const char* prow = row_pointer(src, pr, row_bytes);
    const char* qrow = row_pointer(src, qr, row_bytes);
    const float c32 = (float)log2e_over_T;
    const uint64_t tp_thr = row_keep(dc, pr), tq_thr = row_keep(dc, qr);
    constexpr int EPV = Vec<BF16>::EPV;
    for (int c = c0; c < nc; c += gridDim.y * kDenseWaves) {
        // the chunk's loads go out with the row statistics' (both rows exist
        // whatever their statistics say)
        RawChunk<BF16> xp, xq;
        xp.load(prow, N, c, lane);
        xq.load(qrow, N, c, lane);
        const double Sp = row_S[pr], Sq = row_S[qr];
        const double Ep = row_E[pr], Eq = row_E[qr];
        const bool q_ok = Sq > 0.0;
        double total = 0.0, err = 0.0;
        if (Sp > 0.0) {
            const double rp = Ep / Sp, rq = q_ok ? Eq / Sq : 0.0;
            const ResidualChunk k = residual_chunk(dc, pr, qr, c, (double)row_m[pr], Sp, (double)row_m[qr], Sq, q_ok,
                                                   log2e_over_T);
            const bool light = !KEEP && dc.cerr != nullptr && Ep > 0.0 && (!q_ok || Eq > 0.0);
            double tep, teq, mass_p, mass_q;     // term errors and masses, scaled to the row normalisers
            if (light) {
                double r = 0.0;
#pragma unroll
                for (int i = 0; i < kPerLane; ++i) {
                    float tp, yp, tq, yq;
                    r += (double)residual_weight(k, xp.get(i), q_ok ? xq.get(i) : -INFINITY, true, q_ok, c32, &tp,
                                                 &yp, &tq, &yq);
                }
                total = wave_sum_f64(r);
                const int64_t sp_ = pr * nc + c, sq_ = qr * nc + c;
                const double ep = (double)dc.cerr[sp_], eq = q_ok ? (double)dc.cerr[sq_] : 0.0;
                tep = k.Ap * ep;
                teq = k.Aq * eq;
                mass_p = k.Ap * (dc.csum[sp_] + ep);
                mass_q = q_ok ? k.Aq * (dc.csum[sq_] + eq) : 0.0;
            } else {
                float sp = 0.0f, typ = 0.0f, sq = 0.0f, tyq = 0.0f;
                double r = 0.0;
                // without keep thresholds (KEEP false: no nucleus rows) the
                // per-logit support test is skipped: a NaN or -inf logit's
                // clamped term 2^-200 is far below the bound's 2^-100
#pragma unroll
                for (int i = 0; i < kPerLane; ++i) {
                    const float vp = xp.get(i), vq = xq.get(i);
                    bool kp = true, kq = q_ok;
                    if constexpr (KEEP) {
                        const int64_t id = chunk_elem_id<EPV>(c, i, lane);
                        kp = dense_keeps(tp_thr, vp, id);
                        kq = q_ok && dense_keeps(tq_thr, vq, id);
                    }
                    float tp, yp, tq, yq;
                    const float rw = residual_weight(k, vp, q_ok ? vq : -INFINITY, kp, kq, c32, &tp, &yp, &tq, &yq);
                    sp += tp;
                    typ = fmaf(tp, yp, typ);
                    sq += tq;
                    tyq = fmaf(tq, yq, tyq);
                    r += (double)rw;
                }
                total = wave_sum_f64(r);
                const double SP = wave_sum_f64((double)sp), TYP = wave_sum_f64((double)typ);
                const double SQ = wave_sum_f64((double)sq), TYQ = wave_sum_f64((double)tyq);
                tep = k.Ap * (kFastExpRel * SP - kFastArgRel * TYP);
                teq = k.Aq * (kFastExpRel * SQ - kFastArgRel * TYQ);
                mass_p = k.Ap * SP;
                mass_q = k.Aq * SQ;
            }
            err = (1.0 + 2e-3) * (tep + teq + mass_p * rp + mass_q * rq + 0x1p-22 * (mass_p + mass_q)) + 0x1p-100;
        }
        if (lane == 0) {
            resid[(int64_t)b * nc + c] = total;
            resid_err[(int64_t)b * nc + c] = err;
        }
    }
}

// Residual (or bonus) sample from the fast sums, certified against their
// bounds, and the cycle's outputs for the requests where it is certain; the
// rest are flagged for the exact kernels.
template <bool BF16>
__global__ __launch_bounds__(kWave) void dense_finish_kernel(
    RowSource src, int32_t batch, int32_t B, int64_t N, double log2e_over_T, DenseChunks dc,
    uint64_t seed, uint64_t offset, const uint32_t* req_ids, const float* row_m, const double* row_S,
    const double* row_E, const int32_t* jstar_in, const int32_t* y_in, const uint32_t* flag_in, const double* resid,
    const double* resid_err, int32_t* redo, int64_t* xrows1, int32_t* xreq, LinearOut o, const FilterParams* rowp)
{
    __shared__ double s_exp2[kExp2Entries];
    const int b = blockIdx.x;
    // the request's own reads go out together with its parameter set's, and
    // the p row's sum before the table's, so each costs no round trip of its own
    const int js = jstar_in[b];
    const uint32_t req = req_ids ? req_ids[b] : (uint32_t)b;
    uint32_t fl = flag_in[b];
    if (rowp) {
        const FilterParams& f = rowp[(int64_t)b * B];
        if (f.dense == kRowTopK) {
            if (threadIdx.x == 0) redo[b] = 0;
            return;
        }
        log2e_over_T = 1.4426950408889634074 / (double)f.temperature;
    }
    const int64_t pr = linear_row(batch, B, b, B + js);
    const double Sp = row_S[pr];
    load_exp2_table(s_exp2);
    __syncthreads();
    const int lane = lane_id();
    const DenseExp ex{ log2e_over_T, s_exp2 };
    const int nc = dc.nchunks;
    const int64_t row_bytes = N * Vec<BF16>::ESZ;
    const Draw d = uno_draw(seed, req, (uint32_t)js, offset);
    int32_t fin = -1;
    bool certain = true;
    const char* prow = row_pointer(src, pr, row_bytes);
    if (!(Sp > 0.0)) {
        fl |= 1u;
    } else if (js < B) {
        const int64_t qr = linear_row(batch, B, b, js);
        const double Sq = row_S[qr];
        const bool q_ok = Sq > 0.0;
        const double* R = resid + (int64_t)b * nc;
        const double* RE = resid_err + (int64_t)b * nc;
        // rows of at most 128 chunks keep both lists in registers (two chunks
        // per lane), read once; the sums run in the same order either way
        const bool regs = nc <= 2 * kWave;
        double r0 = 0.0, r1 = 0.0, e0 = 0.0, e1 = 0.0;
        if (regs) {
            if (lane < nc) { r0 = R[lane]; e0 = RE[lane]; }
            if (lane + kWave < nc) { r1 = R[lane + kWave]; e1 = RE[lane + kWave]; }
        }
        double Rtot = 0.0, Etot = 0.0;
        if (regs) {
            Rtot = (Rtot + r0) + r1;
            Etot = (Etot + e0) + e1;
        } else {
            for (int c = lane; c < nc; c += kWave) { Rtot += R[c]; Etot += RE[c]; }
        }
        Rtot = wave_sum_f64(Rtot);
        Etot = wave_sum_f64(Etot);
        certain = false;
        if (Rtot > 2.0 * Etot) {             // certainly a positive residual
            const double t = d.u[2] * Rtot;
            auto rterm = [&](int c) { return regs ? (c < kWave ? r0 : r1) : R[c]; };
            double before;
            const int c = dense_locate(nc, t, rterm, lane, &before);
            if (c >= 0) {
                double eb = 0.0;
                if (regs) {
                    if (lane < c) eb += e0;
                    if (lane + kWave < c) eb += e1;
                } else {
                    for (int k = lane; k < c; k += kWave) eb += RE[k];
                }
                eb = wave_sum_f64(eb);
                const double ec = regs ? lane_value(c < kWave ? e0 : e1, c & (kWave - 1)) : RE[c];
                float xp[kPerLane], xq[kPerLane];
                load_chunk<BF16>(prow, N, c, xp, lane);
                if (q_ok) load_chunk<BF16>(row_pointer(src, qr, row_bytes), N, c, xq, lane);
                const ResidualChunk k = residual_chunk(dc, pr, qr, c, (double)row_m[pr], Sp, (double)row_m[qr], Sq,
                                                       q_ok, log2e_over_T);
                const float c32 = (float)log2e_over_T;
                const uint64_t tp_thr = row_keep(dc, pr), tq_thr = row_keep(dc, qr);
                constexpr int EPV = Vec<BF16>::EPV;
                auto wf = [&](int i) {
                    const int64_t id = chunk_elem_id<EPV>(c, i, lane);
                    float tp, yp, tq, yq;
                    return (double)residual_weight(k, xp[i], q_ok ? xq[i] : -INFINITY, dense_keeps(tp_thr, xp[i], id),
                                                   q_ok && dense_keeps(tq_thr, xq[i], id), c32, &tp, &yp, &tq, &yq);
                };
                double margin = -1.0;
                const int l = pick_in_chunk<EPV>(wf, t - before, lane, &margin);
                const double bound = d.u[2] * Etot + eb + ec + 1e-12 * Rtot;
                if (l >= 0 && margin > bound) {
                    certain = true;
                    fin = (int32_t)(c * (int64_t)kDenseChunk + l);
                }
            }
        }
    } else {
        fin = dense_sample_row<BF16>(prow, N, dc.cmax + pr * nc, dc.csum + pr * nc, nc, row_m[pr], Sp, d.u[2], ex,
                                     lane, row_keep(dc, pr), dc.cerr ? dc.cerr + pr * nc : nullptr, row_E[pr],
                                     &certain);
    }
    if (lane == 0) {
        redo[b] = certain ? 0 : 1;
        if (!certain && dc.xcount != nullptr) {
            xreq[atomicAdd(&dc.xcount[2], 1u)] = b;
            // the rows the exact kernels need exact: p, and q after a rejection
            const int64_t qr = js < B ? linear_row(batch, B, b, js) : -1;
            const bool wp = row_E[pr] > 0.0, wq = qr >= 0 && row_E[qr] > 0.0;
            const uint32_t n = (wp ? 1u : 0u) + (wq ? 1u : 0u);
            if (n > 0) {
                int64_t* out = xrows1 + atomicAdd(&dc.xcount[1], n);
                if (wp) *out++ = pr;
                if (wq) *out = qr;
            }
        }
    }
    if (!certain) return;
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
constexpr int kNucBins = 2048;
constexpr int64_t kNucWideRows = 256;   // nucleus rows up to which a row takes eight waves

// NW waves per row: four, at three workgroups per CU (168 VGPRs; a few
// spills, outside the streaming loops' loads; the LDS of four would not fit),
// or eight when at most one row per CU is cut, where a wave's serial chunks,
// not the chip, set the time.
template <bool BF16, int NW>
__global__ __launch_bounds__(NW * kWave, NW == 4 ? 3 : 2) void nucleus_kernel(
    RowSource src, int64_t N, double log2e_over_T, double top_p, DenseChunks dc, int32_t* out_count,
    double* out_stats, const FilterParams* rowp)
{
    constexpr int kNucWaves = NW;
    constexpr int kNucThreads = NW * kWave;
    constexpr int kNucCand = kNucBins / 2 / kNucWaves;   // collected logits per wave (in s_cnt)
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
    const int64_t r = blockIdx.x;
    if (rowp) {
        // per-row parameters: a full-softmax row keeps the whole vocabulary,
        // a top-k row is not this kernel's
        const FilterParams& f = rowp[r];
        if (f.dense != kRowNucleus) {
            if (f.dense == kRowFull && threadIdx.x == 0) dc.keep[r] = 0ull;
            return;
        }
        log2e_over_T = 1.4426950408889634074 / (double)f.temperature;
        top_p = (double)f.top_p;
    }
    load_exp2_table(s_exp2);
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
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
                    fa = run + lane_value(incl - mb, l);
                    fc = crun + lane_value(cincl - cb, l);
                } else {
                    const uint64_t nz = __ballot(filled);
                    if (nz) {
                        const int l = 63 - __clzll((long long)nz);
                        last = top - l;
                        la = run + lane_value(incl - mb, l);
                        lc = crun + lane_value(cincl - cb, l);
                    }
                    run += lane_value(incl, kWave - 1);
                    crun += lane_value(cincl, kWave - 1);
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
                    run += lane_value(incl, kWave - 1);
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
                const int b = lane_value(run_b, q), e = lane_value(run_e, q);
                const double ab = lane_value(above, q);
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
        // The first level counted nothing (masses only), and s_cnt now holds
        // the waves' lists: at least one counting level must run, even when
        // the chosen bin is a single key (a level of width 1 counts its ties).
        level();
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
                const double tot = lane_value(incl, kWave - 1);
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
// wave per node row over the whole chip, the uniform of the node's depth),
// then one wave per request follows the path as in the sparse walk.
// Every node row's draw for the dense walk, one wave per row over the whole
// chip (a request's nodes side by side on several CUs): the node's depth from
// the request's parent links, held three per lane, the row statistics from
// its chunk sums, and the draw with the uniform of that depth; -1 where the
// walk cannot take it (no valid path to the root, deeper than B, past the
// request's node count, or no mass).
constexpr int kDrawThreads = 256;
constexpr int kDrawWaves = kDrawThreads / kWave;
static_assert(kMaxNodes <= 3 * kWave, "a wave holds a request's parent links three per lane");

template <bool BF16>
__global__ __launch_bounds__(kDrawThreads) void dense_node_draw_kernel(
    RowSource src, int32_t batch, int32_t B, int32_t V, int64_t N, double log2e_over_T, DenseChunks dc,
    uint64_t seed, uint64_t offset, const uint32_t* req_ids, const int32_t* node_parent,
    const int32_t* num_nodes, int32_t* node_draw, const FilterParams* rowp)
{
    __shared__ double s_exp2[kExp2Entries];
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t rows = (int64_t)batch * (V + 1);
    const int64_t r = (int64_t)blockIdx.x * kDrawWaves + w;
    const bool live = r < rows;                                    // wave-uniform
    const int b = live ? (int)(r / (V + 1)) : 0;
    const int n = (int)(r - (int64_t)b * (V + 1));
    const int64_t ob = (int64_t)b * (V + 1);
    // the request's reads go out before the table's
    int nn = live ? num_nodes[b] : 1;
    const uint32_t req = (live && req_ids) ? req_ids[b] : (uint32_t)b;
    int p0 = -1, p1 = -1, p2 = -1;
    if (live) {
        if (lane <= V) p0 = node_parent[ob + lane];
        if (lane + kWave <= V) p1 = node_parent[ob + lane + kWave];
        if (lane + 2 * kWave <= V) p2 = node_parent[ob + lane + 2 * kWave];
    }
    bool dense = live;
    if (live && rowp) {
        const FilterParams& f = rowp[ob];
        dense = f.dense != kRowTopK;
        log2e_over_T = 1.4426950408889634074 / (double)f.temperature;
    }
    load_exp2_table(s_exp2);
    __syncthreads();
    if (!dense) return;
    nn = nn < 1 ? 1 : (nn > V + 1 ? V + 1 : nn);
    // depth: the root is node 0; a node's parent must precede it, so a walk up
    // the links ends at the root or at an invalid link within n steps
    int dep = -1;
    if (n < nn) {
        int x = n, d = 0;
        while (x > 0) {
            const int pr = __builtin_amdgcn_readlane(x < kWave ? p0 : (x < 2 * kWave ? p1 : p2), x & (kWave - 1));
            if (!(pr >= 0 && pr < x)) { d = -1; break; }
            x = pr;
            ++d;
        }
        dep = d;
    }
    int32_t t = -1;
    if (dep >= 0 && dep <= B) {
        const DenseExp ex{ log2e_over_T, s_exp2 };
        const int nc = dc.nchunks;
        const float* cm = dc.cmax + r * nc;
        const double* cs = dc.csum + r * nc;
        float m;
        double S;
        if (dense_row_stat(cm, cs, nc, ex, lane, &m, &S)) {
            const Draw dr = uno_draw(seed, req, (uint32_t)dep, offset);
            t = dense_sample_row<BF16>(row_pointer(src, r, N * Vec<BF16>::ESZ), N, cm, cs, nc, m, S, dr.u[2], ex,
                                       lane, row_keep(dc, r));
        }
    }
    if (lane == 0) node_draw[r] = t;
}

// The dense walk itself, one workgroup per request: the depths and links in
// LDS, then one wave follows the path through the node draws.
constexpr int kFollowThreads = 192;
static_assert(kFollowThreads >= kMaxNodes, "tree_depths takes one thread per node");

__global__ __launch_bounds__(kFollowThreads) void dense_walk_kernel(int32_t B, int32_t V, const int32_t* node_token,
                                                                   const int32_t* node_parent,
                                                                   const int32_t* num_nodes, const int32_t* node_draw,
                                                                   WalkOut o, const FilterParams* rowp)
{
    __shared__ TreeLds L;
    __shared__ int32_t s_t[kMaxNodes];
    const int b = blockIdx.x;
    const int64_t ob = (int64_t)b * (V + 1);
    if (rowp && rowp[ob].dense == kRowTopK) return;
    int nn = num_nodes[b];
    nn = nn < 1 ? 1 : (nn > V + 1 ? V + 1 : nn);
    for (int n = (int)threadIdx.x; n < nn; n += kFollowThreads) s_t[n] = node_draw[ob + n];
    tree_depths(node_token, node_parent, ob, nn, V, L);      // its barriers also publish s_t
    if (threadIdx.x < kWave) follow_path(b, B, nn, s_t, L, o, lane_id());
}

// Tree build over full-vocabulary filters: the top-K supports come normalised
// over their K ids; this rescales them to the full softmax, whose normaliser
// the exact chunk statistics give (one wave per row).
__global__ __launch_bounds__(kDenseThreads) void dense_support_scale_kernel(int64_t rows, double inv_T,
                                                                           DenseChunks dc, const int32_t* limit,
                                                                           SparseOut sup, const FilterParams* rowp)
{
    const int lane = lane_id();
    const int64_t r = (int64_t)blockIdx.x * kDenseWaves + threadIdx.x / kWave;
    if (r >= rows) return;
    if (rowp) {                              // per-row parameters: the full-vocabulary rows only
        if (rowp[r].dense == kRowTopK) return;
        if (rowp[r].dense != kRowNucleus) limit = nullptr;
        inv_T = 1.0 / (double)rowp[r].temperature;
    }
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
                                hipStream_t stream, const FilterParams* rowp)
{
    if (sup.cum == nullptr) return hipErrorInvalidValue;     // needs id-ordered supports
    linear_sparse_kernel<<<dim3((unsigned)batch), kLinThreads, 0, stream>>>(batch, B, sup, seed, offset,
                                                                           request_ids, o, rowp);
    return hipGetLastError();
}

hipError_t launch_linear_dense(const RowSource& src, int32_t batch, int32_t B, int64_t vocab,
                               bool bf16, float temperature, const DenseChunks& dc,
                               const DenseScratch& sc, uint64_t seed, uint64_t offset,
                               const uint32_t* request_ids, const LinearOut& o, bool exact_all,
                               hipStream_t stream, const FilterParams* rowp)
{
    const double c = 1.4426950408889634074 / (double)temperature;
    // about 2048 workgroups: with many requests each wave takes several chunks,
    // so fewer workgroups load the exponential table
    const int per_req = (dc.nchunks + kDenseWaves - 1) / kDenseWaves;
    const int want = (2048 + batch - 1) / batch;
    const int gy = per_req < want ? per_req : want;
    const dim3 rgrid((unsigned)batch, (unsigned)gy);
    // the exact residual runs for the few requests whose last draw was not
    // certain: one chunk per wave for each of them
    const dim3 xgrid((unsigned)kExactJobs, (unsigned)per_req);
    const int64_t rows = (int64_t)batch * (2 * B + 1);
    // the proposals of a request run side by side: one wave each (4 to 8 waves)
    const int pw = B < kDenseWaves ? kDenseWaves : (B > kProposeMaxThreads / kWave ? kProposeMaxThreads / kWave : B);
    const unsigned pthreads = (unsigned)(pw * kWave);
    if (bf16) {
        dense_row_stat_kernel<<<dim3((unsigned)((rows + 2 * kRowStatWaves - 1) / (2 * kRowStatWaves))), kRowStatThreads, 0,
                                stream>>>(rows, c, dc, sc.row_m, sc.row_S, sc.row_E, rowp);
        dense_propose_kernel<true><<<dim3((unsigned)batch), pthreads, 0, stream>>>(
            src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.row_m, sc.row_S, sc.row_E, sc.y, sc.acc,
            sc.flags, sc.xrows, rowp);
        if (dc.xcount && !exact_all)
            dense_exact_list_kernel<true><<<dim3(kListGroups), kDenseThreads, 0, stream>>>(src, vocab, c, dc, sc.xrows,
                                                                                       dc.xcount, rowp);
        dense_settle_kernel<true><<<dim3((unsigned)batch), pthreads, 0, stream>>>(
            src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.row_m, sc.row_S, sc.row_E, sc.y, sc.acc,
            sc.jstar, sc.y, sc.flags, o, rowp);
        if (exact_all) {
            // every row exact already: exact residual and draw for every request
            dense_residual_exact_kernel<true><<<rgrid, kDenseThreads, 0, stream>>>(src, batch, B, vocab, c, dc, sc.jstar,
                                                                                  nullptr, nullptr, sc.resid, rowp);
            dense_finish_exact_kernel<true><<<dim3((unsigned)batch), kFinishThreads, 0, stream>>>(
                src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.jstar, sc.y, sc.flags, nullptr, nullptr,
                sc.resid, o, rowp);
        } else {
            // certified draws from the fast sums; the exact kernels take the uncertain ones
            if (dc.keep)
                dense_residual_kernel<true, true><<<rgrid, kDenseThreads, 0, stream>>>(
                    src, batch, B, vocab, c, dc, sc.row_m, sc.row_S, sc.row_E, sc.jstar, sc.resid, sc.resid_err, rowp);
            else
                dense_residual_kernel<true, false><<<rgrid, kDenseThreads, 0, stream>>>(
                    src, batch, B, vocab, c, dc, sc.row_m, sc.row_S, sc.row_E, sc.jstar, sc.resid, sc.resid_err, rowp);
            dense_finish_kernel<true><<<dim3((unsigned)batch), kWave, 0, stream>>>(
                src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.row_m, sc.row_S, sc.row_E, sc.jstar, sc.y,
                sc.flags, sc.resid, sc.resid_err, sc.fin_redo, sc.xrows + rows, sc.xreq, o, rowp);
            dense_exact_list_kernel<true><<<dim3(kListGroups), kDenseThreads, 0, stream>>>(src, vocab, c, dc,
                                                                                       sc.xrows + rows, dc.xcount + 1,
                                                                                       rowp);
            dense_residual_exact_kernel<true><<<xgrid, kDenseThreads, 0, stream>>>(src, batch, B, vocab, c, dc, sc.jstar,
                                                                                  sc.xreq, dc.xcount + 2, sc.resid, rowp);
            dense_finish_exact_kernel<true><<<dim3(kExactJobs), kFinishThreads, 0, stream>>>(
                src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.jstar, sc.y, sc.flags, sc.xreq,
                dc.xcount + 2, sc.resid, o, rowp);
        }
    } else {
        dense_row_stat_kernel<<<dim3((unsigned)((rows + 2 * kRowStatWaves - 1) / (2 * kRowStatWaves))), kRowStatThreads, 0,
                                stream>>>(rows, c, dc, sc.row_m, sc.row_S, sc.row_E, rowp);
        dense_propose_kernel<false><<<dim3((unsigned)batch), pthreads, 0, stream>>>(
            src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.row_m, sc.row_S, sc.row_E, sc.y, sc.acc,
            sc.flags, sc.xrows, rowp);
        if (dc.xcount && !exact_all)
            dense_exact_list_kernel<false><<<dim3(kListGroups), kDenseThreads, 0, stream>>>(src, vocab, c, dc, sc.xrows,
                                                                                       dc.xcount, rowp);
        dense_settle_kernel<false><<<dim3((unsigned)batch), pthreads, 0, stream>>>(
            src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.row_m, sc.row_S, sc.row_E, sc.y, sc.acc,
            sc.jstar, sc.y, sc.flags, o, rowp);
        if (exact_all) {
            // every row exact already: exact residual and draw for every request
            dense_residual_exact_kernel<false><<<rgrid, kDenseThreads, 0, stream>>>(src, batch, B, vocab, c, dc, sc.jstar,
                                                                                  nullptr, nullptr, sc.resid, rowp);
            dense_finish_exact_kernel<false><<<dim3((unsigned)batch), kFinishThreads, 0, stream>>>(
                src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.jstar, sc.y, sc.flags, nullptr, nullptr,
                sc.resid, o, rowp);
        } else {
            // certified draws from the fast sums; the exact kernels take the uncertain ones
            if (dc.keep)
                dense_residual_kernel<false, true><<<rgrid, kDenseThreads, 0, stream>>>(
                    src, batch, B, vocab, c, dc, sc.row_m, sc.row_S, sc.row_E, sc.jstar, sc.resid, sc.resid_err, rowp);
            else
                dense_residual_kernel<false, false><<<rgrid, kDenseThreads, 0, stream>>>(
                    src, batch, B, vocab, c, dc, sc.row_m, sc.row_S, sc.row_E, sc.jstar, sc.resid, sc.resid_err, rowp);
            dense_finish_kernel<false><<<dim3((unsigned)batch), kWave, 0, stream>>>(
                src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.row_m, sc.row_S, sc.row_E, sc.jstar, sc.y,
                sc.flags, sc.resid, sc.resid_err, sc.fin_redo, sc.xrows + rows, sc.xreq, o, rowp);
            dense_exact_list_kernel<false><<<dim3(kListGroups), kDenseThreads, 0, stream>>>(src, vocab, c, dc,
                                                                                       sc.xrows + rows, dc.xcount + 1,
                                                                                       rowp);
            dense_residual_exact_kernel<false><<<xgrid, kDenseThreads, 0, stream>>>(src, batch, B, vocab, c, dc, sc.jstar,
                                                                                  sc.xreq, dc.xcount + 2, sc.resid, rowp);
            dense_finish_exact_kernel<false><<<dim3(kExactJobs), kFinishThreads, 0, stream>>>(
                src, batch, B, vocab, c, dc, seed, offset, request_ids, sc.jstar, sc.y, sc.flags, sc.xreq,
                dc.xcount + 2, sc.resid, o, rowp);
        }
    }
    return hipGetLastError();
}

hipError_t launch_tree_build(int32_t batch, int32_t B, int32_t K, int32_t V, const SparseOut& sup,
                             const TreeOut& o, hipStream_t stream)
{
    // live frontier entries <= 1 + V
    const dim3 grid((unsigned)batch);
    if (V + 1 <= kWave)
        tree_build_kernel<1><<<grid, kBuildThreads, 0, stream>>>(batch, B, K, V, sup, o);
    else if (V + 1 <= 2 * kWave)
        tree_build_kernel<2><<<grid, kBuildThreads, 0, stream>>>(batch, B, K, V, sup, o);
    else
        tree_build_kernel<3><<<grid, kBuildThreads, 0, stream>>>(batch, B, K, V, sup, o);
    return hipGetLastError();
}

hipError_t launch_tree_walk(int32_t batch, int32_t B, int32_t V, const SparseOut& sup, uint64_t seed,
                            uint64_t offset, const uint32_t* request_ids, const int32_t* node_token,
                            const int32_t* node_parent, const int32_t* num_nodes, const WalkOut& o,
                            hipStream_t stream, const FilterParams* rowp)
{
    if (sup.cum == nullptr) return hipErrorInvalidValue;     // needs id-ordered supports
    tree_walk_kernel<<<dim3((unsigned)batch), kWalkThreads, 0, stream>>>(
        batch, B, V, sup, seed, offset, request_ids, node_token, node_parent, num_nodes, o, rowp);
    return hipGetLastError();
}

hipError_t launch_tree_walk_dense(const RowSource& src, int32_t batch, int32_t B, int32_t V, int64_t vocab,
                                  bool bf16, float temperature, const DenseChunks& dc, uint64_t seed,
                                  uint64_t offset, const uint32_t* request_ids, const int32_t* node_token,
                                  const int32_t* node_parent, const int32_t* num_nodes, int32_t* node_draw,
                                  const WalkOut& o, hipStream_t stream, const FilterParams* rowp)
{
    if (node_draw == nullptr || V + 1 > kMaxNodes) return hipErrorInvalidValue;
    const double c = 1.4426950408889634074 / (double)temperature;
    const int64_t rows = (int64_t)batch * (V + 1);
    const dim3 dgrid((unsigned)((rows + kDrawWaves - 1) / kDrawWaves));
    if (bf16)
        dense_node_draw_kernel<true><<<dgrid, kDrawThreads, 0, stream>>>(src, batch, B, V, vocab, c, dc, seed, offset,
                                                                        request_ids, node_parent, num_nodes,
                                                                        node_draw, rowp);
    else
        dense_node_draw_kernel<false><<<dgrid, kDrawThreads, 0, stream>>>(src, batch, B, V, vocab, c, dc, seed,
                                                                         offset, request_ids, node_parent, num_nodes,
                                                                         node_draw, rowp);
    dense_walk_kernel<<<dim3((unsigned)batch), kFollowThreads, 0, stream>>>(B, V, node_token, node_parent, num_nodes,
                                                                            node_draw, o, rowp);
    return hipGetLastError();
}

hipError_t launch_dense_support_scale(int64_t rows, float temperature, const DenseChunks& dc,
                                      const int32_t* limit, const SparseOut& sup, hipStream_t stream,
                                      const FilterParams* rowp)
{
    if (sup.stats == nullptr) return hipErrorInvalidValue;
    dense_support_scale_kernel<<<dim3((unsigned)((rows + kDenseWaves - 1) / kDenseWaves)), kDenseThreads, 0,
                                 stream>>>(rows, 1.0 / (double)temperature, dc, limit, sup, rowp);
    return hipGetLastError();
}

hipError_t launch_nucleus(const RowSource& src, int64_t rows, int64_t vocab, bool bf16, float temperature,
                          float top_p, const DenseChunks& dc, int32_t* out_count, double* out_stats,
                          hipStream_t stream, const FilterParams* rowp, int64_t active_rows)
{
    if (rows == 0) return hipSuccess;
    if (dc.keep == nullptr) return hipErrorInvalidValue;
    const double c = 1.4426950408889634074 / (double)temperature;
    const dim3 grid((unsigned)rows);
    const bool wide = (active_rows >= 0 ? active_rows : rows) <= kNucWideRows;
    if (bf16 && wide)
        nucleus_kernel<true, 8><<<grid, 8 * kWave, 0, stream>>>(src, vocab, c, (double)top_p, dc, out_count, out_stats,
                                                                rowp);
    else if (bf16)
        nucleus_kernel<true, 4><<<grid, 4 * kWave, 0, stream>>>(src, vocab, c, (double)top_p, dc, out_count, out_stats,
                                                                rowp);
    else if (wide)
        nucleus_kernel<false, 8><<<grid, 8 * kWave, 0, stream>>>(src, vocab, c, (double)top_p, dc, out_count,
                                                                 out_stats, rowp);
    else
        nucleus_kernel<false, 4><<<grid, 4 * kWave, 0, stream>>>(src, vocab, c, (double)top_p, dc, out_count,
                                                                 out_stats, rowp);
    return hipGetLastError();
}

}  // namespace uno
