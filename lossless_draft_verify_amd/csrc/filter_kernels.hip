// filter_kernels.hip -- row filtering for the UNO sampling path on gfx950.
//
// Sparse rows (top-k on, or greedy): one pass over each logit row keeps, per
// wavefront, a candidate buffer in LDS and a running admission threshold; the
// buffer is cut back to the exact top-k (by logit desc, id asc) with a
// radix select whenever it fills.  The filter order itself -- temperature,
// top-k, renormalise, top-p, renormalise -- follows the filter-order review
// thread of SGLang PR #37667 ("native SGLang serving support for UNO").
//
// Dense rows (top-k off, top-p off): per 2048-logit chunk the kernel writes the
// chunk max and the fp64 sum of exp((z - m_chunk)/T); samplers rebuild the row
// normaliser and the inverse CDF from these.
#include "uno_device.h"
#include "uno_internal.h"

#include <math.h>

namespace uno {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kCap = 768;       // candidate entries per wave
constexpr int kPerIter = 16;    // logits per lane per streaming iteration
constexpr int kMaxK = 256;      // UNO_MAX_TOP_K

// kk-th largest value (1-based) among entries i < cnt with pred(i), by an
// 8-bit radix select over a 256-bin LDS histogram.  Requires at least kk such
// entries.  On return *kk_left is the rank of the k-th element among the
// entries equal to the returned value.
template <typename GetV, typename Pred>
__device__ uint32_t wave_kth_largest(int cnt, int kk, GetV getv, Pred pred, uint32_t* hist,
                                     int lane, int* kk_left)
{
    uint32_t prefix = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        const uint32_t hmask = (shift == 24) ? 0u : (0xFFFFFFFFu << (shift + 8));
        for (int b = lane; b < 256; b += kWave) hist[b] = 0u;
        wave_sync();
        for (int i = lane; i < cnt; i += kWave) {
            if (!pred(i)) continue;
            const uint32_t v = getv(i);
            if ((v & hmask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1u);
        }
        wave_sync();
        // lane l owns bins 255-4l .. 252-4l, so lane order walks the bins downward
        const int b0 = 255 - 4 * lane;
        const uint32_t c0 = hist[b0], c1 = hist[b0 - 1], c2 = hist[b0 - 2], c3 = hist[b0 - 3];
        const uint32_t lsum = c0 + c1 + c2 + c3;
        const uint32_t incl = wave_incl_scan_u32(lsum, lane);
        const uint32_t excl = incl - lsum;
        const uint32_t need = (uint32_t)kk;
        int found = -1;
        uint32_t before = 0;
        if (excl < need && incl >= need) {
            uint32_t a = excl;
            if (a + c0 >= need) { found = b0; before = a; }
            else {
                a += c0;
                if (a + c1 >= need) { found = b0 - 1; before = a; }
                else {
                    a += c1;
                    if (a + c2 >= need) { found = b0 - 2; before = a; }
                    else { a += c2; found = b0 - 3; before = a; }
                }
            }
        }
        const uint64_t bal = __ballot(found >= 0);
        const int src = bal ? wave_first_lane(bal) : 0;
        const int bin = __shfl(found, src, kWave);
        const uint32_t bef = __shfl(before, src, kWave);
        prefix |= (uint32_t)(bin & 255) << shift;
        kk -= (int)bef;
        wave_sync();
    }
    *kk_left = kk;
    return prefix;
}

// Cut the wave's candidate buffer to the exact top-k by (key desc, id asc).
// Returns the new count; when the old count was >= k, *kth is the key of the
// k-th entry and *full is set.
__device__ int wave_topk_exact(uint32_t* key, int32_t* id, int cnt, int k, uint32_t* hist,
                               int lane, uint32_t* kth, bool* full)
{
    *full = false;
    if (cnt < k) return cnt;
    int kk;
    const uint32_t T = wave_kth_largest(
        cnt, k, [&](int i) { return key[i]; }, [](int) { return true; }, hist, lane, &kk);
    uint32_t eq = 0;
    for (int i = lane; i < cnt; i += kWave) eq += (key[i] == T) ? 1u : 0u;
    eq = wave_sum_u32(eq);
    int32_t idcut = 0x7FFFFFFF;
    if ((int)eq > kk) {
        int kk2;
        const uint32_t v = wave_kth_largest(
            cnt, kk, [&](int i) { return ~(uint32_t)id[i]; }, [&](int i) { return key[i] == T; },
            hist, lane, &kk2);
        idcut = (int32_t)~v;
    }
    int out = 0;
    for (int base = 0; base < cnt; base += kWave) {
        const int i = base + lane;
        uint32_t kv = 0;
        int32_t iv = 0;
        bool keep = false;
        if (i < cnt) {
            kv = key[i];
            iv = id[i];
            keep = (kv > T) || (kv == T && iv <= idcut);
        }
        const uint64_t m = __ballot(keep);
        wave_sync();
        if (keep) {
            const int pos = out + __popcll(m & lanes_below(lane));
            key[pos] = kv;
            id[pos] = iv;
        }
        out += __popcll(m);
        wave_sync();
    }
    *kth = T;
    *full = true;
    return out;
}

// Sort n entries by (key desc, id asc) into okey/oid (rank by counting).
__device__ void wave_sort_desc(const uint32_t* key, const int32_t* id, int n, uint32_t* okey,
                               int32_t* oid, int lane)
{
    for (int i = lane; i < n; i += kWave) {
        const uint32_t ki = key[i];
        const int32_t ii = id[i];
        int r = 0;
        for (int j = 0; j < n; ++j) {
            const uint32_t kj = key[j];
            const int32_t ij = id[j];
            r += (kj > ki || (kj == ki && ij < ii)) ? 1 : 0;
        }
        okey[r] = ki;
        oid[r] = ii;
    }
    wave_sync();
}

// Softmax over the sorted top-k set, top-p cut, renormalisation; writes the
// row's support.  Same operation order as the filter definition: normaliser
// summed in filter order, pi = e / S, cumulative pi in filter order, kept
// probabilities pi / (kept mass) when top-p is on.
__device__ void finalize_row(const uint32_t* sk, const int32_t* sid, int n, const FilterParams& fp,
                             double* scratch, const SparseOut& out, int64_t r, int lane)
{
    int32_t* oid = out.ids + r * out.cap;
    double* op = out.probs + r * out.cap;
    int n_out;
    double m = NAN, S = NAN;
    if (n <= 0 || sk[0] == kKeyPosInf) {
        n_out = -1;
    } else if (fp.greedy) {
        n_out = 1;
        m = (double)key_float(sk[0]);
        S = 1.0;
        if (lane == 0) { oid[0] = sid[0]; op[0] = 1.0; }
    } else {
        m = (double)key_float(sk[0]);
        const double Td = (double)fp.temperature;
        for (int i = lane; i < n; i += kWave) scratch[i] = exp(((double)key_float(sk[i]) - m) / Td);
        wave_sync();
        S = 0.0;
        for (int i = 0; i < n; ++i) S += scratch[i];
        wave_sync();
        for (int i = lane; i < n; i += kWave) scratch[i] = scratch[i] / S;
        wave_sync();
        int n_keep = n;
        double c = 0.0;
        if (fp.topp_on) {
            const double p = (double)fp.top_p;
            n_keep = 0;
            for (int i = 0; i < n; ++i) {
                if (i > 0 && c >= p) break;
                c += scratch[i];
                ++n_keep;
            }
        }
        int npos = 0;
        for (int base = 0; base < n_keep; base += kWave) {
            const int i = base + lane;
            double v = 0.0;
            if (i < n_keep) v = fp.topp_on ? scratch[i] / c : scratch[i];
            const bool pos = (i < n_keep) && v > 0.0;
            npos += __popcll(__ballot(pos));
            if (pos) { oid[i] = sid[i]; op[i] = v; }
        }
        n_out = npos;
    }
    for (int i = (n_out > 0 ? n_out : 0) + lane; i < out.cap; i += kWave) {
        oid[i] = -1;
        op[i] = 0.0;
    }
    if (lane == 0) {
        out.count[r] = n_out;
        if (out.stats) { out.stats[2 * r] = m; out.stats[2 * r + 1] = S; }
    }
}

// ---- top-k stream ------------------------------------------------------------
// Number of set bits of `c` (< 64) over the wave, and over the lanes below this one.
__device__ __forceinline__ uint32_t wave_count_prefix(uint32_t c, uint32_t* total)
{
    uint32_t tot = 0, excl = 0;
#pragma unroll
    for (int b = 0; b < 6; ++b) {
        const uint64_t m = __ballot((c >> b) & 1u);
        tot += (uint32_t)__popcll(m) << b;
        excl += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
    }
    *total = tot;
    return excl;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads, 5) void topk_stream_kernel(
    RowSource src, int64_t rows, int64_t N, FilterParams fp, SparseOut out, int S,
    uint32_t* part_key, int32_t* part_id, int32_t* part_n)
{
    using V = Vec<BF16>;
    constexpr int EPV = V::EPV, ESZ = V::ESZ;
    constexpr int U = kPerIter / EPV;                  // 16-byte vectors per lane per iteration
    __shared__ uint32_t s_key[kWaves][kCap];
    __shared__ int32_t s_id[kWaves][kCap];
    __shared__ uint32_t s_hist[kWaves][256];
    __shared__ int s_cnt[kWaves];
    __shared__ double s_scratch[kMaxK];

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t r = blockIdx.x;
    const int seg = blockIdx.y;
    const char* row = row_pointer(src, r, N * ESZ);
    if (row == nullptr) {
        if (S == 1 && threadIdx.x == 0) out.count[r] = -1;
        return;
    }
    const RowGeom g = row_geom<BF16>(row, N);
    const int64_t vb = g.nvec * seg / S, ve = g.nvec * (seg + 1) / S;
    const int64_t wb = vb + (ve - vb) * w / kWaves, we = vb + (ve - vb) * (w + 1) / kWaves;

    uint32_t* bk = s_key[w];
    int32_t* bi = s_id[w];
    uint32_t* hist = s_hist[w];
    const int k = fp.k;
    int cnt = 0;
    // Admission: key(z) > thr_key.  thr is the float of thr_key; for logits
    // `z > thr` (an ordered compare, false for NaN) is the same test.  It starts
    // at -inf, passed in as an argument so the compare is never constant-folded.
    uint32_t thr_key = kKeyNegInf;
    float thr = fp.thr_init;

    auto compact = [&]() __attribute__((always_inline)) {
        uint32_t T;
        bool full;
        cnt = wave_topk_exact(bk, bi, cnt, k, hist, lane, &T, &full);
        if (full) { thr_key = T; thr = key_float(T); }
    };
    auto scalar_part = [&](int64_t beg, int64_t n) __attribute__((always_inline)) {   // n <= 64, ids increase with lane
        if (cnt > kCap - kWave) compact();
        uint32_t key = 0;
        if (lane < n) key = float_key(load_scalar<BF16>(row, beg + lane));
        const bool pass = key_admits(key, thr_key);
        const uint64_t m = __ballot(pass);
        if (pass) {
            const int pos = cnt + __popcll(m & lanes_below(lane));
            bk[pos] = key;
            bi[pos] = (int32_t)(beg + lane);
        }
        cnt += __popcll(m);
    };

    if (seg == 0 && w == 0 && g.head > 0) scalar_part(0, g.head);

    const typename V::T* body = reinterpret_cast<const typename V::T*>(row + g.head * ESZ);
    // Fallback for an iteration whose candidates cannot all fit the buffer even
    // after a cut (only while the threshold is still low): vector by vector,
    // re-reading each vector (a cache hit), with a cut whenever the buffer fills.
    auto reload_path = [&](int64_t v0) __attribute__((always_inline)) {
#pragma unroll 1
        for (int u = 0; u < U; ++u) {
            const int64_t vbase = v0 + u * kWave;
            if (vbase >= we) break;
            const int64_t vl = vbase + lane;
            const typename V::T xv = (vl < we) ? body[vl] : V::neg_inf();
            if (cnt > kCap - kWave * EPV) compact();
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const uint32_t key = float_key(V::get(xv, e));
                const bool pass = key_admits(key, thr_key);
                const uint64_t m = __ballot(pass);
                if (m) {
                    if (pass) {
                        const int pos = cnt + __popcll(m & lanes_below(lane));
                        bk[pos] = key;
                        bi[pos] = (int32_t)(g.head + vl * EPV + e);
                    }
                    cnt += __popcll(m);
                }
            }
        }
    };
    auto admit_mask = [&](const typename V::T (&x)[U]) __attribute__((always_inline)) {
        uint32_t mask = 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < EPV; ++e) mask |= (V::get(x[u], e) > thr ? 1u : 0u) << (u * EPV + e);
        return mask;
    };
    // One iteration: U vectors per lane (vector v0 + u*64 + lane), already in x.
    auto process = [&](const typename V::T (&x)[U], int64_t v0) __attribute__((always_inline)) {
        uint32_t mask = admit_mask(x);
        uint32_t total;
        uint32_t excl = wave_count_prefix(__popc(mask), &total);
        if (total == 0) return;
        if (cnt + (int)total > kCap) {
            compact();
            mask = admit_mask(x);
            excl = wave_count_prefix(__popc(mask), &total);
            if (cnt + (int)total > kCap) { reload_path(v0); return; }
        }
        int pos = cnt + (int)excl;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < EPV; ++e)
                if (mask & (1u << (u * EPV + e))) {
                    bk[pos] = float_key(V::get(x[u], e));
                    bi[pos] = (int32_t)(g.head + (v0 + u * kWave + lane) * EPV + e);
                    ++pos;
                }
        cnt += (int)total;
    };

    // whole iterations with the next iteration's loads in flight
    constexpr int64_t kStep = (int64_t)U * kWave;
    const int64_t nfull = (we - wb) / kStep;
    typename V::T xc[U], xn[U];
    if (nfull > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) xc[u] = body[wb + u * kWave + lane];
    }
    for (int64_t it = 0; it < nfull; ++it) {
        const int64_t v0 = wb + it * kStep;
        // unconditional prefetch (the last iteration re-reads its own vectors), so
        // the number of loads in flight is the same on every path
        const int64_t vn = (it + 1 < nfull) ? v0 + kStep : v0;
#pragma unroll
        for (int u = 0; u < U; ++u) xn[u] = body[vn + u * kWave + lane];
        process(xc, v0);
#pragma unroll
        for (int u = 0; u < U; ++u) xc[u] = xn[u];
    }
    {   // last partial iteration
        const int64_t v0 = wb + nfull * kStep;
        if (v0 < we) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t v = v0 + u * kWave + lane;
                xc[u] = (v < we) ? body[v] : V::neg_inf();
            }
            process(xc, v0);
        }
    }

    if (seg == S - 1 && w == kWaves - 1 && g.tail_beg < N) scalar_part(g.tail_beg, N - g.tail_beg);

    if (cnt > k) compact();
    if (lane == 0) s_cnt[w] = cnt;
    __syncthreads();
    if (w != 0) return;

    int tot = cnt;
    for (int ow = 1; ow < kWaves; ++ow) {
        const int c = s_cnt[ow];
        for (int i = lane; i < c; i += kWave) {
            bk[tot + i] = s_key[ow][i];
            bi[tot + i] = s_id[ow][i];
        }
        tot += c;
    }
    wave_sync();
    cnt = tot;
    if (cnt > k) compact();

    if (S == 1) {
        wave_sort_desc(bk, bi, cnt, s_key[1], s_id[1], lane);
        finalize_row(s_key[1], s_id[1], cnt, fp, s_scratch, out, r, lane);
    } else {
        const int64_t base = (r * S + seg) * (int64_t)k;
        for (int i = lane; i < cnt; i += kWave) {
            part_key[base + i] = bk[i];
            part_id[base + i] = bi[i];
        }
        if (lane == 0) part_n[r * S + seg] = cnt;
    }
}

// One wave per row: merge the S segment lists into the row's top-k and finalize.
__global__ __launch_bounds__(kWave) void topk_merge_kernel(
    RowSource src, int64_t rows, FilterParams fp, SparseOut out, int S,
    const uint32_t* part_key, const int32_t* part_id, const int32_t* part_n)
{
    __shared__ uint32_t s_key[kMergeCap];
    __shared__ int32_t s_id[kMergeCap];
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_skey[kMaxK];
    __shared__ int32_t s_sid[kMaxK];
    __shared__ double s_scratch[kMaxK];

    const int lane = lane_id();
    const int64_t r = blockIdx.x;
    if (r >= rows) return;
    if (row_pointer(src, r, 1) == nullptr) {
        if (lane == 0) out.count[r] = -1;
        return;
    }
    const int k = fp.k;
    int cnt = 0;
    for (int seg = 0; seg < S; ++seg) {
        const int c = part_n[r * S + seg];
        const int64_t base = (r * S + seg) * (int64_t)k;
        for (int i = lane; i < c; i += kWave) {
            s_key[cnt + i] = part_key[base + i];
            s_id[cnt + i] = part_id[base + i];
        }
        cnt += c;
    }
    wave_sync();
    if (cnt > k) {
        uint32_t T;
        bool full;
        cnt = wave_topk_exact(s_key, s_id, cnt, k, s_hist, lane, &T, &full);
    }
    wave_sort_desc(s_key, s_id, cnt, s_skey, s_sid, lane);
    finalize_row(s_skey, s_sid, cnt, fp, s_scratch, out, r, lane);
}

// ---- dense chunk statistics --------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void dense_chunk_kernel(
    RowSource src, int64_t rows, int64_t N, double log2e_over_T, DenseChunks dc)
{
    using V = Vec<BF16>;
    constexpr int EPV = V::EPV, ESZ = V::ESZ;
    constexpr int PER_LANE = kDenseChunk / kWave;          // 32 logits per lane
    constexpr int NV = PER_LANE / EPV;                      // vectors per lane
    __shared__ double s_exp2[kWaves][64];
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    fill_exp2_table(s_exp2[w], lane);
    const int64_t r = blockIdx.x;
    const int64_t c = (int64_t)blockIdx.y * kWaves + w;
    if (c >= dc.nchunks) return;
    const char* row = row_pointer(src, r, N * ESZ);
    const int64_t slot = r * dc.nchunks + c;
    if (row == nullptr) {
        if (lane == 0) { dc.cmax[slot] = -INFINITY; dc.csum[slot] = 0.0; dc.ccount[slot] = 0; }
        return;
    }
    const int64_t beg = c * kDenseChunk;
    const int64_t n = (N - beg < kDenseChunk) ? (N - beg) : kDenseChunk;
    float x[PER_LANE];
    const bool vec_ok = (n == kDenseChunk) && ((((uintptr_t)(row + beg * ESZ)) & 15u) == 0);
    if (vec_ok) {
        const typename V::T* p = reinterpret_cast<const typename V::T*>(row + beg * ESZ);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const typename V::T v = p[j * kWave + lane];
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
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) mx = fmaxf(mx, x[i]);
    mx = wave_max_f32(mx);
    double s = 0.0;
    uint32_t cntf = 0;
    if (mx > -INFINITY && mx < INFINITY) {
        const DenseExp ex{ log2e_over_T, s_exp2[w] };
        const double md = (double)mx;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const bool fin = finite_f32(x[i]);
            cntf += fin ? 1u : 0u;
            s += fin ? ex((double)x[i] - md) : 0.0;
        }
    }
    s = wave_sum_f64(s);
    cntf = wave_sum_u32(cntf);
    if (lane == 0) {
        dc.cmax[slot] = mx;
        dc.csum[slot] = (mx < INFINITY) ? s : NAN;
        dc.ccount[slot] = (int32_t)cntf;
    }
}

// Row maximum and normaliser from the chunk statistics (uno_filter, dense mode).
__global__ void dense_row_stats_kernel(int64_t rows, double inv_T, DenseChunks dc, int32_t* out_count,
                                       double* out_stats)
{
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const float* cm = dc.cmax + r * dc.nchunks;
    const double* cs = dc.csum + r * dc.nchunks;
    const int32_t* cc = dc.ccount + r * dc.nchunks;
    float m = -INFINITY;
    int64_t nf = 0;
    bool bad = false;
    for (int c = 0; c < dc.nchunks; ++c) {
        m = fmaxf(m, cm[c]);
        nf += cc[c];
        bad |= (cm[c] == INFINITY);
    }
    if (bad || !(m > -INFINITY)) {
        out_count[r] = -1;
        out_stats[2 * r] = NAN;
        out_stats[2 * r + 1] = NAN;
        return;
    }
    double S = 0.0;
    for (int c = 0; c < dc.nchunks; ++c)
        if (cm[c] > -INFINITY) S += cs[c] * exp(((double)cm[c] - (double)m) * inv_T);
    out_count[r] = (int32_t)nf;
    out_stats[2 * r] = (double)m;
    out_stats[2 * r + 1] = S;
}

}  // namespace

int topk_segments(int64_t rows, int64_t vocab, int k)
{
    // Aim for >= 1024 workgroups (4 per CU) while keeping segments >= 4096
    // logits and the merged candidate list within one merge workgroup.
    int64_t S = (1024 + rows - 1) / rows;
    const int64_t by_len = vocab / 4096;
    if (S > by_len) S = by_len;
    const int64_t by_merge = kMergeCap / (k > 0 ? k : 1);
    if (S > by_merge) S = by_merge;
    if (S > 64) S = 64;
    if (S < 1) S = 1;
    return (int)S;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

hipError_t launch_topk_filter(const RowSource& src, int64_t rows, int64_t vocab, bool bf16,
                              const FilterParams& fp, const SparseOut& out, int S,
                              uint32_t* part_key, int32_t* part_id, int32_t* part_n,
                              hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)rows, (unsigned)S);
    if (bf16)
        topk_stream_kernel<true><<<grid, kThreads, 0, stream>>>(src, rows, vocab, fp, out, S, part_key,
                                                                part_id, part_n);
    else
        topk_stream_kernel<false><<<grid, kThreads, 0, stream>>>(src, rows, vocab, fp, out, S, part_key,
                                                                 part_id, part_n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    topk_merge_kernel<<<dim3((unsigned)rows), kWave, 0, stream>>>(src, rows, fp, out, S, part_key,
                                                                   part_id, part_n);
    return hipGetLastError();
}

hipError_t launch_dense_chunks(const RowSource& src, int64_t rows, int64_t vocab, bool bf16,
                               float temperature, const DenseChunks& dc, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    const double c = 1.4426950408889634074 / (double)temperature;
    dim3 grid((unsigned)rows, (unsigned)((dc.nchunks + kWaves - 1) / kWaves));
    if (bf16)
        dense_chunk_kernel<true><<<grid, kThreads, 0, stream>>>(src, rows, vocab, c, dc);
    else
        dense_chunk_kernel<false><<<grid, kThreads, 0, stream>>>(src, rows, vocab, c, dc);
    return hipGetLastError();
}

hipError_t launch_dense_row_stats(int64_t rows, float temperature, const DenseChunks& dc,
                                  int32_t* out_count, double* out_stats, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((rows + 255) / 256);
    dense_row_stats_kernel<<<blocks, 256, 0, stream>>>(rows, 1.0 / (double)temperature, dc, out_count,
                                                       out_stats);
    return hipGetLastError();
}

}  // namespace uno
