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
constexpr int kCap = 768;       // candidate entries per wave (12 per lane)
constexpr int kCapE = kCap / 64;
constexpr int kStreamVecs = 2;  // 16-byte vectors per lane per streaming iteration
constexpr int kStreamDepth = 3; // iterations whose loads are in flight at once (the one processed included)
constexpr int kMaxK = 256;      // UNO_MAX_TOP_K
constexpr int64_t kSegmentTarget = 1024;   // workgroups the top-k stream aims for (four per CU)
constexpr int64_t kWideBelow = 512;        // launches with fewer segments take eight waves per segment

// ---- candidate buffers and register-resident lists ----------------------------
// A streaming candidate is (raw float bits of the logit, token id); keys are
// formed only when a list is loaded into registers.
using Cand = uint2;

// Entry j*64 + lane of a wave's list lives in kv[j] / iv[j].  Key 0 pads unused
// slots; it ranks below every admitted key (admitted keys exceed the key of -inf).
template <int E>
struct RegList {
    uint32_t kv[E];
    int32_t iv[E];
};

// Loads entries [0, cnt) of buf (which holds at least E*64 entries; slots past
// cnt are read but padded).
template <int E>
__device__ __forceinline__ void reg_load(RegList<E>& L, const Cand* buf, int cnt, int lane)
{
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const int i = j * kWave + lane;
        const bool in = i < cnt;
        const Cand c = buf[i];
        L.kv[j] = in ? float_key(__uint_as_float(c.x)) : 0u;
        L.iv[j] = in ? (int32_t)c.y : 0x7FFFFFFF;
    }
}

// Wave-wide number of entries with key >= t (t >= 1: padding never counts).
template <int E>
__device__ __forceinline__ int reg_count_ge(const RegList<E>& L, uint32_t t)
{
    int c = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) c += __popcll(__ballot(L.kv[j] >= t));
    return c;
}

// Largest t whose bits below min_bit are zero with count(key >= t) >= k
// (requires k <= count of entries): the k-th largest key, truncated.
template <int E>
__device__ __forceinline__ uint32_t reg_kth_key(const RegList<E>& L, int k, int min_bit)
{
    uint32_t prefix = 0;
    for (int b = 31; b >= min_bit; --b) {
        const uint32_t cand = prefix | (1u << b);
        if (reg_count_ge(L, cand) >= k) prefix = cand;
    }
    return prefix;
}

// Write the entries with keep(kv, iv) compactly to buf (as candidates);
// returns their number.  keep must reject key 0 (padding).
template <int E, typename Keep>
__device__ __forceinline__ int reg_store_if(const RegList<E>& L, Keep keep, Cand* buf)
{
    int out = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const bool kp = keep(L.kv[j], L.iv[j]);
        const uint64_t m = __ballot(kp);
        if (kp) {
            const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)out));
            buf[pos] = make_uint2(__float_as_uint(key_float(L.kv[j])), (uint32_t)L.iv[j]);
        }
        out += __popcll(m);
    }
    return out;
}

// Exact top-k by (key desc, id asc) of the >= k entries in L, written to buf
// (unordered); *kth receives the k-th key.
template <int E>
__device__ __forceinline__ int reg_select_exact(const RegList<E>& L, int k, Cand* buf, uint32_t* kth)
{
    const uint32_t T = reg_kth_key(L, k, 0);
    const int ge = reg_count_ge(L, T);
    const int gt = reg_count_ge(L, T + 1u);
    const int need = k - gt;              // entries with key == T to keep, smallest ids first
    uint32_t idcut = 0x7FFFFFFFu;
    if (ge - gt > need) {
        // need-th smallest id among the entries with key == T, bit by bit
        uint32_t x = 0;
        for (int b = 30; b >= 0; --b) {
            const uint32_t y = x | ((1u << b) - 1u);
            int c = 0;
#pragma unroll
            for (int j = 0; j < E; ++j) c += __popcll(__ballot(L.kv[j] == T && (uint32_t)L.iv[j] <= y));
            if (c < need) x |= 1u << b;
        }
        idcut = x;
    }
    *kth = T;
    return reg_store_if(L, [&](uint32_t kv, int32_t iv) {
        return kv > T || (kv == T && (uint32_t)iv <= idcut);
    }, buf);
}

// Cut of a wave's candidate list (cnt >= k entries in buf, cnt <= E*64): keep
// every entry whose key lies in or above the 16-bit key bin holding the k-th
// largest key (at least k stay), or exactly the top-k when more than `limit`
// would.  Returns the new count; *lo receives a key that every kept entry
// reaches and that at least k kept entries reach (the bin's lower edge, or
// the k-th key).  While streaming, admitting only keys above *lo loses
// nothing: the stream visits ids in increasing order, so a later logit whose
// key does not exceed *lo ranks below at least k kept entries.
template <int E>
__device__ __forceinline__ int wave_cut(Cand* buf, int cnt, int k, int limit, int lane, uint32_t* lo)
{
    RegList<E> L;
    reg_load(L, buf, cnt, lane);
    wave_sync();
    const uint32_t b = reg_kth_key(L, k, 16);
    int c;
    if (reg_count_ge(L, b) > limit) {
        c = reg_select_exact(L, k, buf, lo);
    } else {
        c = reg_store_if(L, [&](uint32_t kv, int32_t) { return kv >= b; }, buf);
        *lo = b;
    }
    wave_sync();
    return c;
}

// k-th largest (k <= 64 P) of P keys per lane (P = 2: a, b; P = 4: a to d),
// truncated to its 16-bit bin: the largest t with low 16 bits zero and at
// least k of the keys >= t.
template <int P>
__device__ __forceinline__ uint32_t wave_kth_largest_of_lane_keys(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                                                  int k)
{
    uint32_t prefix = 0;
#pragma unroll 1
    for (int bit = 31; bit >= 16; --bit) {
        const uint32_t t = prefix | (1u << bit);
        int n = __popcll(__ballot(a >= t)) + __popcll(__ballot(b >= t));
        if constexpr (P == 4) n += __popcll(__ballot(c >= t)) + __popcll(__ballot(d >= t));
        if (n >= k) prefix = t;
    }
    return prefix;
}

// Float threshold equivalent to "key > t" for every non-NaN logit.  Key
// 0x7FFFFFFF (the key of -0, which float_key folds onto +0) maps to the
// largest negative float instead.
__device__ __forceinline__ float thr_float(uint32_t t)
{
    return key_float(t == 0x7FFFFFFFu ? 0x7FFFFFFEu : t);
}

// Filter-order position key: larger means earlier (key desc, then id asc).

// Block-wide ranking of the candidates held in L lists (list o: lst[o*stride ..
// o*stride + cnt[o]) in LDS, entries (key, id), distinct ids): the entry at
// filter-order position r < k goes to sk/sid[r], and, when se is given, its
// softmax numerator exp((z - m) / T) to se[r] (m: the largest key's logit).
// Returns min(total, k).  Every thread calls it.  With at most kOkCap
// candidates (the usual case) their order keys are first gathered into ok (LDS
// scratch of kOkCap words, free during the rank) and each rank is a count over
// that one array; otherwise every comparison reads the lists.
constexpr int kOkCap = kMaxK + 1;
template <int L>
__device__ __forceinline__ int block_rank_topk(const uint2* lst, int stride, const int* cnt, int k, uint32_t* sk,
                                               int32_t* sid, double* se, double m, double Td, int tid,
                                               int nthreads, uint64_t* ok)
{
    int n = 0;
#pragma unroll
    for (int o = 0; o < L; ++o) n += cnt[o];
    auto place = [&](uint64_t p, int rank) __attribute__((always_inline)) {
        if (rank < k) {
            const uint32_t key = (uint32_t)(p >> 32);
            sk[rank] = key;
            sid[rank] = (int32_t)~(uint32_t)p;
            if (se) se[rank] = exp(((double)key_float(key) - m) / Td);
        }
    };
    if (n <= kOkCap) {
        for (int g = tid; g < n; g += nthreads) {
            int o = 0, i = g;
            while (i >= cnt[o]) { i -= cnt[o]; ++o; }
            const uint2 c = lst[o * stride + i];
            ok[g] = order_key(c.x, (int32_t)c.y);
        }
        __syncthreads();
        // sixteen keys per step, read as eight 16-byte words (ok is 16-byte aligned)
        const ulonglong2* ok2 = reinterpret_cast<const ulonglong2*>(ok);
        for (int g = tid; g < n; g += nthreads) {
            const uint64_t p = ok[g];
            int rank = 0;
            int j = 0;
            for (; j + 16 <= n; j += 16) {
                ulonglong2 a[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) a[t] = ok2[(j >> 1) + t];
#pragma unroll
                for (int t = 0; t < 8; ++t) rank += (a[t].x > p) + (a[t].y > p);
            }
            for (; j < n; ++j) rank += (ok[j] > p);
            place(p, rank);
        }
        return n < k ? n : k;
    }
    for (int g = tid; g < n; g += nthreads) {
        int o = 0, i = g;
        while (i >= cnt[o]) { i -= cnt[o]; ++o; }
        const uint2 c = lst[o * stride + i];
        const uint64_t p = order_key(c.x, (int32_t)c.y);
        int rank = 0;
#pragma unroll
        for (int o2 = 0; o2 < L; ++o2) {
            const uint2* a = lst + o2 * stride;
            const int mo = cnt[o2];
            int j = 0;
            for (; j + 4 <= mo; j += 4) {
                const uint2 a0 = a[j], a1 = a[j + 1], a2 = a[j + 2], a3 = a[j + 3];
                rank += (order_key(a0.x, (int32_t)a0.y) > p) + (order_key(a1.x, (int32_t)a1.y) > p) +
                        (order_key(a2.x, (int32_t)a2.y) > p) + (order_key(a3.x, (int32_t)a3.y) > p);
            }
            for (; j < mo; ++j) rank += (order_key(a[j].x, (int32_t)a[j].y) > p);
        }
        place(p, rank);
    }
    return n < k ? n : k;
}

// Softmax over the sorted top-k set, top-p cut, renormalisation (one wave);
// writes the row's support.  Same operation order as the filter definition:
// normaliser summed in filter order, pi = e / S, cumulative pi in filter
// order, kept probabilities pi / (kept mass) when top-p is on.  se holds the
// numerators e in filter order (LDS, overwritten with pi); s_cx receives the
// cumulative sums (n + 1 entries).  The in-order sums run in one lane over
// LDS -- one add per step -- and everything else across the wave.
// With out.cum the support is written in ascending id order with its
// inclusive cumulative sums in that order (sk, whose keys are consumed by
// then, serves as the id scratch).
__device__ __forceinline__ void finalize_row(uint32_t* sk, const int32_t* sid, double* se, int n,
                                             const FilterParams fp, const SparseOut out, int64_t r, int lane,
                                             double* s_scal, double* s_cx, bool have_full = false,
                                             double s_full = 0.0)
{
    double* oc = out.cum ? out.cum + r * out.cap : nullptr;
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
        if (lane == 0) {
            oid[0] = sid[0];
            op[0] = 1.0;
            if (oc) oc[0] = 1.0;
        }
    } else {
        m = (double)key_float(sk[0]);
        if (have_full) {
            // joint order, summed by the stream itself (relative to the row maximum)
            S = s_full;
        } else if (fp.full_cmax) {
            // joint order: pi takes the full-vocabulary normaliser, combined from
            // the row's exact chunk sums (each relative to its chunk maximum)
            const float* cm = fp.full_cmax + r * fp.full_nc;
            const double* cs = fp.full_csum + r * fp.full_nc;
            const double T = (double)fp.temperature;
            double part = 0.0;
            for (int c = lane; c < fp.full_nc; c += kWave)
                if (cm[c] > -INFINITY) part += cs[c] * exp(((double)cm[c] - m) / T);
            S = wave_sum_f64(part);
        } else {
            if (lane == 0) {
                double acc = 0.0;
#pragma unroll 8
                for (int i = 0; i < n; ++i) acc += se[i];
                s_scal[0] = acc;
            }
            wave_sync();
            S = s_scal[0];
        }
        for (int i = lane; i < n; i += kWave) se[i] = se[i] / S;
        wave_sync();
        int n_keep = n;
        double c = 1.0;
        if (fp.topp_on) {
            // exclusive cumulative pi in filter order (one lane), then the kept
            // prefix: i == 0 or cumulative < top_p (non-decreasing, so a prefix)
            if (lane == 0) {
                double acc = 0.0;
#pragma unroll 8
                for (int i = 0; i < n; ++i) {
                    s_cx[i] = acc;
                    acc += se[i];
                }
                s_cx[n] = acc;
            }
            wave_sync();
            const double p = (double)fp.top_p;
            n_keep = 0;
            for (int base = 0; base < n; base += kWave) {
                const int i = base + lane;
                n_keep += __popcll(__ballot(i < n && (i == 0 || s_cx[i] < p)));
            }
            c = s_cx[n_keep];
        }
        // the kept entries with positive probability: a prefix in filter order
        int npos = 0;
        for (int base = 0; base < n_keep; base += kWave) {
            const int i = base + lane;
            double v = 0.0;
            if (i < n_keep) v = fp.topp_on ? se[i] / c : se[i];
            const bool pos = (i < n_keep) && v > 0.0;
            npos += __popcll(__ballot(pos));
            if (!oc) {
                if (pos) { oid[i] = sid[i]; op[i] = v; }
            } else if (i < n_keep) {
                se[i] = v;
            }
        }
        if (oc) {
            // id order: an entry's position counts the smaller ids among the kept
            int32_t* s_id = reinterpret_cast<int32_t*>(sk);
            wave_sync();
            for (int base = 0; base < npos; base += kWave) {
                const int i = base + lane;
                if (i < npos) {
                    const int32_t id = sid[i];
                    int rank = 0;
                    int j = 0;
                    for (; j + 4 <= npos; j += 4)
                        rank += (sid[j] < id) + (sid[j + 1] < id) + (sid[j + 2] < id) + (sid[j + 3] < id);
                    for (; j < npos; ++j) rank += (sid[j] < id);
                    s_cx[rank] = se[i];
                    s_id[rank] = id;
                }
            }
            wave_sync();
            if (lane == 0) {
                double acc = 0.0;
#pragma unroll 8
                for (int j = 0; j < npos; ++j) {
                    acc += s_cx[j];
                    se[j] = acc;
                }
            }
            wave_sync();
            for (int j = lane; j < npos; j += kWave) {
                oid[j] = s_id[j];
                op[j] = s_cx[j];
                oc[j] = se[j];
            }
        }
        n_out = npos;
    }
    for (int i = (n_out > 0 ? n_out : 0) + lane; i < out.cap; i += kWave) {
        oid[i] = -1;
        op[i] = 0.0;
        if (oc) oc[i] = 0.0;
    }
    if (lane == 0) {
        out.count[r] = n_out;
        if (out.stats) { out.stats[2 * r] = m; out.stats[2 * r + 1] = S; }
    }
}

// A row the top-k path leaves to the dense kernels: its support slots hold
// -1 / 0 (its count and statistics come from the dense kernels).
__device__ __forceinline__ void pad_skipped_row(const SparseOut& out, int64_t r)
{
    for (int i = threadIdx.x; i < out.cap; i += blockDim.x) {
        out.ids[r * out.cap + i] = -1;
        out.probs[r * out.cap + i] = 0.0;
        if (out.cum) out.cum[r * out.cap + i] = 0.0;
    }
}

// ---- top-k stream ------------------------------------------------------------
// Block (r, seg): NW waves stream equal parts of segment seg of row r, each
// keeping candidates in its own LDS buffer behind a rising admission
// threshold; then every wave cuts its buffer to its exact top-k, the NW
// lists are pruned by the best per-wave k-th entry and ranked together.  With
// one segment the block also finalises the row; otherwise it writes the
// segment's sorted top-k for topk_merge_kernel.  Four waves per block, or
// eight when a launch has few segments (most CUs would hold one block or
// none), which halves each wave's range there.
template <bool BF16, bool JOINT, int NW>
__global__ __launch_bounds__(NW * kWave, JOINT ? 3 : 5) void topk_stream_kernel(
    RowSource src, int64_t rows, int64_t N, FilterParams fp_all, SparseOut out, int S,
    uint32_t* part_key, int32_t* part_id, int32_t* part_n, int part_cap, const FilterParams* rowp)
{
    using V = Vec<BF16>;
    constexpr int EPV = V::EPV, ESZ = V::ESZ;
    constexpr int kT = NW * kWave;                     // threads per workgroup
    static_assert(NW == 4 || NW == 8, "four or eight waves per workgroup");
    // 16-byte vectors per lane per iteration and iterations in flight: the
    // joint variant, fp64-bound, keeps four vectors with one iteration ahead
    // so its running sum is rescaled half as often
    constexpr int U = JOINT ? 4 : kStreamVecs;
    constexpr int DEPTH = JOINT ? 2 : kStreamDepth;
    constexpr int kPerIter = U * EPV;                  // logits per lane per iteration
    // a streaming cut must leave room for one whole vector of candidates per lane
    constexpr int kCutLimit = (kCap - kWave * EPV < kCap / 2) ? kCap - kWave * EPV : kCap / 2;
    __shared__ Cand s_buf[NW * kCap];
    __shared__ uint32_t s_sk[kMaxK];
    __shared__ int32_t s_sid[kMaxK];
    __shared__ double s_e[kMaxK];
    __shared__ __align__(16) double s_cx[kMaxK + 1];
    __shared__ double s_scal[1];
    __shared__ uint32_t s_b[NW];
    __shared__ uint32_t s_mx[NW];
    __shared__ int s_ns[NW];
    __shared__ uint32_t s_jm[NW];
    __shared__ double s_js[NW];
    __shared__ double s_exp2[JOINT ? kExp2Entries : 1];
    if constexpr (JOINT) {
        load_exp2_table(s_exp2);
        __syncthreads();
    }

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // segments of one row are consecutive workgroups, so they run together
    // and the dispatcher hands the next row's segments to whichever CUs free up
    const int64_t r = blockIdx.x / S;
    const int seg = (int)(blockIdx.x - r * S);
    const FilterParams fp = rowp ? rowp[r] : fp_all;              // per-row parameters when given
    if (fp.skip_topk) {
        if (S == 1) pad_skipped_row(out, r);
        return;
    }
    const char* row = row_pointer(src, r, N * ESZ);
    if (row == nullptr) {
        if (S == 1 && threadIdx.x == 0) out.count[r] = -1;
        if (S > 1 && threadIdx.x == 0) part_n[r * S + seg] = -1;
        return;
    }
    const RowGeom g = row_geom<BF16>(row, N);
    const int64_t vb = g.nvec * seg / S, ve = g.nvec * (seg + 1) / S;
    const int64_t wb = vb + (ve - vb) * w / NW, we = vb + (ve - vb) * (w + 1) / NW;

    Cand* buf = s_buf + w * kCap;
    const int k = fp.k;
    int cnt = 0;
    // Admission: key(z) > thr_key.  thr is the float with the same meaning for
    // logits (an ordered compare, false for NaN); it starts at -inf, passed in
    // as an argument so the compare is never constant-folded.
    uint32_t thr_key = kKeyNegInf;
    float thr = fp.thr_init;
    // Joint order in one pass (JOINT, whole rows): each lane keeps the running
    // maximum jm of the finite logits it streams and the sum js of
    // exp((z - jm)/T) over them, rescaled when jm rises.
    const bool jrow = JOINT && fp.joint && !fp.greedy;
    const DenseExp jex{ jrow ? 1.4426950408889634074 / (double)fp.temperature : 1.0, s_exp2 };
    float jm = -INFINITY;
    double js = 0.0;
    auto joint_raise = [&](float mx) __attribute__((always_inline)) {
        if (mx > jm) {
            js = (jm > -INFINITY) ? js * jex((double)jm - (double)mx) : 0.0;
            jm = mx;
        }
    };

    auto compact = [&]() __attribute__((always_inline)) {
        if (cnt < k) return;
        uint32_t t;
        cnt = __builtin_amdgcn_readfirstlane(wave_cut<kCapE>(buf, cnt, k, kCutLimit, lane, &t));
        t = __builtin_amdgcn_readfirstlane(t);
        if (t > thr_key) { thr_key = t; thr = thr_float(t); }
    };
    // An early cut while the list is still short (at most kSmallCut entries,
    // read with four slots per lane): the seed threshold admits the upper tail
    // of the first logits seen, and raising it at kSmallCut entries costs a
    // third of a full-buffer cut and usually leaves none to do.  Only for a
    // wave range of at least kSmallCutRange iterations (a short range seldom
    // fills the buffer at all).
    constexpr int kSmallE = 4, kSmallCut = kSmallE * kWave, kSmallCutRange = 16;
    auto small_cut = [&]() __attribute__((always_inline)) {
        uint32_t t;
        cnt = __builtin_amdgcn_readfirstlane(wave_cut<kSmallE>(buf, cnt, k, kSmallCut / 2, lane, &t));
        t = __builtin_amdgcn_readfirstlane(t);
        if (t > thr_key) { thr_key = t; thr = thr_float(t); }
    };
    auto scalar_part = [&](int64_t beg, int64_t n) __attribute__((always_inline)) {   // n <= 64, ids increase with lane
        if (cnt > kCap - kWave) compact();
        float v = 0.0f;
        uint32_t key = 0;
        if (lane < n) {
            v = load_scalar<BF16>(row, beg + lane);
            key = float_key(v);
        }
        if constexpr (JOINT) {
            if (jrow && lane < n && finite_f32(v)) {
                joint_raise(v);
                js += jex((double)v - (double)jm);
            }
        }
        const bool pass = key_admits(key, thr_key);
        const uint64_t m = __ballot(pass);
        if (pass) {
            const int pos = cnt + __popcll(m & lanes_below(lane));
            buf[pos] = make_uint2(__float_as_uint(v), (uint32_t)(beg + lane));
        }
        cnt += __popcll(m);
    };

    if (seg == 0 && w == 0 && g.head > 0) scalar_part(0, g.head);

    const typename V::T* body = reinterpret_cast<const typename V::T*>(row + g.head * ESZ);
    // Fallback for an iteration whose candidates cannot all fit the buffer even
    // after a cut (only while the threshold is still low): vector by vector,
    // re-reading each vector, with a cut whenever the buffer fills.
    auto reload_path = [&](int64_t v0) __attribute__((always_inline)) {
#pragma unroll 1
        for (int u = 0; u < U; ++u) {
            const int64_t vbase = v0 + u * kWave;
            if (vbase >= we) break;
            const int64_t vl = vbase + lane;
            const typename V::T xv = (vl < we) ? body[vl] : V::neg_inf();
            if (cnt > kCap - kWave * EPV) compact();
            const uint32_t id0 = (uint32_t)(g.head + vl * EPV);
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const float z = V::get(xv, e);
                const bool pass = z > thr;
                const uint64_t m = __ballot(pass);
                if (m) {
                    if (pass) {
                        const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)cnt));
                        buf[pos] = make_uint2(__float_as_uint(z), id0 + e);
                    }
                    cnt += __popcll(m);
                }
            }
        }
    };
    // One iteration: U vectors per lane (vector v0 + u*64 + lane), already in
    // x.  Each logit's test is one compare; its result is both the lane's
    // predicate and, as a wave mask in scalar registers, the source of counts,
    // skips and write positions.
    auto process = [&](const typename V::T (&x)[U], int64_t v0) __attribute__((always_inline)) {
        if constexpr (JOINT) {
            if (jrow) {
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < kPerIter; ++i) {
                    const float z = V::get(x[i / EPV], i % EPV);
                    if (finite_f32(z)) mx = fmaxf(mx, z);
                }
                joint_raise(mx);
                double acc = 0.0;
#pragma unroll
                for (int i = 0; i < kPerIter; ++i) {
                    const float z = V::get(x[i / EPV], i % EPV);
                    if (finite_f32(z)) acc += jex((double)z - (double)jm);
                }
                js += acc;
            }
        }
        bool pass[kPerIter];
        uint64_t m[kPerIter];
        uint64_t any = 0;
#pragma unroll
        for (int i = 0; i < kPerIter; ++i) {
            pass[i] = V::get(x[i / EPV], i % EPV) > thr;
            m[i] = __ballot(pass[i]);
            any |= m[i];
        }
        if (any == 0) return;
        int total = 0;
#pragma unroll
        for (int i = 0; i < kPerIter; ++i) total += __popcll(m[i]);
        if (k <= kSmallCut / 4 && cnt >= 2 * k && cnt <= kSmallCut && cnt + total > kSmallCut &&
            we - wb >= (int64_t)kSmallCutRange * U * kWave) {
            small_cut();
            total = 0;
#pragma unroll
            for (int i = 0; i < kPerIter; ++i) {
                pass[i] = V::get(x[i / EPV], i % EPV) > thr;
                m[i] = __ballot(pass[i]);
                total += __popcll(m[i]);
            }
        }
        if (cnt + total > kCap) {
            compact();
            total = 0;
#pragma unroll
            for (int i = 0; i < kPerIter; ++i) {
                pass[i] = V::get(x[i / EPV], i % EPV) > thr;
                m[i] = __ballot(pass[i]);
                total += __popcll(m[i]);
            }
            if (cnt + total > kCap) { reload_path(v0); return; }
        }
        const uint32_t id0 = (uint32_t)(g.head + (v0 + lane) * EPV);
#pragma unroll
        for (int i = 0; i < kPerIter; ++i) {
            if (m[i]) {
                if (pass[i]) {
                    const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m[i] >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m[i], (uint32_t)cnt));
                    buf[pos] = make_uint2(__float_as_uint(V::get(x[i / EPV], i % EPV)),
                                          id0 + (uint32_t)((i / EPV) * kWave * EPV + (i % EPV)));
                }
                cnt += __popcll(m[i]);
            }
        }
    };

    // Whole iterations, DEPTH - 1 of them loaded ahead of the one being
    // processed: two vectors per lane per iteration with two iterations ahead
    // keep more loads in flight per byte of registers than four vectors with
    // one ahead (a read-only sweep of the same 1088-row split: 104.7 against
    // 112.8 us for 661 MB).
    constexpr int64_t kStep = (int64_t)U * kWave;
    const int64_t nfull = (we - wb) / kStep;
    typename V::T xr[DEPTH][U];
    // Iteration i's vectors.  Past the last whole iteration the loads only keep
    // the pipeline's shape: on 4-byte rows one vector per u for every lane (a
    // few cache lines), on 2-byte rows a re-read of the last iteration
    // (measured faster).
    auto load_iter = [&](int64_t i, typename V::T (&x)[U]) __attribute__((always_inline)) {
        const bool real = i < nfull;
        const typename V::T* p = body + wb + (real ? i : nfull - 1) * kStep + ((real || BF16) ? lane : 0);
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = V::load_stream(p + u * kWave);
    };
    if (nfull > 0) {
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) load_iter(d, xr[d]);
        if (cnt == 0) {
            // Seed the threshold from the first two iterations (only the first
            // when there is no second: a shape-only load holds one lane's data).
            // Each lane keeps its P largest logits (NaN taken as -inf through
            // the maximum with thr_init, which is -inf); the k-th largest of
            // those 64 P values, truncated to its 16-bit key bin, has at least
            // k logits at or above it, all admitted below.  P = 2 for k <= 128
            // and 4 up to k = 256: several per lane put the seed near the k-th
            // largest of all 128 * U * EPV logits read, where the largest per
            // lane alone sat several times lower; four cost more than they save
            // for the smaller k.
            const float ninf = fp.thr_init;
            float m1 = ninf, m2 = ninf, m3 = ninf, m4 = ninf;
            auto seed = [&](auto four) __attribute__((always_inline)) {
                constexpr bool F = decltype(four)::value;
                auto take = [&](float z) __attribute__((always_inline)) {
                    z = fmaxf(z, ninf);
                    if constexpr (F) {
                        m4 = fmaxf(m4, fminf(m3, z));
                        m3 = fmaxf(m3, fminf(m2, z));
                    }
                    m2 = fmaxf(m2, fminf(m1, z));
                    m1 = fmaxf(m1, z);
                };
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        take(V::get(xr[0][u], e));
                        if (DEPTH > 2 && nfull > 1) take(V::get(xr[1][u], e));
                    }
            };
            auto valid = [](uint32_t x) __attribute__((always_inline)) {
                return (x <= kKeyPosInf && x > kKeyNegInf) ? x : kKeyNegInf;
            };
            uint32_t t0;
            if (k <= 2 * kWave) {
                seed(std::false_type());
                t0 = wave_kth_largest_of_lane_keys<2>(valid(float_key(m1)), valid(float_key(m2)), 0u, 0u, k);
            } else {
                seed(std::true_type());
                t0 = wave_kth_largest_of_lane_keys<4>(valid(float_key(m1)), valid(float_key(m2)),
                                                      valid(float_key(m3)), valid(float_key(m4)), k);
            }
            if (t0 > kKeyNegInf + 1u) { thr_key = t0 - 1u; thr = thr_float(thr_key); }
        }
    }
    for (int64_t it = 0; it < nfull; ++it) {
        load_iter(it + DEPTH - 1, xr[DEPTH - 1]);
        process(xr[0], wb + it * kStep);
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d)
#pragma unroll
            for (int u = 0; u < U; ++u) xr[d][u] = xr[d + 1][u];
    }
    typename V::T xc[U];
    {   // last partial iteration
        const int64_t v0 = wb + nfull * kStep;
        if (v0 < we) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t v = v0 + u * kWave + lane;
                xc[u] = (v < we) ? V::load_stream(body + v) : V::neg_inf();
            }
            process(xc, v0);
        }
    }

    if (seg == S - 1 && w == NW - 1 && g.tail_beg < N) scalar_part(g.tail_beg, N - g.tail_beg);

    // Bound: with quota q = ceil(k/NW), each wave finds a key b with at least q
    // of its entries at or above it, so the smallest of the NW waves' bounds
    // has at least k: the block's k-th entry lies at or above it.  Without q
    // entries in every wave there is no bound (B = 0).  For small q, b is the
    // q-th largest of the lane maxima (truncated to its 16-bit key bin); a
    // larger q would push that down to the smallest lane maximum, and the
    // block would rank several times k entries, so there b is the wave's own
    // q-th largest key (truncated to 24 bits).
    const int quota = (k + NW - 1) / NW;
    // the wave's candidates, read once into registers as (key, id); padding
    // slots hold key 0, below every admitted key
    RegList<kCapE> L;
    reg_load(L, buf, cnt, lane);
    uint32_t lmax = 0;
#pragma unroll
    for (int q = 0; q < kCapE; ++q) lmax = L.kv[q] > lmax ? L.kv[q] : lmax;
    uint32_t b = 0;
    if (cnt >= quota && quota > kWave / 2) {
        b = reg_kth_key(L, quota, 8);
    } else if (cnt >= quota) {
        // largest 16-bit prefix t with at least quota lane maxima >= t
        for (int bit = 31; bit >= 16; --bit) {
            const uint32_t cand = b | (1u << bit);
            if (__popcll(__ballot(lmax >= cand)) >= quota) b = cand;
        }
    }
    if constexpr (JOINT) {
        if (jrow) {    // the wave's maximum and sum relative to it
            const uint32_t kw = wave_ext_u32<true>(float_key(jm));
            const float mw = key_float(kw);
            double part = (jm > -INFINITY) ? js * jex((double)jm - (double)mw) : 0.0;
            part = wave_sum_f64(part);
            if (lane == 0) { s_jm[w] = kw; s_js[w] = part; }
        }
    }
    if (lane == 0) s_b[w] = b;
    __syncthreads();
    uint32_t B = s_b[0];
#pragma unroll
    for (int o = 1; o < NW; ++o) B = s_b[o] < B ? s_b[o] : B;
    // this wave's entries with key >= B, compacted in place as (key, id)
    int ns = 0;
#pragma unroll
    for (int q = 0; q < kCapE; ++q) {
        if (q * kWave >= cnt) break;
        const bool keep = L.kv[q] != 0u && L.kv[q] >= B;
        const uint64_t mk = __ballot(keep);
        if (keep)
            buf[(int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, (uint32_t)ns))] =
                make_uint2(L.kv[q], (uint32_t)L.iv[q]);
        ns += __popcll(mk);
    }
    const uint32_t mx = wave_ext_u32<true>(lmax);
    if (lane == 0) { s_ns[w] = ns; s_mx[w] = mx; }
    __syncthreads();
    // softmax numerators are formed during the rank when this block finalises
    uint32_t top = s_mx[0];
#pragma unroll
    for (int o = 1; o < NW; ++o) top = s_mx[o] > top ? s_mx[o] : top;
    const bool want_e = (S == 1) && !fp.greedy;
    // The rank and the one-wave finalisation start at a different wave in each
    // block, so co-resident blocks spread these short serial phases over the
    // four SIMDs instead of stacking them on one.
    const int rot = (int)(blockIdx.x & (NW - 1));
    const int trot = (int)((threadIdx.x + rot * kWave) & (kT - 1));
    const int n = block_rank_topk<NW>(s_buf, kCap, s_ns, k, s_sk, s_sid, want_e ? s_e : nullptr,
                                      (double)key_float(top), (double)fp.temperature, trot, kT,
                                      reinterpret_cast<uint64_t*>(s_cx));
    __syncthreads();
    if (S == 1) {
        if (w == rot) {
            double s_full = 0.0;
            if constexpr (JOINT) {
                if (jrow) {    // the row's full normaliser relative to its maximum
                    uint32_t km = s_jm[0];
#pragma unroll
                    for (int o = 1; o < NW; ++o) km = s_jm[o] > km ? s_jm[o] : km;
                    const double mr = (double)key_float(km);
#pragma unroll
                    for (int o = 0; o < NW; ++o)
                        if (s_jm[o] > kKeyNegInf) s_full += s_js[o] * jex((double)key_float(s_jm[o]) - mr);
                }
            }
            finalize_row(s_sk, s_sid, s_e, n, fp, out, r, lane, s_scal, s_cx, jrow, s_full);
        }
    } else {
        const int64_t base = (r * S + seg) * (int64_t)part_cap;
        for (int i = threadIdx.x; i < n; i += kT) {
            part_key[base + i] = s_sk[i];
            part_id[base + i] = s_sid[i];
        }
        if (threadIdx.x == 0) part_n[r * S + seg] = n;
    }
}

// One workgroup per row: the S segment lists (each sorted, at most k entries)
// are pruned by the best full list's k-th entry, ranked together and
// finalised.  Every global read of the row -- its parameters, whether it is
// present, the segment counts and all S lists (part_cap entries each, the
// largest k) -- is issued before any is used, so the row pays one memory
// round trip before its LDS work.
constexpr int kMergePer = kMergeCap / kThreads;     // list entries per thread
static_assert(kMaxSegments <= kWave, "the merge reduces the per-list bounds in one wave");
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(
    RowSource src, int64_t rows, FilterParams fp_all, SparseOut out, int S,
    const uint32_t* part_key, const int32_t* part_id, const int32_t* part_n, int part_cap,
    const FilterParams* rowp)
{
    __shared__ uint2 s_cand[kMergeCap];
    __shared__ uint32_t s_sk[kMaxK];
    __shared__ int32_t s_sid[kMaxK];
    __shared__ double s_e[kMaxK];
    __shared__ __align__(16) double s_cx[kMaxK + 1];
    __shared__ double s_scal[1];
    __shared__ int s_segn[kMaxSegments];
    __shared__ uint32_t s_first[kMaxSegments];     // per list: its first key
    __shared__ uint64_t s_kth[kMaxSegments];       // per list: order key of entry k - 1
    __shared__ uint64_t s_qth[kMaxSegments];       // per list: order key of entry quota - 1
    __shared__ uint64_t s_bound;
    __shared__ uint32_t s_top;
    __shared__ int s_n;

    const int lane = lane_id();
    const int64_t r = blockIdx.x;
    if (r >= rows) return;
    const int tid = (int)threadIdx.x;
    const int total = S * part_cap;              // <= kMergeCap (topk_segments)
    const int64_t lbase = r * S * (int64_t)part_cap;
    uint32_t ck[kMergePer];
    int32_t ci[kMergePer];
#pragma unroll
    for (int j = 0; j < kMergePer; ++j) {
        const int g = j * kThreads + tid;
        ck[j] = 0u;
        ci[j] = 0;
        if (g < total) {
            ck[j] = part_key[lbase + g];
            ci[j] = part_id[lbase + g];
        }
    }
    const int segn = tid < S ? part_n[r * S + tid] : 0;
    const FilterParams fp = rowp ? rowp[r] : fp_all;
    const bool present = row_pointer(src, r, 1) != nullptr;
    if (fp.skip_topk) {
        pad_skipped_row(out, r);
        return;
    }
    if (!present) {
        if (tid == 0) out.count[r] = -1;
        return;
    }
    const int k = fp.k;
    // Per list: its count, its first key, and two lower bounds on the row's
    // k-th entry -- the k-th entry of a full list, and (quota q = ceil(k/S)) the
    // smallest of the lists' q-th entries, valid when every list holds q.
    const int quota = (k + S - 1) / S;
    if (tid < S) s_segn[tid] = segn;
#pragma unroll
    for (int j = 0; j < kMergePer; ++j) {
        const int g = j * kThreads + tid;
        if (g < total) {
            const int sg = g / part_cap, i = g - sg * part_cap;
            if (i == 0) s_first[sg] = ck[j];
            if (i == k - 1) s_kth[sg] = order_key(ck[j], ci[j]);
            if (i == quota - 1) s_qth[sg] = order_key(ck[j], ci[j]);
        }
    }
    __syncthreads();
    if (tid < kWave) {          // S <= kMaxSegments <= one wave
        uint64_t p = 0, pq = ~0ull;
        uint32_t top = 0;
        if (lane < S) {
            const int ns = s_segn[lane];
            if (ns > 0) top = s_first[lane];    // lists are sorted
            if (ns == k) p = s_kth[lane];
            pq = (ns >= quota) ? s_qth[lane] : 0ull;
        }
        // DPP reductions (the wave_ext_u32 pattern): the results land in lane 63
        auto step = [&](auto ctrl, auto rmask) __attribute__((always_inline)) {
            constexpr int C = decltype(ctrl)::value, M = decltype(rmask)::value;
            const uint64_t po = dpp_u64<C, M>(p, p), qo = dpp_u64<C, M>(pq, pq);
            const uint32_t to = (uint32_t)__builtin_amdgcn_update_dpp((int)top, (int)top, C, M, 0xF, false);
            p = po > p ? po : p;
            pq = qo < pq ? qo : pq;
            top = to > top ? to : top;
        };
        step(std::integral_constant<int, 0xB1>(), std::integral_constant<int, 0xF>());
        step(std::integral_constant<int, 0x4E>(), std::integral_constant<int, 0xF>());
        step(std::integral_constant<int, 0x141>(), std::integral_constant<int, 0xF>());
        step(std::integral_constant<int, 0x140>(), std::integral_constant<int, 0xF>());
        step(std::integral_constant<int, 0x142>(), std::integral_constant<int, 0xA>());
        step(std::integral_constant<int, 0x143>(), std::integral_constant<int, 0xC>());
        if (lane == kWave - 1) {
            s_bound = pq > p ? pq : p;
            s_top = top;
            s_n = 0;
        }
    }
    __syncthreads();
    const uint64_t pstar = s_bound;
    const uint32_t top = s_top;
    // candidates at or above the bound, from the registers, compacted to LDS
#pragma unroll
    for (int j = 0; j < kMergePer; ++j) {
        if (j * kThreads >= total) break;
        const int g = j * kThreads + tid;
        bool keep = false;
        if (g < total) {
            const int sg = g / part_cap, i = g - sg * part_cap;
            keep = i < s_segn[sg] && i < k && order_key(ck[j], ci[j]) >= pstar;
        }
        const uint64_t m = __ballot(keep);
        int pos0 = 0;
        if (lane == 0 && m) pos0 = atomicAdd(&s_n, __popcll(m));
        pos0 = __builtin_amdgcn_readlane(pos0, 0);
        if (keep) s_cand[pos0 + __popcll(m & lanes_below(lane))] = make_uint2(ck[j], (uint32_t)ci[j]);
    }
    __syncthreads();
    const int n = block_rank_topk<1>(s_cand, 0, &s_n, k, s_sk, s_sid, fp.greedy ? nullptr : s_e,
                                     (double)key_float(top), (double)fp.temperature, tid, kThreads,
                                     reinterpret_cast<uint64_t*>(s_cx));
    __syncthreads();
    if (tid < kWave) finalize_row(s_sk, s_sid, s_e, n, fp, out, r, lane, s_scal, s_cx);
}

// ---- dense chunk statistics --------------------------------------------------
template <bool BF16, bool COUNT>
__global__ __launch_bounds__(kThreads, 5) void dense_chunk_kernel(
    RowSource src, int64_t rows, int64_t N, double log2e_over_T, int64_t exact_rows, DenseChunks dc,
    const FilterParams* rowp, int select)
{
    using V = Vec<BF16>;
    constexpr int EPV = V::EPV, ESZ = V::ESZ;
    constexpr int PER_LANE = kDenseChunk / kWave;          // 32 logits per lane
    constexpr int NV = PER_LANE / EPV;                      // vectors per lane
    __shared__ double s_exp2[kExp2Entries];
    // the samplers' exact-row list counters start every call at 0
    if (dc.xcount != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 3) dc.xcount[threadIdx.x] = 0u;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t r = blockIdx.x;
    // rows below exact_rows take the exact (fp64-bound) sums, the rest the fast
    // ones, which need no table
    bool exact = r < exact_rows;
    if (rowp != nullptr) {
        // per-row parameters: only the rows the pass is for, each at its own
        // temperature; joint-order and nucleus rows are cut on these sums
        const float* fc = rowp[r].full_cmax;
        const int32_t dn = rowp[r].dense;
        if (select == kChunkJointRows ? fc == nullptr : dn == kRowTopK) return;
        log2e_over_T = 1.4426950408889634074 / (double)rowp[r].temperature;
        exact = exact || fc != nullptr || dn == kRowNucleus;
    }
    const int nc = dc.nchunks;
    // a row's chunks are dealt over gridDim.y workgroups (more than one when
    // there are few rows), round robin over all their waves
    const int c0 = (int)blockIdx.y * kWaves + w;
    const int cstep = (int)gridDim.y * kWaves;
    if (exact) load_exp2_table(s_exp2);
    __syncthreads();
    const char* row = row_pointer(src, r, N * ESZ);
    if (row == nullptr) {
        for (int c = c0; c < nc; c += cstep)
            if (lane == 0) {
                const int64_t slot = r * nc + c;
                dc.cmax[slot] = -INFINITY; dc.csum[slot] = 0.0;
                if (COUNT) dc.ccount[slot] = 0;
                if (dc.cerr) dc.cerr[slot] = 0.0f;
            }
        return;
    }
    const DenseExp ex{ log2e_over_T, s_exp2 };
    // whole chunks of a 16-byte aligned row are loaded as vectors, the next
    // chunk of this wave while the current one is summed
    const bool aligned = (((uintptr_t)row) & 15u) == 0;
    const int nvec_chunks = aligned ? (int)(N / kDenseChunk) : 0;
    // vectors of chunk c (all lanes read one vector per j when `shape` only:
    // a load that keeps the pipeline's shape at its end)
    auto load_vec = [&](int c, typename V::T (&v)[NV], bool shape) __attribute__((always_inline)) {
        const typename V::T* p = reinterpret_cast<const typename V::T*>(row + (int64_t)c * kDenseChunk * ESZ) +
                                 (shape ? 0 : lane);
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] = V::load_stream(p + j * kWave);
    };
    // statistics of one chunk held as x[PER_LANE] (element (j*64 + lane)*EPV + e
    // at x[j*EPV + e])
    const float log2e_over_T32 = (float)log2e_over_T;
    auto chunk_stats = [&](int c, const float (&x)[PER_LANE]) __attribute__((always_inline)) {
        float mx;
        double s;
        uint32_t cntf;
        float err = 0.0f;
        if (exact) chunk_stats_exact<COUNT>(x, ex, &mx, &s, &cntf);
        else chunk_stats_fast<COUNT>(x, log2e_over_T32, &mx, &s, &cntf, &err);
        if (lane == 0) {
            const int64_t slot = r * nc + c;
            dc.cmax[slot] = mx;
            dc.csum[slot] = (mx < INFINITY) ? s : NAN;
            if (COUNT) dc.ccount[slot] = (int32_t)cntf;
            if (dc.cerr) dc.cerr[slot] = err;
        }
    };
    int c = c0;
    if (c < nvec_chunks) {
        typename V::T cur[NV], nxt[NV];
        load_vec(c, cur, false);
        for (;;) {
            const int cn = c + cstep;
            const bool more = cn < nvec_chunks;
            load_vec(more ? cn : c, nxt, !more);
            float x[PER_LANE];
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int e = 0; e < EPV; ++e) x[j * EPV + e] = V::get(cur[j], e);
            chunk_stats(c, x);
            c = cn;
            if (!more) break;
#pragma unroll
            for (int j = 0; j < NV; ++j) cur[j] = nxt[j];
        }
    }
    // remaining chunks (ragged tail, or a row off 16-byte alignment) element by
    // element, element i of the chunk in lane i % 64: one pass for the maximum,
    // one (reloading) for the count and the sum, in loops that keep this rare
    // path from setting the kernel's register count
    for (; c < nc; c += cstep) {
        const int64_t beg = (int64_t)c * kDenseChunk;
        const int n = (int)((N - beg < kDenseChunk) ? (N - beg) : kDenseChunk);
        const char* base = row + beg * ESZ;
        float mx = -INFINITY;
#pragma unroll 1
        for (int i = lane; i < n; i += kWave) mx = fmaxf(mx, load_scalar<BF16>(base, i));
        mx = wave_max_f32_lds(mx);
        double sum = 0.0, ty = 0.0;
        uint32_t cntf = 0;
        if (mx > -INFINITY && mx < INFINITY) {
            const double md = (double)mx;
#pragma unroll 1
            for (int i0 = 0; i0 < n; i0 += kWave) {
                const int i = i0 + lane;
                const float v = i < n ? load_scalar<BF16>(base, i) : -INFINITY;
                if (COUNT) cntf += (uint32_t)__popcll(__ballot(finite_f32(v)));
                if (i < n) {
                    // as in the whole-chunk sums: NaN and -inf add a vanishing term
                    if (exact) {
                        sum += ex((double)v - md);
                    } else {
                        const float y = fmaxf((v - mx) * log2e_over_T32, -200.0f);
                        const float t = __builtin_amdgcn_exp2f(y);
                        sum += (double)t;
                        ty += (double)t * (double)y;
                    }
                }
            }
        }
        sum = wave_sum_f64_lds(sum);
        ty = wave_sum_f64_lds(ty);
        if (lane == 0) {
            const int64_t slot = r * nc + c;
            dc.cmax[slot] = mx;
            dc.csum[slot] = (mx < INFINITY) ? sum : NAN;
            if (COUNT) dc.ccount[slot] = (int32_t)cntf;
            if (dc.cerr)
                dc.cerr[slot] = exact ? 0.0f : (float)((1.0 + 2e-3) * (kFastExpRel * sum - kFastArgRel * ty) + 0x1p-114);
        }
    }
}

// Row maximum and normaliser from the chunk statistics (uno_filter, dense mode).
__global__ void dense_row_stats_kernel(int64_t rows, double inv_T, DenseChunks dc, int32_t* out_count,
                                       double* out_stats, const FilterParams* rowp)
{
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    if (rowp != nullptr) {
        if (rowp[r].dense != kRowFull) return;
        inv_T = 1.0 / (double)rowp[r].temperature;
    }
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
    // About kSegmentTarget workgroups: one full round over the chip, all
    // resident at once.  More segments would balance CUs that stream at
    // different rates, but each segment pays a serial epilogue and a split row
    // a merge, which cost more than the balance gains on 151936-logit rows.
    // A segment keeps >= 16384 logits (each wave streams several iterations)
    // and the merged candidate list fits one merge workgroup.
    int64_t S = (kSegmentTarget + rows - 1) / rows;
    const int64_t by_len = vocab / 16384;
    if (S > by_len) S = by_len;
    const int64_t by_merge = kMergeCap / (k > 0 ? k : 1);
    if (S > by_merge) S = by_merge;
    if (S > kMaxSegments) S = kMaxSegments;
    if (S < 1) S = 1;
    return (int)S;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// One workgroup per request of the launch: request first + blockIdx.x gets the
// set a.p[blockIdx.x] on each of its rows (the row layout of map).
__global__ __launch_bounds__(kThreads) void expand_params_kernel(ParamArgs a, int64_t first, RowMap map,
                                                                FilterParams* out)
{
    const int64_t q = first + blockIdx.x;
    const FilterParams p = a.p[blockIdx.x];
    if (map.kind == 0) {
        if (threadIdx.x == 0) out[q] = p;
    } else if (map.kind == 1) {
        const int n = 2 * map.B + 1;
        for (int j = threadIdx.x; j < n; j += kThreads) {
            const int64_t row = j < map.B ? q * map.B + j : map.batch * map.B + q * (map.B + 1) + (j - map.B);
            out[row] = p;
        }
    } else {
        for (int j = threadIdx.x; j < map.rows_per_req; j += kThreads) out[q * map.rows_per_req + j] = p;
    }
}

hipError_t launch_expand_params(const ParamArgs& a, int64_t first, int n, const RowMap& map, FilterParams* out,
                                hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    expand_params_kernel<<<dim3((unsigned)n), kThreads, 0, stream>>>(a, first, map, out);
    return hipGetLastError();
}

hipError_t launch_topk_filter(const RowSource& src, int64_t rows, int64_t vocab, bool bf16,
                              const FilterParams& fp, const SparseOut& out, int S,
                              uint32_t* part_key, int32_t* part_id, int32_t* part_n, int part_cap,
                              const FilterParams* rowp, bool joint_sums, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    if (joint_sums && S != 1) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(rows * S));
    // eight waves per segment when the launch would leave most CUs idle
    const bool wide = !joint_sums && rows * S < kWideBelow;
    if (joint_sums) {
        if (bf16)
            topk_stream_kernel<true, true, 4><<<grid, 4 * kWave, 0, stream>>>(src, rows, vocab, fp, out, S, part_key,
                                                                              part_id, part_n, part_cap, rowp);
        else
            topk_stream_kernel<false, true, 4><<<grid, 4 * kWave, 0, stream>>>(src, rows, vocab, fp, out, S, part_key,
                                                                               part_id, part_n, part_cap, rowp);
    } else if (wide) {
        if (bf16)
            topk_stream_kernel<true, false, 8><<<grid, 8 * kWave, 0, stream>>>(src, rows, vocab, fp, out, S, part_key,
                                                                               part_id, part_n, part_cap, rowp);
        else
            topk_stream_kernel<false, false, 8><<<grid, 8 * kWave, 0, stream>>>(src, rows, vocab, fp, out, S,
                                                                                part_key, part_id, part_n, part_cap,
                                                                                rowp);
    } else {
        if (bf16)
            topk_stream_kernel<true, false, 4><<<grid, 4 * kWave, 0, stream>>>(src, rows, vocab, fp, out, S, part_key,
                                                                               part_id, part_n, part_cap, rowp);
        else
            topk_stream_kernel<false, false, 4><<<grid, 4 * kWave, 0, stream>>>(src, rows, vocab, fp, out, S,
                                                                                part_key, part_id, part_n, part_cap,
                                                                                rowp);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    topk_merge_kernel<<<dim3((unsigned)rows), kThreads, 0, stream>>>(src, rows, fp, out, S, part_key,
                                                                   part_id, part_n, part_cap, rowp);
    return hipGetLastError();
}

hipError_t launch_dense_chunks(const RowSource& src, int64_t rows, int64_t vocab, bool bf16,
                               float temperature, const DenseChunks& dc, int64_t exact_rows, hipStream_t stream,
                               const FilterParams* rowp, int select, int64_t active_rows)
{
    if (rows == 0) return hipSuccess;
    const double c = 1.4426950408889634074 / (double)temperature;
    // about two rounds of workgroups over the chip at least: few rows (or few
    // selected rows) are split over several workgroups each (at most one
    // chunk per wave)
    const int64_t per_row_max = (dc.nchunks + kWaves - 1) / kWaves;
    const int64_t busy = (active_rows >= 0 && active_rows < rows) ? (active_rows > 0 ? active_rows : 1) : rows;
    int64_t g = (2048 + busy - 1) / busy;
    if (g > per_row_max) g = per_row_max;
    if (g < 1) g = 1;
    dim3 grid((unsigned)rows, (unsigned)g);
    const bool counts = dc.ccount != nullptr;
    if (bf16 && counts)
        dense_chunk_kernel<true, true><<<grid, kThreads, 0, stream>>>(src, rows, vocab, c, exact_rows, dc, rowp,
                                                                       select);
    else if (bf16)
        dense_chunk_kernel<true, false><<<grid, kThreads, 0, stream>>>(src, rows, vocab, c, exact_rows, dc, rowp,
                                                                        select);
    else if (counts)
        dense_chunk_kernel<false, true><<<grid, kThreads, 0, stream>>>(src, rows, vocab, c, exact_rows, dc, rowp,
                                                                        select);
    else
        dense_chunk_kernel<false, false><<<grid, kThreads, 0, stream>>>(src, rows, vocab, c, exact_rows, dc, rowp,
                                                                         select);
    return hipGetLastError();
}

hipError_t launch_dense_row_stats(int64_t rows, float temperature, const DenseChunks& dc,
                                  int32_t* out_count, double* out_stats, hipStream_t stream,
                                  const FilterParams* rowp)
{
    if (rows == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((rows + 255) / 256);
    dense_row_stats_kernel<<<blocks, 256, 0, stream>>>(rows, 1.0 / (double)temperature, dc, out_count,
                                                       out_stats, rowp);
    return hipGetLastError();
}

}  // namespace uno
