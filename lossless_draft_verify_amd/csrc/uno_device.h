// uno_device.h -- device helpers shared by the UNO sampling kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uno_internal.h"

namespace uno {

constexpr int kWave = 64;

// Wave-level ordering point for LDS traffic between lanes of one wave.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint64_t lanes_below(int lane)
{
    return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// Order-preserving unsigned key of a float: a > b (as floats, -0 == +0) iff
// key(a) > key(b).  -0 is folded onto +0 first.  NaN never reaches a key.
__device__ __forceinline__ uint32_t float_key(float v)
{
    const uint32_t b = __float_as_uint(v + 0.0f);
    return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// 64-bit order key of (logit key, id): larger keys first, then smaller ids --
// the filter order (z desc, id asc) as one unsigned compare.
__device__ __forceinline__ uint64_t order_key(uint32_t key, int32_t id)
{
    return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)id);
}

constexpr uint32_t kKeyPosInf = 0xFF800000u;   // float_key(+inf)
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;   // float_key(-inf)

// Predicates that must treat NaN exactly are integer tests on the bit pattern
// or the key: float compares feeding a ballot are not lowered consistently
// for NaN operands.
// Admission test on keys: above `thr_key` and not NaN (NaN keys lie above
// +inf or below -inf).
__device__ __forceinline__ bool key_admits(uint32_t key, uint32_t thr_key)
{
    return (key > thr_key) & (key <= kKeyPosInf);
}

// Finite (neither NaN nor +-inf).
__device__ __forceinline__ bool finite_f32(float v)
{
    return (__float_as_uint(v) & 0x7FFFFFFFu) < 0x7F800000u;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Philox4x32-10, Salmon et al. (SC'11): 10 rounds, key bumped by the Weyl
// constants between rounds.  Counter (c0..c3), key (k0, k1).
struct Philox4 { uint32_t w[4]; };

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                  uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    Philox4 o;
    o.w[0] = c0; o.w[1] = c1; o.w[2] = c2; o.w[3] = c3;
    return o;
}

// Uniform in [0, 1) from one Philox word (exact in double).
__device__ __forceinline__ double unit_uniform(uint32_t w) { return (double)w * 0x1p-32; }

// The four uniforms of draw (request, position) at cycle `offset`.
struct Draw { double u[4]; };

__device__ __forceinline__ Draw uno_draw(uint64_t seed, uint32_t req, uint32_t pos, uint64_t offset)
{
    const Philox4 p = philox4x32_10(req, pos, (uint32_t)offset, (uint32_t)(offset >> 32),
                                    (uint32_t)seed, (uint32_t)(seed >> 32));
    Draw d;
#pragma unroll
    for (int i = 0; i < 4; ++i) d.u[i] = unit_uniform(p.w[i]);
    return d;
}

// ---- wave reductions --------------------------------------------------------
// All on the VALU's DPP lane moves (no LDS round trips): within each 16-lane
// row first, then across rows by broadcasting lane 15 of a row into the next
// row and lane 31 into rows 2-3.  DPP controls: quad_perm [1,0,3,2] 0xB1,
// [2,3,0,1] 0x4E; row_shr:n 0x110+n; row_mirror 0x140; row_half_mirror 0x141;
// row_bcast:15 0x142; row_bcast:31 0x143.  A lane whose row the row mask
// leaves out, or whose row_shr source lies before its row, receives `old`.

// Value of lane l (l uniform).
__device__ __forceinline__ double readlane_f64(double v, int l)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ int lane_value(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ double lane_value(double v, int l) { return readlane_f64(v, l); }

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v, double old)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v), o = (uint64_t)__double_as_longlong(old);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)o, (int)(uint32_t)b, CTRL, ROW_MASK, 0xF,
                                                              false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(o >> 32), (int)(uint32_t)(b >> 32), CTRL,
                                                              ROW_MASK, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v, uint64_t old)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)old, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF,
                                                              false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(old >> 32), (int)(uint32_t)(v >> 32), CTRL,
                                                              ROW_MASK, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v, float old)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xF,
                                                      false));
}

// Inclusive prefix sum over the wave's lanes (in lane order).
__device__ __forceinline__ double wave_incl_scan_f64(double v, int lane)
{
    (void)lane;
    v += dpp_f64<0x111>(v, 0.0);
    v += dpp_f64<0x112>(v, 0.0);
    v += dpp_f64<0x114>(v, 0.0);
    v += dpp_f64<0x118>(v, 0.0);
    v += dpp_f64<0x142, 0xA>(v, 0.0);
    v += dpp_f64<0x143, 0xC>(v, 0.0);
    return v;
}

// Sum over the wave, returned to every lane.
__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_f64<0xB1>(v, 0.0);
    v += dpp_f64<0x4E>(v, 0.0);
    v += dpp_f64<0x141>(v, 0.0);
    v += dpp_f64<0x140>(v, 0.0);
    v += dpp_f64<0x142, 0xA>(v, 0.0);
    v += dpp_f64<0x143, 0xC>(v, 0.0);
    return readlane_f64(v, kWave - 1);
}

// Maximum over the wave, returned to every lane.
__device__ __forceinline__ int wave_max_i32(int v)
{
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(v, kWave - 1);
}

// Maximum over the wave (NaN lanes ignored, as fmaxf does), returned to every lane.
__device__ __forceinline__ float wave_max_f32(float v)
{
    v = fmaxf(v, dpp_f32<0xB1>(v, v));
    v = fmaxf(v, dpp_f32<0x4E>(v, v));
    v = fmaxf(v, dpp_f32<0x141>(v, v));
    v = fmaxf(v, dpp_f32<0x140>(v, v));
    v = fmaxf(v, dpp_f32<0x142, 0xA>(v, v));
    v = fmaxf(v, dpp_f32<0x143, 0xC>(v, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// The same sum and maximum by LDS butterflies (ds_bpermute): slower to
// return, but they leave the VALU to a kernel that streams at the HBM rate
// with fp32 work per element (the dense chunk pass).
__device__ __forceinline__ double wave_sum_f64_lds(double v)
{
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

__device__ __forceinline__ float wave_max_f32_lds(float v)
{
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
    return v;
}

__device__ __forceinline__ int wave_first_lane(uint64_t mask) { return __ffsll((long long)mask) - 1; }

// Wave-wide maximum / minimum of a u32, returned to every lane: within each
// 16-lane row by DPP (swap neighbours, swap pairs, mirror halves, mirror the
// row), then lane 15 of each row into the next row and lane 31 into rows 2-3,
// which leaves the result in lane 63.  (The in-row steps have a source for
// every lane, so their old value is never used and they fuse into one DPP op.)
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v)
{
    auto pick = [](uint32_t a, uint32_t b) __attribute__((always_inline)) {
        return MAX ? (a > b ? a : b) : (a < b ? a : b);
    };
    v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
    v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// ---- logit rows --------------------------------------------------------------
template <bool BF16> struct Vec;
// load_stream: a 16-byte load marked non-temporal (the logits are read once;
// keeping them out of the caches' normal replacement lets the stream run
// closer to the HBM rate).
template <> struct Vec<false> {
    using T = float4;
    static constexpr int EPV = 4, ESZ = 4;
    __device__ __forceinline__ static T load_stream(const T* p)
    {
        typedef float v4 __attribute__((ext_vector_type(4)));
        const v4 r = __builtin_nontemporal_load(reinterpret_cast<const v4*>(p));
        return make_float4(r.x, r.y, r.z, r.w);
    }
    __device__ __forceinline__ static T neg_inf() { return make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY); }
    __device__ __forceinline__ static float get(const T& v, int e)
    {
        return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    }
};
template <> struct Vec<true> {
    using T = uint4;
    static constexpr int EPV = 8, ESZ = 2;
    __device__ __forceinline__ static T load_stream(const T* p)
    {
        typedef uint32_t v4 __attribute__((ext_vector_type(4)));
        const v4 r = __builtin_nontemporal_load(reinterpret_cast<const v4*>(p));
        return make_uint4(r.x, r.y, r.z, r.w);
    }
    __device__ __forceinline__ static T neg_inf() { return make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u); }
    __device__ __forceinline__ static float get(const T& v, int e)
    {
        const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
        return (e & 1) ? bf16_hi(w) : bf16_lo(w);
    }
};

template <bool BF16>
__device__ __forceinline__ float load_scalar(const char* row, int64_t i)
{
    if constexpr (BF16) {
        const uint16_t h = reinterpret_cast<const uint16_t*>(row)[i];
        return __uint_as_float((uint32_t)h << 16);
    } else {
        return reinterpret_cast<const float*>(row)[i];
    }
}

// Row pointer; returns nullptr for rows skipped by tree verification.
__device__ __forceinline__ const char* row_pointer(const RowSource s, int64_t r, int64_t row_bytes)
{
    if (r < s.rows0) {
        if (s.num_nodes) {
            const int64_t req = r / s.rows_per_req;
            if (r - req * s.rows_per_req >= (int64_t)s.num_nodes[req]) return nullptr;
        }
        return s.src0 + r * row_bytes;
    }
    return s.src1 + (r - s.rows0) * row_bytes;
}

// Split of a row into a scalar head (up to the first 16-byte boundary), whole
// 16-byte vectors, and a scalar tail.
struct RowGeom { int64_t head, nvec, tail_beg; };

template <bool BF16>
__device__ __forceinline__ RowGeom row_geom(const char* row, int64_t N)
{
    constexpr int ESZ = Vec<BF16>::ESZ, EPV = Vec<BF16>::EPV;
    int64_t head = (int64_t)(((16u - ((uintptr_t)row & 15u)) & 15u) / ESZ);
    if (head > N) head = N;
    const int64_t nvec = (N - head) / EPV;
    return { head, nvec, head + nvec * EPV };
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// ---- double-precision exp for the dense path ---------------------------------
// Table-driven exponential (P. T. P. Tang, "Table-driven implementation of the
// exponential function in IEEE floating-point arithmetic", ACM TOMS 15(2),
// 1989).  exp(d / T) = 2^y with y = d * log2(e) / T <= 0.  y = k/2048 + r with
// k the integer nearest 2048*y, read from the low bits of fma(d, c, 1.5*2^41)
// (whose ulp is 2^-11), and r = fma(d, c, -k/2048) rounded once, |r| <= 2^-12;
// then 2^y = 2^(k>>11) * 2^((k&2047)/2048) * 2^r, the middle factor from a
// 2048-entry table of nearest doubles and 2^r from the Taylor series of
// exp(r ln 2) to degree 3 (truncation below 4e-17).  d is clamped so that
// y >= -1000 (NaN and -inf land on the clamp as well).
constexpr int kExp2Entries = 2048;
static __constant__ double kExp2Table[kExp2Entries] = {
#include "exp2_table.inc"
};

// Copy the table into LDS (tab: kExp2Entries doubles); the caller synchronises.
__device__ __forceinline__ void load_exp2_table(double* tab)
{
    for (int i = (int)threadIdx.x; i < kExp2Entries; i += (int)blockDim.x) tab[i] = kExp2Table[i];
}

struct DenseExp {
    double c;              // log2(e) / T
    const double* tab;     // LDS copy of kExp2Table
    __device__ __forceinline__ double operator()(double d) const
    {
        constexpr double kC1 = 0.69314718055994530942;     // ln 2
        constexpr double kC2 = 0.24022650695910071233;     // (ln 2)^2 / 2
        constexpr double kC3 = 0.055504108664821579953;    // (ln 2)^3 / 6
        constexpr double kMagic = 0x1.8p41;
        d = fmax(d, -1000.0 / c);
        const double t = fma(d, c, kMagic);
        const double r = fma(d, c, -(t - kMagic));
        const int32_t k = (int32_t)(uint32_t)(uint64_t)__double_as_longlong(t);
        const double p = fma(fma(fma(r, kC3, kC2), r, kC1), r, 1.0);
        return ldexp(tab[k & (kExp2Entries - 1)] * p, k >> 11);
    }
};

// ---- per-chunk statistics of dense rows ----------------------------------------
// x: one chunk held by a wave (entry i of each lane; NaN and -inf allowed).
// Outputs are wave-uniform: the chunk max m, the fp64 sum of exp((z - m)/T)
// over the chunk and the number of finite logits.  With no finite logit the
// sum is 0; with +inf the max is +inf (the caller marks the row invalid).

// The finite count costs a compare and a ballot per logit, so it is taken
// only when COUNT is set (*cnt_out is 0 otherwise).

// Exact: every term from DenseExp.
template <bool COUNT, int PER_LANE>
__device__ __forceinline__ void chunk_stats_exact(const float (&x)[PER_LANE], const DenseExp& ex, float* m_out,
                                                  double* s_out, uint32_t* cnt_out)
{
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) mx = fmaxf(mx, x[i]);
    mx = wave_max_f32_lds(mx);
    double s0 = 0.0, s1 = 0.0;
    uint32_t cntf = 0;
    if (mx > -INFINITY && mx < INFINITY) {
        const double md = (double)mx;
        // groups of eight exps (two sums) bound how many are in flight, and
        // with them the registers
#pragma unroll
        for (int g = 0; g < PER_LANE; g += 8) {
#pragma unroll
            for (int i = g; i < g + 8; ++i) {
                // NaN and -inf reach the exp's lower clamp, whose term (2^-1000)
                // vanishes next to the chunk maximum's 1
                if (COUNT) cntf += (uint32_t)__popcll(__ballot(finite_f32(x[i])));
                const double e = ex((double)x[i] - md);
                if (i & 1) s1 += e; else s0 += e;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    *m_out = mx;
    *s_out = wave_sum_f64_lds(s0 + s1);
    *cnt_out = cntf;
}

// Fast: terms t = 2^y from the fp32 exponential, y = fl(fl(z - m) * c) with
// c = fl(log2(e)/T), summed in fp64, with a bound on the chunk sum's error.
// The bound (a certificate for callers that invert a CDF from these sums):
//  - v_exp_f32 is within 0.712 * 2^-23 relative of 2^y for every fp32 y in
//    [-126, 0) (checked exhaustively on gfx950 against exp2 in double), so
//    kFastExpRel = 2^-23 bounds it;
//  - y carries three fp32 roundings (difference, constant, product):
//    |y - y_exact| <= 3.0002 * 2^-24 * |y|, which moves the term by at most
//    kFastArgRel * |y| relative (ln 2 * 3.0002 * 2^-24, with room for the
//    exponential's curvature at |y| <= 200);
//  - y is clamped at -200 (NaN, -inf and negligible terms) and results below
//    2^-126 may flush to 0: at most 2^-126 per term.
//  - the terms are added four at a time in fp32 (a two-level tree of
//    non-negative values: within 2^-23 relative of each group's sum, plus at
//    most 2^-126 per addition flushed) before each group joins the fp64 sum:
//    kFastSumRel = 2^-23 of the sum.
// So |sum - exact| <= (kFastExpRel + kFastSumRel) * sum + kFastArgRel * sum(t * |y|)
// + 3584 * 2^-126; the factor (1 + 2e-3) covers the fp32 sum of t * |y|, the
// fp64 sums and the rounding of the result to float.
constexpr double kFastExpRel = 0x1p-23;
constexpr double kFastArgRel = 1.2397e-7;
constexpr double kFastSumRel = 0x1p-23;

template <bool COUNT, int PER_LANE>
__device__ __forceinline__ void chunk_stats_fast(const float (&x)[PER_LANE], float log2e_over_T, float* m_out,
                                                 double* s_out, uint32_t* cnt_out, float* err_out)
{
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) mx = fmaxf(mx, x[i]);
    mx = wave_max_f32_lds(mx);
    double s = 0.0;
    float a = 0.0f;            // sum of t * y (every y <= 0)
    uint32_t cntf = 0;
    if (mx > -INFINITY && mx < INFINITY) {
        static_assert(PER_LANE % 4 == 0, "terms are summed four at a time");
#pragma unroll
        for (int i = 0; i < PER_LANE; i += 4) {
            float t4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (COUNT) cntf += (uint32_t)__popcll(__ballot(finite_f32(x[i + e])));
                // NaN and -inf give y = NaN or -inf, which the clamp maps to -200
                const float y = fmaxf((x[i + e] - mx) * log2e_over_T, -200.0f);
                t4[e] = __builtin_amdgcn_exp2f(y);
                a = fmaf(t4[e], y, a);
            }
            s += (double)((t4[0] + t4[1]) + (t4[2] + t4[3]));
        }
    }
    *m_out = mx;
    s = wave_sum_f64_lds(s);
    const double ty = wave_sum_f64_lds((double)a);
    *s_out = s;
    *err_out = (float)((1.0 + 2e-3) * ((kFastExpRel + kFastSumRel) * s - kFastArgRel * ty) + 0x1p-114);
    *cnt_out = cntf;
}

}  // namespace uno
