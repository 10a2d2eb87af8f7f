// attention_kernels.hip -- tree-suffix attention merged with the prefix
// attention state, for UNO tree verification on gfx950.
//
// Method: SGLang PR #37667, Modifications (an UNO-only fused kernel for
// tree-suffix attention and LSE merge) and Changes to shared SGLang
// infrastructure (the fused merge serves UNO tree verification; cascade
// attention computes the shared prefix once).  The verify tokens of a request
// are the tree's nodes; node i attends, among the suffix keys, to itself and
// its ancestors, and that suffix attention (o_s, lse_s) is merged with the
// query's prefix state (o_p, lse_p):
//   lse = log(exp(lse_p) + exp(lse_s)),  o = exp(lse_p - lse) o_p + exp(lse_s - lse) o_s.
//
// Workgroups per (request, key/value head, group of four query pairs).  The
// head's suffix keys and values are staged in LDS; a wave scores its query
// against 64 keys at once, one key per lane (16-byte key reads, the query
// broadcast from LDS), and sums the values of the visible keys only, found in
// ancestor bitsets built by pointer doubling.  Scores, softmax and sums run in
// fp32; outputs are bf16 (o) and fp32 (lse).
#include "uno_device.h"
#include "uno_internal.h"

#include <math.h>

namespace uno {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kAttnD = 128;                   // head dimension
constexpr int kAttnMaxNodes = 129;            // V + 1 with V <= 128
constexpr int kAttnWords = (kAttnMaxNodes + 63) / 64;
constexpr int kAttnKRow = kAttnD + 8;         // key row stride in LDS (bf16): 16-byte reads spread over the banks

__device__ __forceinline__ float bf16_at(const uint16_t* p, int64_t i)
{
    return __uint_as_float((uint32_t)p[i] << 16);
}

// float -> bf16, round to nearest even (finite inputs; NaN kept quiet)
__device__ __forceinline__ uint16_t to_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// LDS of one workgroup for n nodes: keys [n][kAttnKRow] and values [n][D]
// (bf16), ancestor sets [2][n][words], jumps [2][n], the waves' queries.
__host__ __device__ constexpr size_t attn_lds_bytes(int n)
{
    return ((size_t)n * kAttnKRow * 2 + 15) / 16 * 16 + ((size_t)n * kAttnD * 2 + 15) / 16 * 16 +
           (size_t)2 * n * kAttnWords * 8 + ((size_t)2 * n * 4 + 15) / 16 * 16 + (size_t)kAttnWaves * kAttnD * 4;
}

// Grid (request, kv head, pair group): each wave takes up to `ppw` (query
// node, head of the group) pairs; every workgroup stages the head's suffix
// keys and values in LDS and builds the ancestor sets.
__global__ __launch_bounds__(kAttnThreads) void tree_attention_kernel(
    const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o_prefix, const float* lse_prefix,
    const int32_t* node_parent, const int32_t* num_nodes, int32_t n, int32_t Hq, int32_t Hkv, float scale,
    int32_t ppw, uint16_t* out, float* out_lse)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t s_raw[];
    uint16_t* s_k = reinterpret_cast<uint16_t*>(s_raw);
    uint16_t* s_v = s_k + ((size_t)n * kAttnKRow * 2 + 15) / 16 * 8;
    uint64_t* s_anc = reinterpret_cast<uint64_t*>(s_v + ((size_t)n * kAttnD * 2 + 15) / 16 * 8);
    int32_t* s_jump = reinterpret_cast<int32_t*>(s_anc + (size_t)2 * n * kAttnWords);
    float* s_qall = reinterpret_cast<float*>(s_jump + ((size_t)2 * n * 4 + 15) / 16 * 4);
    auto anc = [&](int c, int i, int wd) -> uint64_t& { return s_anc[((size_t)c * n + i) * kAttnWords + wd]; };
    auto jump = [&](int c, int i) -> int32_t& { return s_jump[(size_t)c * n + i]; };

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x;
    const int hk = blockIdx.y;
    const int G = Hq / Hkv;
    int nn = num_nodes ? num_nodes[b] : n;
    nn = nn < 0 ? 0 : (nn > n ? n : nn);
    const int64_t t0 = (int64_t)b * n;
    const int pbeg = (int)blockIdx.z * kAttnWaves * ppw;           // this workgroup's pairs
    if (pbeg >= nn * G) return;                                    // the whole workgroup is idle
    const int pend = min(pbeg + kAttnWaves * ppw, nn * G);
    // a pair's own inputs (query, prefix output and lse) go to registers, the
    // next pair's while the current one is processed; the first pair's load
    // overlaps the staging below
    auto pair_token = [&](int pr) -> int64_t {
        const int pc = pr < pend ? pr : pbeg;                      // past the end: a valid pair (shape only)
        const int ii = pc / G;
        return (t0 + ii) * Hq + hk * G + (pc - ii * G);
    };
    float cq0, cq1, cp0, cp1, clp;
    auto load_pair = [&](int pr, float& q0, float& q1, float& p0, float& p1, float& lp) __attribute__((always_inline)) {
        const int64_t tq = pair_token(pr);
        q0 = bf16_at(q, tq * kAttnD + lane);
        q1 = bf16_at(q, tq * kAttnD + lane + kWave);
        p0 = bf16_at(o_prefix, tq * kAttnD + lane);
        p1 = bf16_at(o_prefix, tq * kAttnD + lane + kWave);
        lp = lse_prefix[tq];
    };
    load_pair(pbeg + w, cq0, cq1, cp0, cp1, clp);

    // keys and values of this head into LDS, 16 bytes at a time
    for (int idx = threadIdx.x; idx < nn * (kAttnD / 8); idx += kAttnThreads) {
        const int j = idx / (kAttnD / 8), c = idx - j * (kAttnD / 8);
        const int64_t src = ((t0 + j) * Hkv + hk) * kAttnD + c * 8;
        *reinterpret_cast<uint4*>(&s_k[j * kAttnKRow + c * 8]) = *reinterpret_cast<const uint4*>(&k[src]);
        *reinterpret_cast<uint4*>(&s_v[j * kAttnD + c * 8]) = *reinterpret_cast<const uint4*>(&v[src]);
    }
    // ancestor-or-self sets by pointer doubling: after round r, anc[i] holds
    // the nodes within 2^r steps above i and jump[i] the node 2^r steps up
    for (int i = threadIdx.x; i < nn; i += kAttnThreads) {
        const int p = node_parent[t0 + i];
        const int pj = (p >= 0 && p < i) ? p : -1;                 // parents precede children
        for (int wd = 0; wd < kAttnWords; ++wd) anc(0, i, wd) = 0ull;
        anc(0, i, i >> 6) |= 1ull << (i & 63);
        if (pj >= 0) anc(0, i, pj >> 6) |= 1ull << (pj & 63);
        jump(0, i) = pj;
    }
    __syncthreads();
    int cur = 0;
    int rounds = 0;                                                // 2^rounds >= nn covers every depth
    while ((1 << rounds) < nn) ++rounds;
    for (int round = 0; round < rounds; ++round) {
        for (int i = threadIdx.x; i < nn; i += kAttnThreads) {
            const int jp = jump(cur, i);
            for (int wd = 0; wd < kAttnWords; ++wd)
                anc(cur ^ 1, i, wd) = anc(cur, i, wd) | (jp >= 0 ? anc(cur, jp, wd) : 0ull);
            jump(cur ^ 1, i) = jp >= 0 ? jump(cur, jp) : -1;
        }
        __syncthreads();
        cur ^= 1;
    }
    float* s_q = s_qall + w * kAttnD;
    for (int pr = pbeg + w; pr < pend; pr += kAttnWaves) {        // no barrier in this loop
    float nq0, nq1, np0, np1, nlp;
    load_pair(pr + kAttnWaves, nq0, nq1, np0, np1, nlp);
    const int i = pr / G, g = pr - i * G;
    const int h = hk * G + g;
    const int64_t tq = (t0 + i) * Hq + h;
    // the query into this wave's LDS row, pre-scaled
    s_q[lane] = scale * cq0;
    s_q[lane + kWave] = scale * cq1;
    wave_sync();
    const float4* q4 = reinterpret_cast<const float4*>(s_q);
    // scores of up to three 64-key blocks, one key per lane (16-byte key reads)
    float sc[kAttnWords];
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < kAttnWords; ++blk) {
        const int j = blk * kWave + lane;
        float s = -INFINITY;
        if (blk * kWave < nn) {
            const bool vis = j < nn && ((anc(cur, i, j >> 6) >> (j & 63)) & 1ull);
            const uint4* kr = reinterpret_cast<const uint4*>(&s_k[(j < nn ? j : 0) * kAttnKRow]);
            float acc = 0.0f;
#pragma unroll 4
            for (int c = 0; c < kAttnD / 8; ++c) {
                const uint4 kv = kr[c];
                const float4 qa = q4[2 * c], qb = q4[2 * c + 1];
                acc = fmaf(qa.x, bf16_lo(kv.x), acc);
                acc = fmaf(qa.y, bf16_hi(kv.x), acc);
                acc = fmaf(qa.z, bf16_lo(kv.y), acc);
                acc = fmaf(qa.w, bf16_hi(kv.y), acc);
                acc = fmaf(qb.x, bf16_lo(kv.z), acc);
                acc = fmaf(qb.y, bf16_hi(kv.z), acc);
                acc = fmaf(qb.z, bf16_lo(kv.w), acc);
                acc = fmaf(qb.w, bf16_hi(kv.w), acc);
            }
            s = vis ? acc : -INFINITY;
        }
        sc[blk] = s;
        mx = fmaxf(mx, s);
    }
    mx = wave_max_f32(mx);
    float sum = 0.0f;
#pragma unroll
    for (int blk = 0; blk < kAttnWords; ++blk) {
        const float e = (sc[blk] > -INFINITY) ? __expf(sc[blk] - mx) : 0.0f;
        sc[blk] = e;
        sum += e;
    }
    for (int o = kWave / 2; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, kWave);
    const float lse_s = mx + __logf(sum);
    const float inv = 1.0f / sum;
    // o_s over the visible keys (dimensions lane and lane + 64)
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int wd = 0; wd < kAttnWords; ++wd) {
        uint64_t bits = anc(cur, i, wd);
        while (bits) {
            const int jb = __ffsll((long long)bits) - 1;
            bits &= bits - 1;
            const int j = wd * 64 + jb;
            const float pj = __shfl(sc[wd], jb, kWave) * inv;
            o0 = fmaf(pj, __uint_as_float((uint32_t)s_v[j * kAttnD + lane] << 16), o0);
            o1 = fmaf(pj, __uint_as_float((uint32_t)s_v[j * kAttnD + lane + kWave] << 16), o1);
        }
    }
    // merge with the prefix state
    const float lp = clp;
    float lse = lse_s, wp = 0.0f, ws = 1.0f;
    if (lp > -INFINITY) {
        const float hi = fmaxf(lp, lse_s), lo = fminf(lp, lse_s);
        lse = hi + log1pf(__expf(lo - hi));
        wp = __expf(lp - lse);
        ws = __expf(lse_s - lse);
    }
    const int64_t ob = tq * kAttnD;
    const float r0 = wp * cp0 + ws * o0;
    const float r1 = wp * cp1 + ws * o1;
    out[ob + lane] = to_bf16(r0);
    out[ob + lane + kWave] = to_bf16(r1);
    if (lane == 0) out_lse[tq] = lse;
    wave_sync();                                                   // s_q is rewritten by the next pair
    cq0 = nq0; cq1 = nq1; cp0 = np0; cp1 = np1; clp = nlp;
    }
}

}  // namespace

hipError_t launch_tree_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o_prefix,
                                 const float* lse_prefix, const int32_t* node_parent, const int32_t* num_nodes,
                                 int32_t batch, int32_t n, int32_t Hq, int32_t Hkv, float scale, uint16_t* out,
                                 float* out_lse, hipStream_t stream)
{
    if (batch == 0) return hipSuccess;
    // about 1024 workgroups in all; each wave then takes ppw pairs
    const int64_t pairs = (int64_t)n * (Hq / Hkv);
    const int64_t per_head = (int64_t)batch * Hkv;
    int64_t groups = (1024 + per_head - 1) / per_head;
    const int64_t max_groups = (pairs + kAttnWaves - 1) / kAttnWaves;
    groups = groups < 1 ? 1 : (groups > max_groups ? max_groups : groups);
    const int ppw = (int)((pairs + groups * kAttnWaves - 1) / (groups * kAttnWaves));
    const size_t lds = attn_lds_bytes(n);
    if (lds > 65536) {       // beyond the default dynamic LDS limit (the largest trees)
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&tree_attention_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    tree_attention_kernel<<<dim3((unsigned)batch, (unsigned)Hkv, (unsigned)groups), kAttnThreads, lds, stream>>>(
        q, k, v, o_prefix, lse_prefix, node_parent, num_nodes, n, Hq, Hkv, scale, ppw, out, out_lse);
    return hipGetLastError();
}

}  // namespace uno
