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
// One workgroup per (request, key/value head).  The head's suffix keys sit in
// LDS transposed (dimension-major), so a wave scores one query against 64
// keys at once, one key per lane, with the query broadcast from LDS.  The
// visible keys come from ancestor bitsets built by pointer doubling.  Values
// are read from global memory only for the visible keys.  Scores, softmax and
// accumulation run in fp32; outputs are bf16 (o) and fp32 (lse).
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
constexpr int kAttnKeyPad = 3 * kWave;        // key columns in LDS (>= kAttnMaxNodes)

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

__global__ __launch_bounds__(kAttnThreads) void tree_attention_kernel(
    const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o_prefix, const float* lse_prefix,
    const int32_t* node_parent, const int32_t* num_nodes, int32_t n, int32_t Hq, int32_t Hkv, float scale,
    uint16_t* out, float* out_lse)
{
    __shared__ uint16_t s_kt[kAttnD * kAttnKeyPad];               // K^T: [d][node]
    __shared__ uint64_t s_anc[2][kAttnMaxNodes][kAttnWords];      // ancestor-or-self bitsets
    __shared__ int32_t s_jump[2][kAttnMaxNodes];
    __shared__ float s_q[kAttnWaves][kAttnD];

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x;
    const int hk = blockIdx.y;
    const int G = Hq / Hkv;
    int nn = num_nodes ? num_nodes[b] : n;
    nn = nn < 0 ? 0 : (nn > n ? n : nn);
    const int64_t t0 = (int64_t)b * n;

    // keys of this head, transposed into LDS
    for (int idx = threadIdx.x; idx < nn * kAttnD; idx += kAttnThreads) {
        const int j = idx / kAttnD, d = idx - j * kAttnD;
        s_kt[d * kAttnKeyPad + j] = k[((t0 + j) * Hkv + hk) * kAttnD + d];
    }
    // ancestor-or-self sets by pointer doubling: after round r, anc[i] holds
    // the nodes within 2^r steps above i and jump[i] the node 2^r steps up
    for (int i = threadIdx.x; i < nn; i += kAttnThreads) {
        const int p = node_parent[t0 + i];
        const int pj = (p >= 0 && p < i) ? p : -1;                 // parents precede children
        for (int wd = 0; wd < kAttnWords; ++wd) s_anc[0][i][wd] = 0ull;
        s_anc[0][i][i >> 6] |= 1ull << (i & 63);
        if (pj >= 0) s_anc[0][i][pj >> 6] |= 1ull << (pj & 63);
        s_jump[0][i] = pj;
    }
    __syncthreads();
    int cur = 0;
    for (int round = 0; round < 8; ++round) {                     // 2^8 > kAttnMaxNodes
        for (int i = threadIdx.x; i < nn; i += kAttnThreads) {
            const int jp = s_jump[cur][i];
            for (int wd = 0; wd < kAttnWords; ++wd)
                s_anc[cur ^ 1][i][wd] = s_anc[cur][i][wd] | (jp >= 0 ? s_anc[cur][jp][wd] : 0ull);
            s_jump[cur ^ 1][i] = jp >= 0 ? s_jump[cur][jp] : -1;
        }
        __syncthreads();
        cur ^= 1;
    }

    // (query node i, head g of this group) pairs, round robin over the waves
    for (int pr = w; pr < nn * G; pr += kAttnWaves) {
        const int i = pr / G, g = pr - i * G;
        const int h = hk * G + g;
        const int64_t tq = (t0 + i) * Hq + h;
        // the query into this wave's LDS row, pre-scaled
        for (int d = lane; d < kAttnD; d += kWave) s_q[w][d] = scale * bf16_at(q, tq * kAttnD + d);
        wave_sync();                      // the wave's own LDS row: in-order within the wave
        // scores of up to three 64-key blocks, one key per lane
        float sc[3];
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 3; ++blk) {
            const int j = blk * kWave + lane;
            const bool vis = j < nn && ((s_anc[cur][i][j >> 6] >> (j & 63)) & 1ull);
            float s = -INFINITY;
            if (blk * kWave < nn) {
                float acc = 0.0f;
#pragma unroll 8
                for (int d = 0; d < kAttnD; ++d) acc = fmaf(s_q[w][d], __uint_as_float((uint32_t)s_kt[d * kAttnKeyPad + j] << 16), acc);
                s = vis ? acc : -INFINITY;
            }
            sc[blk] = s;
            mx = fmaxf(mx, s);
        }
        mx = wave_max_f32(mx);
        float sum = 0.0f;
#pragma unroll
        for (int blk = 0; blk < 3; ++blk) {
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
            uint64_t bits = s_anc[cur][i][wd];
            while (bits) {
                const int jb = __ffsll((long long)bits) - 1;
                bits &= bits - 1;
                const int j = wd * 64 + jb;
                const float pj = __shfl(sc[wd], jb, kWave) * inv;
                const int64_t vr = ((t0 + j) * Hkv + hk) * kAttnD;
                o0 = fmaf(pj, bf16_at(v, vr + lane), o0);
                o1 = fmaf(pj, bf16_at(v, vr + lane + kWave), o1);
            }
        }
        // merge with the prefix state
        const float lp = lse_prefix[tq];
        float lse = lse_s, wp = 0.0f, ws = 1.0f;
        if (lp > -INFINITY) {
            const float hi = fmaxf(lp, lse_s), lo = fminf(lp, lse_s);
            lse = hi + log1pf(__expf(lo - hi));
            wp = __expf(lp - lse);
            ws = __expf(lse_s - lse);
        }
        const int64_t ob = tq * kAttnD;
        const float r0 = wp * bf16_at(o_prefix, ob + lane) + ws * o0;
        const float r1 = wp * bf16_at(o_prefix, ob + lane + kWave) + ws * o1;
        out[ob + lane] = to_bf16(r0);
        out[ob + lane + kWave] = to_bf16(r1);
        if (lane == 0) out_lse[tq] = lse;
        wave_sync();                      // s_q is rewritten by the next pair
    }
}

}  // namespace

hipError_t launch_tree_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o_prefix,
                                 const float* lse_prefix, const int32_t* node_parent, const int32_t* num_nodes,
                                 int32_t batch, int32_t n, int32_t Hq, int32_t Hkv, float scale, uint16_t* out,
                                 float* out_lse, hipStream_t stream)
{
    if (batch == 0) return hipSuccess;
    tree_attention_kernel<<<dim3((unsigned)batch, (unsigned)Hkv), kAttnThreads, 0, stream>>>(
        q, k, v, o_prefix, lse_prefix, node_parent, num_nodes, n, Hq, Hkv, scale, out, out_lse);
    return hipGetLastError();
}

}  // namespace uno
