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
// One workgroup per (request, key/value head, block of up to 64 query rows),
// where the rows stack the G query heads that share the key/value head (row m
// is node m / G, head m % G).  The workgroup stages the head's keys and values
// (transposed) in LDS, wave 0 walks every node's ancestor chain meanwhile, and
// after that single barrier each wave takes one 16-row tile alone: S = Q K^T
// on the matrix cores (16x16x16 bf16 tiles, fp32 accumulation, Q straight from
// memory into the A operands), the ancestor mask and the softmax in registers
// (rows reduced over 16 lanes), P through the wave's own LDS tile into the A
// layout, split into two bf16 parts (P = hi + lo, 16 significant bits), and
// O_s = P V on the matrix cores, merged with the prefix state held in
// registers since the start.  Outputs are bf16 (o) and fp32 (lse).
#include "uno_device.h"
#include "uno_internal.h"

#include <math.h>

#include <mutex>

namespace uno {

namespace {

typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kAttnD = 128;                   // head dimension
constexpr int kAttnMaxTreeNodes = 129;        // V + 1 with V <= 128
constexpr int kAttnWords = 3;                 // ancestor-set words
constexpr int kAttnRows = kAttnWaves * 16;    // query rows per workgroup at most: a 16-row tile per wave
constexpr int kAttnKRow = kAttnD + 8;         // bf16 per key row in LDS (16-byte rows, spread over the banks)
constexpr int kDTiles = kAttnD / 16;

// float -> bf16 bits, round to nearest even (the hardware conversion)
__device__ __forceinline__ uint16_t to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Maximum / sum over the 16 lanes of a row (lanes 16 g .. 16 g + 15), returned
// to all of them: DPP swaps of neighbours and pairs within each quad, then the
// half-row and row mirrors.
template <bool MAX>
__device__ __forceinline__ float row16_reduce(float v)
{
    auto op = [](float a, float b) __attribute__((always_inline)) { return MAX ? fmaxf(a, b) : a + b; };
    v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
    return v;
}

// LDS of one workgroup for trees of up to n nodes (keys padded to npad, a
// multiple of 16): keys [npad][kAttnKRow] and values transposed [D][npad + 8]
// (bf16), the parents [npad] and ancestor sets [npad][3], and per wave a
// 16-row P tile [16][npad + 4] of packed bf16 parts (hi | lo << 16) and its
// rows' prefix outputs [16][kAttnKRow] (bf16).  (129 nodes: 138 KB.)
struct AttnLds {
    int npad, vt_stride, p_stride;
    size_t off_vt, off_par, off_anc, off_p, off_op, total;
};

__host__ __device__ inline AttnLds attn_lds(int n)
{
    AttnLds L;
    L.npad = (n + 15) / 16 * 16;
    L.vt_stride = L.npad + 8;
    L.p_stride = L.npad + 4;
    size_t o = (size_t)L.npad * kAttnKRow * 2;
    L.off_vt = o;
    o += (size_t)kAttnD * L.vt_stride * 2;
    L.off_par = o;
    o += (size_t)L.npad * 4;
    L.off_anc = o;
    o += (size_t)L.npad * kAttnWords * 8;
    L.off_p = o;
    o += (size_t)kAttnWaves * 16 * L.p_stride * 4;
    L.off_op = o;
    o += (size_t)kAttnWaves * 16 * kAttnKRow * 2;
    L.total = o;
    return L;
}

// KT: key tiles of 16 (ceil of the tree's nodes / 16), a compile-time count so
// the score tiles stay in registers with loops of exactly that length.
template <int KT>
__global__ __launch_bounds__(kAttnThreads) void tree_attention_kernel(
    const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o_prefix, const float* lse_prefix,
    const int32_t* node_parent, const int32_t* num_nodes, int32_t n, int32_t Hq, int32_t Hkv, float scale,
    int32_t rows_wg, uint16_t* out, float* out_lse)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t s_raw[];
    const AttnLds L = attn_lds(n);
    uint16_t* s_k = reinterpret_cast<uint16_t*>(s_raw);
    uint16_t* s_vt = reinterpret_cast<uint16_t*>(s_raw + L.off_vt);
    uint64_t* s_anc = reinterpret_cast<uint64_t*>(s_raw + L.off_anc);
    int32_t* s_par = reinterpret_cast<int32_t*>(s_raw + L.off_par);

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int tid = (int)threadIdx.x;
    uint16_t* s_op = reinterpret_cast<uint16_t*>(s_raw + L.off_op) + (size_t)w * 16 * kAttnKRow;   // this wave's rows
    const int b = blockIdx.x;
    const int hk = blockIdx.y;
    const int G = Hq / Hkv;
    int nn = num_nodes ? num_nodes[b] : n;
    nn = nn < 0 ? 0 : (nn > n ? n : nn);
    const int M = nn * G;                                          // query rows of this head group
    const int m0 = (int)blockIdx.z * rows_wg;
    if (m0 >= M) return;                                           // the whole workgroup is idle
    const int mrows = min(rows_wg, M - m0);
    const int ktiles = (nn + 15) / 16;                            // <= KT
    const int64_t t0 = (int64_t)b * n;
    const int r0 = w * 16;                                         // this wave's first row in the block
    const bool active = r0 < mrows;                                // wave-uniform
    // lane l of a 16x16x16 tile supplies A[l % 16][4 (l / 16) + e] and
    // B[4 (l / 16) + e][l % 16] and receives D[4 (l / 16) + e][l % 16], e = 0..3
    const int lr = lane & 15, lk = 4 * (lane >> 4);
    auto row_token = [&](int r) -> int64_t {                       // (token, head) of block row r
        const int m = m0 + r, i = m / G;
        return (t0 + i) * Hq + hk * G + (m - i * G);
    };

    int par0 = -1, par1 = -1, par2 = -1;                           // wave 0: the parents, loaded first
    if (w == 0) {
        if (lane < nn) par0 = node_parent[t0 + lane];
        if (lane + kWave < nn) par1 = node_parent[t0 + lane + kWave];
        if (lane + 2 * kWave < nn) par2 = node_parent[t0 + lane + 2 * kWave];
    }

    // ---- this wave's own inputs, straight to registers (issued first) ----
    // Q rows in the A layout (row r0 + lr), the lane's four C-layout rows
    // (r0 + lk + e): their token offsets, prefix lse and prefix outputs
    bf16x4 qa[kDTiles];
    int64_t ctok[4];
    float clp[4];
    uint4 opv[4];                                                  // the wave's 16 prefix rows, 16 bytes a piece
    {
        const int ra = r0 + lr;
        const int64_t qb = (active && ra < mrows) ? row_token(ra) * kAttnD : -1;
#pragma unroll
        for (int ks = 0; ks < kDTiles; ++ks) {
            bf16x4 z = { 0, 0, 0, 0 };
            qa[ks] = qb >= 0 ? *reinterpret_cast<const bf16x4*>(&q[qb + ks * 16 + lk]) : z;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = r0 + lk + e;
            ctok[e] = (active && r < mrows) ? row_token(r) : -1;
            clp[e] = ctok[e] >= 0 ? lse_prefix[ctok[e]] : -INFINITY;
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = lane + it * kWave, r = idx / (kAttnD / 8), c = idx - r * (kAttnD / 8);
            const bool ok = active && r0 + r < mrows;
            opv[it] = ok ? *reinterpret_cast<const uint4*>(&o_prefix[row_token(r0 + r) * kAttnD + c * 8])
                         : make_uint4(0u, 0u, 0u, 0u);
        }
    }

    // ---- shared staging: keys, values transposed (zero past the tree, where
    // P is 0); wave 0 meanwhile builds the ancestor-or-self set of every node
    // by walking up the parent links in registers ----
    constexpr int kKvBatch = 4;
    for (int base = 0; base < ktiles * 16 * (kAttnD / 8); base += kKvBatch * kAttnThreads) {
        uint4 kv[kKvBatch], vv[kKvBatch];
#pragma unroll
        for (int it = 0; it < kKvBatch; ++it) {
            const int idx = base + tid + it * kAttnThreads;
            const int j = idx / (kAttnD / 8), c = idx - j * (kAttnD / 8);
            kv[it] = make_uint4(0u, 0u, 0u, 0u);
            vv[it] = kv[it];
            if (j < nn) {
                const int64_t src = ((t0 + j) * Hkv + hk) * kAttnD + c * 8;
                kv[it] = *reinterpret_cast<const uint4*>(&k[src]);
                vv[it] = *reinterpret_cast<const uint4*>(&v[src]);
            }
        }
#pragma unroll
        for (int it = 0; it < kKvBatch; ++it) {
            const int idx = base + tid + it * kAttnThreads;
            const int j = idx / (kAttnD / 8), c = idx - j * (kAttnD / 8);
            if (j >= ktiles * 16) continue;
            *reinterpret_cast<uint4*>(&s_k[j * kAttnKRow + c * 8]) = kv[it];
            const uint32_t vw[4] = { vv[it].x, vv[it].y, vv[it].z, vv[it].w };
#pragma unroll
            for (int e = 0; e < 8; ++e)
                s_vt[(c * 8 + e) * L.vt_stride + j] = (uint16_t)(vw[e >> 1] >> ((e & 1) * 16));
        }
    }
    if (w == 0) {
        // the ancestor-or-self set of node i (lanes take i = lane, lane + 64, ...):
        // walk up the parent links, which precede their children, so every walk
        // ends at the root within i steps
        const int pv[kAttnWords] = { par0, par1, par2 };
#pragma unroll
        for (int c = 0; c < kAttnWords; ++c) {
            const int i = lane + kWave * c;
            if (i < nn) s_par[i] = (pv[c] >= 0 && pv[c] < i) ? pv[c] : -1;
        }
        wave_sync();
        for (int i = lane; i < nn; i += kWave) {
            uint64_t a0 = 0ull, a1 = 0ull, a2 = 0ull;
            for (int x = i; x >= 0; x = s_par[x]) {
                const uint64_t bit = 1ull << (x & 63);
                if ((x >> 6) == 0) a0 |= bit; else if ((x >> 6) == 1) a1 |= bit; else a2 |= bit;
            }
            s_anc[i * kAttnWords] = a0;
            s_anc[i * kAttnWords + 1] = a1;
            s_anc[i * kAttnWords + 2] = a2;
        }
    }
    // the wave's prefix rows into its own tile (read back after the barrier)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = lane + it * kWave, r = idx / (kAttnD / 8), c = idx - r * (kAttnD / 8);
        *reinterpret_cast<uint4*>(&s_op[r * kAttnKRow + c * 8]) = opv[it];
    }
    __syncthreads();
    if (!active) return;                                           // no barrier follows

    // ---- S = scale * Q K^T over every key tile, masked to the row's ancestors ----
    f32x4 sc[KT];
#pragma unroll
    for (int ct = 0; ct < KT; ++ct) {
        sc[ct] = (f32x4){ 0.0f, 0.0f, 0.0f, 0.0f };
        if (ct < ktiles) {
            const uint16_t* kb = s_k + (ct * 16 + lr) * kAttnKRow + lk;
#pragma unroll
            for (int ks = 0; ks < kDTiles; ++ks)
                sc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qa[ks], *reinterpret_cast<const bf16x4*>(kb + ks * 16),
                                                                   sc[ct], 0, 0, 0);
        }
    }
    uint64_t rw[4][kAttnWords];                                    // ancestor sets of the lane's rows' nodes
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int node = ctok[e] >= 0 ? (m0 + r0 + lk + e) / G : 0;
#pragma unroll
        for (int wd = 0; wd < kAttnWords; ++wd) rw[e][wd] = ctok[e] >= 0 ? s_anc[node * kAttnWords + wd] : 0ull;
    }
    float mx[4] = { -INFINITY, -INFINITY, -INFINITY, -INFINITY };
#pragma unroll
    for (int ct = 0; ct < KT; ++ct) {
        const int j = ct * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint64_t word = (j >> 6) == 0 ? rw[e][0] : ((j >> 6) == 1 ? rw[e][1] : rw[e][2]);
            const bool vis = ct < ktiles && j < nn && ((word >> (j & 63)) & 1ull);
            const float x = vis ? sc[ct][e] * scale : -INFINITY;
            sc[ct][e] = x;
            mx[e] = fmaxf(mx[e], x);
        }
    }
    // a row's keys are spread over the 16 lanes of its group
#pragma unroll
    for (int e = 0; e < 4; ++e) mx[e] = row16_reduce<true>(mx[e]);
    float sm[4] = { 0.0f, 0.0f, 0.0f, 0.0f };
#pragma unroll
    for (int ct = 0; ct < KT; ++ct) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = sc[ct][e];
            const float pe = (x > -INFINITY) ? __expf(x - mx[e]) : 0.0f;
            sc[ct][e] = pe;
            sm[e] += pe;
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sm[e] = row16_reduce<false>(sm[e]);
    // the merge with the prefix state, per row: with t = exp(min - max) of the
    // two lse and d = 1 + t, lse = max + log d and the weights are 1/d and t/d
    float wp[4], ws[4], inv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float ls = mx[e] + __logf(sm[e]), lp = clp[e];
        inv[e] = sm[e] > 0.0f ? 1.0f / sm[e] : 0.0f;
        float lse = ls;
        wp[e] = 0.0f;
        ws[e] = 1.0f;
        if (lp > -INFINITY) {
            const bool pbig = lp >= ls;
            const float t = __expf(pbig ? ls - lp : lp - ls), d = 1.0f + t, rd = 1.0f / d;
            lse = (pbig ? lp : ls) + __logf(d);
            wp[e] = pbig ? rd : t * rd;
            ws[e] = pbig ? t * rd : rd;
        }
        if (lr == 0 && ctok[e] >= 0) out_lse[ctok[e]] = lse;
    }
    // P (C layout) into the wave's tile as packed bf16 parts, then read back in
    // the A layout
    uint32_t* s_p = reinterpret_cast<uint32_t*>(s_raw + L.off_p) + (size_t)w * 16 * L.p_stride;
#pragma unroll
    for (int ct = 0; ct < KT; ++ct) {
        if (ct < ktiles) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pj = sc[ct][e] * inv[e];
                const uint16_t hi = to_bf16(pj);
                const uint16_t lo = to_bf16(pj - __uint_as_float((uint32_t)hi << 16));
                s_p[(lk + e) * L.p_stride + ct * 16 + lr] = (uint32_t)hi | ((uint32_t)lo << 16);
            }
        }
    }
    wave_sync();

    // ---- O_s = P V (P's two bf16 parts), merged with the prefix state ----
    // every dimension tile at once: per key tile the P operands are read once
    // and the eight tiles' products are independent chains
    f32x4 acc[kDTiles];
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) acc[dt] = (f32x4){ 0.0f, 0.0f, 0.0f, 0.0f };
    const uint32_t* pa = s_p + lr * L.p_stride + lk;
    const uint16_t* vb = s_vt + lr * L.vt_stride + lk;
    for (int ks = 0; ks < ktiles; ++ks) {
        const uint4 pw = *reinterpret_cast<const uint4*>(pa + ks * 16);
        bf16x4 bv[kDTiles];
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt)
            bv[dt] = *reinterpret_cast<const bf16x4*>(vb + (size_t)dt * 16 * L.vt_stride + ks * 16);
        bf16x4 hi, lo;
        hi.x = (short)(pw.x & 0xFFFFu); hi.y = (short)(pw.y & 0xFFFFu); hi.z = (short)(pw.z & 0xFFFFu); hi.w = (short)(pw.w & 0xFFFFu);
        lo.x = (short)(pw.x >> 16); lo.y = (short)(pw.y >> 16); lo.z = (short)(pw.z >> 16); lo.w = (short)(pw.w >> 16);
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt) acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, bv[dt], acc[dt], 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt) acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, bv[dt], acc[dt], 0, 0, 0);
    }
    uint16_t opr[kDTiles][4];
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) opr[dt][e] = s_op[(lk + e) * kAttnKRow + dt * 16 + lr];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (ctok[e] < 0) continue;
        uint16_t* orow = out + ctok[e] * kAttnD + lr;
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt)
            orow[dt * 16] = to_bf16(wp[e] * __uint_as_float((uint32_t)opr[dt][e] << 16) + ws[e] * acc[dt][e]);
    }
}

}  // namespace

hipError_t launch_tree_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o_prefix,
                                 const float* lse_prefix, const int32_t* node_parent, const int32_t* num_nodes,
                                 int32_t batch, int32_t n, int32_t Hq, int32_t Hkv, float scale, uint16_t* out,
                                 float* out_lse, hipStream_t stream)
{
    if (batch == 0) return hipSuccess;
    // query rows per workgroup: 64 (a 16-row tile per wave), or fewer when the
    // batch gives too few workgroups to spread over the chip (one request: 16)
    const int64_t rows = (int64_t)n * (Hq / Hkv);
    int rows_wg = kAttnRows;
    while (rows_wg > 16 && (int64_t)batch * Hkv * ((rows + rows_wg - 1) / rows_wg) < 512) rows_wg /= 2;
    const int64_t blocks = (rows + rows_wg - 1) / rows_wg;
    const size_t lds = attn_lds(n).total;
    if (lds > 65536) {
        // beyond the default dynamic LDS limit (trees of more than about 70
        // nodes): raised once per process to what the largest tree needs
        static std::once_flag once;
        static hipError_t raised = hipSuccess;
        std::call_once(once, [] {
            const int most = (int)attn_lds(kAttnMaxTreeNodes).total;
            const void* fns[] = { reinterpret_cast<const void*>(&tree_attention_kernel<1>),
                                  reinterpret_cast<const void*>(&tree_attention_kernel<2>),
                                  reinterpret_cast<const void*>(&tree_attention_kernel<3>),
                                  reinterpret_cast<const void*>(&tree_attention_kernel<4>),
                                  reinterpret_cast<const void*>(&tree_attention_kernel<5>),
                                  reinterpret_cast<const void*>(&tree_attention_kernel<6>),
                                  reinterpret_cast<const void*>(&tree_attention_kernel<7>),
                                  reinterpret_cast<const void*>(&tree_attention_kernel<8>),
                                  reinterpret_cast<const void*>(&tree_attention_kernel<9>) };
            for (const void* f : fns)
                if (raised == hipSuccess)
                    raised = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, most);
        });
        if (raised != hipSuccess) return raised;
    }
    const dim3 grid((unsigned)batch, (unsigned)Hkv, (unsigned)blocks);
    switch ((n + 15) / 16) {
#define UNO_ATTN_CASE(KT)                                                                                            \
    case KT:                                                                                                         \
        tree_attention_kernel<KT><<<grid, kAttnThreads, lds, stream>>>(q, k, v, o_prefix, lse_prefix, node_parent,   \
                                                                       num_nodes, n, Hq, Hkv, scale, rows_wg, out,   \
                                                                       out_lse);                                     \
        break;
        UNO_ATTN_CASE(1)
        UNO_ATTN_CASE(2)
        UNO_ATTN_CASE(3)
        UNO_ATTN_CASE(4)
        UNO_ATTN_CASE(5)
        UNO_ATTN_CASE(6)
        UNO_ATTN_CASE(7)
        UNO_ATTN_CASE(8)
        UNO_ATTN_CASE(9)
#undef UNO_ATTN_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace uno
