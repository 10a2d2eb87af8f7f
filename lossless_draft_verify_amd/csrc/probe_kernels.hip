// probe_kernels.hip -- read-only streaming reference for the HBM roofline.
//
// Each workgroup reads its own contiguous range once with 16-byte non-temporal
// loads (four per lane per iteration, the next iteration's loads in flight
// while one is folded, each of the four waves a quarter of the range) and does
// nothing with the data but fold it into one word, so its duration is what
// streaming those bytes costs on this chip.  With one range per logit row it
// has the top-k stream's decomposition; with many equal ranges it measures the
// chip's streaming rate.
#include "uno_device.h"
#include "uno_internal.h"

namespace uno {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeWaves = kProbeThreads / kWave;
constexpr int kProbeU = 4;              // 16-byte vectors per lane per iteration

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* buf, int64_t nvec, int64_t wg_vec,
                                                                   uint32_t* out)
{
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t b0 = (int64_t)blockIdx.x * wg_vec;
    const int64_t b1 = (b0 + wg_vec < nvec) ? b0 + wg_vec : nvec;
    const int64_t wb = b0 + (b1 - b0) * w / kProbeWaves, we = b0 + (b1 - b0) * (w + 1) / kProbeWaves;
    constexpr int64_t kStep = (int64_t)kProbeU * kWave;
    const int64_t nfull = (we - wb) / kStep;
    uint32_t acc = 0;
    // two buffers in turn, each at a fixed place: copying the next buffer into
    // the current one would wait on its loads (111.3 against 102.5 us for the
    // 1088-row split of 661 MB)
    uint4 xa[kProbeU], xb[kProbeU];
    if (nfull > 0) {
#pragma unroll
        for (int u = 0; u < kProbeU; ++u) xa[u] = Vec<true>::load_stream(buf + wb + u * kWave + lane);
    }
    auto step = [&](int64_t it, uint4 (&cur)[kProbeU], uint4 (&nxt)[kProbeU]) __attribute__((always_inline)) {
        const bool more = it + 1 < nfull;
        const uint4* pn = buf + wb + (more ? (it + 1) * kStep : it * kStep) + lane;
#pragma unroll
        for (int u = 0; u < kProbeU; ++u) nxt[u] = Vec<true>::load_stream(pn + u * kWave);
#pragma unroll
        for (int u = 0; u < kProbeU; ++u) acc ^= cur[u].x ^ cur[u].y ^ cur[u].z ^ cur[u].w;
    };
    for (int64_t it = 0; it < nfull; it += 2) {
        step(it, xa, xb);
        if (it + 1 < nfull) step(it + 1, xb, xa);
    }
    for (int64_t v = wb + nfull * kStep + lane; v < we; v += kWave) {
        const uint4 x = Vec<true>::load_stream(buf + v);
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, kWave);
    __shared__ uint32_t s_acc[kProbeWaves];
    if (lane == 0) s_acc[w] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, int64_t wg_bytes, uint32_t* out, hipStream_t stream)
{
    const int64_t nvec = bytes / 16, wg_vec = wg_bytes / 16;
    const int64_t groups = (nvec + wg_vec - 1) / wg_vec;
    stream_read_kernel<<<dim3((unsigned)groups), kProbeThreads, 0, stream>>>(static_cast<const uint4*>(buf), nvec,
                                                                           wg_vec, out);
    return hipGetLastError();
}

}  // namespace uno
