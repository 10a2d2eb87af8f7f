// uno_noalloc.cpp -- allocation-free variant of uno_sample_linear for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Its workspace is a
// file-scope device array of fixed size; every call on one GPU shares that
// GPU's copy.
#include "uno.h"

#include <hip/hip_runtime.h>

#include <mutex>

// The workspace of uno_sample_linear_noalloc.  Host code never passes this
// name to a kernel or a copy: on the host it is only a handle for the symbol
// lookup below, which yields the device's own address of its copy.
static __device__ __align__(256) unsigned char scratch[UNO_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = (size_t)UNO_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_lock;
void* g_scratch[kMaxDevices];        // per device: the address of its copy of `scratch`

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current.
int scratch_address(hipStream_t stream, void** out)
{
    int dev = -1;
    if (stream == nullptr || hipStreamGetDevice(stream, &dev) != hipSuccess) {
        if (hipGetDevice(&dev) != hipSuccess) return UNO_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return UNO_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> g(g_lock);
    if (g_scratch[dev] == nullptr) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return UNO_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return UNO_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return UNO_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return UNO_OK;
}

}  // namespace

extern "C" int uno_sample_linear_noalloc(const void* draft, const void* target, int32_t dtype, int32_t batch,
                                         int32_t B, int64_t vocab, const uno_sampling_t* sp, uint64_t seed,
                                         uint64_t offset, const uint32_t* request_ids, int32_t* out_tokens,
                                         int32_t* out_accept_len, int32_t* out_proposals, uint32_t* out_flags,
                                         hipStream_t stream)
{
    size_t need = 0;
    int st = uno_workspace_bytes(UNO_OP_SAMPLE_LINEAR, batch, B, 1, B, vocab, dtype, sp, &need);
    if (st != UNO_OK) return st;
    if (need > kScratchBytes) return UNO_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_address(stream, &ws);
        if (st != UNO_OK) return st;
    }
    // the sampling path reads nothing from its workspace that it has not
    // written in the same call, so the last call's contents need no clearing
    return uno_sample_linear(draft, target, dtype, batch, B, vocab, sp, seed, offset, request_ids, out_tokens,
                             out_accept_len, out_proposals, out_flags, ws, kScratchBytes, stream);
}
