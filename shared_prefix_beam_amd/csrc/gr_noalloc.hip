// Device scratch of gr_decode_attn_noalloc: the context-split counters and
// partials live in one file-scope device array, so that the call allocates
// nothing (for callers that cannot allocate: code under graph capture,
// serving loops that forbid it).  Each device holds its own copy of the
// array at its own address; the host looks that address up once per device
// (with the device current) and passes it to the kernels like a workspace.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "gr_attn_internal.h"

namespace gr {

static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

__global__ void zero_words(uint32_t *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];
bool g_cleared[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void **out, hipStream_t s)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    if (!g_cleared[dev]) {
        // the counters must start at zero (each call leaves them at zero);
        // cleared with a kernel, ahead of the first call on this stream
        constexpr int n = NOALLOC_COUNTER_BYTES / 4;
        hipLaunchKernelGGL(zero_words, dim3((n + 255) / 256), dim3(256), 0, s,
                           static_cast<uint32_t *>(g_ptr[dev]), n);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        g_cleared[dev] = true;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace gr
