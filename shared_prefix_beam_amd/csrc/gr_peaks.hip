// Measured denominators for the roofline fractions (entry points declared in
// gr_peaks.h): sustained bf16 matrix throughput, streaming HBM copy and read
// bandwidth, and the fp32 exp2 rate of one gfx950.  These kernels are
// measurement probes, not part of the decode path; the benchmark reports
// their figures beside the vendor peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gr_peaks {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave,
// so the matrix pipe never waits on a result; 32768 flops per instruction.
__global__ __launch_bounds__(THREADS) void mfma_chain(float *out, int iters)
{
    const int t = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)((t + i) & 7));
        b[i] = (__bf16)(0.001f * (float)((t * 3 + i) & 7));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        s += c0[i] + c1[i] + c2[i] + c3[i];
    out[blockIdx.x * THREADS + t] = s;
}

// Eight independent chains x <- 2^-x per lane (x stays in [0.5, 1]).
__global__ __launch_bounds__(THREADS) void exp2_chain(float *out, int iters)
{
    const int t = threadIdx.x;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        x[j] = 0.5f + 0.01f * (float)((t + j) & 15);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = __builtin_amdgcn_exp2f(-x[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        s += x[j];
    out[blockIdx.x * THREADS + t] = s;
}

// Grid-stride streaming copy and read of n 16-byte words.
__global__ __launch_bounds__(THREADS) void stream_copy(const u32x4 *src, u32x4 *dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

__global__ __launch_bounds__(THREADS) void stream_read(const u32x4 *src, int64_t n, uint32_t *out)
{
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n; i += stride) {
        const u32x4 v = src[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[blockIdx.x * THREADS + threadIdx.x] = acc;
}

}  // namespace gr_peaks

extern "C" {

// Each entry point enqueues one launch on `stream` and returns the HIP
// status (0 = success).  `out` holds grid * 256 elements (caller-owned
// device memory); the copy buffers hold n 16-byte words each.
int gr_peak_mfma(float *out, int grid, int iters, void *stream)
{
    if (!out || grid <= 0 || iters <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(gr_peaks::mfma_chain, dim3(grid), dim3(gr_peaks::THREADS), 0,
                       static_cast<hipStream_t>(stream), out, iters);
    return (int)hipGetLastError();
}

int gr_peak_exp2(float *out, int grid, int iters, void *stream)
{
    if (!out || grid <= 0 || iters <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(gr_peaks::exp2_chain, dim3(grid), dim3(gr_peaks::THREADS), 0,
                       static_cast<hipStream_t>(stream), out, iters);
    return (int)hipGetLastError();
}

int gr_peak_copy(const void *src, void *dst, int64_t n16, int grid, void *stream)
{
    if (!src || !dst || n16 <= 0 || grid <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(gr_peaks::stream_copy, dim3(grid), dim3(gr_peaks::THREADS), 0,
                       static_cast<hipStream_t>(stream),
                       static_cast<const gr_peaks::u32x4 *>(src),
                       static_cast<gr_peaks::u32x4 *>(dst), n16);
    return (int)hipGetLastError();
}

int gr_peak_read(const void *src, int64_t n16, uint32_t *out, int grid, void *stream)
{
    if (!src || !out || n16 <= 0 || grid <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(gr_peaks::stream_read, dim3(grid), dim3(gr_peaks::THREADS), 0,
                       static_cast<hipStream_t>(stream),
                       static_cast<const gr_peaks::u32x4 *>(src), n16, out);
    return (int)hipGetLastError();
}

}  // extern "C"
