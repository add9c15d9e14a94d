// Device code of one decode step of the per-beam state: BeamKV append and
// BeamPath update (GR-Inference blog, section on system design: BeamKV holds
// the short per-beam history and BeamPath records beam forking and reordering
// by index, so the long context is never copied; xGR review, section
// "xAttention": the unshared cache is managed per token through direct
// indices, with no block copies).
//
// gfx950 mapping: one wave per new beam row, four rows per workgroup.  The
// wave finds its request by a binary search of row_offset_new (wave-uniform
// scalar loads), copies its parent's path entries (one int per lane), and
// copies its current token's K and V rows (Hkv*D bf16 each, contiguous in
// source and destination) with 16-byte vector loads and stores, so both
// sides are fully coalesced.  The kernel is a copy: HBM-bound.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gr_attn_internal.h"

namespace gr {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t cint32;

// Wave-uniform reads of metadata that this kernel never writes, through the
// constant address space: scalar loads, counted apart from the vector loads
// of the K/V rows, so that they do not wait for each other.
__device__ __forceinline__ int ld_uniform(const int32_t *p, int64_t i)
{
    return ((cint32 *)(uintptr_t)p)[i];
}

constexpr int STEP_ROWS = 4;   // beam rows (waves) per workgroup
constexpr int PRE = 2;         // K/V chunks per lane loaded ahead (rows of up to 1024 bf16)

__global__ __launch_bounds__(64 * STEP_ROWS) void beam_step(const StepParams p)
{
    // the first workgroup also writes every request's new path length
    if (blockIdx.x == 0) {
        for (int b = threadIdx.x; b < p.B; b += 64 * STEP_ROWS) {
            const int w_new = p.row_offset_new[b + 1] - p.row_offset_new[b];
            p.len_new[b] = w_new > 0 ? p.len_old[b] + 1 : p.len_old[b];
        }
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * STEP_ROWS + wave;
    if (r >= p.R_new)
        return;

    // The new token's K and V rows depend on r alone: their first PRE
    // 16-byte chunks per lane are loaded before the metadata chain (request,
    // length, parent, path), so both latencies overlap.
    const int64_t row = (int64_t)p.Hkv * p.D;            // bf16 elements per token
    const int n16 = (int)(row / 8);                      // 16-byte chunks per token
    const u32x4_t *sk = reinterpret_cast<const u32x4_t *>(p.new_k + (int64_t)r * row);
    const u32x4_t *sv = reinterpret_cast<const u32x4_t *>(p.new_v + (int64_t)r * row);
    u32x4_t kk[PRE], vv[PRE];
#pragma unroll
    for (int i = 0; i < PRE; ++i) {
        const int c = lane + 64 * i;
        kk[i] = c < n16 ? sk[c] : u32x4_t{0, 0, 0, 0};
        vv[i] = c < n16 ? sv[c] : u32x4_t{0, 0, 0, 0};
    }

    // request b with row_offset_new[b] <= r < row_offset_new[b+1]: the
    // invariant holds for lo = 0, hi = B and every halving keeps it
    int lo = 0, hi = p.B;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ld_uniform(p.row_offset_new, mid) <= r)
            lo = mid;
        else
            hi = mid;
    }
    const int b = lo;
    const int k = r - ld_uniform(p.row_offset_new, b);
    const int s = ld_uniform(p.len_old, b);
    const int ro_b = ld_uniform(p.row_offset_old, b);
    const int w_old = ld_uniform(p.row_offset_old, b + 1) - ro_b;
    const int par = s > 0 ? ld_uniform(p.parent, r) : 0;
    const int src_row = ro_b + par;
    const int64_t slot = (int64_t)s * p.W_cap + k;
    // the last two terms only matter for row offsets that break their
    // precondition: they keep every access inside its buffer
    const bool ok = s >= 0 && s < p.T_cap && k < p.W_cap && slot < p.beam_cap &&
                    (s == 0 || (par >= 0 && par < w_old)) && k >= 0 &&
                    (s == 0 || (src_row >= 0 && src_row < p.R_old));
    if (!ok) {
        if (lane == 0 && p.violations)
            atomicAdd(p.violations, 1);
        return;
    }

    // BeamPath: the parent's first s entries, then this beam's own slot
    int32_t *dst_path = p.path_new + (int64_t)r * p.T_cap;
    if (s > 0) {
        const int32_t *src_path = p.path_old + (int64_t)src_row * p.T_cap;
        for (int t = lane; t < s; t += 64)
            dst_path[t] = src_path[t];
    }
    if (lane == 0)
        dst_path[s] = (int32_t)slot;

    // BeamKV append: the current token's K and V rows, all KV heads
    u32x4_t *dk = reinterpret_cast<u32x4_t *>(p.beam_k + ((int64_t)b * p.beam_cap + slot) * row);
    u32x4_t *dv = reinterpret_cast<u32x4_t *>(p.beam_v + ((int64_t)b * p.beam_cap + slot) * row);
#pragma unroll
    for (int i = 0; i < PRE; ++i) {
        const int c = lane + 64 * i;
        if (c < n16) {
            dk[c] = kk[i];
            dv[c] = vv[i];
        }
    }
    for (int c = lane + 64 * PRE; c < n16; c += 64) {   // rows beyond PRE*64 chunks
        const u32x4_t k2 = sk[c];
        const u32x4_t v2 = sv[c];
        dk[c] = k2;
        dv[c] = v2;
    }
}

hipError_t launch_beam_step(const StepParams &p, hipStream_t s)
{
    const int grid = (p.R_new + STEP_ROWS - 1) / STEP_ROWS;
    hipLaunchKernelGGL(beam_step, dim3(grid > 0 ? grid : 1), dim3(64 * STEP_ROWS), 0, s, p);
    return hipGetLastError();
}

}  // namespace gr
