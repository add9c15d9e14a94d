// Stand-ins for the few HIP runtime calls and kernel launchers that the
// host-side C ABI (gr_attn_api.cpp) makes, so that it can be built with g++
// under AddressSanitizer and UndefinedBehaviorSanitizer and run on a machine
// without a GPU.  The device queries report one gfx950 device; every
// launcher checks the launch it is given against the buffers the caller
// passed (recorded for the test program in `g_call`) and enqueues nothing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "gr_attn_internal.h"
#include "stub_state.h"

StubCall g_call;
long g_launches = 0;

#define REQUIRE(c)                                                                       \
    do {                                                                                 \
        if (!(c)) {                                                                      \
            std::fprintf(stderr, "launch check failed at %s:%d: %s\n", __FILE__, __LINE__, #c); \
            std::abort();                                                                \
        }                                                                                \
    } while (0)

extern "C" hipError_t hipGetDeviceCount(int *n)
{
    *n = 1;
    return hipSuccess;
}

extern "C" hipError_t hipGetDevice(int *d)
{
    *d = 0;
    return hipSuccess;
}

extern "C" hipError_t hipGetDeviceProperties(hipDeviceProp_t *prop, int dev)
{
    std::memset(prop, 0, sizeof(*prop));
    std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
    return dev == 0 ? hipSuccess : hipErrorInvalidDevice;
}

namespace gr {

// The fused grid: every workgroup id decodes to (pair, query tile, split)
// inside the unit range, and every split's wave partials lie inside the
// caller's workspace.
hipError_t launch_fused(const Params &p, int nqt, int nks, int grid, hipStream_t)
{
    ++g_launches;
    REQUIRE(grid > 0 && nqt > 0 && nks > 0 && p.n_split >= 1 && p.n_split <= 8);
    REQUIRE(fused_lds_bytes(p.D, nqt, nks) > 0);
    const int64_t pairs = (int64_t)p.B * p.Hkv;
    REQUIRE((int64_t)grid == 8 * ((pairs + 7) / 8) * p.n_qt * p.n_split);
    REQUIRE((int64_t)p.n_qt * 32 * nqt >= (int64_t)g_call.W_max * p.G);
    if (p.n_split > 1) {
        const uintptr_t ws = (uintptr_t)g_call.workspace, end = ws + g_call.workspace_bytes;
        const size_t units = (size_t)pairs * p.n_qt;
        REQUIRE((uintptr_t)p.ws_count >= ws && (uintptr_t)(p.ws_count + units) <= end);
        const size_t part = units * p.n_split * nqt * (size_t)fused_part_bytes(p.D);
        REQUIRE((uintptr_t)p.ws_part >= (uintptr_t)(p.ws_count + units) &&
                (uintptr_t)p.ws_part + part <= end);
    }
    return hipSuccess;
}

// The 16-row-wave grid: one workgroup per (pair, 16*nqt-row tile), no split.
hipError_t launch_fused16(const Params &p, int nqt, int nks, int grid, hipStream_t)
{
    ++g_launches;
    REQUIRE(grid > 0 && nqt > 0 && nks > 0 && p.n_split == 1);
    REQUIRE(fused16_lds_bytes(p.D, nqt, nks) > 0);
    const int64_t pairs = (int64_t)p.B * p.Hkv;
    REQUIRE((int64_t)grid == 8 * ((pairs + 7) / 8) * p.n_qt);
    REQUIRE((int64_t)p.n_qt * 16 * nqt >= (int64_t)g_call.W_max * p.G);
    return hipSuccess;
}

hipError_t launch_generic(const Params &p, hipStream_t)
{
    ++g_launches;
    REQUIRE(p.ctx_cap + p.T_cap <= GENERIC_MAX_KEYS);
    return hipSuccess;
}

hipError_t launch_check(const MetaCheck &, hipStream_t)
{
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_beam_step(const StepParams &p, hipStream_t)
{
    ++g_launches;
    REQUIRE(p.B > 0 && p.Hkv > 0 && (p.D == 64 || p.D == 128));
    return hipSuccess;
}

// The selection's six workspace tables lie inside the caller's workspace.
hipError_t launch_beam_select(const SelParams &p, hipStream_t)
{
    ++g_launches;
    const uintptr_t ws = (uintptr_t)g_call.workspace, end = ws + g_call.workspace_bytes;
    const size_t R = (size_t)p.R_old;
    REQUIRE((uintptr_t)p.ws_list >= ws);
    REQUIRE((uintptr_t)(p.ws_e0 + R) <= end);
    REQUIRE((uintptr_t)(p.ws_surv + R * (size_t)p.K_max) <= (uintptr_t)p.ws_n);
    return hipSuccess;
}

// The no-alloc scratch: a host array standing in for the device one, of the
// same size, so that the stubbed launch can check the split's layout in it.
static char g_scratch[NOALLOC_SCRATCH_BYTES] __attribute__((aligned(256)));

hipError_t noalloc_scratch(void **out, hipStream_t)
{
    *out = g_scratch;
    g_call.workspace = g_scratch;
    g_call.workspace_bytes = NOALLOC_SCRATCH_BYTES;
    return hipSuccess;
}

}  // namespace gr
