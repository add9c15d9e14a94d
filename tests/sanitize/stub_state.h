// What the sanitizer test program tells the launch stubs about the current call.
#pragma once
#include <cstddef>
#include <cstdint>

struct StubCall {
    const void *workspace;
    size_t workspace_bytes;
    int32_t W_max;
};
extern StubCall g_call;
extern long g_launches;
