// Shared between the HIP stub and the host-only C-ABI driver.
#pragma once
#include <stdint.h>

#include "kernels.h"

constexpr uintptr_t STUB_DEV_LO = (uintptr_t)1 << 44;
constexpr uintptr_t STUB_DEV_HI = (uintptr_t)1 << 45;

struct StubRecord {
    char last[32];
    int launches;
    int H, dim;
    double lambda_init;
    diffattn::PrefillArgs prefill;
    diffattn::DecodeArgs decode;
};
extern StubRecord g_stub;
