// Test double for a host-only build of the C-ABI layer (api.cpp + shapes.cpp)
// under the address, undefined-behaviour and thread sanitizers.  It replaces
// the three HIP runtime calls api.cpp makes and the kernel launchers: no GPU
// code is built or run.  Addresses in [STUB_DEV_LO, STUB_DEV_HI) count as
// device memory; the launchers only record their arguments for the driver.
#include <hip/hip_runtime.h>

#include <cstring>

#include "kernels.h"
#include "hip_stub.h"

StubRecord g_stub;

extern "C" hipError_t hipPointerGetAttributes(hipPointerAttribute_t* attr, const void* ptr) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(ptr);
    if (a < STUB_DEV_LO || a >= STUB_DEV_HI) return hipErrorInvalidValue;
    std::memset(attr, 0, sizeof *attr);
    attr->type = hipMemoryTypeDevice;
    return hipSuccess;
}
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace diffattn {

static hipError_t record(const char* what) {
    std::strncpy(g_stub.last, what, sizeof g_stub.last - 1);
    g_stub.launches++;
    return hipSuccess;
}

hipError_t launch_lambda(const float*, const float*, const float*, const float*, int H, int dim,
                         double lambda_init, float*, hipStream_t) {
    g_stub.H = H;
    g_stub.dim = dim;
    g_stub.lambda_init = lambda_init;
    return record("lambda");
}
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t) {
    g_stub.prefill = a;
    return record("prefill_bf16");
}
hipError_t launch_attention_pp(const PrefillArgs& a, hipStream_t) {
    g_stub.prefill = a;
    return record("attention_pp");
}
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t) {
    g_stub.prefill = a;
    return record("prefill_f32");
}
hipError_t launch_combine(const float*, const float*, const float*, int, int, int, int dv, int,
                          float, float, const float*, float*, hipStream_t) {
    g_stub.dim = dv;
    return record("combine");
}
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
    g_stub.decode = a;
    return record("decode");
}
hipError_t launch_decode_noalloc(const DecodeArgs& a, hipStream_t) {
    g_stub.decode = a;
    return record("decode_noalloc");
}

}  // namespace diffattn
