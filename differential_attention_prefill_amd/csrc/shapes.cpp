// Host-side shape logic of libdiffattn: which (d, dv) each kernel family is
// built for, and the decode workspace layout.  Plain C++ with no HIP calls,
// shared by the library and by the host-only sanitizer build of the C ABI.
#include "kernels.h"

namespace diffattn {

// Instantiations of the fused bf16 prefill kernels (prefill_pp.hip).
bool prefill_bf16_supported(int d, int dv) {
    return (d == 64 && dv == 128) || (d == 64 && dv == 64) || (d == 32 && dv == 64) ||
           (d == 128 && dv == 128);
}

// Single-map instantiations of the same schedule (the unfused path).
bool attention_pp_supported(int d, int dv) {
    return (d == 64 && dv == 128) || (d == 64 && dv == 64);
}

// Instantiations of the fp32 vector-ALU prefill (prefill_f32.hip).
bool prefill_f32_supported(int d, int dv) {
    return (d == 32 || d == 64 || d == 128) && (dv == 64 || dv == 128);
}

bool decode_supported(int D) { return D == DECODE_D; }

// A segment of L <= max_len keys meets at most ceil(L / R) + 1 key ranges of
// R >= DECODE_RANGE_MIN keys.
int decode_max_splits(int max_len) {
    return (max_len + DECODE_RANGE_MIN - 1) / DECODE_RANGE_MIN + 1;
}

size_t decode_state_floats(int B, int Hq, int max_len) {
    return (size_t)B * Hq * decode_max_splits(max_len) * DECODE_STATE;
}

size_t decode_workspace_floats(int B, int Hq, int D, int max_len) {
    (void)D;
    return decode_state_floats(B, Hq, max_len) + (size_t)B * Hq;
}

}  // namespace diffattn
