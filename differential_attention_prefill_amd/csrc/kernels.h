// Internal launch interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/diffattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace diffattn {

// Arguments of one V1-layout prefill launch, already validated by the caller.
struct PrefillArgs {
    const void* q1;
    const void* q2;
    const void* k1;
    const void* k2;
    const void* v;
    int64_t ldq, ldk, ldv;   // elements between consecutive tokens
    int B, H, N, d, dv;
    int causal;
    const float* lambda;     // [H]
    int rmsnorm;
    float eps, norm_scale;
    const float* norm_weight;  // [dv] or nullptr
    float* out;              // [B][H][N][dv]
};

// Arguments of one V2-layout decode launch, already validated by the caller.
struct DecodeArgs {
    const void* q;           // bf16 [B][Hq][D]
    const void* k_cache;     // bf16 [B][Hkv][max_len][D]
    const void* v_cache;
    const int32_t* seq_lens; // [B]
    int B, Hq, Hkv, D, max_len;
    const float* lambda;     // [Hq/2]
    float* workspace;        // partial states, see decode_workspace_floats
    float* out;              // [B][Hq/2][D]
};

hipError_t launch_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                         int H, int dim, double lambda_init, float* out, hipStream_t stream);

bool prefill_bf16_supported(int d, int dv);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
// Ping-pong schedule (d <= 64); launch_prefill_bf16 dispatches to it.
bool prefill_pp_supported(int d, int dv);
hipError_t launch_prefill_pp(const PrefillArgs& a, hipStream_t stream);

bool prefill_f32_supported(int d, int dv);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);

bool decode_supported(int D);
int decode_max_splits(int max_len);
size_t decode_workspace_floats(int B, int Hq, int D, int max_len);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace diffattn
