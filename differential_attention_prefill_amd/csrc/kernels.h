// Internal launch interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/diffattn.h.  The
// shape predicates and workspace sizing are plain host code (shapes.cpp); the
// launch_* functions live with their kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "diffattn.h"

namespace diffattn {

// Where the rows of diff head (b, h) start, in elements: q1 and q2 at
// b*qb + h*qh, k1 and k2 at b*kb + g*kh, v at b*vb + g*vh, with K/V head
// g = h / kv_group.  Rows within a head are ldq / ldk / ldv apart.
struct HeadStrides {
    int64_t qb, qh;
    int64_t kb, kh;
    int64_t vb, vh;
    int kv_group;
};

// Arguments of one prefill launch, already validated by the caller.
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
    HeadStrides hs;
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
    // V1 layout when qhalf > 0: q is [B][Hkv][D] packed [q1 | q2] with
    // qhalf = d = D/2, Hq = 2*Hkv, and the caches hold [k1 | k2] and v rows.
    int qhalf = 0;
    int rmsnorm = 0;
    float eps = 0.f, norm_scale = 1.f;
    const float* norm_weight = nullptr;   // [D] or null
    // Plain single-map attention when single != 0: every query head is its
    // own softmax over its KV head's rows, out [B][Hq][D], lambda unused.
    int single = 0;
};

hipError_t launch_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                         int H, int dim, double lambda_init, float* out, hipStream_t stream);

bool prefill_bf16_supported(int d, int dv);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
// Single-map softmax attention on the same schedule (q1, k1, v; out = A V).
bool attention_pp_supported(int d, int dv);
hipError_t launch_attention_pp(const PrefillArgs& a, hipStream_t stream);

// out = o1 - lambda_h * o2 per row of [B][H][N][dv], then the optional RMS
// norm (rmsnorm, eps, norm_scale, norm_weight as for prefill).
hipError_t launch_combine(const float* o1, const float* o2, const float* lambda, int B, int H,
                          int N, int dv, int rmsnorm, float eps, float norm_scale,
                          const float* norm_weight, float* out, hipStream_t stream);

bool prefill_f32_supported(int d, int dv);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);

// Decode geometry shared by the kernels and the host-side sizing (shapes.cpp).
constexpr int DECODE_D = 128;            // head width the decode kernels are built for
constexpr int DECODE_RANGE_MIN = 4096;   // shortest key range per split workgroup
constexpr int DECODE_STATE = DECODE_D + 2;   // floats per partial state: O[D], m*c, l

bool decode_supported(int D);
// Pieces (partial states) one (sequence, KV head) segment can be cut into.
int decode_max_splits(int max_len);
// Floats of partial states [B][Hq][decode_max_splits][DECODE_STATE]; the
// piece counts (one int32 per (sequence, query head) slot) follow them.
size_t decode_state_floats(int B, int Hq, int max_len);
size_t decode_workspace_floats(int B, int Hq, int D, int max_len);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// The same decode with its partial states in the library's fixed per-device
// scratch array (a.workspace is ignored); the caller has checked that the
// workspace size fits DECODE_SCRATCH_BYTES.
constexpr size_t DECODE_SCRATCH_BYTES = DIFFATTN_DECODE_SCRATCH_BYTES;
hipError_t launch_decode_noalloc(const DecodeArgs& a, hipStream_t stream);

}  // namespace diffattn
