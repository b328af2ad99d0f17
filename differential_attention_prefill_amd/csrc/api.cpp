// C ABI of libdiffattn: argument validation and dispatch to the HIP kernels.
// The contract of every entry point is documented in include/diffattn.h.
#include "diffattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

diffattn_status_t fail(diffattn_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

diffattn_status_t ok() {
    g_last_error[0] = '\0';
    return DIFFATTN_OK;
}

// True if p is device (or managed) memory the current device can address.
// Runs only after every pure-argument check, so argument errors are reported
// without touching the HIP runtime.
bool is_device_ptr(const void* p) {
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // an unknown pointer is not a sticky error
        return false;
    }
    return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged ||
           attr.type == hipMemoryTypeUnified;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

diffattn_status_t check_device(const void* p, const char* name) {
    if (!is_device_ptr(p))
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "%s is not device memory", name);
    return DIFFATTN_OK;
}

// The bf16 kernels address a tile of 64 token rows with 32-bit byte offsets
// (copy offsets, tile strides and buffer extents of up to 64 * ld * 2
// bytes), so every token stride must keep 64 rows below 2^31 bytes.
constexpr int64_t BF16_MAX_LD = ((int64_t)1 << 31) / (64 * 2) - 1;

bool bf16_ld_ok(int64_t ldq, int64_t ldk, int64_t ldv) {
    return ldq <= BF16_MAX_LD && ldk <= BF16_MAX_LD && ldv <= BF16_MAX_LD;
}

// The kernels run 1-D grids of at most 2^31 - 1 workgroups, one per `rows`
// query rows of one (b, h): at least 128 rows for the bf16 prefill kernels,
// 32 for the fp32 kernel, 4 for the combine kernel.  The caller has bounded
// B*H*N by 2^40, so the products stay in int64.
constexpr int64_t MAX_GRID = 0x7fffffff;

bool grid_fits(int B, int H, int N, int rows) {
    return (int64_t)B * H * (((int64_t)N + rows - 1) / rows) <= MAX_GRID;
}

diffattn_status_t hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(DIFFATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

double diffattn_lambda_init(int layer) {
    if (layer < 1) return NAN;
    return 0.8 - 0.6 * std::exp(-0.3 * (double)(layer - 1));
}

diffattn_status_t diffattn_lambda(const float* lq1, const float* lk1, const float* lq2,
                                  const float* lk2, int H, int dim, int layer, float* lambda_out,
                                  void* stream) {
    if (!lq1 || !lk1 || !lq2 || !lk2 || !lambda_out)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_lambda: null pointer");
    if (H < 1 || dim < 1)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_lambda: H=%d dim=%d must be >= 1", H, dim);
    if (layer < 1)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_lambda: layer=%d must be >= 1", layer);
    const void* ptrs[5] = {lq1, lk1, lq2, lk2, lambda_out};
    const char* names[5] = {"lq1", "lk1", "lq2", "lk2", "lambda_out"};
    for (int i = 0; i < 5; ++i) {
        diffattn_status_t s = check_device(ptrs[i], names[i]);
        if (s != DIFFATTN_OK) return s;
    }
    return hip_status(diffattn::launch_lambda(lq1, lk1, lq2, lk2, H, dim, diffattn_lambda_init(layer),
                                              lambda_out, (hipStream_t)stream),
                      "diffattn_lambda launch");
}

diffattn_status_t diffattn_prefill(const void* q1, const void* q2, const void* k1, const void* k2,
                                   const void* v, int64_t ldq, int64_t ldk, int64_t ldv,
                                   int dtype, int B, int H, int N, int d, int dv,
                                   int causal, const float* lambda, int rmsnorm, float eps,
                                   float norm_scale, const float* norm_weight, float* out,
                                   void* stream) {
    if (!q1 || !q2 || !k1 || !k2 || !v || !lambda || !out)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill: null pointer");
    if (B < 1 || H < 1 || N < 1 || d < 1 || dv < 1)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_prefill: B=%d H=%d N=%d d=%d dv=%d must be >= 1", B, H, N, d, dv);
    if (dtype != DIFFATTN_FP32 && dtype != DIFFATTN_BF16)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill: unknown dtype %d", dtype);
    if (ldq < d || ldk < d || ldv < dv)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_prefill: strides ldq=%lld ldk=%lld ldv=%lld below widths d=%d dv=%d",
                    (long long)ldq, (long long)ldk, (long long)ldv, d, dv);
    const int esize = dtype == DIFFATTN_BF16 ? 2 : 4;
    if ((ldq * esize) % 16 || (ldk * esize) % 16 || (ldv * esize) % 16)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_prefill: token strides must be multiples of 16 bytes");
    const void* ptrs[7] = {q1, q2, k1, k2, v, out, lambda};
    const char* names[7] = {"q1", "q2", "k1", "k2", "v", "out", "lambda"};
    for (int i = 0; i < 6; ++i)   // vector-loaded tensors; lambda is read as scalars
        if (!aligned16(ptrs[i]))
            return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill: %s not 16-byte aligned",
                        names[i]);
    if ((reinterpret_cast<uintptr_t>(lambda) & 3u) != 0)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill: lambda not 4-byte aligned");
    if (rmsnorm && !(eps >= 0.f))
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill: eps must be >= 0");
    const bool supported = dtype == DIFFATTN_BF16 ? diffattn::prefill_bf16_supported(d, dv)
                                                  : diffattn::prefill_f32_supported(d, dv);
    if (!supported)
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_prefill: (d=%d, dv=%d) not built for %s", d,
                    dv, dtype == DIFFATTN_BF16 ? "bf16" : "fp32");
    if (dtype == DIFFATTN_BF16 && !bf16_ld_ok(ldq, ldk, ldv))
        return fail(DIFFATTN_ERR_UNSUPPORTED,
                    "diffattn_prefill: bf16 token strides must be at most %lld elements",
                    (long long)BF16_MAX_LD);
    if ((int64_t)B * H * N > (int64_t)1 << 40)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill: B*H*N too large");
    if (!grid_fits(B, H, N, dtype == DIFFATTN_BF16 ? 128 : 32))
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_prefill: B*H row tiles exceed the launch grid");
    for (int i = 0; i < 7; ++i) {
        diffattn_status_t s = check_device(ptrs[i], names[i]);
        if (s != DIFFATTN_OK) return s;
    }
    if (rmsnorm && norm_weight) {
        diffattn_status_t s = check_device(norm_weight, "norm_weight");
        if (s != DIFFATTN_OK) return s;
    }
    diffattn::PrefillArgs a;
    a.q1 = q1; a.q2 = q2; a.k1 = k1; a.k2 = k2; a.v = v;
    a.ldq = ldq; a.ldk = ldk; a.ldv = ldv;
    a.B = B; a.H = H; a.N = N; a.d = d; a.dv = dv;
    a.causal = causal ? 1 : 0;
    a.lambda = lambda;
    a.rmsnorm = rmsnorm ? 1 : 0;
    a.eps = eps;
    a.norm_scale = norm_scale;
    a.norm_weight = rmsnorm ? norm_weight : nullptr;
    a.out = out;
    const int64_t HN = (int64_t)H * N;
    a.hs = {HN * ldq, (int64_t)N * ldq, HN * ldk, (int64_t)N * ldk, HN * ldv, (int64_t)N * ldv, 1};
    hipError_t e = dtype == DIFFATTN_BF16 ? diffattn::launch_prefill_bf16(a, (hipStream_t)stream)
                                          : diffattn::launch_prefill_f32(a, (hipStream_t)stream);
    return hip_status(e, "diffattn_prefill launch");
}

diffattn_status_t diffattn_prefill_v2(const void* q, const void* k, const void* v,
                                      int dtype, int B, int Hq, int Hkv, int N, int D,
                                      int causal, const float* lambda, float* out, void* stream) {
    if (!q || !k || !v || !lambda || !out)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill_v2: null pointer");
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_prefill_v2: B=%d Hq=%d Hkv=%d N=%d D=%d must be >= 1", B, Hq, Hkv, N, D);
    if (Hq % (2 * Hkv) != 0)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_prefill_v2: Hq=%d must be a multiple of 2*Hkv=%d", Hq, 2 * Hkv);
    if (dtype != DIFFATTN_FP32 && dtype != DIFFATTN_BF16)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill_v2: unknown dtype %d", dtype);
    const int esize = dtype == DIFFATTN_BF16 ? 2 : 4;
    if ((D * esize) % 16)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_prefill_v2: rows of D=%d elements must be multiples of 16 bytes", D);
    const void* ptrs[5] = {q, k, v, out, lambda};
    const char* names[5] = {"q", "k", "v", "out", "lambda"};
    for (int i = 0; i < 4; ++i)
        if (!aligned16(ptrs[i]))
            return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill_v2: %s not 16-byte aligned",
                        names[i]);
    if ((reinterpret_cast<uintptr_t>(lambda) & 3u) != 0)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill_v2: lambda not 4-byte aligned");
    const bool supported = dtype == DIFFATTN_BF16 ? diffattn::prefill_bf16_supported(D, D)
                                                  : diffattn::prefill_f32_supported(D, D);
    if (!supported)
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_prefill_v2: D=%d not built for %s", D,
                    dtype == DIFFATTN_BF16 ? "bf16" : "fp32");
    if ((int64_t)B * Hq * N > (int64_t)1 << 40)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_prefill_v2: B*Hq*N too large");
    if (!grid_fits(B, Hq / 2, N, dtype == DIFFATTN_BF16 ? 128 : 32))
        return fail(DIFFATTN_ERR_UNSUPPORTED,
                    "diffattn_prefill_v2: B*Hq/2 row tiles exceed the launch grid");
    for (int i = 0; i < 5; ++i) {
        diffattn_status_t s = check_device(ptrs[i], names[i]);
        if (s != DIFFATTN_OK) return s;
    }
    // Pair p: queries of heads 2p (map 1) and 2p+1 (map 2), over K/V head
    // p / (Hq / (2 Hkv)) for both maps.
    const int64_t ND = (int64_t)N * D;
    diffattn::PrefillArgs a;
    a.q1 = q;
    a.q2 = static_cast<const char*>(q) + ND * esize;
    a.k1 = k; a.k2 = k; a.v = v;
    a.ldq = D; a.ldk = D; a.ldv = D;
    a.B = B; a.H = Hq / 2; a.N = N; a.d = D; a.dv = D;
    a.causal = causal ? 1 : 0;
    a.lambda = lambda;
    a.rmsnorm = 0;
    a.eps = 0.f;
    a.norm_scale = 1.f;
    a.norm_weight = nullptr;
    a.out = out;
    a.hs = {(int64_t)Hq * ND, 2 * ND, (int64_t)Hkv * ND, ND, (int64_t)Hkv * ND, ND, Hq / (2 * Hkv)};
    hipError_t e = dtype == DIFFATTN_BF16 ? diffattn::launch_prefill_bf16(a, (hipStream_t)stream)
                                          : diffattn::launch_prefill_f32(a, (hipStream_t)stream);
    return hip_status(e, "diffattn_prefill_v2 launch");
}

diffattn_status_t diffattn_attention(const void* q, const void* k, const void* v, int64_t ldq,
                                     int64_t ldk, int64_t ldv, int dtype, int B,
                                     int H, int N, int d, int dv, int causal, float* out,
                                     void* stream) {
    if (!q || !k || !v || !out)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_attention: null pointer");
    if (B < 1 || H < 1 || N < 1 || d < 1 || dv < 1)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_attention: B=%d H=%d N=%d d=%d dv=%d must be >= 1", B, H, N, d, dv);
    if (dtype != DIFFATTN_BF16)
        return fail(dtype == DIFFATTN_FP32 ? DIFFATTN_ERR_UNSUPPORTED : DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_attention: bf16 only");
    if (ldq < d || ldk < d || ldv < dv)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_attention: strides below widths");
    if ((ldq * 2) % 16 || (ldk * 2) % 16 || (ldv * 2) % 16)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_attention: token strides must be multiples of 16 bytes");
    const void* ptrs[4] = {q, k, v, out};
    const char* names[4] = {"q", "k", "v", "out"};
    for (int i = 0; i < 4; ++i)
        if (!aligned16(ptrs[i]))
            return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_attention: %s not 16-byte aligned",
                        names[i]);
    if (!diffattn::attention_pp_supported(d, dv))
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_attention: (d=%d, dv=%d) not built", d, dv);
    if (!bf16_ld_ok(ldq, ldk, ldv))
        return fail(DIFFATTN_ERR_UNSUPPORTED,
                    "diffattn_attention: bf16 token strides must be at most %lld elements",
                    (long long)BF16_MAX_LD);
    if ((int64_t)B * H * N > (int64_t)1 << 40)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_attention: B*H*N too large");
    if (!grid_fits(B, H, N, 128))
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_attention: B*H row tiles exceed the launch grid");
    for (int i = 0; i < 4; ++i) {
        diffattn_status_t s = check_device(ptrs[i], names[i]);
        if (s != DIFFATTN_OK) return s;
    }
    diffattn::PrefillArgs a;
    a.q1 = q; a.q2 = q; a.k1 = k; a.k2 = k; a.v = v;
    a.ldq = ldq; a.ldk = ldk; a.ldv = ldv;
    a.B = B; a.H = H; a.N = N; a.d = d; a.dv = dv;
    a.causal = causal ? 1 : 0;
    a.lambda = nullptr;
    a.rmsnorm = 0; a.eps = 0.f; a.norm_scale = 1.f; a.norm_weight = nullptr;
    a.out = out;
    const int64_t HN = (int64_t)H * N;
    a.hs = {HN * ldq, (int64_t)N * ldq, HN * ldk, (int64_t)N * ldk, HN * ldv, (int64_t)N * ldv, 1};
    return hip_status(diffattn::launch_attention_pp(a, (hipStream_t)stream),
                      "diffattn_attention launch");
}

diffattn_status_t diffattn_combine(const float* o1, const float* o2, const float* lambda, int B,
                                   int H, int N, int dv, int rmsnorm, float eps, float norm_scale,
                                   const float* norm_weight, float* out, void* stream) {
    if (!o1 || !o2 || !lambda || !out)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_combine: null pointer");
    if (B < 1 || H < 1 || N < 1 || dv < 1)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_combine: B=%d H=%d N=%d dv=%d must be >= 1", B, H, N, dv);
    if (rmsnorm && !(eps >= 0.f))
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_combine: eps must be >= 0");
    const void* ptrs[4] = {o1, o2, lambda, out};
    const char* names[4] = {"o1", "o2", "lambda", "out"};
    for (int i = 0; i < 4; ++i)
        if ((reinterpret_cast<uintptr_t>(ptrs[i]) & 3u) != 0)
            return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_combine: %s not 4-byte aligned",
                        names[i]);
    if (dv != 64 && dv != 128)
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_combine: dv=%d not built", dv);
    if ((int64_t)B * H * N > (int64_t)1 << 40)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_combine: B*H*N too large");
    if (!grid_fits(B, H, N, 4))
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_combine: B*H*N rows exceed the launch grid");
    for (int i = 0; i < 4; ++i) {
        diffattn_status_t s = check_device(ptrs[i], names[i]);
        if (s != DIFFATTN_OK) return s;
    }
    if (rmsnorm && norm_weight) {
        diffattn_status_t s = check_device(norm_weight, "norm_weight");
        if (s != DIFFATTN_OK) return s;
    }
    return hip_status(diffattn::launch_combine(o1, o2, lambda, B, H, N, dv, rmsnorm ? 1 : 0, eps,
                                               norm_scale, rmsnorm ? norm_weight : nullptr, out,
                                               (hipStream_t)stream),
                      "diffattn_combine launch");
}

size_t diffattn_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_len) {
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || max_len < 1) return 0;
    return diffattn::decode_workspace_floats(B, Hq, D, max_len) * sizeof(float);
}

}  // extern "C"

namespace {

// Pure-argument checks shared by the V2 decode entry points (everything but
// the workspace), in the order the contract lists them.
// `paired`: differential heads (query heads 2p, 2p+1 over one KV head, a
// lambda per pair); otherwise plain single-map heads (no lambda).
diffattn_status_t check_decode_args(const char* fn, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* seq_lens, int B, int Hq,
                                    int Hkv, int D, int max_len, const float* lambda,
                                    const float* out, bool paired = true) {
    if (!q || !k_cache || !v_cache || !seq_lens || (paired && !lambda) || !out)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || max_len < 1)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "%s: B=%d Hq=%d Hkv=%d D=%d max_len=%d must be >= 1", fn, B, Hq, Hkv, D,
                    max_len);
    const int group = paired ? 2 * Hkv : Hkv;
    if (Hq % group != 0)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "%s: Hq=%d must be a multiple of %s=%d", fn,
                    Hq, paired ? "2*Hkv" : "Hkv", group);
    const void* ptrs[6] = {q, k_cache, v_cache, seq_lens, out, lambda};
    const char* names[6] = {"q", "k_cache", "v_cache", "seq_lens", "out", "lambda"};
    for (int i = 0; i < 3; ++i)   // vector-loaded tensors
        if (!aligned16(ptrs[i]))
            return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "%s: %s not 16-byte aligned", fn, names[i]);
    for (int i = 3; i < (paired ? 6 : 5); ++i)   // read or written as 4-byte scalars
        if ((reinterpret_cast<uintptr_t>(ptrs[i]) & 3u) != 0)
            return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "%s: %s not 4-byte aligned", fn, names[i]);
    if (!diffattn::decode_supported(D))
        return fail(DIFFATTN_ERR_UNSUPPORTED, "%s: head width D=%d not built", fn, D);
    if (Hq / Hkv > 16)
        return fail(DIFFATTN_ERR_UNSUPPORTED, "%s: %d query heads per KV head (at most 16)", fn,
                    Hq / Hkv);
    if ((int64_t)B * Hkv * max_len > ((int64_t)1 << 40))
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "%s: cache too large", fn);
    if (max_len > (1 << 30))
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "%s: max_len too large", fn);
    return DIFFATTN_OK;
}

diffattn_status_t check_decode_devices(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* seq_lens, const float* lambda,
                                       const float* out) {
    const void* ptrs[6] = {q, k_cache, v_cache, seq_lens, out, lambda};
    const char* names[6] = {"q", "k_cache", "v_cache", "seq_lens", "out", "lambda"};
    for (int i = 0; i < (lambda ? 6 : 5); ++i) {
        diffattn_status_t s = check_device(ptrs[i], names[i]);
        if (s != DIFFATTN_OK) return s;
    }
    return DIFFATTN_OK;
}

diffattn::DecodeArgs decode_args(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                 int max_len, const float* lambda, void* workspace, float* out) {
    diffattn::DecodeArgs a;
    a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.seq_lens = seq_lens;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.max_len = max_len;
    a.lambda = lambda;
    a.workspace = static_cast<float*>(workspace);
    a.out = out;
    return a;
}

}  // namespace

extern "C" {

diffattn_status_t diffattn_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                  int max_len, const float* lambda, void* workspace,
                                  size_t workspace_bytes, float* out, void* stream) {
    diffattn_status_t s = check_decode_args("diffattn_decode", q, k_cache, v_cache, seq_lens, B,
                                            Hq, Hkv, D, max_len, lambda, out);
    if (s != DIFFATTN_OK) return s;
    const size_t need = diffattn_decode_workspace_bytes(B, Hq, Hkv, D, max_len);
    if (!workspace || workspace_bytes < need)
        return fail(DIFFATTN_ERR_WORKSPACE, "diffattn_decode: workspace needs %zu bytes, got %zu",
                    need, workspace ? workspace_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_decode: workspace not 256-byte aligned");
    s = check_decode_devices(q, k_cache, v_cache, seq_lens, lambda, out);
    if (s != DIFFATTN_OK) return s;
    s = check_device(workspace, "workspace");
    if (s != DIFFATTN_OK) return s;
    return hip_status(diffattn::launch_decode(decode_args(q, k_cache, v_cache, seq_lens, B, Hq,
                                                          Hkv, D, max_len, lambda, workspace, out),
                                              (hipStream_t)stream),
                      "diffattn_decode launch");
}

diffattn_status_t diffattn_attention_decode(const void* q, const void* k_cache,
                                            const void* v_cache, const int32_t* seq_lens, int B,
                                            int Hq, int Hkv, int D, int max_len, void* workspace,
                                            size_t workspace_bytes, float* out, void* stream) {
    diffattn_status_t s = check_decode_args("diffattn_attention_decode", q, k_cache, v_cache,
                                            seq_lens, B, Hq, Hkv, D, max_len, nullptr, out, false);
    if (s != DIFFATTN_OK) return s;
    const size_t need = diffattn_decode_workspace_bytes(B, Hq, Hkv, D, max_len);
    if (!workspace || workspace_bytes < need)
        return fail(DIFFATTN_ERR_WORKSPACE,
                    "diffattn_attention_decode: workspace needs %zu bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_attention_decode: workspace not 256-byte aligned");
    s = check_decode_devices(q, k_cache, v_cache, seq_lens, nullptr, out);
    if (s != DIFFATTN_OK) return s;
    s = check_device(workspace, "workspace");
    if (s != DIFFATTN_OK) return s;
    diffattn::DecodeArgs a = decode_args(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, D, max_len,
                                         nullptr, workspace, out);
    a.single = 1;
    return hip_status(diffattn::launch_decode(a, (hipStream_t)stream),
                      "diffattn_attention_decode launch");
}

diffattn_status_t diffattn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                          int max_len, const float* lambda, float* out,
                                          void* stream) {
    diffattn_status_t s = check_decode_args("diffattn_decode_noalloc", q, k_cache, v_cache,
                                            seq_lens, B, Hq, Hkv, D, max_len, lambda, out);
    if (s != DIFFATTN_OK) return s;
    const size_t need = diffattn_decode_workspace_bytes(B, Hq, Hkv, D, max_len);
    if (need > DIFFATTN_DECODE_SCRATCH_BYTES)
        return fail(DIFFATTN_ERR_WORKSPACE,
                    "diffattn_decode_noalloc: these sizes need %zu bytes of partial states, the "
                    "fixed scratch holds %zu; use diffattn_decode with a workspace",
                    need, (size_t)DIFFATTN_DECODE_SCRATCH_BYTES);
    s = check_decode_devices(q, k_cache, v_cache, seq_lens, lambda, out);
    if (s != DIFFATTN_OK) return s;
    return hip_status(diffattn::launch_decode_noalloc(decode_args(q, k_cache, v_cache, seq_lens, B,
                                                                  Hq, Hkv, D, max_len, lambda,
                                                                  nullptr, out),
                                                      (hipStream_t)stream),
                      "diffattn_decode_noalloc launch");
}

size_t diffattn_decode_v1_workspace_bytes(int B, int H, int max_len) {
    if (B < 1 || H < 1 || max_len < 1) return 0;
    // Two query columns (one per map) per head.
    return diffattn::decode_workspace_floats(B, 2 * H, 128, max_len) * sizeof(float);
}

diffattn_status_t diffattn_decode_v1(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* seq_lens, int B, int H, int d, int dv,
                                     int max_len, const float* lambda, int rmsnorm, float eps,
                                     float norm_scale, const float* norm_weight, void* workspace,
                                     size_t workspace_bytes, float* out, void* stream) {
    if (!q || !k_cache || !v_cache || !seq_lens || !lambda || !out)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_decode_v1: null pointer");
    if (B < 1 || H < 1 || d < 1 || dv < 1 || max_len < 1)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_decode_v1: B=%d H=%d d=%d dv=%d max_len=%d must be >= 1", B, H, d, dv,
                    max_len);
    if (rmsnorm && !(eps >= 0.f))
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_decode_v1: eps must be >= 0");
    const void* ptrs[6] = {q, k_cache, v_cache, seq_lens, lambda, out};
    const char* names[6] = {"q", "k_cache", "v_cache", "seq_lens", "lambda", "out"};
    for (int i = 0; i < 3; ++i)
        if (!aligned16(ptrs[i]))
            return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_decode_v1: %s not 16-byte aligned",
                        names[i]);
    for (int i = 3; i < 6; ++i)
        if ((reinterpret_cast<uintptr_t>(ptrs[i]) & 3u) != 0)
            return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_decode_v1: %s not 4-byte aligned",
                        names[i]);
    if (rmsnorm && norm_weight && (reinterpret_cast<uintptr_t>(norm_weight) & 3u) != 0)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_decode_v1: norm_weight not 4-byte aligned");
    if (!(d == 64 && dv == 128))
        return fail(DIFFATTN_ERR_UNSUPPORTED,
                    "diffattn_decode_v1: (d=%d, dv=%d) not built (d=64, dv=128 only)", d, dv);
    if ((int64_t)B * H * max_len > ((int64_t)1 << 40) || max_len > (1 << 30))
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "diffattn_decode_v1: cache too large");
    const size_t need = diffattn_decode_v1_workspace_bytes(B, H, max_len);
    if (!workspace || workspace_bytes < need)
        return fail(DIFFATTN_ERR_WORKSPACE, "diffattn_decode_v1: workspace needs %zu bytes, got %zu",
                    need, workspace ? workspace_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                    "diffattn_decode_v1: workspace not 256-byte aligned");
    for (int i = 0; i < 6; ++i) {
        diffattn_status_t s = check_device(ptrs[i], names[i]);
        if (s != DIFFATTN_OK) return s;
    }
    {
        diffattn_status_t s = check_device(workspace, "workspace");
        if (s != DIFFATTN_OK) return s;
    }
    if (rmsnorm && norm_weight) {
        diffattn_status_t s = check_device(norm_weight, "norm_weight");
        if (s != DIFFATTN_OK) return s;
    }
    diffattn::DecodeArgs a;
    a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.seq_lens = seq_lens;
    a.B = B; a.Hq = 2 * H; a.Hkv = H; a.D = 2 * d; a.max_len = max_len;
    a.lambda = lambda;
    a.workspace = static_cast<float*>(workspace);
    a.out = out;
    a.qhalf = d;
    a.rmsnorm = rmsnorm ? 1 : 0;
    a.eps = eps;
    a.norm_scale = norm_scale;
    a.norm_weight = rmsnorm ? norm_weight : nullptr;
    return hip_status(diffattn::launch_decode(a, (hipStream_t)stream), "diffattn_decode_v1 launch");
}

const char* diffattn_status_string(int status) {
    switch (status) {
        case DIFFATTN_OK: return "ok";
        case DIFFATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
        case DIFFATTN_ERR_UNSUPPORTED: return "unsupported shape or type";
        case DIFFATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case DIFFATTN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* diffattn_last_error(void) { return g_last_error; }

}  // extern "C"
