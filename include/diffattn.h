/*
 * libdiffattn -- differential attention on AMD Instinct MI355X (gfx950).
 *
 * The operator (page "差分注意力" (aiknowledge.cn), part 一 "差分思路" and
 * part 二 Step 2):
 *     A1 = softmax(Q1 K1^T / sqrt(d)),   A2 = softmax(Q2 K2^T / sqrt(d)),
 *     out = (A1 - lambda * A2) V,
 * with d the length of the query/key dot product and lambda a per-head scalar
 * (part 二 Step 4) whose initial value follows a depth schedule (page
 * "【架构革新】Differential Transformer：用“差分降噪”重塑LLM注意力机制"
 * (mcipr.com), section 3).  Two head layouts are served (page "差分注意力",
 * "V1 到 V2 的 diff"): V1 splits each head's query and key into halves
 * Q = (Q1, Q2), K = (K1, K2) over one value of full width and may normalise
 * each head's output; V2 keeps full-width heads and doubles the query heads
 * over the same KV heads.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers (memory from hipMalloc or a
 *    caller's allocator such as PyTorch).  The library allocates nothing and
 *    never frees caller memory.  Between calls it keeps only per-device
 *    caches (the CU count, a kernel's LDS limit, the address of the
 *    allocation-free decode's fixed scratch array); no result of one call
 *    depends on an earlier call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously; results are valid once the stream has
 *    reached that point.  Calls on different streams may run concurrently;
 *    every call only reads its inputs and writes its own outputs/workspace.
 *  - Arguments are validated on the host before anything is enqueued.  On any
 *    error no kernel is launched and no output is touched; the call returns a
 *    status code and diffattn_last_error() (thread-local) describes it.
 *  - Element strides are counted in elements of the tensor's own type.
 *  - Element types are passed as an int holding a diffattn_dtype_t value;
 *    any other value is rejected with INVALID_ARGUMENT.
 *  - No C++ exception crosses this interface.
 */
#ifndef DIFFATTN_H_
#define DIFFATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DIFFATTN_OK = 0,
    DIFFATTN_ERR_INVALID_ARGUMENT = 1, /* null/host pointer, bad size, misalignment */
    DIFFATTN_ERR_UNSUPPORTED = 2,      /* valid but not built: head width, dtype  */
    DIFFATTN_ERR_WORKSPACE = 3,        /* workspace missing or too small          */
    DIFFATTN_ERR_HIP = 4               /* the HIP runtime reported an error        */
} diffattn_status_t;

typedef enum {
    DIFFATTN_FP32 = 0, /* fp32 inputs, fp32 arithmetic                           */
    DIFFATTN_BF16 = 1  /* bf16 inputs, bf16 matrix products, fp32 accumulation   */
} diffattn_dtype_t;

/*
 * lambda_init = 0.8 - 0.6 * exp(-0.3 * (layer - 1)), computed on the host in
 * double.  `layer` is the 1-based layer index (page "【架构革新】...",
 * section 3, initialisation strategy).  Returns NaN for layer < 1.
 */
double diffattn_lambda_init(int layer);

/*
 * Per-head lambda (page "差分注意力", part 二 Step 4 re-parameterisation):
 *     lambda_h = exp(lq1_h . lk1_h) - exp(lq2_h . lk2_h) + lambda_init(layer).
 * lq1, lk1, lq2, lk2: device fp32 [H][dim], row-major.
 * lambda_out:         device fp32 [H].
 * Each dot product is summed in double in index order, the exponentials and
 * the sum are taken in double, and the result is rounded once to fp32.
 * lambda may be negative or exceed 1; it is not clamped.
 * Errors: INVALID_ARGUMENT for null or non-device pointers, H < 1, dim < 1,
 * layer < 1.
 */
diffattn_status_t diffattn_lambda(const float* lq1, const float* lk1, const float* lq2,
                                  const float* lk2, int H, int dim, int layer,
                                  float* lambda_out, void* stream);

/*
 * Fused differential-attention prefill, V1 layout (page "差分注意力", part 一
 * "差分思路" and "V1 到 V2 的 diff"; page "【架构革新】...", section 3: both
 * softmaxes share their intermediates in one fused kernel).
 *
 * Tensors are [B][H][N][ld] (token-major inside each head): element (b,h,n,c)
 * of q1 is q1[((b*H + h)*N + n)*ldq + c].  A packed [B][H][N][2d] query
 * tensor is passed as q1 = base, q2 = base + d, ldq = 2d; the same for keys.
 *   q1, q2, k1, k2 : d columns each (dtype), ldq/ldk >= d
 *   v              : dv columns (dtype), ldv >= dv
 *   lambda         : device fp32 [H] (e.g. from diffattn_lambda)
 *   out            : device fp32 [B][H][N][dv], contiguous
 * causal != 0: query n sees keys 0..n; otherwise all N keys.
 * rmsnorm != 0: each output row of a head becomes
 *     y_c = o_c / sqrt(mean_c o_c^2 + eps) * w_c * norm_scale,
 * with w = norm_weight (device fp32 [dv]) or 1 if norm_weight is NULL; pass
 * norm_scale = 1 - lambda_init for the V1 head normalisation.
 * Supported: BF16 with (d, dv) in {(64,128), (64,64), (32,64), (128,128)};
 * FP32 with d in {32, 64, 128} and dv in {64, 128}.  Other shapes return
 * UNSUPPORTED.  BF16 token strides ldq, ldk, ldv above 2^24 - 1 elements
 * also return UNSUPPORTED (the kernels address 64-row tiles with 32-bit byte
 * offsets).  Pointers must be 16-byte aligned and ld*sizeof(elem) a
 * multiple of 16 (INVALID_ARGUMENT otherwise).  B, H, N >= 1, and B*H*N at
 * most 2^40 (INVALID_ARGUMENT otherwise).  The launch grid holds at most
 * 2^31 - 1 workgroups: B*H*ceil(N/128) (BF16) or B*H*ceil(N/32) (FP32) above
 * that returns UNSUPPORTED.
 */
diffattn_status_t diffattn_prefill(const void* q1, const void* q2, const void* k1,
                                   const void* k2, const void* v, int64_t ldq, int64_t ldk,
                                   int64_t ldv, int dtype, int B, int H, int N,
                                   int d, int dv, int causal, const float* lambda, int rmsnorm,
                                   float eps, float norm_scale, const float* norm_weight,
                                   float* out, void* stream);

/*
 * Fused differential-attention prefill, V2 layout (page "差分注意力",
 * "V1 到 V2 的 diff": the query heads are doubled over a shared key/value
 * cache, each map keeps the full head width, and no per-head norm follows).
 * Diff head (pair) p takes query heads 2p (map 1) and 2p+1 (map 2); both maps
 * use K/V head g = p / (Hq / (2*Hkv)) (grouped-query sharing).
 *   q      : device [B][Hq][N][D] (dtype)
 *   k, v   : device [B][Hkv][N][D] (dtype)
 *   lambda : device fp32 [Hq/2]
 *   out    : device fp32 [B][Hq/2][N][D]
 * out[b,p,n] = (A1 - lambda_p A2) V with A1, A2 the softmaxes of the two
 * maps' scores / sqrt(D); causal != 0 restricts query n to keys 0..n.
 * Supported: BF16 and FP32 with D in {64, 128} (UNSUPPORTED otherwise),
 * with the size and grid limits of diffattn_prefill for H = Hq/2.
 * Hq must be a multiple of 2*Hkv, pointers 16-byte aligned, D*sizeof(elem)
 * a multiple of 16 (INVALID_ARGUMENT otherwise).  Asynchronous on stream.
 */
diffattn_status_t diffattn_prefill_v2(const void* q, const void* k, const void* v,
                                      int dtype, int B, int Hq, int Hkv, int N, int D,
                                      int causal, const float* lambda, float* out, void* stream);

/*
 * Plain single-map softmax attention, out = softmax(q k^T / sqrt d) v, on the
 * prefill kernel's schedule.  With diffattn_combine it forms the unfused
 * two-pass differential attention that the fused kernels replace (page
 * "【架构革新】...", section 3: separate passes keep two full intermediate
 * outputs and read the values twice; page "差分注意力", "V1 到 V2 的 diff").
 * Layouts as for diffattn_prefill: q, k [B][H][N][ld] with d columns, v with
 * dv columns, out fp32 [B][H][N][dv].  causal != 0: query n sees keys 0..n.
 * Supported: BF16 with (d, dv) in {(64,128), (64,64)}; FP32 and other
 * shapes return UNSUPPORTED, as do token strides above 2^24 - 1 elements
 * and the BF16 grid limit of diffattn_prefill.
 * Other errors as for diffattn_prefill.
 */
diffattn_status_t diffattn_attention(const void* q, const void* k, const void* v, int64_t ldq,
                                     int64_t ldk, int64_t ldv, int dtype, int B,
                                     int H, int N, int d, int dv, int causal, float* out,
                                     void* stream);

/*
 * Second pass of the unfused path: out = o1 - lambda_h * o2 row by row over
 * fp32 [B][H][N][dv] tensors (page "差分注意力", part 一 "差分思路"), then the
 * optional RMS norm exactly as in diffattn_prefill.  lambda: device fp32 [H].
 * out may alias o1.  Supported dv: 64, 128 (UNSUPPORTED otherwise); pointers
 * 4-byte aligned (INVALID_ARGUMENT otherwise).  B*H*N at most 2^40
 * (INVALID_ARGUMENT), and B*H*ceil(N/4) at most 2^31 - 1 (UNSUPPORTED).
 */
diffattn_status_t diffattn_combine(const float* o1, const float* o2, const float* lambda, int B,
                                   int H, int N, int dv, int rmsnorm, float eps, float norm_scale,
                                   const float* norm_weight, float* out, void* stream);

/*
 * Bytes of device workspace diffattn_decode needs for these sizes (partial
 * softmax states of every KV piece, ceil(max_len/4096)+1 per sequence and
 * query head, and a piece count per sequence and KV head).  Returns 0 for
 * invalid sizes.
 */
size_t diffattn_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_len);

/*
 * One-token differential-attention decode over a KV cache, V2 layout (page
 * "差分注意力", "V1 到 V2 的 diff": twice the query heads over unchanged KV
 * heads, so one pass over the cache serves both maps; part 五 exercise 3 on
 * decode arithmetic intensity).
 *   q        : device bf16 [B][Hq][D]
 *   k_cache,
 *   v_cache  : device bf16 [B][Hkv][max_len][D]; positions 0..L_b-1 are read
 *   seq_lens : device int32 [B], 1 <= L_b <= max_len
 *   lambda   : device fp32 [Hq/2], one per pair
 *   out      : device fp32 [B][Hq/2][D]
 * Pair p takes query head 2p for A1 and 2p+1 for A2, both over KV head
 * floor(2p / (Hq/Hkv)); Hq must be a multiple of 2*Hkv.  There is no output
 * normalisation in this layout.
 * workspace: device memory of at least diffattn_decode_workspace_bytes(...)
 * bytes, 256-byte aligned, owned by the caller, overwritten by the call.
 * Supported: D = 128.  A sequence whose device-side length lies outside
 * [1, max_len] (the host cannot see it) yields zeros for its outputs.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (D), WORKSPACE (missing/too small).
 */
diffattn_status_t diffattn_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                  int max_len, const float* lambda, void* workspace,
                                  size_t workspace_bytes, float* out, void* stream);

/*
 * Plain single-map softmax attention decode over the same GQA cache layout:
 * every query head h is its own softmax over KV head h / (Hq/Hkv),
 *     out[b,h] = softmax(q[b,h] K^T / sqrt(D)) V.
 * It is the baseline decode that page "差分注意力" compares the V2 layout
 * with ("V1 到 V2 的 diff", part 三 and part 五 exercise 3: doubling the
 * query heads over the same KV heads keeps decode at the baseline's speed);
 * a baseline model with half the query heads runs this over the cache a V2
 * model reads.
 *   q        : device bf16 [B][Hq][D]
 *   k_cache,
 *   v_cache  : device bf16 [B][Hkv][max_len][D]; positions 0..L_b-1 are read
 *   seq_lens : device int32 [B]
 *   out      : device fp32 [B][Hq][D]
 * Hq must be a multiple of Hkv (at most 16 query heads per KV head).
 * workspace: at least diffattn_decode_workspace_bytes(B, Hq, Hkv, D, max_len)
 * bytes, 256-byte aligned, caller-owned.  Supported: D = 128.  A sequence
 * whose device-side length is outside [1, max_len] yields zeros.  Errors as
 * for diffattn_decode.
 */
diffattn_status_t diffattn_attention_decode(const void* q, const void* k_cache,
                                            const void* v_cache, const int32_t* seq_lens, int B,
                                            int Hq, int Hkv, int D, int max_len, void* workspace,
                                            size_t workspace_bytes, float* out, void* stream);

/*
 * diffattn_decode without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * and harnesses that forbid hipMalloc.  Arguments, layouts, results and
 * errors are those of diffattn_decode, less the workspace.  The partial
 * states go to a fixed array of DIFFATTN_DECODE_SCRATCH_BYTES inside the
 * library: one per device, created with the library's code on that device
 * and held until the process ends.  Sizes whose
 * diffattn_decode_workspace_bytes(...) exceed it return WORKSPACE (nothing is
 * launched).  Nothing is allocated by this call.  Every call on one device
 * shares that device's array, so calls that overlap on one device (on other
 * streams or from other threads) race and must be ordered by the caller.
 */
#define DIFFATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
diffattn_status_t diffattn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                          int max_len, const float* lambda, float* out,
                                          void* stream);

/*
 * Bytes of device workspace diffattn_decode_v1 needs (two partial softmax
 * states, one per map, per head and KV piece, and a piece count per head).
 * Returns 0 for invalid sizes.
 */
size_t diffattn_decode_v1_workspace_bytes(int B, int H, int max_len);

/*
 * Split-KV differential-attention decode, V1 layout (page "差分注意力", part 一
 * "差分思路" and "V1 到 V2 的 diff": half-width maps and per-head RMS norm).
 * One query token per sequence and head, attending to cache positions
 * 0 .. seq_lens[b]-1; the value cache is read once for both maps.
 *   q        : bf16 [B][H][2d], packed [q1 | q2]
 *   k_cache  : bf16 [B][H][max_len][2d], packed [k1 | k2]
 *   v_cache  : bf16 [B][H][max_len][dv]
 *   seq_lens : device int32 [B], each in [1, max_len]
 *   lambda   : device fp32 [H]
 *   out      : device fp32 [B][H][dv]
 * out = (softmax(q1 K1^T / sqrt d) - lambda_h softmax(q2 K2^T / sqrt d)) V,
 * then, if rmsnorm != 0, y_c = out_c / sqrt(mean_c out_c^2 + eps) * w_c *
 * norm_scale with w = norm_weight (device fp32 [dv]) or 1 when NULL; pass
 * norm_scale = 1 - lambda_init.
 * Supported: d = 64, dv = 128 (UNSUPPORTED otherwise).  workspace: device
 * memory of at least diffattn_decode_v1_workspace_bytes(B, H, max_len)
 * bytes, 256-byte aligned, owned by the caller (WORKSPACE if missing or
 * small).  A sequence whose device-side length is outside [1, max_len]
 * yields zeros.  Other argument errors as for diffattn_decode.
 */
diffattn_status_t diffattn_decode_v1(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* seq_lens, int B, int H, int d, int dv,
                                     int max_len, const float* lambda, int rmsnorm, float eps,
                                     float norm_scale, const float* norm_weight, void* workspace,
                                     size_t workspace_bytes, float* out, void* stream);

/* Static text for a status code (a diffattn_status_t value; any other int
 * gives "unknown status"). */
const char* diffattn_status_string(int status);

/* Detail of the last error reported on the calling thread ("" if none). */
const char* diffattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H_ */
