// Differential-attention prefill, fp32 inputs and fp32 arithmetic.
//
// Computes, per query row i of head (b,h):
//     A1 = softmax(q1_i K1^T / sqrt d),  A2 = softmax(q2_i K2^T / sqrt d),
//     o_i = (A1 - lambda_h A2) V,  then optionally the per-head RMS norm
// (page "差分注意力" (aiknowledge.cn), part 一 "差分思路", part 二 Step 2, and
// "V1 到 V2 的 diff" for the per-head normalisation after the difference).
//
// This is the full-precision path: small shapes where exactness to about
// 1e-6 matters more than throughput.  It runs on the vector ALUs: a
// workgroup of 128 threads owns 32 query rows, four threads per row.  Each
// thread keeps a quarter of the row's query halves and a quarter of both
// output accumulators in registers; keys and values stream through LDS in
// tiles of 16 keys shared by the workgroup.  Per key, each thread forms a
// partial dot product over its quarter, the quad sums them with two lane
// exchanges, and both softmax states (running maximum m, normaliser l,
// accumulator O) are updated exactly, one key at a time.
#include "kernels.h"

namespace diffattn {
namespace {

constexpr int F32_ROWS = 32;     // query rows per workgroup
constexpr int F32_THREADS = 128; // four threads per row
constexpr int F32_BN = 16;       // keys per LDS tile

template <int D, int DV>
__global__ void __launch_bounds__(F32_THREADS)
prefill_f32_kernel(const float* __restrict__ q1, const float* __restrict__ q2,
                   const float* __restrict__ k1, const float* __restrict__ k2,
                   const float* __restrict__ v, int64_t ldq, int64_t ldk, int64_t ldv, int H,
                   int N, int causal, const float* __restrict__ lambda, int rmsnorm, float eps,
                   float norm_scale, const float* __restrict__ norm_weight,
                   float* __restrict__ out, int row_tiles, HeadStrides hs) {
    constexpr int DQ = D / 4;    // query/key elements per thread
    constexpr int DVQ = DV / 4;  // output channels per thread
    __shared__ float sk1[F32_BN][D];
    __shared__ float sk2[F32_BN][D];
    __shared__ float sv[F32_BN][DV];

    const int tid = threadIdx.x;
    const int sub = tid & 3;         // position inside the row's quad
    const int r_local = tid >> 2;    // row inside the workgroup
    const int bh = blockIdx.x / row_tiles;
    const int tile = blockIdx.x % row_tiles;
    const int h = bh % H;
    const int row = tile * F32_ROWS + r_local;
    const bool row_ok = row < N;
    const int64_t head_tok0 = (int64_t)bh * N;           // output rows
    const int64_t qoff = (bh / H) * hs.qb + h * hs.qh;
    const int64_t koff = (bh / H) * hs.kb + (h / hs.kv_group) * hs.kh;
    const int64_t voff = (bh / H) * hs.vb + (h / hs.kv_group) * hs.vh;

    // Thread `sub` owns elements sub, sub+4, sub+8, ... of each vector.
    float qa[DQ], qb[DQ];
    for (int i = 0; i < DQ; ++i) {
        qa[i] = row_ok ? q1[qoff + (int64_t)row * ldq + sub + 4 * i] : 0.f;
        qb[i] = row_ok ? q2[qoff + (int64_t)row * ldq + sub + 4 * i] : 0.f;
    }
    // Scores are kept in raw units; exp(x/sqrt d) = exp2(x * log2(e)/sqrt d).
    const float c = 1.4426950408889634f / sqrtf((float)D);
    float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
    float o1[DVQ], o2[DVQ];
    for (int i = 0; i < DVQ; ++i) { o1[i] = 0.f; o2[i] = 0.f; }

    const int last_row = min(N - 1, tile * F32_ROWS + F32_ROWS - 1);
    const int kv_end = causal ? last_row + 1 : N;
    const int my_end = row_ok ? (causal ? row + 1 : N) : 0;

    for (int kb = 0; kb < kv_end; kb += F32_BN) {
        __syncthreads();  // previous tile fully consumed
        for (int e = tid; e < F32_BN * D; e += F32_THREADS) {
            int j = e / D, cc = e % D;
            bool ok = kb + j < N;
            sk1[j][cc] = ok ? k1[koff + (int64_t)(kb + j) * ldk + cc] : 0.f;
            sk2[j][cc] = ok ? k2[koff + (int64_t)(kb + j) * ldk + cc] : 0.f;
        }
        for (int e = tid; e < F32_BN * DV; e += F32_THREADS) {
            int j = e / DV, cc = e % DV;
            sv[j][cc] = (kb + j < N) ? v[voff + (int64_t)(kb + j) * ldv + cc] : 0.f;
        }
        __syncthreads();
        const int jn = min(F32_BN, kv_end - kb);
        for (int j = 0; j < jn; ++j) {
            float s1 = 0.f, s2 = 0.f;
            for (int i = 0; i < DQ; ++i) {
                s1 = fmaf(qa[i], sk1[j][sub + 4 * i], s1);
                s2 = fmaf(qb[i], sk2[j][sub + 4 * i], s2);
            }
            s1 += __shfl_xor(s1, 1);
            s2 += __shfl_xor(s2, 1);
            s1 += __shfl_xor(s1, 2);
            s2 += __shfl_xor(s2, 2);
            if (kb + j >= my_end) continue;  // masked key (quad-uniform)
            float n1 = fmaxf(m1, s1), n2 = fmaxf(m2, s2);
            float a1 = __builtin_amdgcn_exp2f((m1 - n1) * c);  // 0 on the first key
            float a2 = __builtin_amdgcn_exp2f((m2 - n2) * c);
            float p1 = __builtin_amdgcn_exp2f((s1 - n1) * c);
            float p2 = __builtin_amdgcn_exp2f((s2 - n2) * c);
            m1 = n1;
            m2 = n2;
            l1 = fmaf(l1, a1, p1);
            l2 = fmaf(l2, a2, p2);
            for (int i = 0; i < DVQ; ++i) {
                float vv = sv[j][sub + 4 * i];
                o1[i] = fmaf(o1[i], a1, p1 * vv);
                o2[i] = fmaf(o2[i], a2, p2 * vv);
            }
        }
    }
    if (!row_ok) return;
    const float lam = lambda[h];
    const float w1 = 1.f / l1;
    const float w2 = lam / l2;
    float y[DVQ];
    float ss = 0.f;
    for (int i = 0; i < DVQ; ++i) {
        y[i] = o1[i] * w1 - o2[i] * w2;
        ss = fmaf(y[i], y[i], ss);
    }
    if (rmsnorm) {
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        const float r = norm_scale / sqrtf(ss / (float)DV + eps);
        for (int i = 0; i < DVQ; ++i)
            y[i] *= r * (norm_weight ? norm_weight[sub + 4 * i] : 1.f);
    }
    float* orow = out + (head_tok0 + row) * DV;
    for (int i = 0; i < DVQ; ++i) orow[sub + 4 * i] = y[i];
}

template <int D, int DV>
hipError_t launch_f32(const PrefillArgs& a, hipStream_t stream) {
    const int row_tiles = (a.N + F32_ROWS - 1) / F32_ROWS;
    const int64_t blocks = (int64_t)a.B * a.H * row_tiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_f32_kernel<D, DV>), dim3((unsigned)blocks), dim3(F32_THREADS), 0,
                       stream, (const float*)a.q1, (const float*)a.q2, (const float*)a.k1,
                       (const float*)a.k2, (const float*)a.v, a.ldq, a.ldk, a.ldv, a.H, a.N,
                       a.causal, a.lambda, a.rmsnorm, a.eps, a.norm_scale, a.norm_weight, a.out,
                       row_tiles, a.hs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
#define DIFFATTN_F32_CASE(DD, VV) \
    if (a.d == DD && a.dv == VV) return launch_f32<DD, VV>(a, stream);
    DIFFATTN_F32_CASE(32, 64)
    DIFFATTN_F32_CASE(32, 128)
    DIFFATTN_F32_CASE(64, 64)
    DIFFATTN_F32_CASE(64, 128)
    DIFFATTN_F32_CASE(128, 64)
    DIFFATTN_F32_CASE(128, 128)
#undef DIFFATTN_F32_CASE
    return hipErrorInvalidValue;
}

}  // namespace diffattn
