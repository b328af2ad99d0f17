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
// tiles of 16 keys shared by the workgroup.  Per tile, each thread forms the
// partial dot products of the 16 keys over its quarter, the quad sums them
// with two lane exchanges, and both softmax states (running maximum m,
// normaliser l, accumulator O) take one update for the whole tile.
#include "kernels.h"

namespace diffattn {
namespace {

// x from the lane whose index differs in bit 0 (CTRL 0xB1) or bit 1 (0x4E)
// inside its group of four: a DPP quad permutation, no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float quad_swap(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

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
    __shared__ __attribute__((aligned(16))) float sk1[F32_BN][D];
    __shared__ __attribute__((aligned(16))) float sk2[F32_BN][D];
    __shared__ __attribute__((aligned(16))) float sv[F32_BN][DV];

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

    // Thread `sub` owns the contiguous quarter sub*DQ .. sub*DQ+DQ-1 of each
    // query/key vector and sub*DVQ .. sub*DVQ+DVQ-1 of each value/output row,
    // so its LDS reads and global accesses are 16 bytes wide.
    float qa[DQ], qb[DQ];
    for (int i = 0; i < DQ; ++i) {
        qa[i] = row_ok ? q1[qoff + (int64_t)row * ldq + sub * DQ + i] : 0.f;
        qb[i] = row_ok ? q2[qoff + (int64_t)row * ldq + sub * DQ + i] : 0.f;
    }
    // Scores are kept in raw units; exp(x/sqrt d) = exp2(x * log2(e)/sqrt d).
    const float c = 1.4426950408889634f / sqrtf((float)D);
    float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
    float o1[DVQ], o2[DVQ];
    for (int i = 0; i < DVQ; ++i) { o1[i] = 0.f; o2[i] = 0.f; }

    const int last_row = min(N - 1, tile * F32_ROWS + F32_ROWS - 1);
    const int kv_end = causal ? last_row + 1 : N;
    const int my_end = row_ok ? (causal ? row + 1 : N) : 0;

    // Tiles are staged through registers one tile ahead: 16-byte loads of
    // tile kb+16 are in flight while tile kb is computed from LDS.  Rows past
    // N read as zeros.
    constexpr int KPT = F32_BN * D / 4 / F32_THREADS;    // float4s per thread, per key half
    constexpr int VPT = F32_BN * DV / 4 / F32_THREADS;   // float4s per thread of values
    static_assert(KPT >= 1 && VPT >= 1 && KPT * 4 * F32_THREADS == F32_BN * D &&
                  VPT * 4 * F32_THREADS == F32_BN * DV, "tile staging");
    float4 rk1[KPT], rk2[KPT], rv[VPT];
    auto load_tile = [&](int kb) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int e = tid + u * F32_THREADS, j = e / (D / 4), cc = (e % (D / 4)) * 4;
            const bool ok = kb + j < N;
            const int64_t o = koff + (int64_t)(ok ? kb + j : 0) * ldk + cc;
            rk1[u] = ok ? *reinterpret_cast<const float4*>(k1 + o) : make_float4(0.f, 0.f, 0.f, 0.f);
            rk2[u] = ok ? *reinterpret_cast<const float4*>(k2 + o) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int e = tid + u * F32_THREADS, j = e / (DV / 4), cc = (e % (DV / 4)) * 4;
            const bool ok = kb + j < N;
            rv[u] = ok ? *reinterpret_cast<const float4*>(v + voff + (int64_t)(ok ? kb + j : 0) * ldv + cc)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    if (kv_end > 0) load_tile(0);
    for (int kb = 0; kb < kv_end; kb += F32_BN) {
        __syncthreads();  // previous tile fully consumed
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int e = tid + u * F32_THREADS, j = e / (D / 4), cc = (e % (D / 4)) * 4;
            *reinterpret_cast<float4*>(&sk1[j][cc]) = rk1[u];
            *reinterpret_cast<float4*>(&sk2[j][cc]) = rk2[u];
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int e = tid + u * F32_THREADS, j = e / (DV / 4), cc = (e % (DV / 4)) * 4;
            *reinterpret_cast<float4*>(&sv[j][cc]) = rv[u];
        }
        __syncthreads();
        if (kb + F32_BN < kv_end) load_tile(kb + F32_BN);
        const int jn = min(F32_BN, kv_end - kb);
        // The tile's 16 scores of both maps at once (independent dot
        // products and lane exchanges), then one online-softmax update per
        // tile: new maximum, one rescale factor, 16 probabilities.
        float s1[F32_BN], s2[F32_BN];
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int i = 0; i < DQ; i += 4) {
                const float4 x = *reinterpret_cast<const float4*>(&sk1[j][sub * DQ + i]);
                const float4 y = *reinterpret_cast<const float4*>(&sk2[j][sub * DQ + i]);
                a = fmaf(qa[i], x.x, a);
                a = fmaf(qa[i + 1], x.y, a);
                a = fmaf(qa[i + 2], x.z, a);
                a = fmaf(qa[i + 3], x.w, a);
                b = fmaf(qb[i], y.x, b);
                b = fmaf(qb[i + 1], y.y, b);
                b = fmaf(qb[i + 2], y.z, b);
                b = fmaf(qb[i + 3], y.w, b);
            }
            s1[j] = a;
            s2[j] = b;
        }
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            s1[j] += quad_swap<0xB1>(s1[j]);
            s2[j] += quad_swap<0xB1>(s2[j]);
        }
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            s1[j] += quad_swap<0x4E>(s1[j]);
            s2[j] += quad_swap<0x4E>(s2[j]);
        }
        // Keys past the tile or (causally) past this row are masked
        // (quad-uniform).
        float t1 = m1, t2 = m2;
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            if (j >= jn || kb + j >= my_end) {
                s1[j] = -INFINITY;
                s2[j] = -INFINITY;
            }
            t1 = fmaxf(t1, s1[j]);
            t2 = fmaxf(t2, s2[j]);
        }
        if (t1 == -INFINITY) continue;   // no visible key yet (both maps alike)
        const float a1 = __builtin_amdgcn_exp2f((m1 - t1) * c);  // 0 before the first key
        const float a2 = __builtin_amdgcn_exp2f((m2 - t2) * c);
        m1 = t1;
        m2 = t2;
        float p1[F32_BN], p2[F32_BN];
        float sum1 = 0.f, sum2 = 0.f;
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            p1[j] = __builtin_amdgcn_exp2f((s1[j] - t1) * c);
            p2[j] = __builtin_amdgcn_exp2f((s2[j] - t2) * c);
            sum1 += p1[j];
            sum2 += p2[j];
        }
        l1 = fmaf(l1, a1, sum1);
        l2 = fmaf(l2, a2, sum2);
#pragma unroll
        for (int i = 0; i < DVQ; i += 4) {
            float4 x1 = make_float4(0.f, 0.f, 0.f, 0.f), x2 = x1;
#pragma unroll
            for (int j = 0; j < F32_BN; ++j) {
                const float4 vv = *reinterpret_cast<const float4*>(&sv[j][sub * DVQ + i]);
                x1.x = fmaf(p1[j], vv.x, x1.x);
                x1.y = fmaf(p1[j], vv.y, x1.y);
                x1.z = fmaf(p1[j], vv.z, x1.z);
                x1.w = fmaf(p1[j], vv.w, x1.w);
                x2.x = fmaf(p2[j], vv.x, x2.x);
                x2.y = fmaf(p2[j], vv.y, x2.y);
                x2.z = fmaf(p2[j], vv.z, x2.z);
                x2.w = fmaf(p2[j], vv.w, x2.w);
            }
            o1[i] = fmaf(o1[i], a1, x1.x);
            o1[i + 1] = fmaf(o1[i + 1], a1, x1.y);
            o1[i + 2] = fmaf(o1[i + 2], a1, x1.z);
            o1[i + 3] = fmaf(o1[i + 3], a1, x1.w);
            o2[i] = fmaf(o2[i], a2, x2.x);
            o2[i + 1] = fmaf(o2[i + 1], a2, x2.y);
            o2[i + 2] = fmaf(o2[i + 2], a2, x2.z);
            o2[i + 3] = fmaf(o2[i + 3], a2, x2.w);
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
        ss += quad_swap<0xB1>(ss);
        ss += quad_swap<0x4E>(ss);
        const float r = norm_scale / sqrtf(ss / (float)DV + eps);
        for (int i = 0; i < DVQ; ++i)
            y[i] *= r * (norm_weight ? norm_weight[sub * DVQ + i] : 1.f);
    }
    float* orow = out + (head_tok0 + row) * DV;
    for (int i = 0; i < DVQ; i += 4)
        *reinterpret_cast<float4*>(orow + sub * DVQ + i) = make_float4(y[i], y[i + 1], y[i + 2], y[i + 3]);
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
