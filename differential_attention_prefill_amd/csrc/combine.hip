// Second pass of the unfused two-pass path: out = o1 - lambda_h * o2 for every
// row of [B][H][N][dv] (fp32), then the optional per-head RMS norm
// (page "差分注意力", part 一 "差分思路" for the difference, "V1 到 V2 的 diff"
// for the norm).  The fused kernels do this in their epilogue; here it reads
// the two single-map outputs back from memory.
//
// One wave per row: lane i holds channels i*R .. i*R + R-1 (R = dv/64), the
// row's sum of squares is one wave reduction.  Reads 2*dv*4 bytes and writes
// dv*4 bytes per row: bound by HBM.
#include "kernels.h"

namespace diffattn {
namespace {

constexpr int CMB_ROWS = 4;                  // rows (waves) per workgroup

template <int DV>
__global__ void __launch_bounds__(64 * CMB_ROWS)
combine_kernel(const float* __restrict__ o1, const float* __restrict__ o2,
               const float* __restrict__ lambda, int H, int N, int64_t rows, int rmsnorm,
               float eps, float norm_scale, const float* __restrict__ norm_weight,
               float* __restrict__ out) {
    constexpr int R = DV / 64;
    const int64_t row = (int64_t)blockIdx.x * CMB_ROWS + (threadIdx.x >> 6);
    if (row >= rows) return;                 // whole wave leaves together
    const int lane = threadIdx.x & 63;
    const int h = (int)((row / N) % H);
    const float lam = lambda[h];
    const int64_t base = row * DV + lane * R;
    float y[R];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < R; ++e) {
        y[e] = o1[base + e] - lam * o2[base + e];
        ss = fmaf(y[e], y[e], ss);
    }
    float scale = 1.f;
    if (rmsnorm) {
        for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
        scale = norm_scale / sqrtf(ss / (float)DV + eps);
    }
#pragma unroll
    for (int e = 0; e < R; ++e) {
        const float w = (rmsnorm && norm_weight) ? norm_weight[lane * R + e] : 1.f;
        out[base + e] = y[e] * scale * w;
    }
}

}  // namespace

hipError_t launch_combine(const float* o1, const float* o2, const float* lambda, int B, int H,
                          int N, int dv, int rmsnorm, float eps, float norm_scale,
                          const float* norm_weight, float* out, hipStream_t stream) {
    const int64_t rows = (int64_t)B * H * N;
    const int64_t blocks = (rows + CMB_ROWS - 1) / CMB_ROWS;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (dv == 128)
        hipLaunchKernelGGL(combine_kernel<128>, dim3((unsigned)blocks), dim3(64 * CMB_ROWS), 0,
                           stream, o1, o2, lambda, H, N, rows, rmsnorm, eps, norm_scale,
                           norm_weight, out);
    else if (dv == 64)
        hipLaunchKernelGGL(combine_kernel<64>, dim3((unsigned)blocks), dim3(64 * CMB_ROWS), 0,
                           stream, o1, o2, lambda, H, N, rows, rmsnorm, eps, norm_scale,
                           norm_weight, out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace diffattn
