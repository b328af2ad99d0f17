// Per-head lambda of differential attention.
//
// lambda_h = exp(lq1_h . lk1_h) - exp(lq2_h . lk2_h) + lambda_init
// (page "差分注意力" (aiknowledge.cn), part 二 Step 4: a learnable, possibly
// negative scalar per head; lambda_init from the depth schedule of page
// "【架构革新】Differential Transformer..." (mcipr.com), section 3).
//
// One thread per head.  Each product of two fp32 values is exact in double;
// the dot products are summed in double in index order, the exponentials and
// the sum are taken in double, and the result is rounded once to fp32.  The
// work is a few hundred flops per head, so the launch is latency-bound and a
// serial double loop costs nothing measurable.
#include "kernels.h"

namespace diffattn {

__global__ void __launch_bounds__(64) lambda_kernel(const float* __restrict__ lq1,
                                                    const float* __restrict__ lk1,
                                                    const float* __restrict__ lq2,
                                                    const float* __restrict__ lk2, int H,
                                                    int dim, double lambda_init,
                                                    float* __restrict__ out) {
    int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    const int64_t base = (int64_t)h * dim;
    double d1 = 0.0, d2 = 0.0;
    for (int i = 0; i < dim; ++i) {
        // fma(a, b, acc) would round once instead of twice; the product is
        // exact in double anyway, so a separate multiply and add is identical.
        double p1 = (double)lq1[base + i] * (double)lk1[base + i];
        double p2 = (double)lq2[base + i] * (double)lk2[base + i];
        d1 = d1 + p1;
        d2 = d2 + p2;
    }
    out[h] = (float)(exp(d1) - exp(d2) + lambda_init);
}

hipError_t launch_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                         int H, int dim, double lambda_init, float* out, hipStream_t stream) {
    int blocks = (H + 63) / 64;
    hipLaunchKernelGGL(lambda_kernel, dim3(blocks), dim3(64), 0, stream, lq1, lk1, lq2, lk2, H,
                       dim, lambda_init, out);
    return hipGetLastError();
}

}  // namespace diffattn
