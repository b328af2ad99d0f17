// Fused differential-attention prefill on gfx950 matrix cores (bf16 in, fp32
// accumulate).
//
// Per head (b,h) and query row i:
//     A1 = softmax(q1_i K1^T / sqrt d),   A2 = softmax(q2_i K2^T / sqrt d),
//     o_i = (A1 - lambda_h A2) V,   optional y_i = RMSNorm(o_i) * w * s
// (page "差分注意力" (aiknowledge.cn), part 一 "差分思路" and part 二 Step 2;
// per-head normalisation after the difference: "V1 到 V2 的 diff").
//
// One pass over a shared key/value stream (page "【架构革新】...", section 3:
// the two softmaxes share intermediates inside one fused kernel):
//  - A workgroup owns BM = 32*WAVES query rows of one head; each wave owns 32
//    rows.  Keys and values stream through LDS in tiles of 32 keys, double
//    buffered: the next tile's global loads are issued before the current
//    tile is computed.  Keys hold both halves K1|K2 in one LDS row; values are
//    written into LDS transposed (channel-major) because the P.V product
//    contracts over keys.
//  - Scores are formed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_bf16: a lane then holds 16 keys of ONE query, so
//    each softmax row statistic is a per-lane quantity plus a single exchange
//    with the lane 32 apart.
//  - Keys are loaded into the A operand in a bit-permuted order (bits 2 and 3
//    of the row index swapped), which makes the score accumulator's register
//    order coincide with the B-operand order of the next product: the
//    probabilities feed O^T += V^T . P^T straight from registers, no LDS
//    round trip.
//  - Each map keeps its own running maximum, normaliser and fp32 accumulator
//    (the two maps rescale independently, so an exact single pass needs two
//    accumulators); lambda combines them once, in the epilogue, followed by
//    the optional RMS norm.
//  - Rescaling is lazy: an accumulator is rescaled only when a row maximum
//    grows by more than 8 (base 2) over the reference it was built on, so
//    probabilities stay <= 2^8.  Results are the same exact quantity.
//  - Causal: tiles wholly above a wave's rows are skipped; only tiles that
//    straddle the diagonal or the sequence end are masked.  Heavy query tiles
//    are scheduled first, and consecutive workgroups take different heads so
//    that each XCD's L2 serves a fixed set of heads.
#include "kernels.h"

namespace diffattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int QROWS = 32;      // query rows per wave (MFMA N dimension)
constexpr int BN = 32;         // keys per tile (MFMA M dimension of S^T)
constexpr float TAU = 8.0f;    // lazy-rescale threshold, base-2 exponent units

template <int D, int DV, int WAVES>
struct Cfg {
    static constexpr int THREADS = WAVE * WAVES;
    static constexpr int BM = QROWS * WAVES;
    static constexpr int KROW = 2 * D * 2 + 16;   // bytes per key row in LDS: K1|K2 + pad
    static constexpr int VROW = BN * 2 + 16;      // bytes per channel row of V^T + pad
    static constexpr int KBYTES = BN * KROW;
    static constexpr int VBYTES = DV * VROW;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int KCHUNKS = BN * (2 * D) / 8;   // 16-byte chunks per key tile
    static constexpr int KPT = (KCHUNKS + THREADS - 1) / THREADS;
    static constexpr int VITEMS = (BN / 2) * (DV / 8); // (2 keys x 8 channels) items
    static constexpr int VPT = (VITEMS + THREADS - 1) / THREADS;
    static constexpr int KSTEPS = D / 16;             // MFMA k-steps for one score map
    static constexpr int VBLK = DV / 32;              // 32-channel blocks of O^T
};

// Row slot rho of the S^T tile holds key kappa(rho): bits 2 and 3 swapped.
__device__ __forceinline__ int kappa(int rho) {
    return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

template <int D, int DV, int WAVES>
__global__ void __launch_bounds__(WAVE * WAVES)
prefill_bf16_kernel(const __bf16* __restrict__ q1, const __bf16* __restrict__ q2,
                    const __bf16* __restrict__ k1, const __bf16* __restrict__ k2,
                    const __bf16* __restrict__ v, int64_t ldq, int64_t ldk, int64_t ldv,
                    int BH, int H, int N, int causal, const float* __restrict__ lambda,
                    int rmsnorm, float eps, float norm_scale,
                    const float* __restrict__ norm_weight, float* __restrict__ out,
                    int row_tiles) {
    using C = Cfg<D, DV, WAVES>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;   // query column inside the wave's 32 rows
    const int half = lane >> 5;  // which 8-element half of each 16-element k-step

    // Consecutive workgroups take consecutive heads (so each XCD sees a fixed
    // subset of heads); within a head the heaviest causal tiles come first.
    const int bh = blockIdx.x % BH;
    const int tile = row_tiles - 1 - (int)(blockIdx.x / BH);
    const int h = bh % H;
    const int q0 = tile * C::BM;
    const int64_t tok0 = (int64_t)bh * N;

    const int wrow0 = q0 + wave * QROWS;          // first row of this wave
    const int my_row = wrow0 + col;                // this lane's query row
    const int wrow_last = min(wrow0 + QROWS, N) - 1;  // < wrow0 if the wave is idle

    // Query fragments (B operand of S^T = K . Q^T): lane holds 8 consecutive
    // elements of its row for each 16-element k-step of each map.
    bf16x8 qf[2][C::KSTEPS];
    {
        const bool ok = my_row < N;
        const __bf16* r1 = q1 + (tok0 + (ok ? my_row : 0)) * ldq + half * 8;
        const __bf16* r2 = q2 + (tok0 + (ok ? my_row : 0)) * ldq + half * 8;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            uint4 a = ok ? load16(r1 + s * 16) : make_uint4(0, 0, 0, 0);
            uint4 b = ok ? load16(r2 + s * 16) : make_uint4(0, 0, 0, 0);
            qf[0][s] = __builtin_bit_cast(bf16x8, a);
            qf[1][s] = __builtin_bit_cast(bf16x8, b);
        }
    }

    const float c = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)
    float mref[2] = {-INFINITY, -INFINITY};   // reference maxima (raw score units)
    float lsum[2] = {0.f, 0.f};               // this lane's share of the normalisers
    f32x16 acc[2][C::VBLK];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb)
            for (int r = 0; r < 16; ++r) acc[m][nb][r] = 0.f;

    const int kv_end = causal ? min(N, q0 + C::BM) : N;
    const int ntiles = (kv_end + BN - 1) / BN;

    // ---- global -> register prefetch of one key/value tile --------------
    uint4 kreg[C::KPT];
    uint4 vreg[C::VPT][2];
    auto fetch = [&](int t) {
        const int kb = t * BN;
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int ch = tid + i * C::THREADS;
            const int key = ch / (D / 4);
            const int part = ch % (D / 4);           // 16-byte chunk of K1|K2
            uint4 val = make_uint4(0, 0, 0, 0);
            if (ch < C::KCHUNKS && kb + key < N) {
                const __bf16* src = (part < D / 8) ? k1 + (tok0 + kb + key) * ldk + part * 8
                                                   : k2 + (tok0 + kb + key) * ldk + (part - D / 8) * 8;
                val = load16(src);
            }
            kreg[i] = val;
        }
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
            const int it = tid + i * C::THREADS;
            const int kp = it / (DV / 8);            // key pair
            const int ch = it % (DV / 8);            // 8-channel chunk
            uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
            if (it < C::VITEMS) {
                const int key = kb + 2 * kp;
                if (key < N) a = load16(v + (tok0 + key) * ldv + ch * 8);
                if (key + 1 < N) b = load16(v + (tok0 + key + 1) * ldv + ch * 8);
            }
            vreg[i][0] = a;
            vreg[i][1] = b;
        }
    };
    auto stash = [&](int stage) {
        unsigned char* base = smem + stage * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int ch = tid + i * C::THREADS;
            if (ch < C::KCHUNKS) {
                const int key = ch / (D / 4);
                const int part = ch % (D / 4);
                *reinterpret_cast<uint4*>(base + key * C::KROW + part * 16) = kreg[i];
            }
        }
        unsigned char* vt = base + C::KBYTES;
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
            const int it = tid + i * C::THREADS;
            if (it < C::VITEMS) {
                const int kp = it / (DV / 8);
                const int ch = it % (DV / 8);
                const unsigned aw[4] = {vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w};
                const unsigned bw[4] = {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // channel ch*8+e of keys 2kp and 2kp+1 -> one dword of V^T
                    const unsigned lo = (e & 1) ? (aw[e >> 1] >> 16) : (aw[e >> 1] & 0xffffu);
                    const unsigned hi = (e & 1) ? (bw[e >> 1] & 0xffff0000u) : (bw[e >> 1] << 16);
                    *reinterpret_cast<unsigned*>(vt + (ch * 8 + e) * C::VROW + kp * 4) = lo | hi;
                }
            }
        }
    };

    if (ntiles > 0) fetch(0);
    for (int t = 0; t < ntiles; ++t) {
        const int stage = t & 1;
        stash(stage);
        if (t + 1 < ntiles) fetch(t + 1);
        __syncthreads();

        const int kb = t * BN;
        // Skip tiles wholly above this wave's rows (or an idle wave).
        if (wrow_last < wrow0 || (causal && kb > wrow_last)) continue;

        const unsigned char* kt = smem + stage * C::STAGE;
        const unsigned char* vt = kt + C::KBYTES;

        // ---- S^T = K . Q^T for both maps --------------------------------
        f32x16 s[2];
        const unsigned char* krow = kt + kappa(col) * C::KROW + half * 16;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            for (int r = 0; r < 16; ++r) s[m][r] = 0.f;
#pragma unroll
            for (int st = 0; st < C::KSTEPS; ++st) {
                bf16x8 kf = __builtin_bit_cast(bf16x8, load16(krow + (m * D + st * 16) * 2));
                s[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[m][st], s[m], 0, 0, 0);
            }
        }

        // ---- mask the diagonal / ragged tile ----------------------------
        const bool need_mask = (kb + BN > N) || (causal && kb + BN - 1 > wrow0);
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rho = (r >> 2) * 8 + half * 4 + (r & 3);
                const int key = kb + kappa(rho);
                const bool dead = key >= N || (causal && key > my_row);
                if (dead) {
                    s[0][r] = -INFINITY;
                    s[1][r] = -INFINITY;
                }
            }
        }

        // ---- online softmax, both maps, and P^T fragments ---------------
        bf16x8 pf[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            float mx = s[m][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[m][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(mref[m], mx);
            const bool grow = mnew > -INFINITY && (mref[m] == -INFINITY || (mnew - mref[m]) * c > TAU);
            if (__any(grow)) {
                const float alpha = (mnew == -INFINITY) ? 1.f
                                                         : __builtin_amdgcn_exp2f((mref[m] - mnew) * c);
                mref[m] = mnew;
                lsum[m] *= alpha;
#pragma unroll
                for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[m][nb][r] *= alpha;
            }
            const float mc = (mref[m] == -INFINITY) ? 0.f : mref[m] * c;
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s[m][r], c, -mc));
            float ls = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) ls += p[r];
            lsum[m] += ls;
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    f32x2 pr = {p[t2 * 8 + e], p[t2 * 8 + e + 1]};
                    bf16x2 pb = __builtin_convertvector(pr, bf16x2);
                    pf[m][t2][e] = pb[0];
                    pf[m][t2][e + 1] = pb[1];
                }
            }
        }

        // ---- O^T += V^T . P^T for both maps (shared V fragments) ---------
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb) {
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                bf16x8 vf = __builtin_bit_cast(
                    bf16x8, load16(vt + (nb * 32 + col) * C::VROW + (t2 * 16 + half * 8) * 2));
                acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[0][t2], acc[0][nb], 0, 0, 0);
                acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[1][t2], acc[1][nb], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: combine the maps with lambda, optional RMS norm ----------
    if (my_row >= N) return;
    const float l1 = lsum[0] + __shfl_xor(lsum[0], 32);
    const float l2 = lsum[1] + __shfl_xor(lsum[1], 32);
    const float w1 = 1.f / l1;
    const float w2 = lambda[h] / l2;
    float ss = 0.f;
#pragma unroll
    for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float y = acc[0][nb][r] * w1 - acc[1][nb][r] * w2;
            acc[0][nb][r] = y;
            ss = fmaf(y, y, ss);
        }
    float scale = 1.f;
    if (rmsnorm) {
        ss += __shfl_xor(ss, 32);
        scale = norm_scale / sqrtf(ss / (float)DV + eps);
    }
    float* orow = out + (tok0 + my_row) * DV;
#pragma unroll
    for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int ch = nb * 32 + g * 8 + half * 4;   // 4 consecutive channels
            f32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float w = (rmsnorm && norm_weight) ? norm_weight[ch + e] : 1.f;
                y[e] = acc[0][nb][g * 4 + e] * scale * w;
            }
            *reinterpret_cast<f32x4*>(orow + ch) = y;
        }
}

template <int D, int DV, int WAVES>
hipError_t launch_bf16(const PrefillArgs& a, hipStream_t stream) {
    using C = Cfg<D, DV, WAVES>;
    const int row_tiles = (a.N + C::BM - 1) / C::BM;
    const int BH = a.B * a.H;
    const int64_t blocks = (int64_t)BH * row_tiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = 2 * (size_t)C::STAGE;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, WAVES>), dim3((unsigned)blocks),
                       dim3(C::THREADS), lds, stream, (const __bf16*)a.q1, (const __bf16*)a.q2,
                       (const __bf16*)a.k1, (const __bf16*)a.k2, (const __bf16*)a.v, a.ldq, a.ldk,
                       a.ldv, BH, a.H, a.N, a.causal, a.lambda, a.rmsnorm, a.eps, a.norm_scale,
                       a.norm_weight, a.out, row_tiles);
    return hipGetLastError();
}

}  // namespace

bool prefill_bf16_supported(int d, int dv) {
    return (d == 64 && dv == 128) || (d == 64 && dv == 64) || (d == 32 && dv == 64) ||
           (d == 128 && dv == 128);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    if (a.d == 64 && a.dv == 128) return launch_bf16<64, 128, 4>(a, stream);
    if (a.d == 64 && a.dv == 64) return launch_bf16<64, 64, 4>(a, stream);
    if (a.d == 32 && a.dv == 64) return launch_bf16<32, 64, 4>(a, stream);
    if (a.d == 128 && a.dv == 128) return launch_bf16<128, 128, 4>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
