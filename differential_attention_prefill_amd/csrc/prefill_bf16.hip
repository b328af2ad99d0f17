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
//    tile is computed.  Keys hold both halves K1|K2 in one LDS row; values
//    stay token-major, and the P.V product, which contracts over keys, reads
//    its V^T operand with the gfx950 LDS transpose load (ds_read_b64_tr_b16):
//    each 16-lane group reads a 4-key x 16-channel block and every lane
//    receives 4 keys of one channel.
//  - Two workgroups share a CU (<= 256 registers per lane), so one wave's
//    softmax arithmetic overlaps the other's matrix products.
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
    // Row pitches in LDS.  A key row (K1|K2) is padded by 16 bytes so that
    // the 16 rows read by one 16-lane quarter land in distinct banks; a value
    // row is padded so consecutive rows start 16 banks apart, which keeps the
    // 4-row x 32-byte blocks of the transpose load conflict-free.
    static constexpr int KROW = 2 * D * 2 + 16;
    static constexpr int VROW = DV * 2 + 64;
    static constexpr int KBYTES = BN * KROW;
    static constexpr int VBYTES = BN * VROW;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int KCHUNKS = BN * (2 * D) / 8;   // 16-byte chunks per key tile
    static constexpr int KPT = (KCHUNKS + THREADS - 1) / THREADS;
    static constexpr int VCHUNKS = BN * DV / 8;        // 16-byte chunks per value tile
    static constexpr int VPT = (VCHUNKS + THREADS - 1) / THREADS;
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

// max(a, b, c) in one instruction.  Written out because fmaxf chains get an
// extra quieting max per operand in IEEE mode; scores are never NaN here.
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// gfx950 LDS transpose load: within each 16-lane group, lane j supplies an
// 8-byte segment (4 bf16) at `p`; lane i receives element i%4 of the
// segments supplied by lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ bf16x4 lds_read_tr(const unsigned char* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<unsigned char*>(p)));
    return __builtin_bit_cast(bf16x4, v);
}

// OCC: waves per SIMD the register budget is cut for (2 lets one wave's
// softmax overlap the other's matrix products; d = 128 keeps 1 so that its
// larger query fragments stay in registers).
template <int D, int DV, int WAVES, int OCC>
__global__ void __launch_bounds__(WAVE * WAVES) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
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
    // Let the query loads land before the loop: otherwise the wait inserted
    // for their first use inside the loop also waits for the tile prefetch.
    __builtin_amdgcn_s_waitcnt(0);

    const float c = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)
    float mref[2] = {-INFINITY, -INFINITY};   // reference maxima (raw score units)
    float lsum[2] = {0.f, 0.f};               // this lane's share of the normalisers
    f32x16 acc[2][C::VBLK];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][nb][r] = 0.f;

    const int kv_end = causal ? min(N, q0 + C::BM) : N;
    const int ntiles = (kv_end + BN - 1) / BN;

    // Lane-constant LDS offsets.
    // K fragment: row kappa(col), 8 elements at half*8 of each k-step.
    const int k_lane_off = kappa(col) * C::KROW + half * 16;
    // V^T fragment through the transpose load: group g = lane/16 covers
    // channels 16*(g%2) .. +15 of a 32-channel block and keys 8*(g/2) .. +7 of
    // a 16-key step; lane j of the group points at key 4*r + j/4, channels
    // 4*(j%4) .. +3 for the two loads r = 0, 1.
    const int grp = lane >> 4, gl = lane & 15;
    const int v_lane_off = ((grp >> 1) * 8 + (gl >> 2)) * C::VROW + (16 * (grp & 1) + 4 * (gl & 3)) * 2;

    // ---- global -> register prefetch of one key/value tile --------------
    uint4 kreg[C::KPT];
    uint4 vreg[C::VPT];
    auto fetch = [&](int t) {
        const int kb = t * BN;
        // Positions past the sequence end load row 0 of the head instead:
        // their scores are masked to -inf, so their probabilities are exactly
        // zero and the row contributes nothing.  (Selecting zeros here would
        // make every load wait for its data immediately.)
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int ch = tid + i * C::THREADS;
            const int key = ch / (D / 4);
            const int part = ch % (D / 4);           // 16-byte chunk of K1|K2
            const bool ok = (C::KCHUNKS % C::THREADS == 0 || ch < C::KCHUNKS) && kb + key < N;
            const int64_t row = tok0 + (ok ? kb + key : 0);
            kreg[i] = load16((part < D / 8) ? k1 + row * ldk + part * 8
                                            : k2 + row * ldk + (part - D / 8) * 8);
        }
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
            const int ch = tid + i * C::THREADS;
            const int key = ch / (DV / 8);
            const int part = ch % (DV / 8);
            const bool ok = (C::VCHUNKS % C::THREADS == 0 || ch < C::VCHUNKS) && kb + key < N;
            vreg[i] = load16(v + (tok0 + (ok ? kb + key : 0)) * ldv + part * 8);
        }
    };
    auto stash = [&](int stage) {
        unsigned char* base = smem + stage * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int ch = tid + i * C::THREADS;
            if (ch < C::KCHUNKS)
                *reinterpret_cast<uint4*>(base + (ch / (D / 4)) * C::KROW + (ch % (D / 4)) * 16) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
            const int ch = tid + i * C::THREADS;
            if (ch < C::VCHUNKS)
                *reinterpret_cast<uint4*>(base + C::KBYTES + (ch / (DV / 8)) * C::VROW + (ch % (DV / 8)) * 16) = vreg[i];
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
        const bool need_mask = (kb + BN > N) || (causal && kb + BN - 1 > wrow0);

        // ---- per map: S^T = K . Q^T, online softmax, P^T fragments --------
        bf16x8 pf[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
            for (int st = 0; st < C::KSTEPS; ++st) {
                bf16x8 kf = __builtin_bit_cast(bf16x8, load16(kt + k_lane_off + (m * D + st * 16) * 2));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[m][st], s, 0, 0, 0);
            }
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb + kappa((r >> 2) * 8 + half * 4 + (r & 3));
                    if (key >= N || (causal && key > my_row)) s[r] = -INFINITY;
                }
            }
            float mx = max3(s[0], s[1], s[2]);
#pragma unroll
            for (int r = 3; r < 15; r += 2) mx = max3(mx, s[r], s[r + 1]);
            mx = max3(mx, s[15], s[15]);
            // Row maximum: this lane's 16 keys, the partner lane's 16, and the
            // reference the accumulator was built on.
            const float mnew = max3(mref[m], mx, __shfl_xor(mx, 32));
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
            float ls = lsum[m];
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    f32x2 pr = {__builtin_amdgcn_exp2f(fmaf(s[t2 * 8 + e], c, -mc)),
                                __builtin_amdgcn_exp2f(fmaf(s[t2 * 8 + e + 1], c, -mc))};
                    bf16x2 pb = __builtin_convertvector(pr, bf16x2);
                    // The normaliser sums the same bf16 probabilities the
                    // product uses.
                    ls = __builtin_amdgcn_fdot2_f32_bf16(pb, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, ls, false);
                    pf[m][t2][e] = pb[0];
                    pf[m][t2][e + 1] = pb[1];
                }
            }
            lsum[m] = ls;
        }

        // ---- O^T += V^T . P^T for both maps (shared V fragments) ---------
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb) {
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const unsigned char* vp = vt + v_lane_off + t2 * 16 * C::VROW + nb * 64;
                bf16x4 lo = lds_read_tr(vp);
                bf16x4 hi = lds_read_tr(vp + 4 * C::VROW);
                bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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

template <int D, int DV, int WAVES, int OCC>
hipError_t launch_bf16(const PrefillArgs& a, hipStream_t stream) {
    using C = Cfg<D, DV, WAVES>;
    const int row_tiles = (a.N + C::BM - 1) / C::BM;
    const int BH = a.B * a.H;
    const int64_t blocks = (int64_t)BH * row_tiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = 2 * (size_t)C::STAGE;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, WAVES, OCC>), dim3((unsigned)blocks),
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
    if (a.d == 64 && a.dv == 128) return launch_bf16<64, 128, 4, 2>(a, stream);
    if (a.d == 64 && a.dv == 64) return launch_bf16<64, 64, 4, 2>(a, stream);
    if (a.d == 32 && a.dv == 64) return launch_bf16<32, 64, 4, 2>(a, stream);
    if (a.d == 128 && a.dv == 128) return launch_bf16<128, 128, 4, 1>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
