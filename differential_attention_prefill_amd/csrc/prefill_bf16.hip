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
//    rows.  Keys and values stream through LDS in tiles of 64 keys, double
//    buffered, copied by buffer loads that write LDS directly (no staging
//    registers); the copy of tile T+1 runs while tile T is computed, and
//    one barrier per tile hands a stage over.  Rows are XOR-swizzled in
//    16-byte chunks so that fragment reads hit distinct banks.  Values stay
//    token-major, and the P.V product, which contracts over keys, reads its
//    V^T operand with the gfx950 LDS transpose load (ds_read_b64_tr_b16):
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
    static constexpr int TK = 2 * BN;                 // keys per stage (two 32-key sub-tiles)
    static constexpr int KC = D / 8;                  // 16-byte chunks per key half-row
    static constexpr int VC = DV / 8;                 // 16-byte chunks per value row
    static constexpr int KROWB = D * 2;               // bytes per key half-row (K1 or K2)
    static constexpr int VROWB = DV * 2;              // bytes per value row
    static constexpr int K1_OFF = 0;
    static constexpr int K2_OFF = TK * KROWB;
    static constexpr int V_OFF = 2 * TK * KROWB;
    static constexpr int STAGE = 2 * TK * KROWB + TK * VROWB;
    // One LDS-DMA instruction moves 1 KB (64 lanes x 16 bytes).
    static constexpr int KI = TK * KROWB / 1024 / WAVES;   // per wave, per key half
    static constexpr int VI = TK * VROWB / 1024 / WAVES;   // per wave
    static constexpr int KRPI = 1024 / KROWB;              // key rows per DMA instruction
    static constexpr int VRPI = 1024 / VROWB;              // value rows per DMA instruction
    static constexpr int KSTEPS = D / 16;                  // MFMA k-steps for one score map
    static constexpr int VBLK = DV / 32;                   // 32-channel blocks of O^T
    static_assert(KI >= 1 && VI >= 1, "tile must give every wave whole DMA instructions");
};

// Chunk swizzles (physical chunk = logical chunk ^ swizzle(row)).
// Keys: the 16 rows read by one 16-lane quarter must land in 16 distinct
// 16-byte bank groups of a 256-byte bank line.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
    constexpr int KC = D / 8, RPB = 256 / (D * 2);     // rows per 256-byte bank line
    return (row / RPB) % KC;
}
// Values: a transpose load reads 4 consecutive rows x 32 bytes per 16-lane
// group; the swizzle spreads them (and the neighbouring group's) over
// distinct bank groups.
template <int DV>
__device__ __forceinline__ int v_swz(int row) {
    if constexpr (DV == 128) return 4 * (row & 3);
    else return 2 * ((row >> 1) & 1);
}

// Row slot rho of the S^T tile holds key kappa(rho): bits 2 and 3 swapped.
__device__ __forceinline__ int kappa(int rho) {
    return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// max(a, b, c): this file is compiled with IEEE mode off and NaNs not
// honoured, so the chain lowers to one v_max3_f32 with no quieting of its
// inputs.  (It must stay visible to the compiler: reading matrix-core
// results needs wait states that only the compiler inserts.)
__device__ __forceinline__ float max3(float a, float b, float c) {
    return fmaxf(fmaxf(a, b), c);
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
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (gfx9-family layout): base, stride 0, byte extent.
// Loads at offsets >= `bytes` return zeros.  Scalar registers throughout.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int bytes) {
    const unsigned long long a = (unsigned long long)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000;
    return r;
}

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)((__attribute__((address_space(3))) const unsigned char*)p);
}

// 16 bytes per lane from global memory straight into LDS at
// lds_base + 16*lane (lds_base wave-uniform).  Written as an instruction the
// compiler does not track: it would otherwise wait for every copy in flight
// before each LDS read.  Completion is awaited explicitly (vmcnt) before the
// barrier that publishes a stage.
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, unsigned lds_base, int voff) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base)
                 : "memory");
}

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
    // Wave-uniform values live in scalar registers, so tile skipping and
    // masking decisions are scalar branches rather than per-lane selects.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // Lane-constant LDS offsets (within a stage, sub-tile 0; sub-tile 1 adds
    // 32 rows, which leaves both swizzles unchanged).
    // K fragment of k-step st: row kappa(col), logical chunk 2*st + half.
    int k_frag[C::KSTEPS];
    {
        const int row = kappa(col);
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st)
            k_frag[st] = row * C::KROWB + (((2 * st + half) ^ k_swz<D>(row)) * 16);
    }
    // V^T fragment through the transpose load: group g = lane/16 covers
    // channels 16*(g%2) .. +15 of a 32-channel block and keys 8*(g/2) .. +7 of
    // a 16-key step; lane j of the group points at key 4*r + j/4, channels
    // 4*(j%4) .. +3 for the two loads r = 0, 1.
    const int grp = lane >> 4, gl = lane & 15;
    int v_frag[C::VBLK];
    {
        const int row = (grp >> 1) * 8 + (gl >> 2);          // + t2*16 + r*4 (+32 per sub-tile)
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb) {
            const int chunk = nb * 4 + 2 * (grp & 1) + ((gl & 3) >> 1);
            v_frag[nb] = C::V_OFF + row * C::VROWB + ((chunk ^ v_swz<DV>(row)) * 16) + 8 * (gl & 1);
        }
    }

    // ---- global -> LDS copies of one 64-key tile ------------------------
    // Buffer descriptors start at the tile's first key and end at the
    // sequence end: rows past N read as zeros (their scores are masked).
    auto rsrc = [&](const __bf16* base, int64_t ld, int kb) {
        const int rows = max(0, min(N - kb, C::TK));
        return make_rsrc(base + (tok0 + kb) * ld, rows * (int)ld * 2);
    };
    // Lane-constant source offsets of this wave's DMA instructions.
    int koff[C::KI], voff[C::VI];
#pragma unroll
    for (int j = 0; j < C::KI; ++j) {
        const int row = (wave * C::KI + j) * C::KRPI + lane / C::KC;
        const int chunk = (lane % C::KC) ^ k_swz<D>(row);
        koff[j] = row * (int)ldk * 2 + chunk * 16;
    }
#pragma unroll
    for (int j = 0; j < C::VI; ++j) {
        const int row = (wave * C::VI + j) * C::VRPI + lane / C::VC;
        const int chunk = (lane % C::VC) ^ v_swz<DV>(row);
        voff[j] = row * (int)ldv * 2 + chunk * 16;
    }
    auto issue_tile = [&](int T) {
        const int kb = T * C::TK;
        const unsigned st = __builtin_amdgcn_readfirstlane(lds_addr(smem) + (T & 1) * C::STAGE);
        const i32x4 r1 = rsrc(k1, ldk, kb);
        const i32x4 r2 = rsrc(k2, ldk, kb);
        const i32x4 rv = rsrc(v, ldv, kb);
#pragma unroll
        for (int j = 0; j < C::KI; ++j) {
            const unsigned dst = st + (wave * C::KI + j) * 1024;
            copy16_to_lds(r1, dst + C::K1_OFF, koff[j]);
            copy16_to_lds(r2, dst + C::K2_OFF, koff[j]);
        }
#pragma unroll
        for (int j = 0; j < C::VI; ++j)
            copy16_to_lds(rv, st + C::V_OFF + (wave * C::VI + j) * 1024, voff[j]);
    };

    // One key tile: scores, online softmax and both P.V products.
    auto tile_body = [&](const unsigned char* stg, int sub, int kb, bool masked) {
        const unsigned char* kt = stg + sub * BN * C::KROWB;
        const unsigned char* vt = stg + sub * BN * C::VROWB;
        // ---- per map: S^T = K . Q^T, online softmax, P^T fragments --------
        bf16x8 pf[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
            // Matrix sections run at raised wave priority: when both waves of
            // a SIMD are ready, the one feeding the matrix core issues first
            // and the other wave's softmax fills the gaps.
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int st = 0; st < C::KSTEPS; ++st) {
                bf16x8 kf = __builtin_bit_cast(bf16x8, load16(kt + k_frag[st] + (m ? C::K2_OFF : C::K1_OFF)));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[m][st], s, 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
            // Rare (diagonal / last tile), uniform: kept as a real branch.
            if (__builtin_expect(masked, 0)) {
                // key kb + kappa(rho) is visible iff kappa(rho) < lim.
                const int lim = causal ? min(N - kb, my_row - kb + 1) : N - kb;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kappa((r >> 2) * 8 + half * 4 + (r & 3)) >= lim) s[r] = -INFINITY;
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
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb) {
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const unsigned char* vp = vt + v_frag[nb] + t2 * 16 * C::VROWB;
                bf16x4 lo = lds_read_tr(vp);
                bf16x4 hi = lds_read_tr(vp + 4 * C::VROWB);
                bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[0][t2], acc[0][nb], 0, 0, 0);
                acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[1][t2], acc[1][nb], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    const int ntiles = (kv_end + C::TK - 1) / C::TK;
    if (ntiles > 0) issue_tile(0);
    for (int T = 0; T < ntiles; ++T) {
        // Tile T's copies (the only vector-memory operations in flight) have
        // landed for this wave; the barrier makes every wave's copies visible
        // and shows that every wave is done reading the stage copied into next.
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (T + 1 < ntiles) issue_tile(T + 1);
        const unsigned char* stg = smem + (T & 1) * C::STAGE;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int kb = T * C::TK + sub * BN;
            // Skip sub-tiles past the keys this wave can see (uniform).
            if (wrow_last < wrow0 || kb >= kv_end || (causal && kb > wrow_last)) continue;
            // Only tiles that straddle the diagonal or the sequence end need a mask.
            tile_body(stg, sub, kb, (kb + BN > N) || (causal && kb + BN - 1 > wrow0));
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
    static bool attr_set = false;    // raise the dynamic-LDS limit once per process
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)prefill_bf16_kernel<D, DV, WAVES, OCC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
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
