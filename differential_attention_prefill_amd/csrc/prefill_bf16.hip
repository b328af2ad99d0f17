// Fused differential-attention prefill on gfx950 matrix cores (bf16 in, fp32
// accumulate), map-split schedule: used for d = 128, whose query fragments of
// both maps do not fit one wave's registers next to two accumulators (the
// ping-pong schedule in prefill_pp.hip serves d <= 64).
//
// Per head (b,h) and query row i:
//     A1 = softmax(q1_i K1^T / sqrt d),   A2 = softmax(q2_i K2^T / sqrt d),
//     o_i = (A1 - lambda_h A2) V,   optional y_i = RMSNorm(o_i) * w * s
// (page "差分注意力" (aiknowledge.cn), part 一 "差分思路" and part 二 Step 2;
// per-head normalisation after the difference: "V1 到 V2 的 diff").
//
// One pass over a shared key/value stream (page "【架构革新】...", section 3:
// the two softmaxes share intermediates inside one fused kernel):
//  - A workgroup owns 128 query rows of one head, as 4 row blocks of 32, and
//    runs 8 waves: wave w computes map 1 + (w >= 4) for row block w % 4.  The
//    two maps of a row block live in different waves.  Each wave keeps one
//    fp32 accumulator (the maps rescale independently, so an exact single
//    pass needs one per map), one query half and one score tile: about half
//    the registers of a wave that does both maps, so twice as many waves fit
//    on a SIMD and the hardware hides one wave's softmax arithmetic behind
//    other waves' matrix products.  At the end the map-2 waves hand their
//    lambda-scaled accumulators to the map-1 waves through LDS, which take
//    the difference and apply the optional RMS norm.
//  - Keys and values stream through LDS in tiles of 64 keys, double
//    buffered, copied by buffer loads that write LDS directly (no staging
//    registers): map-1 waves copy both key halves, map-2 waves the values.
//    The copy of tile T+1 runs while tile T is computed, and one barrier per
//    tile hands a stage over.  Rows are XOR-swizzled in 16-byte chunks so
//    that fragment reads hit distinct banks.  Values stay token-major; the
//    P.V product, which contracts over keys, reads its V^T operand with the
//    gfx950 LDS transpose load (ds_read_b64_tr_b16): each 16-lane group reads
//    a 4-key x 16-channel block and every lane receives 4 keys of one channel.
//  - Scores are formed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_bf16: a lane then holds 16 keys of ONE query, so
//    each softmax row statistic is a per-lane quantity plus one exchange with
//    the lane 32 apart.
//  - Keys are loaded into the A operand in a bit-permuted order (bits 2 and 3
//    of the row index swapped), which makes the score accumulator's register
//    order coincide with the B-operand order of the next product: the
//    probabilities feed O^T += V^T . P^T straight from registers.
//  - Rescaling is lazy: an accumulator is rescaled only when a row maximum
//    grows by more than 8 (base 2) over the reference it was built on, so
//    probabilities stay <= 2^8.  Results are the same exact quantity.
//  - Causal: sub-tiles wholly above a row block are skipped; only those that
//    straddle the diagonal or the sequence end are masked.  Heavy query tiles
//    are scheduled first, and consecutive workgroups take different heads so
//    that each XCD's L2 serves a fixed set of heads.
#include "kernels.h"
#include "bf16_tile.h"

namespace diffattn {
namespace {

using namespace tile;

constexpr int RBLK = 4;        // row blocks per workgroup
constexpr int WAVES = 2 * RBLK;
constexpr int THREADS = WAVE * WAVES;
constexpr int BM = QROWS * RBLK;

template <int D, int DV>
struct Cfg {
    static constexpr int KC = D / 8;                  // 16-byte chunks per key half-row
    static constexpr int VC = DV / 8;                 // 16-byte chunks per value row
    static constexpr int KROWB = D * 2;               // bytes per key half-row (K1 or K2)
    static constexpr int VROWB = DV * 2;              // bytes per value row
    static constexpr int K1_OFF = 0;
    static constexpr int K2_OFF = TK * KROWB;
    static constexpr int V_OFF = 2 * TK * KROWB;
    static constexpr int STAGE = 2 * TK * KROWB + TK * VROWB;
    // One LDS-DMA instruction moves 1 KB (64 lanes x 16 bytes).
    static constexpr int KPW = TK * KROWB / 1024 / RBLK;   // per map-1 wave, per key half
    static constexpr int VPW = TK * VROWB / 1024 / RBLK;   // per map-2 wave
    static constexpr int CPW = KPW > VPW ? KPW : VPW;
    static constexpr int KRPI = 1024 / KROWB;              // key rows per DMA instruction
    static constexpr int VRPI = 1024 / VROWB;              // value rows per DMA instruction
    static constexpr int KSTEPS = D / 16;                  // MFMA k-steps of one score map
    static constexpr int VBLK = DV / 32;                   // 32-channel blocks of O^T
    static constexpr int XBYTES = RBLK * QROWS * DV * 4;   // epilogue hand-over buffer
    static constexpr int LDS = 2 * STAGE > XBYTES ? 2 * STAGE : XBYTES;
    static_assert(KPW >= 1 && VPW >= 1, "tile must give every copying wave whole instructions");
};

// Wait for this wave's LDS accesses and copies, then a workgroup barrier.
__device__ __forceinline__ void sync_stage() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// OCC: waves per SIMD the register budget is cut for.
template <int D, int DV, int OCC>
__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
prefill_bf16_kernel(const __bf16* __restrict__ q1, const __bf16* __restrict__ q2,
                    const __bf16* __restrict__ k1, const __bf16* __restrict__ k2,
                    const __bf16* __restrict__ v, int64_t ldq, int64_t ldk, int64_t ldv,
                    int BH, int H, int N, int causal, const float* __restrict__ lambda,
                    int rmsnorm, float eps, float norm_scale,
                    const float* __restrict__ norm_weight, float* __restrict__ out,
                    int row_tiles, HeadStrides hs) {
    using C = Cfg<D, DV>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave-uniform values live in scalar registers, so tile skipping and
    // masking decisions are scalar branches rather than per-lane selects.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int map = wave / RBLK;   // 0: A1 from (q1, k1); 1: A2 from (q2, k2)
    const int rb = wave % RBLK;    // row block
    const int col = lane & 31;     // query column inside the row block
    const int half = lane >> 5;    // which 8-element half of each 16-element k-step

    // Consecutive workgroups take consecutive heads (so each XCD sees a fixed
    // subset of heads); within a head the heaviest causal tiles come first.
    const int bh = blockIdx.x % BH;
    const int tile = row_tiles - 1 - (int)(blockIdx.x / BH);
    const int h = bh % H;
    const int q0 = tile * BM;
    const int64_t tok0 = (int64_t)bh * N;                 // output rows
    const int64_t qoff = (bh / H) * hs.qb + h * hs.qh;
    const int64_t koff = (bh / H) * hs.kb + (h / hs.kv_group) * hs.kh;
    const int64_t voff = (bh / H) * hs.vb + (h / hs.kv_group) * hs.vh;

    const int wrow0 = q0 + rb * QROWS;                // first row of the row block
    const int my_row = wrow0 + col;                   // this lane's query row
    const int wrow_last = min(wrow0 + QROWS, N) - 1;  // < wrow0 if the block is empty

    // Query fragments of this wave's map (B operand of S^T = K . Q^T): the
    // lane holds 8 consecutive elements of its row per 16-element k-step.
    bf16x8 qf[C::KSTEPS];
    {
        const bool ok = my_row < N;
        const __bf16* qr = (map ? q2 : q1) + qoff + (int64_t)(ok ? my_row : 0) * ldq + half * 8;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s)
            qf[s] = __builtin_bit_cast(bf16x8, ok ? load16(qr + s * 16) : make_uint4(0, 0, 0, 0));
    }
    // Let the query loads land before the loop: otherwise the wait inserted
    // for their first use inside the loop also waits for the tile copies.
    __builtin_amdgcn_s_waitcnt(0);

    const float c = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)
    float mref = -INFINITY;   // reference maximum (raw score units)
    float lsum = 0.f;         // this lane's share of the normaliser
    f32x16 acc[C::VBLK];
#pragma unroll
    for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;

    const int kv_end = causal ? min(N, q0 + BM) : N;

    // ---- lane-constant LDS fragment offsets (stage-relative, sub-tile 0;
    // sub-tile 1 adds 32 rows, which leaves both swizzles unchanged) --------
    // K fragment of k-step st: row kappa(col), logical chunk 2*st + half.
    // The swizzle acts on chunk bits only, so its offset is kx ^ (32*st).
    const int krow = kappa(col);
    const int kx = (map ? C::K2_OFF : C::K1_OFF) + krow * C::KROWB + ((half ^ k_swz<D>(krow)) * 16);
    // V^T fragment through the transpose load: group g = lane/16 covers
    // channels 16*(g%2) .. +15 of a 32-channel block and keys 8*(g/2) .. +7 of
    // a 16-key step; lane j of the group points at key 4*r + j/4, channels
    // 4*(j%4) .. +3, for the two loads r = 0, 1.  The swizzle acts on chunk
    // bits below the channel-block bits, so block nb sits at vx ^ (64*nb).
    const int grp = lane >> 4, gl = lane & 15;
    const int vrow = (grp >> 1) * 8 + (gl >> 2);
    const int vx = C::V_OFF + vrow * C::VROWB +
                   (((2 * (grp & 1) + ((gl & 3) >> 1)) ^ v_swz<DV>(vrow)) * 16) + 8 * (gl & 1);

    // ---- global -> LDS copies of one 64-key tile -------------------------
    // Descriptors start at the tile's first key and end at the sequence end:
    // rows past N read as zeros (their scores are masked anyway).
    auto rsrc = [&](const __bf16* base, int64_t ld, int kb) {
        const int rows = max(0, min(N - kb, TK));
        return make_rsrc(base + (int64_t)kb * ld, rows * (int)ld * 2);
    };
    int coff[C::CPW];   // lane-constant source offsets of this wave's copies
#pragma unroll
    for (int j = 0; j < C::CPW; ++j) {
        if (map == 0) {
            const int row = (rb * C::KPW + j) * C::KRPI + lane / C::KC;
            coff[j] = row * (int)ldk * 2 + (((lane % C::KC) ^ k_swz<D>(row)) * 16);
        } else {
            const int row = (rb * C::VPW + j) * C::VRPI + lane / C::VC;
            coff[j] = row * (int)ldv * 2 + (((lane % C::VC) ^ v_swz<DV>(row)) * 16);
        }
    }
    auto issue_tile = [&](int T) {
        const int kb = T * TK;
        const unsigned st = __builtin_amdgcn_readfirstlane(lds_addr(smem) + (T & 1) * C::STAGE);
        if (map == 0) {
            const i32x4 r1 = rsrc(k1 + koff, ldk, kb);
            const i32x4 r2 = rsrc(k2 + koff, ldk, kb);
#pragma unroll
            for (int j = 0; j < C::KPW; ++j) {
                const unsigned dst = st + (rb * C::KPW + j) * 1024;
                copy16_to_lds(r1, dst + C::K1_OFF, coff[j]);
                copy16_to_lds(r2, dst + C::K2_OFF, coff[j]);
            }
        } else {
            const i32x4 rv = rsrc(v + voff, ldv, kb);
#pragma unroll
            for (int j = 0; j < C::VPW; ++j)
                copy16_to_lds(rv, st + C::V_OFF + (rb * C::VPW + j) * 1024, coff[j]);
        }
    };

    // One 32-key sub-tile of this wave's map: scores, online softmax, P.V.
    auto sub_tile = [&](const unsigned char* stg, int sub, int kb, bool masked) {
        const unsigned char* ks = stg + sub * BN * C::KROWB;
        const unsigned char* vs = stg + sub * BN * C::VROWB;
        // Matrix sections run at raised wave priority: when several waves of
        // a SIMD are ready, one feeding the matrix core issues first.
        __builtin_amdgcn_s_setprio(1);
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st) {
            const bf16x8 kf = __builtin_bit_cast(bf16x8, load16(ks + (kx ^ (32 * st))));
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s, 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        // Rare (diagonal / last tile), uniform: kept as a real branch.
        if (__builtin_expect(masked, 0)) {
            // Register r holds key kb + key_of_reg(r) + 8*half, visible iff
            // that offset is below lim.
            const int lim = causal ? min(N - kb, my_row - kb + 1) : N - kb;
            const int limh = lim - 8 * half;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (key_of_reg(r) >= limh) s[r] = -INFINITY;
        }
        float mx = max3(s[0], s[1], s[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) mx = max3(mx, s[r], s[r + 1]);
        mx = max3(mx, s[15], s[15]);
        // Row maximum: this lane's 16 keys, the partner lane's 16, and the
        // reference the accumulator was built on.
        const float mnew = max3(mref, mx, __shfl_xor(mx, 32));
        const bool grow = mnew > -INFINITY && (mref == -INFINITY || (mnew - mref) * c > TAU);
        if (__any(grow)) {
            const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((mref - mnew) * c);
            mref = mnew;
            lsum *= alpha;
#pragma unroll
            for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[nb][r] *= alpha;
        }
        const float mc = (mref == -INFINITY) ? 0.f : mref * c;
        bf16x8 pf[2];
        float ls = lsum;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const f32x2 pr = {__builtin_amdgcn_exp2f(fmaf(s[t2 * 8 + e], c, -mc)),
                                  __builtin_amdgcn_exp2f(fmaf(s[t2 * 8 + e + 1], c, -mc))};
                const bf16x2 pb = __builtin_convertvector(pr, bf16x2);
                // The normaliser sums the same bf16 probabilities the product uses.
                ls = __builtin_amdgcn_fdot2_f32_bf16(pb, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, ls, false);
                pf[t2][e] = pb[0];
                pf[t2][e + 1] = pb[1];
            }
        }
        lsum = ls;
        // O^T += V^T . P^T
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb) {
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const unsigned char* vp = vs + (vx ^ (64 * nb)) + t2 * 16 * C::VROWB;
                const bf16x4 lo = lds_read_tr(vp);
                const bf16x4 hi = lds_read_tr(vp + 4 * C::VROWB);
                const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t2], acc[nb], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    const int ntiles = __builtin_amdgcn_readfirstlane((kv_end + TK - 1) / TK);   // uniform
    if (ntiles > 0) issue_tile(0);
    for (int T = 0; T < ntiles; ++T) {
        // Tile T's copies (the only vector-memory operations in flight) have
        // landed for this wave; the barrier makes every wave's copies visible
        // and shows that every wave is done reading the stage copied into next.
        sync_stage();
        if (T + 1 < ntiles) issue_tile(T + 1);
        const unsigned char* stg = smem + (T & 1) * C::STAGE;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int kb = T * TK + sub * BN;
            // Skip sub-tiles past the keys this row block can see (uniform).
            if (wrow_last < wrow0 || kb >= kv_end || (causal && kb > wrow_last)) continue;
            // Only sub-tiles that straddle the diagonal or the sequence end need a mask.
            sub_tile(stg, sub, kb, (kb + BN > N) || (causal && kb + BN - 1 > wrow0));
        }
    }

    // ---- epilogue: map 2 hands over, lambda combine, optional RMS norm ----
    const float l = lsum + __shfl_xor(lsum, 32);
    // The stages are free once every wave passes this barrier (no copy is in
    // flight after the last tile).  They become the hand-over buffer, in the
    // accumulator's own lane order: 16 bytes per lane per 4 registers.
    sync_stage();
    float* xb = reinterpret_cast<float*>(smem) + rb * (QROWS * DV);
    if (map == 1) {
        const float w2 = lambda[h] / l;
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = acc[nb][g * 4 + e] * w2;
                *reinterpret_cast<f32x4*>(xb + ((nb * 4 + g) * WAVE + lane) * 4) = y;
            }
    }
    sync_stage();
    if (map == 1 || my_row >= N) return;
    const float w1 = 1.f / l;
    float ss = 0.f;
#pragma unroll
    for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 o2 = *reinterpret_cast<const f32x4*>(xb + ((nb * 4 + g) * WAVE + lane) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float y = acc[nb][g * 4 + e] * w1 - o2[e];
                acc[nb][g * 4 + e] = y;
                ss = fmaf(y, y, ss);
            }
        }
    float scale = 1.f;
    if (rmsnorm) {
        ss += __shfl_xor(ss, 32);
        scale = norm_scale / sqrtf(ss / (float)DV + eps);
    }
    float* orow = out + (tok0 + my_row) * DV;
    // Lane (col, half) holds channels nb*32 + g*8 + half*4 .. +3 in registers
    // 4g .. 4g+3 of block nb.
    auto store = [&](auto weight) {
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ch = nb * 32 + g * 8 + half * 4;
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = acc[nb][g * 4 + e] * scale * weight(ch + e);
                *reinterpret_cast<f32x4*>(orow + ch) = y;
            }
    };
    if (rmsnorm && norm_weight) store([&](int ch) { return norm_weight[ch]; });
    else store([](int) { return 1.f; });
}

template <int D, int DV, int OCC>
hipError_t launch_bf16(const PrefillArgs& a, hipStream_t stream) {
    using C = Cfg<D, DV>;
    const int row_tiles = (a.N + BM - 1) / BM;
    const int BH = a.B * a.H;
    const int64_t blocks = (int64_t)BH * row_tiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = (size_t)C::LDS;
    static bool attr_set = false;    // raise the dynamic-LDS limit once per process
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)prefill_bf16_kernel<D, DV, OCC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((prefill_bf16_kernel<D, DV, OCC>), dim3((unsigned)blocks), dim3(THREADS), lds,
                       stream, (const __bf16*)a.q1, (const __bf16*)a.q2, (const __bf16*)a.k1,
                       (const __bf16*)a.k2, (const __bf16*)a.v, a.ldq, a.ldk, a.ldv, BH, a.H, a.N,
                       a.causal, a.lambda, a.rmsnorm, a.eps, a.norm_scale, a.norm_weight, a.out,
                       row_tiles, a.hs);
    return hipGetLastError();
}

}  // namespace

bool prefill_bf16_supported(int d, int dv) {
    return prefill_pp_supported(d, dv) || (d == 128 && dv == 128);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    if (prefill_pp_supported(a.d, a.dv)) return launch_prefill_pp(a, stream);
    if (a.d == 128 && a.dv == 128) return launch_bf16<128, 128, 2>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
