// Fused differential-attention prefill on gfx950 matrix cores, ping-pong
// schedules (bf16 in, fp32 accumulate): both maps per wave for d <= 64, one
// map per wave (map-split) for d = 128.
//
// Per head (b,h) and query row i:
//     A1 = softmax(q1_i K1^T / sqrt d),   A2 = softmax(q2_i K2^T / sqrt d),
//     o_i = (A1 - lambda_h A2) V,   optional y_i = RMSNorm(o_i) * w * s
// (page "差分注意力" (aiknowledge.cn), part 一 "差分思路" and part 二 Step 2;
// per-head normalisation after the difference: "V1 到 V2 的 diff"), in one
// pass over a shared key/value stream (page "【架构革新】...", section 3: the
// two softmaxes share intermediates inside one fused kernel).
//
// Work split and schedule:
//  - A workgroup owns 256 query rows of one head, as 8 row blocks of 32, one
//    per wave.  Each wave runs both maps for its rows: two score tiles, two
//    running maxima and normalisers, two fp32 accumulators (the maps rescale
//    independently, so an exact single pass needs one per map).
//  - Each 32-key sub-tile j is two phases per wave: M(j) issues the matrix
//    products (P.V of sub-tile j-1 and the scores of sub-tile j, both maps,
//    as one pipeline over operand units), V(j) runs both online softmaxes of sub-tile
//    j on the vector ALU.  The waves form two groups that meet at one
//    workgroup barrier per interval: interval j holds group 0's M(j) and
//    V(j) and group 1's V(j-1) and M(j) (group 1 places its barrier between
//    its M and V phases, group 0 after its V phase), so while one group's
//    matrix products occupy a SIMD's matrix core, the other group's softmax
//    occupies its vector ALU.  Waves w and w+4 share a SIMD and take
//    adjacent row blocks 2w and 2w+1, so they have the same causal extent
//    and stay balanced.
//  - Keys and values stream through LDS in tiles of 64 keys, three stages
//    deep, copied by buffer loads that write LDS directly.  Tile t is read
//    by the M phases of steps 2t .. 2t+2 (intervals 2t .. 2t+2).  Every wave
//    copies the same number of 1 KB blocks of it, in one burst at the end of
//    its M phase of step 2t-3, into the stage that tile t-3 left in interval
//    2t-4, and waits for it at the end of its M phase of step 2t-1 with
//    exactly the copies of tile t+1, issued just before, still in flight
//    (copies complete in issue order); the barrier ending interval 2t-1
//    publishes the tile.  The softmax phase carries no copy work.
//  - Scores are formed transposed, S^T = K . Q^T (v_mfma_f32_32x32x16_bf16):
//    a lane holds 16 keys of ONE query, so each softmax row statistic is a
//    per-lane quantity plus one exchange with the lane 32 apart.  Keys enter
//    the A operand with bits 2 and 3 of the row index swapped, which makes
//    the score registers line up with the B operand of O^T += V^T . P^T: the
//    probabilities feed the next product straight from registers.  Values
//    stay token-major in LDS and the V^T operand comes from the gfx950
//    transpose load (ds_read_b64_tr_b16).  Rows are XOR-swizzled in 16-byte
//    chunks so fragment reads hit distinct banks.
//  - Rescaling is lazy: an accumulator is rescaled only when a row maximum
//    grows by more than 8 (base 2) over the reference it was built on, so
//    probabilities stay <= 2^8; the result is the same exact quantity.
//  - Causal: sub-tiles wholly above a row block are skipped (the wave still
//    takes part in every barrier); only those that straddle the diagonal or
//    the sequence end are masked.  Heavy query tiles are scheduled first, and
//    consecutive workgroups take different heads.
#include <atomic>

#include "kernels.h"
#include "bf16_tile.h"

namespace diffattn {
namespace {

using namespace tile;

constexpr int PP_WAVES = 8;                  // two groups of four
constexpr int PP_THREADS = WAVE * PP_WAVES;
constexpr int PP_BM = QROWS * PP_WAVES;      // 256 rows per workgroup
constexpr int PP_NSTAGE = 3;

// MAPS = 2: differential attention (both maps share the K/V stream).
// MAPS = 1: plain single-map attention with the same schedule, the building
// block of the unfused two-pass comparison path.
template <int D, int DV, int MAPS>
struct PPCfg {
    static constexpr int KC = D / 8;                  // 16-byte chunks per key half-row
    static constexpr int VC = DV / 8;                 // 16-byte chunks per value row
    static constexpr int KROWB = D * 2;               // bytes per key half-row (K1 or K2)
    static constexpr int VROWB = DV * 2;              // bytes per value row
    static constexpr int K2_OFF = TK * KROWB;         // stage layout: K1 | K2 | V
    static constexpr int V_OFF = MAPS * TK * KROWB;
    static constexpr int STAGE = MAPS * TK * KROWB + TK * VROWB;
    static constexpr int KBLK = TK * KROWB / 1024;    // 1 KB copy blocks per key half
    static constexpr int NCOPY = STAGE / 1024;        // copy blocks per tile
    static constexpr int CPW = NCOPY / PP_WAVES;      // per wave
    static constexpr int KRPI = 1024 / KROWB;         // key rows per copy block
    static constexpr int VRPI = 1024 / VROWB;         // value rows per copy block
    static constexpr int KSTEPS = D / 16;             // MFMA k-steps of one score map
    static constexpr int VBLK = DV / 32;              // 32-channel blocks of O^T
    static constexpr int LDS = PP_NSTAGE * STAGE;
    static_assert(NCOPY % PP_WAVES == 0, "every wave must copy the same number of blocks");
    static_assert(LDS <= 160 * 1024, "stages exceed LDS");
};

// Workgroup barrier; the scheduler may not move work across it.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Wait until at most CNT of this wave's copies are in flight.
template <int CNT>
__device__ __forceinline__ void wait_copies() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CNT) : "memory");
}

// A constant the compiler must rematerialise (one scalar move) at each use
// instead of hoisting a per-lane copy of every derived address out of the
// loop: the loop runs at the vector-register limit.
__device__ __forceinline__ int fresh(int c) {
    asm volatile("" : "+s"(c));
    return c;
}

// Units of the pipelined M phase: 0 .. VB-1 are V^T blocks (4 LDS reads,
// 2*MAPS products), VB .. NU-1 are key k-steps (MAPS reads, MAPS products).
// unit_at(p) is the unit at pipeline position p.  V^T units 0 and 1 come first
// (they are read at the end of the previous M phase); with IL the key
// k-steps then alternate with the remaining V^T units, so that every load has
// at least one V^T unit's products between its issue and its use.
__host__ __device__ constexpr int unit_at(int p, int VB, int NU, bool IL) {
    if (!IL || p < 2) return p;
    int v = 2, k = 0;
    for (int q = 2; q < NU; ++q) {
        const bool take_k = (k < NU - VB) && ((q % 2 == 0) || v >= VB);
        if (q == p) return take_k ? VB + k : v;
        if (take_k) ++k;
        else ++v;
    }
    return -1;
}

// Scheduling groups of the pipelined M phase: for each position p the
// products of its unit, then the loads of the unit at position p+PD.
template <int P, int NU, int VB, int MAPS, bool IL, int PD>
struct PipeGroupsN {
    static __device__ __forceinline__ void run() {
        __builtin_amdgcn_sched_group_barrier(0x008, unit_at(P, VB, NU, IL) < VB ? 2 * MAPS : MAPS, 0);
        if constexpr (P + PD < NU)
            __builtin_amdgcn_sched_group_barrier(0x100, unit_at(P + PD, VB, NU, IL) < VB ? 4 : MAPS, 0);
        if constexpr (P + 1 < NU) PipeGroupsN<P + 1, NU, VB, MAPS, IL, PD>::run();
    }
};

template <int D, int DV, int MAPS>
__global__ void __launch_bounds__(PP_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_pp_kernel(const __bf16* __restrict__ q1, const __bf16* __restrict__ q2,
                  const __bf16* __restrict__ k1, const __bf16* __restrict__ k2,
                  const __bf16* __restrict__ v, int64_t ldq, int64_t ldk, int64_t ldv,
                  int BH, int H, int N, int causal, const float* __restrict__ lambda,
                  int rmsnorm, float eps, float norm_scale,
                  const float* __restrict__ norm_weight, float* __restrict__ out,
                  int row_tiles, HeadStrides hs) {
    using C = PPCfg<D, DV, MAPS>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave-uniform values live in scalar registers: every phase decision is a
    // scalar branch.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;                 // 0 leads, 1 trails by one phase
    const int rb = 2 * (wave & 3) + grp;       // row block
    const int col = lane & 31;                 // query column inside the row block
    const int half = lane >> 5;                // which 8-element half of a 16-element k-step

    // Consecutive workgroups take consecutive heads (so each XCD sees a fixed
    // subset of heads); within a head the heaviest causal tiles come first.
    const int bh = blockIdx.x % BH;
    const int tile = row_tiles - 1 - (int)(blockIdx.x / BH);
    const int h = bh % H;
    const int q0 = tile * PP_BM;
    const int64_t tok0 = (int64_t)bh * N;                 // output rows
    const int b = bh / H;
    const int64_t qoff = b * hs.qb + h * hs.qh;
    const int64_t koff = b * hs.kb + (h / hs.kv_group) * hs.kh;
    const int64_t voff = b * hs.vb + (h / hs.kv_group) * hs.vh;

    const int wrow0 = q0 + rb * QROWS;                // first row of the row block
    const int my_row = wrow0 + col;                   // this lane's query row
    const int wrow_last = min(wrow0 + QROWS, N) - 1;  // < wrow0 if the block is empty

    const int kv_end = causal ? min(N, q0 + PP_BM) : N;
    const int nsub = __builtin_amdgcn_readfirstlane((kv_end + BN - 1) / BN);
    const int ntile = __builtin_amdgcn_readfirstlane((kv_end + TK - 1) / TK);
    // This row block sees sub-tiles 0 .. jmax-1.
    const int jmax = __builtin_amdgcn_readfirstlane(
        wrow_last < wrow0 ? 0 : (causal ? min(nsub, wrow_last / BN + 1) : nsub));
    // Sub-tiles j >= jmask need masking: they reach past the sequence end
    // (j*BN + BN > N) or, causally, past the row block's first row
    // (j*BN + BN - 1 > wrow0).
    const int jmask = __builtin_amdgcn_readfirstlane(
        min(N >= BN ? (N - BN) / BN + 1 : 0,
            causal ? (wrow0 - BN + 1 < 0 ? 0 : (wrow0 - BN + 1) / BN + 1) : (1 << 30)));

    // Query fragments of both maps (B operand of S^T = K . Q^T): the lane
    // holds 8 consecutive elements of its row per 16-element k-step.
    bf16x8 qf[MAPS][C::KSTEPS];
    {
        const bool ok = my_row < N;
        const int64_t off = qoff + (int64_t)(ok ? my_row : 0) * ldq + half * 8;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            qf[0][s] = __builtin_bit_cast(bf16x8, ok ? load16(q1 + off + s * 16) : make_uint4(0, 0, 0, 0));
            if constexpr (MAPS == 2)
                qf[1][s] = __builtin_bit_cast(bf16x8, ok ? load16(q2 + off + s * 16) : make_uint4(0, 0, 0, 0));
        }
    }
    // The query loads land before any copy is issued, so the copy waits
    // below count copies only.
    __builtin_amdgcn_s_waitcnt(0);

    const float c = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)
    float mref[MAPS];   // reference maxima (raw score units; -inf until a row
                        // has seen a visible key)
    // A new maximum above mref + TAU/c triggers a rescale.
    const float tau_raw = TAU / c;
    float lsum[MAPS];   // this lane's share of the normalisers
#pragma unroll
    for (int m = 0; m < MAPS; ++m) {
        mref[m] = -INFINITY;
        lsum[m] = 0.f;
    }
    f32x16 acc[MAPS][C::VBLK];
#pragma unroll
    for (int m = 0; m < MAPS; ++m)
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][nb][r] = 0.f;
    f32x16 s[MAPS];       // scores of the current sub-tile
    bf16x8 pf[MAPS][2];   // probabilities of the previous sub-tile (B operand)
    bf16x8 vnext[2][2];   // V^T units 0 and 1 of the next M phase, read ahead
#pragma unroll
    for (int m = 0; m < MAPS; ++m) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[m][r] = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[m][t][e] = (__bf16)0.f;
    }

    // ---- lane-constant LDS fragment offsets (stage-relative, sub-tile 0;
    // sub-tile 1 adds 32 rows, which leaves both swizzles unchanged) --------
    // K fragment of k-step st: row kappa(col), logical chunk 2*st + half; the
    // swizzle acts on chunk bits only, so its offset is kx ^ (32*st).
    const int krow = kappa(col);
    const int kx = krow * C::KROWB + ((half ^ k_swz<D>(krow)) * 16);
    // V^T fragment through the transpose load: group g = lane/16 covers
    // channels 16*(g%2) .. +15 of a 32-channel block and keys 8*(g/2) .. +7 of
    // a 16-key step; lane j of the group points at key 4*r + j/4, channels
    // 4*(j%4) .. +3, for the two loads r = 0, 1.  The swizzle acts on chunk
    // bits below the channel-block bits, so block nb sits at vx ^ (64*nb).
    const int lg = lane >> 4, gl = lane & 15;
    const int vrow = (lg >> 1) * 8 + (gl >> 2);
    const int vx = C::V_OFF + vrow * C::VROWB +
                   (((2 * (lg & 1) + ((gl & 3) >> 1)) ^ v_swz<DV>(vrow)) * 16) + 8 * (gl & 1);

    // ---- global -> LDS copies ----------------------------------------------
    // Copy block id (0 .. NCOPY-1) of a tile moves 1 KB: ids below KBLK are
    // K1 rows, then K2 rows, then V rows, in stage order, so block id lands at
    // stage + 1024*id.  Wave w copies ids w, w+8, ...  Descriptors start at the
    // tile's first key and end at the sequence end: rows past N read as zeros.
    int coff[C::CPW];
#pragma unroll
    for (int j = 0; j < C::CPW; ++j) {
        const int id = wave + PP_WAVES * j;
        if (id < MAPS * C::KBLK) {
            const int row = (id % C::KBLK) * C::KRPI + lane / C::KC;
            coff[j] = row * (int)ldk * 2 + (((lane % C::KC) ^ k_swz<D>(row)) * 16);
        } else {
            const int row = (id - MAPS * C::KBLK) * C::VRPI + lane / C::VC;
            coff[j] = row * (int)ldv * 2 + (((lane % C::VC) ^ v_swz<DV>(row)) * 16);
        }
    }
    // Copy block b of this wave has a fixed source: its region's base for
    // this head, the byte stride from one tile to the next, and the row pitch.
    unsigned long long cbase[C::CPW];
    unsigned cstride[C::CPW];
    int cpitch[C::CPW];
#pragma unroll
    for (int b = 0; b < C::CPW; ++b) {
        const int id = wave + PP_WAVES * b;
        const __bf16* src = id < C::KBLK ? k1 : (id < MAPS * C::KBLK ? k2 : v);
        const int64_t ld = id < MAPS * C::KBLK ? ldk : ldv;
        // Uniform values: kept in scalar registers.
        const unsigned long long a64 = (unsigned long long)(src + (id < MAPS * C::KBLK ? koff : voff));
        const unsigned alo = __builtin_amdgcn_readfirstlane((unsigned)(a64 & 0xffffffffu));
        const unsigned ahi = __builtin_amdgcn_readfirstlane((unsigned)(a64 >> 32));
        cbase[b] = ((unsigned long long)ahi << 32) | alo;
        cstride[b] = __builtin_amdgcn_readfirstlane((unsigned)(TK * ld * 2));
        cpitch[b] = __builtin_amdgcn_readfirstlane((int)(ld * 2));
    }
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
    // All CPW blocks of tile t.  Rows past the sequence end read as zeros
    // (their scores are masked).
    auto issue_tile = [&](int t) {
        const int rows = min(N - t * TK, TK);
        const unsigned st = lds0 + (unsigned)((t % PP_NSTAGE) * C::STAGE);
#pragma unroll
        for (int bb = 0; bb < C::CPW; ++bb) {
            const i32x4 r = make_rsrc((const void*)(cbase[bb] + (unsigned long long)t * cstride[bb]),
                                      rows * cpitch[bb]);
            copy16_to_lds(r, st + (wave + PP_WAVES * bb) * 1024, coff[bb]);
        }
    };
    static_assert(C::CPW >= 1 && C::CPW <= 15, "copies per wave must fit the vmcnt field");


    // M(j), for j <= jmax: P.V of sub-tile j-1 (both maps share each V^T
    // fragment) and the scores of sub-tile j for both maps, as one software
    // pipeline over units in unit_at order (V^T blocks 0 and 1, then the key
    // k-steps alternating with the other V^T blocks) with the loads two
    // positions ahead.  V^T units 0 and 1 arrive in registers from the end of
    // M(j-1) (from the prologue for M(0)), so the phase starts on products;
    // at its end M(j) reads them for M(j+1).  At j = 0 the probabilities are
    // all zero and the values of sub-tile 0 stand in, adding exact zeros; at
    // j = jmax the scores come from whatever the stage holds and are never
    // used.  One code path for every step keeps the accumulators in place.
    // The derived LDS offsets are rematerialised per use (fresh) rather than
    // kept per lane.
    auto read_v = [&](const unsigned char* vs, int u, bf16x8 (&dst)[2]) {
        // One lane address per unit; the four reads differ by constants.
        const unsigned char* vu = vs + (u ? (vx ^ fresh(64 * u)) : vx);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            const unsigned char* vp = vu + t2 * 16 * C::VROWB;
            const bf16x4 lo = lds_read_tr(vp);
            const bf16x4 hi = lds_read_tr(vp + 4 * C::VROWB);
            dst[t2] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    // so_j, so_v: byte offsets of the stages holding sub-tiles j and j - 1.
    auto m_phase = [&](int j, int so_j, int so_v) {
        if (j > jmax) return;
        const int jv = j > 0 ? j - 1 : 0;
        const unsigned char* vs = smem + so_v + (jv & 1) * BN * C::VROWB;
        const unsigned char* ks = smem + so_j + (j & 1) * BN * C::KROWB;
        constexpr int NU = C::VBLK + C::KSTEPS;
        bf16x8 vf[C::VBLK][2];
        bf16x8 kf[MAPS][C::KSTEPS];
        auto load_unit = [&](int u) {
            if (u < C::VBLK) {
                read_v(vs, u, vf[u < C::VBLK ? u : 0]);
            } else {
                const int st = u - C::VBLK;
                // One lane address for both maps' reads of this k-step.
                const unsigned char* ku = ks + (st ? (kx ^ fresh(32 * st)) : kx);
#pragma unroll
                for (int m = 0; m < MAPS; ++m)
                    kf[m][st] = __builtin_bit_cast(bf16x8, load16(ku + m * C::K2_OFF));
            }
        };
#pragma unroll
        for (int m = 0; m < MAPS; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[m][r] = 0.f;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            vf[0][t2] = vnext[0][t2];
            vf[1][t2] = vnext[1][t2];
        }
#pragma unroll
        for (int p = 0; p < NU; ++p) {
            const int u = unit_at(p, C::VBLK, NU, true);
            if (u < C::VBLK) {
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                    for (int m = 0; m < MAPS; ++m)
                        acc[m][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u][t2], pf[m][t2], acc[m][u], 0, 0, 0);
            } else {
                const int st = u - C::VBLK;
#pragma unroll
                for (int m = 0; m < MAPS; ++m)
                    s[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[m][st], qf[m][st], s[m], 0, 0, 0);
            }
            if (p + 2 < NU) load_unit(unit_at(p + 2, C::VBLK, NU, true));
        }
        // Units 0 and 1 of M(j+1): the values of sub-tile j, visible now (its
        // keys were read above) and not overwritten before M(j+1).
        const unsigned char* vsn = smem + so_j + (j & 1) * BN * C::VROWB;
        read_v(vsn, 0, vnext[0]);
        read_v(vsn, 1, vnext[1]);
        PipeGroupsN<0, NU, C::VBLK, MAPS, true, 2>::run();
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    };

    // V(j): both online softmaxes of sub-tile j -> probabilities for M(j+1).
    auto v_phase = [&](int j) {
        if (j >= jmax) return;
        // Rare (diagonal / last sub-tile), uniform: a real branch.
        if (__builtin_expect(j >= jmask, 0)) {
            const int kb = j * BN;
            // Register r holds key kb + key_of_reg(r) + 8*half, visible iff
            // that offset is below lim.
            const int lim = causal ? min(N - kb, my_row - kb + 1) : N - kb;
            const int limh = lim - 8 * half;
#pragma unroll
            for (int m = 0; m < MAPS; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (key_of_reg(r) >= limh) s[m][r] = -INFINITY;
        }
        // Row maxima of both maps: both lanes of a row (16 keys each) and the
        // reference each accumulator was built on.
        float mnew[MAPS];
        bool grow[MAPS];
        bool any_grow = false;
#pragma unroll
        for (int m = 0; m < MAPS; ++m) {
            // A tree of three-way maxima: short dependency chains.
            const float a0 = max3(s[m][0], s[m][1], s[m][2]);
            const float a1 = max3(s[m][3], s[m][4], s[m][5]);
            const float a2 = max3(s[m][6], s[m][7], s[m][8]);
            const float a3 = max3(s[m][9], s[m][10], s[m][11]);
            const float a4 = max3(s[m][12], s[m][13], s[m][14]);
            const float mx = max3(max3(a0, a1, a2), a3, max3(a4, s[m][15], s[m][15]));
            const f32x2 hm = halves(mx);
            mnew[m] = max3(mref[m], hm[0], hm[1]);
            grow[m] = mnew[m] > mref[m] + tau_raw;
            any_grow = any_grow | grow[m];
        }
        // Rare: one uniform branch for both maps keeps the common path in one block.
        if (__any(any_grow)) {
#pragma unroll
            for (int m = 0; m < MAPS; ++m) {
                if (__any(grow[m])) {
                    // Lanes that do not grow keep their reference (alpha = 1);
                    // a first visible key gives alpha = exp2(-inf) = 0 on an
                    // all-zero accumulator.
                    const float alpha = grow[m] ? __builtin_amdgcn_exp2f((mref[m] - mnew[m]) * c) : 1.f;
                    mref[m] = grow[m] ? mnew[m] : mref[m];
                    lsum[m] *= alpha;
#pragma unroll
                    for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[m][nb][r] *= alpha;
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MAPS; ++m) {
            const float mc = (mref[m] == -INFINITY) ? 0.f : mref[m] * c;
            float ls = lsum[m];
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const f32x2 pr = {__builtin_amdgcn_exp2f(fmaf(s[m][t2 * 8 + e], c, -mc)),
                                      __builtin_amdgcn_exp2f(fmaf(s[m][t2 * 8 + e + 1], c, -mc))};
                    const bf16x2 pb = __builtin_convertvector(pr, bf16x2);
                    // The normaliser sums the same bf16 probabilities the product uses.
                    ls = __builtin_amdgcn_fdot2_f32_bf16(pb, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, ls, false);
                    pf[m][t2][e] = pb[0];
                    pf[m][t2][e + 1] = pb[1];
                }
            }
            lsum[m] = ls;
        }
    };

    // ---- the schedule ------------------------------------------------------
    // Interval j ends with the workgroup's j-th loop barrier and holds both
    // groups' M(j).  Tile t (sub-tiles 2t, 2t+1) is read by M(2t) .. M(2t+2),
    // intervals 2t .. 2t+2.  M(2t-3) copies it into the stage tile t-3 left
    // in interval 2t-4; M(2t-1) waits for it, and the barrier ending interval
    // 2t-1 publishes it.  (tests/test_copy_schedule.py models both groups over
    // every key extent up to 2560 and at 4k/32k/64k: each copy issued once
    // into a free stage, complete and published before its first read, none
    // in flight at the end.)
    issue_tile(0);
    if (ntile > 1) {
        issue_tile(1);
        wait_copies<C::CPW>();
    } else {
        wait_copies<0>();
    }
    phase_barrier();            // tile 0 visible
    read_v(smem, 0, vnext[0]);  // M(0): values of sub-tile 0 (times zero probabilities)
    read_v(smem, 1, vnext[1]);
    // The wave in its matrix phase takes issue priority over the one in its
    // softmax phase on the same SIMD, so the matrix core is fed first.  The
    // stage ring advances every second sub-tile; its offsets are carried
    // through the loop rather than recomputed modulo the stage count.
    int so_j = 0, so_v = 0;
    auto m_and_copies = [&](int j) {
        __builtin_amdgcn_s_setprio(1);
        m_phase(j, so_j, so_v);
        if (j & 1) {
            // Copy tile (j+3)/2, then wait for tile (j+1)/2 with only the
            // copies just issued still in flight.
            const int ti = (j + 3) >> 1, tw = (j + 1) >> 1;
            if (ti < ntile) issue_tile(ti);
            if (tw + 1 < ntile) wait_copies<C::CPW>();
            else wait_copies<0>();
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // Both groups run M(j) then V(j); group 0 ends interval j after V(j),
    // group 1 after M(j), so interval j holds group 0's M(j), V(j) and group
    // 1's V(j-1), M(j).
    for (int j = 0; j <= nsub; ++j) {
        m_and_copies(j);
        if (grp) {
            phase_barrier();
            so_v = so_j;
            if (j & 1) so_j = (so_j + C::STAGE == PP_NSTAGE * C::STAGE) ? 0 : so_j + C::STAGE;
        }
        v_phase(j);
        if (!grp) {
            phase_barrier();
            so_v = so_j;
            if (j & 1) so_j = (so_j + C::STAGE == PP_NSTAGE * C::STAGE) ? 0 : so_j + C::STAGE;
        }
    }
    __builtin_amdgcn_s_setprio(0);

    // ---- epilogue: combine the maps with lambda, optional RMS norm ----------
    if (my_row >= N) return;
    const f32x2 h1 = halves(lsum[0]);
    const float w1 = 1.f / (h1[0] + h1[1]);
    float ss = 0.f;
    if constexpr (MAPS == 2) {
        const f32x2 h2 = halves(lsum[1]);
        const float w2 = lambda[h] / (h2[0] + h2[1]);
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float y = acc[0][nb][r] * w1 - acc[1][nb][r] * w2;
                acc[0][nb][r] = y;
                ss = fmaf(y, y, ss);
            }
    } else {
#pragma unroll
        for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[0][nb][r] *= w1;
    }
    float scale = 1.f;
    if (MAPS == 2 && rmsnorm) {
        const f32x2 hs = halves(ss);
        scale = norm_scale / sqrtf((hs[0] + hs[1]) / (float)DV + eps);
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
                for (int e = 0; e < 4; ++e) y[e] = acc[0][nb][g * 4 + e] * scale * weight(ch + e);
                *reinterpret_cast<f32x4*>(orow + ch) = y;
            }
    };
    if (MAPS == 2 && rmsnorm && norm_weight) store([&](int ch) { return norm_weight[ch]; });
    else store([](int) { return 1.f; });
}

// Raises a kernel's dynamic-LDS limit on the current device.  The attribute
// belongs to the device, so it is set once on each device; `done` only caches
// that (setting it again is harmless, so concurrent first calls are safe).
constexpr int MAX_DEVICES = 64;
template <typename K>
hipError_t ensure_lds_limit(K kernel, int bytes, std::atomic<bool>* done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < MAX_DEVICES;
    if (cached && done[dev].load(std::memory_order_acquire)) return hipSuccess;
    e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && cached) done[dev].store(true, std::memory_order_release);
    return e;
}

template <int D, int DV, int MAPS>
hipError_t launch_pp(const PrefillArgs& a, hipStream_t stream) {
    using C = PPCfg<D, DV, MAPS>;
    const int row_tiles = (a.N + PP_BM - 1) / PP_BM;
    const int64_t blocks = (int64_t)a.B * a.H * row_tiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const int BH = a.B * a.H;   // at most `blocks`, so it fits
    static std::atomic<bool> lds_ok[MAX_DEVICES];
    const hipError_t e = ensure_lds_limit(prefill_pp_kernel<D, DV, MAPS>, C::LDS, lds_ok);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_pp_kernel<D, DV, MAPS>), dim3((unsigned)blocks), dim3(PP_THREADS),
                       (size_t)C::LDS, stream, (const __bf16*)a.q1, (const __bf16*)a.q2,
                       (const __bf16*)a.k1, (const __bf16*)a.k2, (const __bf16*)a.v, a.ldq, a.ldk,
                       a.ldv, BH, a.H, a.N, a.causal, a.lambda, a.rmsnorm, a.eps, a.norm_scale,
                       a.norm_weight, a.out, row_tiles, a.hs);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Map-split ping-pong (d = 128): 8 waves own 128 rows.  Wave w runs map
// w >> 2 for row block w & 3; the map-2 waves form the second group (its
// barrier sits between its matrix and softmax phases), so each SIMD holds the
// two maps of one row block, one in its matrix phase while the other is in
// its softmax phase.  A wave keeps one
// map's query fragments and accumulator (d = 128 does not fit both).
constexpr int PS_WAVES = 8;
constexpr int PS_THREADS = WAVE * PS_WAVES;
constexpr int PS_BM = QROWS * 4;
constexpr int PS_PD = 4;   // M-phase read-ahead distance, in pipeline units

// SK: both maps read one key tensor (the V2 layout, where the two query heads
// of a pair share their K/V head): the stage holds it once and both waves of
// a row block read the same key rows.
template <int D, int DV, bool SK>
struct PSCfg {
    static constexpr int KC = D / 8;
    static constexpr int VC = DV / 8;
    static constexpr int KROWB = D * 2;
    static constexpr int VROWB = DV * 2;
    static constexpr int NK = SK ? 1 : 2;             // key regions per stage
    static constexpr int K2_OFF = SK ? 0 : TK * KROWB;
    static constexpr int V_OFF = NK * TK * KROWB;
    static constexpr int STAGE = NK * TK * KROWB + TK * VROWB;
    static constexpr int KBLK = TK * KROWB / 1024;
    static constexpr int NCOPY = STAGE / 1024;
    static constexpr int CPW = NCOPY / PS_WAVES;
    static constexpr int KRPI = 1024 / KROWB;
    static constexpr int VRPI = 1024 / VROWB;
    static constexpr int KSTEPS = D / 16;
    static constexpr int VBLK = DV / 32;
    static constexpr int XBYTES = 4 * QROWS * DV * 4;   // map-2 hand-over, 4 row blocks
    static constexpr int LDS = (PP_NSTAGE * STAGE > XBYTES) ? PP_NSTAGE * STAGE : XBYTES;
    static_assert(NCOPY % PS_WAVES == 0 && CPW >= 1, "copy schedule");
    static_assert(LDS <= 160 * 1024, "LDS");
};

template <int D, int DV, bool SK>
__global__ void __launch_bounds__(PS_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_ps_kernel(const __bf16* __restrict__ q1, const __bf16* __restrict__ q2,
                   const __bf16* __restrict__ k1, const __bf16* __restrict__ k2,
                   const __bf16* __restrict__ v, int64_t ldq, int64_t ldk, int64_t ldv,
                   int BH, int H, int N, int causal, const float* __restrict__ lambda,
                   int rmsnorm, float eps, float norm_scale,
                   const float* __restrict__ norm_weight, float* __restrict__ out,
                   int row_tiles, HeadStrides hs) {
    using C = PSCfg<D, DV, SK>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int map = grp;
    const int rb = wave & 3;
    const int col = lane & 31;
    const int half = lane >> 5;

    const int bh = blockIdx.x % BH;
    const int tile = row_tiles - 1 - (int)(blockIdx.x / BH);
    const int h = bh % H;
    const int q0 = tile * PS_BM;
    const int64_t tok0 = (int64_t)bh * N;
    const int b = bh / H;
    const int64_t qoff = b * hs.qb + h * hs.qh;
    const int64_t koff = b * hs.kb + (h / hs.kv_group) * hs.kh;
    const int64_t voff = b * hs.vb + (h / hs.kv_group) * hs.vh;

    const int wrow0 = q0 + rb * QROWS;
    const int my_row = wrow0 + col;
    const int wrow_last = min(wrow0 + QROWS, N) - 1;
    const int kv_end = causal ? min(N, q0 + PS_BM) : N;
    const int nsub = __builtin_amdgcn_readfirstlane((kv_end + BN - 1) / BN);
    const int ntile = __builtin_amdgcn_readfirstlane((kv_end + TK - 1) / TK);
    const int jmax = __builtin_amdgcn_readfirstlane(
        wrow_last < wrow0 ? 0 : (causal ? min(nsub, wrow_last / BN + 1) : nsub));

    bf16x8 qf[C::KSTEPS];
    {
        const bool ok = my_row < N;
        const int64_t off = qoff + (int64_t)(ok ? my_row : 0) * ldq + half * 8;
        const __bf16* qs = map ? q2 : q1;
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st)
            qf[st] = __builtin_bit_cast(bf16x8, ok ? load16(qs + off + st * 16) : make_uint4(0, 0, 0, 0));
    }
    __builtin_amdgcn_s_waitcnt(0);

    const float c = 1.4426950408889634f / sqrtf((float)D);
    const float tau_raw = TAU / c;
    float mref = -INFINITY, lsum = 0.f;
    f32x16 acc[C::VBLK];
#pragma unroll
    for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
    f32x16 s;
    bf16x8 pf[2];
    // The M phase's loads run PS_PD units ahead; its first PS_PD units (V^T
    // blocks) are read at the end of the previous M phase.
    static_assert(PS_PD >= 1 && PS_PD <= C::VBLK, "read-ahead units must be V^T blocks");
    bf16x8 vnext[PS_PD][2];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[t][e] = (__bf16)0.f;

    const int krow = kappa(col);
    const int kx = map * C::K2_OFF + krow * C::KROWB + ((half ^ k_swz<D>(krow)) * 16);
    const int lg = lane >> 4, gl = lane & 15;
    const int vrow = (lg >> 1) * 8 + (gl >> 2);
    const int vx = C::V_OFF + vrow * C::VROWB +
                   (((2 * (lg & 1) + ((gl & 3) >> 1)) ^ v_swz<DV>(vrow)) * 16) + 8 * (gl & 1);

    int coff[C::CPW];
    unsigned long long cbase[C::CPW];
    unsigned cstride[C::CPW];
    int cpitch[C::CPW];
#pragma unroll
    // Copy blocks as in the d <= 64 kernel: block id of a tile moves 1 KB
    // (K1 rows, then K2 rows, then V rows), and wave w copies ids w, w+8, ...
    for (int bb = 0; bb < C::CPW; ++bb) {
        const int id = wave + PS_WAVES * bb;
        if (id < C::NK * C::KBLK) {
            const int row = (id % C::KBLK) * C::KRPI + lane / C::KC;
            coff[bb] = row * (int)ldk * 2 + (((lane % C::KC) ^ k_swz<D>(row)) * 16);
        } else {
            const int row = (id - C::NK * C::KBLK) * C::VRPI + lane / C::VC;
            coff[bb] = row * (int)ldv * 2 + (((lane % C::VC) ^ v_swz<DV>(row)) * 16);
        }
        const __bf16* src = id < C::KBLK ? k1 : (id < C::NK * C::KBLK ? k2 : v);
        const int64_t ld = id < C::NK * C::KBLK ? ldk : ldv;
        const unsigned long long a64 = (unsigned long long)(src + (id < C::NK * C::KBLK ? koff : voff));
        const unsigned alo = __builtin_amdgcn_readfirstlane((unsigned)(a64 & 0xffffffffu));
        const unsigned ahi = __builtin_amdgcn_readfirstlane((unsigned)(a64 >> 32));
        cbase[bb] = ((unsigned long long)ahi << 32) | alo;
        cstride[bb] = __builtin_amdgcn_readfirstlane((unsigned)(TK * ld * 2));
        cpitch[bb] = __builtin_amdgcn_readfirstlane((int)(ld * 2));
    }
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
    auto issue_tile = [&](int t) {
        const int rows = min(N - t * TK, TK);
        const unsigned st = lds0 + (unsigned)((t % PP_NSTAGE) * C::STAGE);
#pragma unroll
        for (int bb = 0; bb < C::CPW; ++bb) {
            const i32x4 r = make_rsrc((const void*)(cbase[bb] + (unsigned long long)t * cstride[bb]),
                                      rows * cpitch[bb]);
            copy16_to_lds(r, st + (wave + PS_WAVES * bb) * 1024, coff[bb]);
        }
    };

    // M(j), j <= jmax: this map's P.V of sub-tile j-1 (4 V^T blocks) and its
    // scores of sub-tile j (8 key k-steps), one pipeline with the loads PS_PD
    // units ahead; at j = 0 the probabilities are zero, at j = jmax the scores
    // are dropped (as in the d <= 64 kernel).
    auto read_v = [&](const unsigned char* vs, int u, bf16x8 (&dst)[2]) {
        const unsigned char* vu = vs + (u ? (vx ^ fresh(64 * u)) : vx);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            const unsigned char* vp = vu + t2 * 16 * C::VROWB;
            const bf16x4 lo = lds_read_tr(vp);
            const bf16x4 hi = lds_read_tr(vp + 4 * C::VROWB);
            dst[t2] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    // so_j, so_v: byte offsets of the stages holding sub-tiles j and j - 1.
    auto m_phase = [&](int j, int so_j, int so_v) {
        if (j > jmax) return;
        const int jv = j > 0 ? j - 1 : 0;
        const unsigned char* vs = smem + so_v + (jv & 1) * BN * C::VROWB;
        const unsigned char* ks = smem + so_j + (j & 1) * BN * C::KROWB;
        constexpr int NU = C::VBLK + C::KSTEPS;
        bf16x8 vf[C::VBLK][2];
        bf16x8 kf[C::KSTEPS];
        auto load_unit = [&](int u) {
            if (u < C::VBLK) {
                read_v(vs, u, vf[u < C::VBLK ? u : 0]);
            } else {
                const int st = u - C::VBLK;
                kf[st] = __builtin_bit_cast(bf16x8, load16(ks + (st ? (kx ^ fresh(32 * st)) : kx)));
            }
        };
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int u = 0; u < PS_PD; ++u)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) vf[u][t2] = vnext[u][t2];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            if (u < C::VBLK) {
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2)
                    acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u][t2], pf[t2], acc[u], 0, 0, 0);
            } else {
                const int st = u - C::VBLK;
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s, 0, 0, 0);
            }
            if (u + PS_PD < NU) load_unit(u + PS_PD);
        }
        // The first units of M(j+1): the values of sub-tile j.
        const unsigned char* vsn = smem + so_j + (j & 1) * BN * C::VROWB;
#pragma unroll
        for (int u = 0; u < PS_PD; ++u) read_v(vsn, u, vnext[u]);
        PipeGroupsN<0, NU, C::VBLK, 1, false, PS_PD>::run();
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * PS_PD, 0);
    };

    // V(j): this map's online softmax of sub-tile j (mask, row maximum, lazy
    // rescale, probabilities for M(j+1)).
    auto v_phase = [&](int j) {
        if (j >= jmax) return;
        const int kb = fresh(j * BN);
        if (__builtin_expect((kb + BN > N) || (causal && kb + BN - 1 > wrow0), 0)) {
            const int lim = causal ? min(N - kb, my_row - kb + 1) : N - kb;
            const int limh = lim - 8 * half;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (key_of_reg(r) >= limh) s[r] = -INFINITY;
        }
        const float a0 = max3(s[0], s[1], s[2]);
        const float a1 = max3(s[3], s[4], s[5]);
        const float a2 = max3(s[6], s[7], s[8]);
        const float a3 = max3(s[9], s[10], s[11]);
        const float a4 = max3(s[12], s[13], s[14]);
        const float mx = max3(max3(a0, a1, a2), a3, max3(a4, s[15], s[15]));
        const f32x2 hm = halves(mx);
        const float mnew = max3(mref, hm[0], hm[1]);
        const bool grow = mnew > mref + tau_raw;
        if (__any(grow)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f((mref - mnew) * c) : 1.f;
            mref = grow ? mnew : mref;
            lsum *= alpha;
#pragma unroll
            for (int nb = 0; nb < C::VBLK; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[nb][r] *= alpha;
        }
        const float mc = (mref == -INFINITY) ? 0.f : mref * c;
        float ls = lsum;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const f32x2 pr = {__builtin_amdgcn_exp2f(fmaf(s[t2 * 8 + e], c, -mc)),
                                  __builtin_amdgcn_exp2f(fmaf(s[t2 * 8 + e + 1], c, -mc))};
                const bf16x2 pb = __builtin_convertvector(pr, bf16x2);
                ls = __builtin_amdgcn_fdot2_f32_bf16(pb, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, ls, false);
                pf[t2][e] = pb[0];
                pf[t2][e + 1] = pb[1];
            }
        }
        lsum = ls;
    };

    issue_tile(0);
    if (ntile > 1) {
        issue_tile(1);
        wait_copies<C::CPW>();
    } else {
        wait_copies<0>();
    }
    phase_barrier();            // tile 0 visible
#pragma unroll
    for (int u = 0; u < PS_PD; ++u)  // M(0): values of sub-tile 0 (times zero probabilities)
        read_v(smem, u, vnext[u]);
    // Intervals and barriers as in the d <= 64 kernel: the map-1 group ends
    // interval j after V(j), the map-2 group after M(j).
    int so_j = 0, so_v = 0;   // stage ring offsets, carried as in the d <= 64 kernel
    for (int j = 0; j <= nsub; ++j) {
        __builtin_amdgcn_s_setprio(1);
        m_phase(j, so_j, so_v);
        if (j & 1) {
            // Copy tile (j+3)/2, then wait for tile (j+1)/2 with only the
            // copies just issued still in flight.
            const int ti = (j + 3) >> 1, tw = (j + 1) >> 1;
            if (ti < ntile) issue_tile(ti);
            if (tw + 1 < ntile) wait_copies<C::CPW>();
            else wait_copies<0>();
        }
        __builtin_amdgcn_s_setprio(0);
        if (grp) {
            phase_barrier();
            so_v = so_j;
            if (j & 1) so_j = (so_j + C::STAGE == PP_NSTAGE * C::STAGE) ? 0 : so_j + C::STAGE;
        }
        v_phase(j);
        if (!grp) {
            phase_barrier();
            so_v = so_j;
            if (j & 1) so_j = (so_j + C::STAGE == PP_NSTAGE * C::STAGE) ? 0 : so_j + C::STAGE;
        }
    }

    // Epilogue: map-2 waves hand lambda-scaled accumulators to map-1 waves.
    const f32x2 hl = halves(lsum);
    const float l = hl[0] + hl[1];
    phase_barrier();   // every wave is done with the stages (no copy in flight)
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
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
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
        const f32x2 hs2 = halves(ss);
        scale = norm_scale / sqrtf((hs2[0] + hs2[1]) / (float)DV + eps);
    }
    float* orow = out + (tok0 + my_row) * DV;
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

template <int D, int DV, bool SK>
hipError_t launch_ps(const PrefillArgs& a, hipStream_t stream) {
    using C = PSCfg<D, DV, SK>;
    const int row_tiles = (a.N + PS_BM - 1) / PS_BM;
    const int64_t blocks = (int64_t)a.B * a.H * row_tiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const int BH = a.B * a.H;   // at most `blocks`, so it fits
    static std::atomic<bool> lds_ok[MAX_DEVICES];
    const hipError_t e = ensure_lds_limit(prefill_ps_kernel<D, DV, SK>, C::LDS, lds_ok);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_ps_kernel<D, DV, SK>), dim3((unsigned)blocks), dim3(PS_THREADS),
                       (size_t)C::LDS, stream, (const __bf16*)a.q1, (const __bf16*)a.q2,
                       (const __bf16*)a.k1, (const __bf16*)a.k2, (const __bf16*)a.v, a.ldq, a.ldk,
                       a.ldv, BH, a.H, a.N, a.causal, a.lambda, a.rmsnorm, a.eps, a.norm_scale,
                       a.norm_weight, a.out, row_tiles, a.hs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    if (a.d == 64 && a.dv == 128) return launch_pp<64, 128, 2>(a, stream);
    if (a.d == 64 && a.dv == 64) return launch_pp<64, 64, 2>(a, stream);
    if (a.d == 32 && a.dv == 64) return launch_pp<32, 64, 2>(a, stream);
    if (a.d == 128 && a.dv == 128)
        return a.k1 == a.k2 ? launch_ps<128, 128, true>(a, stream) : launch_ps<128, 128, false>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_attention_pp(const PrefillArgs& a, hipStream_t stream) {
    if (a.d == 64 && a.dv == 128) return launch_pp<64, 128, 1>(a, stream);
    if (a.d == 64 && a.dv == 64) return launch_pp<64, 64, 1>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace diffattn
