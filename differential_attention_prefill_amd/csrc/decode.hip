// Split-KV differential-attention decode, V2 layout (bf16 cache, fp32 math).
//
// One new query token per sequence.  Pair p of a sequence uses query head 2p
// for A1 and query head 2p+1 for A2, both over KV head g = floor(2p/(Hq/Hkv)):
//     out_p = (softmax(q_2p K_g^T / sqrt D) - lambda_p softmax(q_2p+1 K_g^T / sqrt D)) V_g
// (page "差分注意力" (aiknowledge.cn), "V1 到 V2 的 diff": twice the query heads
// over the same KV heads, so one pass over the cache serves both maps and all
// query heads of a group; part 二 Step 2 for the operator).
//
// The cache is read exactly once, which makes the kernel HBM-bound:
//  - split kernel: about two workgroups per CU, each with an equal share of
//    the keys.  The cached rows of all (sequence, KV head) segments, laid end
//    to end (sequence-major, head-minor), are cut into gridDim.x contiguous
//    ranges of one length R (a multiple of the 128 keys one loop step covers,
//    at least DEC_RANGE_MIN), so every workgroup streams the same number of
//    keys whatever the length mix; fixed chunks dealt round-robin leave the
//    workgroups that draw one chunk more as the tail of the launch.  A
//    workgroup takes its range as one piece per segment it touches; piece k
//    of a segment is its k-th range, so a segment has at most
//    ceil(max_len / DEC_RANGE_MIN) + 1 pieces.  One piece streams its rows of
//    K_g and V_g for ALL Hq/Hkv query heads of the group (both heads of every
//    pair).  Each of its 4 waves takes every 4th 32-key tile of the piece.  Scores come from v_mfma_f32_16x16x32_bf16
//    as S^T = K . Q^T (keys x query heads, the 16 columns padded with zero
//    heads); probabilities go from registers into O^T += V^T . P^T.  Each V
//    tile is copied from global memory straight into one of the wave's two
//    LDS tiles (buffer loads that write LDS, one tile ahead) and its V^T
//    fragments are read with the transpose load.  Each head keeps
//    its own running maximum / normaliser / accumulator; the waves' states are
//    merged in LDS and one partial state (O, m, l) per head and piece is
//    written to the workspace.
//    The workgroup that streams the last piece of a segment also writes the
//    segment's piece count.
//  - merge kernel: grid (pair, sequence).  Merges the pieces of the pair's
//    segment for both heads of the pair by log-sum-exp weights in a fixed
//    order (deterministic for a given grid), then
//    combines the two maps with lambda and optionally applies the per-head
//    RMS norm.
//
// V1 layout (half-width maps: q = [q1 | q2] and each key row = [k1 | k2],
// d = D/2; page "差分注意力", part 一 and "V1 到 V2 的 diff") runs on the same
// kernels: head h is a group of two query columns over its own K/V rows,
// column 0 holding q1 in the first d channels and zeros in the rest, column 1
// zeros then q2, so the D-wide dot products are q1.k1 and q2.k2 and V is read
// once for both maps.  Scores are scaled by 1/sqrt(d).
#include <atomic>

#include "kernels.h"

namespace diffattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int DEC_D = DECODE_D;        // head width
constexpr int DEC_WAVES = 4;
constexpr int DEC_THREADS = 64 * DEC_WAVES;
constexpr int DEC_TILE = 32;           // keys per wave iteration
constexpr int DEC_STEP = DEC_TILE * DEC_WAVES;   // keys per loop step of a workgroup
constexpr int DEC_RANGE_MIN = DECODE_RANGE_MIN;   // shortest key range per workgroup
constexpr int DEC_GROUP_MAX = 16;      // query heads per KV head that fit the MFMA columns
constexpr int DEC_VROWB = DEC_D * 2;            // bytes per cached V row
constexpr int DEC_VBYTES = DEC_TILE * DEC_VROWB; // one V tile, token-major (8 KB)
constexpr int DEC_STATE = DECODE_STATE;         // floats per partial state: O[D], m*c, l
constexpr float DEC_TAU = 8.0f;

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Cache stream: every byte is read once, so the loads carry the non-temporal
// hint (no reuse to keep in the caches; measured 6.5-7.4 TB/s for a plain
// streaming read on this device against 6.1-6.3 TB/s without it).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// V tiles reach LDS straight from global memory (buffer loads that write LDS:
// no staging registers) and leave it through the gfx950 transpose load, which
// hands each lane 4 consecutive keys of one channel.  Rows are stored with
// their 32-byte channel slots XOR-swizzled so that the 4 rows one 16-lane
// group reads (rows 8G + 0..3, or + 4..7) and the 4 rows of the neighbouring
// group (8(G+1) + the same) take 8 distinct slots: the 32 lanes served
// together touch every bank once.
__device__ __forceinline__ int vslot_swz(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }

// Raw buffer descriptor (gfx9-family layout): base, stride 0, byte extent;
// loads at offsets >= `bytes` return zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int bytes) {
    const unsigned long long a = (unsigned long long)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000;
    return r;
}
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)((__attribute__((address_space(3))) const unsigned char*)p);
}
// 16 bytes per lane from global memory into LDS at lds_base + 16*lane, with the
// non-temporal hint.  The compiler does not track these loads.  Inside the key
// loop the kernel relies on the waits it emits for the key loads issued after
// each tile's copies (loads complete in issue order); before the LDS is reused
// for the merge it waits for every load explicitly.
__device__ __forceinline__ void copy16_to_lds_nt(i32x4 rsrc, unsigned lds_base, int voff) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base)
                 : "memory");
}
__device__ __forceinline__ bf16x4 lds_read_tr(const unsigned char* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<unsigned char*>(p)));
    return __builtin_bit_cast(bf16x4, v);
}

// Row slot rho of score tile t holds key (rho/4)*8 + t*4 + rho%4 of the
// 32-key tile, so that the accumulator registers of tiles 0 and 1 line up as
// 8 consecutive keys per lane group: the B operand of the next product.
__device__ __forceinline__ int slot_key(int rho, int t) { return (rho >> 2) * 8 + t * 4 + (rho & 3); }

// Length of sequence bb, 0 when outside [1, max_len] (such a sequence has no
// keys and its outputs are zeros).
__device__ __forceinline__ int valid_len(const int32_t* seq_lens, int bb, int max_len) {
    const int Lb = seq_lens[bb];
    return (Lb < 1 || Lb > max_len) ? 0 : Lb;
}
// Keys per workgroup range for `total` keys over `nranges` ranges.
__device__ __forceinline__ int64_t range_len(int64_t total, int nranges) {
    int64_t r = (total + nranges - 1) / nranges;
    r = (r + DEC_STEP - 1) / DEC_STEP * DEC_STEP;
    return r < DEC_RANGE_MIN ? DEC_RANGE_MIN : r;
}

__global__ void __launch_bounds__(DEC_THREADS)
decode_split_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ kc,
                    const __bf16* __restrict__ vc, const int32_t* __restrict__ seq_lens, int B,
                    int Hq, int Hkv, int max_len, int max_splits, float* __restrict__ ws,
                    int* __restrict__ piece_count, int qhalf, float c) {
    // Two V tiles per wave during the stream; reused as the wave-merge buffer.
    // Each lane stores 16 bytes per block; head rows are padded to 132 floats
    // (528 bytes), so the 16 heads of one store's 16 lanes start 4 banks apart
    // and fill all 64 banks.
    __shared__ __attribute__((aligned(16))) unsigned char lds[DEC_WAVES * 2 * DEC_VBYTES];
    __shared__ float merge_m[DEC_WAVES][DEC_GROUP_MAX];
    __shared__ float merge_l[DEC_WAVES][DEC_GROUP_MAX];
    constexpr int MROW = DEC_D + 4;
    static_assert(DEC_WAVES * DEC_GROUP_MAX * MROW * 4 <= DEC_WAVES * 2 * DEC_VBYTES,
                  "merge buffer must fit in the V tiles");
    float (*merge_o)[DEC_GROUP_MAX][MROW] = reinterpret_cast<float (*)[DEC_GROUP_MAX][MROW]>(lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;      // query head inside the group (MFMA column)
    const int grp = lane >> 4;      // 4 lane groups
    const int G = Hq / Hkv;         // query heads in this KV group
    const bool col_ok = col < G;

    // This workgroup's key range [r0, r1) (uniform).
    int64_t total = 0;
    for (int bb = 0; bb < B; ++bb) total += (int64_t)valid_len(seq_lens, bb, max_len) * Hkv;
    const int64_t R = range_len(total, gridDim.x);
    const int64_t r0 = (int64_t)blockIdx.x * R;
    if (r0 >= total) return;
    const int64_t r1 = min(total, r0 + R);
    // The segment holding r0: sequence b (keys from base on), head g.  The walk
    // stops at a sequence with keys because r0 < total.
    int b = 0, L = valid_len(seq_lens, 0, max_len);
    int64_t base = 0;
    while (base + (int64_t)L * Hkv <= r0) {
        base += (int64_t)L * Hkv;
        ++b;
        L = valid_len(seq_lens, b, max_len);
    }
    int g = (int)((r0 - base) / L);
    int64_t seg0 = base + (int64_t)g * L;   // first key of segment (b, g)
    for (int64_t pos = r0; pos < r1;) {
        // Piece: positions c0 .. cend-1 of segment (b, g); it is the
        // (blockIdx.x - seg0/R)-th range that touches the segment.
        const int c0 = (int)(pos - seg0);
        const int cend = (int)min((int64_t)L, r1 - seg0);
        const int split = (int)(blockIdx.x - seg0 / R);
        const int n_it = (cend - c0 + DEC_STEP - 1) / DEC_STEP;
        const int64_t kv0 = ((int64_t)b * Hkv + g) * max_len;   // row of position 0
        // c = log2(e) / sqrt(dot length), from the host.

        // Q^T fragments: lane (col, grp) holds q[head col][s*32 + grp*8 .. +8].
        // V1 (qhalf > 0): both columns read the packed row [q1 | q2] of head g and
        // keep only their own half.
        bf16x8 qf[4];
        {
            const __bf16* qr = qhalf > 0 ? q + ((int64_t)b * Hkv + g) * DEC_D + grp * 8
                                         : q + ((int64_t)b * Hq + g * G + (col_ok ? col : 0)) * DEC_D + grp * 8;
    #pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bool mine = qhalf > 0 ? ((s * 32 + grp * 8 < qhalf) == (col == 0)) : true;
                uint4 v = col_ok && mine ? ld16(qr + s * 32) : make_uint4(0, 0, 0, 0);
                qf[s] = __builtin_bit_cast(bf16x8, v);
            }
        }

        float mref = -INFINITY, lsum = 0.f;
        f32x4 acc[8];
    #pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Prefetch registers: K fragments in A-operand order.  V tiles go to
        // this wave's two LDS tiles (tile it in tile it % 2).
        uint4 kreg[2][4];
        auto fetch_k = [&](int it) {
            const int kb = c0 + (it * DEC_WAVES + wave) * DEC_TILE;
    #pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int key = kb + slot_key(col, t);
                const bool ok = key < cend;
                const __bf16* src = kc + (kv0 + (ok ? key : 0)) * DEC_D + grp * 8;
    #pragma unroll
                for (int s = 0; s < 4; ++s) kreg[t][s] = ok ? ld16_stream(src + s * 32) : make_uint4(0, 0, 0, 0);
            }
        };
        const unsigned vlds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds + wave * 2 * DEC_VBYTES));
        auto fetch_v = [&](int it) {
            const int kb = c0 + (it * DEC_WAVES + wave) * DEC_TILE;
            // Rows past the piece end read as zeros (their probabilities are 0).
            const int rows = max(0, min(DEC_TILE, cend - kb));
            const i32x4 r = make_rsrc(vc + (kv0 + kb) * DEC_D, rows * DEC_VROWB);
            const unsigned dst = vlds0 + (unsigned)((it & 1) * DEC_VBYTES);
    #pragma unroll
            for (int bb = 0; bb < DEC_VBYTES / 1024; ++bb) {
                // Lane l of block bb fills physical row 4*bb + l/16, 16-byte
                // chunk l%16, which holds logical chunk (l%16) ^ 2*swz(row).
                const int row = 4 * bb + (lane >> 4);
                const int lc = (lane & 15) ^ (2 * vslot_swz(row));
                copy16_to_lds_nt(r, dst + bb * 1024, row * DEC_VROWB + lc * 16);
            }
        };
        // V^T fragment of 16 channels (block blk) from the tile at vt: lane
        // (i = lane % 16, G = lane / 16) gets keys 8G .. 8G+7 of channel
        // 16*blk + i; within a 16-lane group lane j points at row 8G + j/4 (+4),
        // channels 16*blk + 4*(j%4) .. +3.
        const int vr0 = 8 * grp + (col >> 2);
        const int vcb = 8 * (col & 3);                 // byte offset of the 4 channels in the slot
        auto vfrag = [&](const unsigned char* vt, int blk) -> bf16x8 {
            const unsigned char* p0 = vt + vr0 * DEC_VROWB + ((blk ^ vslot_swz(vr0)) * 32) + vcb;
            const unsigned char* p1 = vt + (vr0 + 4) * DEC_VROWB + ((blk ^ vslot_swz(vr0 + 4)) * 32) + vcb;
            const bf16x4 lo = lds_read_tr(p0);
            const bf16x4 hi = lds_read_tr(p1);
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };

        fetch_v(0);
        fetch_k(0);
        for (int it = 0; it < n_it; ++it) {
            const int kb = c0 + (it * DEC_WAVES + wave) * DEC_TILE;
            const bool active = kb < cend;
            // S^T = K . Q^T for the two 16-key halves of the tile.  The waits the
            // compiler emits for kreg also cover this tile's V copies, issued
            // before its keys.
            f32x4 s[2];
    #pragma unroll
            for (int t = 0; t < 2; ++t) {
                s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                for (int st = 0; st < 4; ++st)
                    s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[t][st]),
                                                                   qf[st], s[t], 0, 0, 0);
            }
            // The next tile: its values into the other LDS tile (last read by
            // the products of tile it-1, complete before this iteration), then
            // its keys into kreg.
            if (it + 1 < n_it) {
                fetch_v(it + 1);
                fetch_k(it + 1);
            }
            const unsigned char* vt = lds + wave * 2 * DEC_VBYTES + (it & 1) * DEC_VBYTES;
            if (!active) continue;

            // Mask positions past the piece end; online softmax per head.
            float sv[8];
    #pragma unroll
            for (int t = 0; t < 2; ++t)
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = kb + slot_key(grp * 4 + r, t);
                    sv[t * 4 + r] = key < cend ? s[t][r] : -INFINITY;
                }
            float mx = sv[0];
    #pragma unroll
            for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(mref, mx);
            const bool grow = mref == -INFINITY || (mnew - mref) * c > DEC_TAU;
            if (__any(grow)) {
                const float alpha = __builtin_amdgcn_exp2f((mref - mnew) * c);  // 0 on first use
                mref = mnew;
                lsum *= alpha;
    #pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] *= alpha;
            }
            const float mc = mref * c;
            bf16x8 pf;
            float ls = 0.f;
    #pragma unroll
            for (int e = 0; e < 8; e += 2) {
                f32x2 pr = {__builtin_amdgcn_exp2f(fmaf(sv[e], c, -mc)),
                            __builtin_amdgcn_exp2f(fmaf(sv[e + 1], c, -mc))};
                bf16x2 pb = __builtin_convertvector(pr, bf16x2);
                // The normaliser sums the same bf16 probabilities the product uses.
                ls = __builtin_amdgcn_fdot2_f32_bf16(pb, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, ls, false);
                pf[e] = pb[0];
                pf[e + 1] = pb[1];
            }
            lsum += ls;
            // O^T += V^T . P^T over 8 blocks of 16 channels.
    #pragma unroll
            for (int blk = 0; blk < 8; ++blk) {
                const bf16x8 vf = vfrag(vt, blk);
                acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[blk], 0, 0, 0);
            }
        }

        // Every wave saw at least one key of the piece only if its first tile was
        // inside it; idle waves carry m = -inf, l = 0, O = 0 and merge as nothing.
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        // The merge buffer below overlays the V tiles, which the untracked
        // LDS copies write: every copy of this wave has landed before the
        // barrier, whatever waits the compiler placed for the key loads.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();   // every wave is done reading its V tiles
        if (col_ok) {
            if (grp == 0) {
                merge_m[wave][col] = mref;
                merge_l[wave][col] = lsum;
            }
    #pragma unroll
            for (int blk = 0; blk < 8; ++blk)
                *reinterpret_cast<f32x4*>(&merge_o[wave][col][blk * 16 + grp * 4]) = acc[blk];
        }
        __syncthreads();
        // Merge the waves: thread = (head, channel).
        float* ws_split = ws + (((int64_t)b * Hq + g * G) * max_splits + split) * DEC_STATE;
        for (int e = tid; e < G * DEC_D; e += DEC_THREADS) {
            const int hh = e / DEC_D, ch = e % DEC_D;
            float M = -INFINITY;
    #pragma unroll
            for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, merge_m[w][hh]);
            float o = 0.f, l = 0.f;
    #pragma unroll
            for (int w = 0; w < DEC_WAVES; ++w) {
                const float mw = merge_m[w][hh];
                const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mw - M) * c);
                o = fmaf(merge_o[w][hh][ch], f, o);
                l = fmaf(merge_l[w][hh], f, l);
            }
            float* st = ws_split + (int64_t)hh * max_splits * DEC_STATE;
            st[ch] = o;
            if (ch == 0) {
                st[DEC_D] = M * c;
                st[DEC_D + 1] = l;
            }
        }
        if (cend == L && tid == 0) piece_count[b * Hkv + g] = split + 1;
        __syncthreads();   // the merge buffer is read before the next piece's V tiles
        // Next segment (a piece that ends before r1 ends its segment); sequences
        // without keys are skipped, and one with keys follows because pos < r1.
        pos = seg0 + cend;
        if (pos < r1) {
            seg0 += L;
            if (++g == Hkv) {
                g = 0;
                do {
                    ++b;
                    L = valid_len(seq_lens, b, max_len);
                } while (L == 0);
            }
        }
    }
}

// Merge the pieces of both heads of a pair and combine them with lambda.
// 256 threads: thread (m, ch) owns channel ch of head 2p+m.  The split maxima
// are reduced once through LDS; each thread then sums its channel over the
// splits with independent loads (unrolled), so the kernel is not a chain of
// dependent global reads.  With `single` the two heads are independent
// single-map heads (plain attention): each is normalised and written to
// out [B][Hq][D], with no pairing, lambda or norm.
constexpr int MERGE_THREADS = 2 * DEC_D;
constexpr int MERGE_LDS_SPLITS = 1024;   // splits whose weights are cached in LDS

__global__ void __launch_bounds__(MERGE_THREADS)
decode_merge_kernel(const float* __restrict__ ws, const int* __restrict__ piece_count,
                    const int32_t* __restrict__ seq_lens, int Hq, int Hkv, int max_len,
                    int max_splits, const float* __restrict__ lambda,
                    float* __restrict__ out, int rmsnorm, float eps, float norm_scale,
                    const float* __restrict__ norm_weight, int single) {
    const int p = blockIdx.x;
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int m = tid / DEC_D;        // 0: head 2p (A1), 1: head 2p+1 (A2)
    const int ch = tid % DEC_D;
    const int P = Hq / 2;
    const int L = seq_lens[b];
    const int head = 2 * p + m;
    const bool head_ok = head < Hq;   // an odd single-map head count leaves one idle
    float* o = single ? out + ((int64_t)b * Hq + head) * DEC_D : out + ((int64_t)b * P + p) * DEC_D;
    if (L < 1 || L > max_len) {       // block-uniform
        if (single ? head_ok : tid < DEC_D) o[ch] = 0.f;
        return;
    }
    __shared__ float w_lds[2][MERGE_LDS_SPLITS];
    __shared__ float red[2][MERGE_THREADS / 64];
    __shared__ float res[DEC_D];
    // Pieces of segment (b, g) of this thread's head, written by the split
    // kernel (both heads of a pair share g).
    const int nsplit = head_ok ? min(piece_count[b * Hkv + head / (Hq / Hkv)], max_splits) : 0;
    const float* st = ws + ((int64_t)b * Hq + (head_ok ? head : 0)) * max_splits * DEC_STATE;

    // Maximum of the split maxima of this thread's head (both heads at once:
    // threads 0..127 scan head 0, 128..255 head 1).
    float M = -INFINITY;
    for (int s = ch; s < nsplit; s += DEC_D) M = fmaxf(M, st[(int64_t)s * DEC_STATE + DEC_D]);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if ((tid & 63) == 0) red[m][(tid % DEC_D) / 64] = M;
    __syncthreads();
    M = fmaxf(red[m][0], red[m][1]);
    // Split weights 2^(m_s - M), cached for the first MERGE_LDS_SPLITS splits.
    for (int s = ch; s < min(nsplit, MERGE_LDS_SPLITS); s += DEC_D)
        w_lds[m][s] = __builtin_amdgcn_exp2f(st[(int64_t)s * DEC_STATE + DEC_D] - M);
    __syncthreads();
    float acc = 0.f, l = 0.f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) {
        const float f = s < MERGE_LDS_SPLITS ? w_lds[m][s]
                                             : __builtin_amdgcn_exp2f(st[(int64_t)s * DEC_STATE + DEC_D] - M);
        acc = fmaf(st[(int64_t)s * DEC_STATE + ch], f, acc);
        l = fmaf(st[(int64_t)s * DEC_STATE + DEC_D + 1], f, l);
    }
    const float r = acc / l;
    if (single) {                     // block-uniform
        if (head_ok) o[ch] = r;
        return;
    }
    if (m == 1) res[ch] = r;
    __syncthreads();
    const float y = r - lambda[p] * res[ch];     // meaningful for m == 0
    if (!rmsnorm) {
        if (m == 0) o[ch] = y;
        return;
    }
    // RMS norm over the DEC_D channels of the row (threads 0..127, two waves).
    float ss = m == 0 ? y * y : 0.f;
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) red[0][tid / 64] = ss;
    __syncthreads();
    const float scale = norm_scale / sqrtf((red[0][0] + red[0][1]) / (float)DEC_D + eps);
    if (m == 0) o[ch] = y * scale * (norm_weight ? norm_weight[ch] : 1.f);
}

}  // namespace

// Workgroups (= key ranges) of the split kernel: two per CU (its register
// use allows two per CU), never more than ranges of DEC_RANGE_MIN keys can be
// non-empty.
static int decode_split_grid(int B, int Hkv, int max_len) {
    // CU count per device, cached (a repeated first query is harmless).
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    int n = dev >= 0 && dev < 64 ? cus[dev].load(std::memory_order_relaxed) : 0;
    if (n == 0) {
        if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            n = 256;
        if (dev >= 0 && dev < 64) cus[dev].store(n, std::memory_order_relaxed);
    }
    const int64_t ranges = (int64_t)B * Hkv * ((max_len + DEC_RANGE_MIN - 1) / DEC_RANGE_MIN);
    const int64_t want = 2 * (int64_t)n;
    return (int)(ranges < want ? ranges : want);
}

// Fixed decode workspace for callers that cannot allocate: one copy of this
// array per device, held until the process ends, shared by every
// allocation-free call on that device (so such calls must not overlap).  The
// kernels keep nothing in it across calls: every piece count and partial
// state the merge reads is written by the same call's split kernel, so it
// needs no clearing.  In host code the name is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[DECODE_SCRATCH_BYTES / sizeof(float)];

constexpr int SCRATCH_DEVICES = 64;

// Device address of `scratch` on the current device, looked up on the first
// call there (a repeated first lookup from two threads stores the same value).
static hipError_t scratch_address(float** out) {
    static std::atomic<float*> addr[SCRATCH_DEVICES];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_DEVICES) return hipErrorInvalidDevice;
    float* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(reinterpret_cast<void**>(&p), HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_decode_noalloc(const DecodeArgs& args, hipStream_t stream) {
    if (decode_workspace_floats(args.B, args.Hq, args.D, args.max_len) * sizeof(float) >
        DECODE_SCRATCH_BYTES)
        return hipErrorInvalidValue;
    DecodeArgs a = args;
    const hipError_t e = scratch_address(&a.workspace);
    if (e != hipSuccess) return e;
    return launch_decode(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.D != DEC_D || a.Hq / a.Hkv > DEC_GROUP_MAX) return hipErrorInvalidValue;
    const int S = decode_max_splits(a.max_len);
    const float c = 1.4426950408889634f / sqrtf((float)(a.qhalf > 0 ? a.qhalf : DEC_D));
    const int grid = decode_split_grid(a.B, a.Hkv, a.max_len);
    int* counts = reinterpret_cast<int*>(a.workspace + decode_state_floats(a.B, a.Hq, a.max_len));
    if (grid > 0)
        hipLaunchKernelGGL(decode_split_kernel, dim3(grid), dim3(DEC_THREADS), 0, stream,
                           (const __bf16*)a.q, (const __bf16*)a.k_cache, (const __bf16*)a.v_cache,
                           a.seq_lens, a.B, a.Hq, a.Hkv, a.max_len, S, a.workspace, counts, a.qhalf, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel, dim3((a.Hq + 1) / 2, a.B), dim3(MERGE_THREADS), 0, stream,
                       a.workspace, counts, a.seq_lens, a.Hq, a.Hkv, a.max_len, S, a.lambda, a.out, a.rmsnorm,
                       a.eps, a.norm_scale, a.norm_weight, a.single);
    return hipGetLastError();
}

}  // namespace diffattn
