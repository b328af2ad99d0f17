// Device helpers shared by the bf16 prefill kernels: operand types, the LDS
// tile layout (chunk swizzles, key permutation), the gfx950 LDS transpose
// load, and global->LDS copies through raw buffer descriptors.
//
// Translation units that include this file are compiled with IEEE mode off
// and NaNs not honoured (see max3).
#pragma once

#include <hip/hip_runtime.h>

namespace diffattn {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int QROWS = 32;      // query rows per row block (MFMA N dimension)
constexpr int BN = 32;         // keys per sub-tile (MFMA M dimension of S^T)
constexpr int TK = 2 * BN;     // keys per LDS stage
constexpr float TAU = 8.0f;    // lazy-rescale threshold, base-2 exponent units

// Chunk swizzles (physical 16-byte chunk = logical chunk ^ swizzle(row)).
// Keys: the 16 rows read by one 16-lane quarter land in 16 distinct 16-byte
// bank groups of a 256-byte bank line.
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
// Score register r of lane (col, half) then holds key
// 16*(r/8) + 8*half + 4*((r/4)%2) + r%4 of the sub-tile.
__device__ __forceinline__ int kappa(int rho) {
    return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}
__device__ __forceinline__ constexpr int key_of_reg(int r) {
    return 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);   // + 8*half
}

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// max(a, b, c): with IEEE mode off and NaNs not honoured the chain lowers to
// one v_max3_f32 with no quieting of its inputs.  (It must stay visible to
// the compiler: reading matrix-core results needs wait states that only the
// compiler inserts.)
__device__ __forceinline__ float max3(float a, float b, float c) {
    return fmaxf(fmaxf(a, b), c);
}

// Both halves of a wave, broadcast: lanes l and l^32 exchange through
// v_permlane32_swap (no LDS round trip).  Returns {x[l % 32], x[l % 32 + 32]}.
__device__ __forceinline__ f32x2 halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// gfx950 LDS transpose load: within each 16-lane group, lane j supplies an
// 8-byte segment (4 bf16) at `p`; lane i receives element i%4 of the
// segments supplied by lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ bf16x4 lds_read_tr(const unsigned char* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<unsigned char*>(p)));
    return __builtin_bit_cast(bf16x4, v);
}

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
// barrier that publishes the data.
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, unsigned lds_base, int voff) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base)
                 : "memory");
}

}  // namespace tile
}  // namespace diffattn
