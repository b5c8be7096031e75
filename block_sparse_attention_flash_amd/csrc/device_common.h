// Device-side building blocks shared by the gfx950 kernels of libblasst.
//
// Lane layouts below were checked on MI355X hardware:
//  * v_mfma_f32_16x16x32_bf16: lane l holds A[l&15][8*(l>>4)+i] and
//    B[8*(l>>4)+i][l&15] (i = 0..7); the result C[4*(l>>4)+i][l&15] (i = 0..3).
//  * v_mfma_f32_32x32x16_bf16: lane l holds A[l&31][8*(l>>5)+i] and
//    B[8*(l>>5)+i][l&31]; the result C[8*(i>>2) + 4*(l>>5) + (i&3)][l&31].
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, lane 4r+c names 4
//    consecutive 16-bit values (row r, columns 4c..4c+3 of a 4x16 block) and
//    lane j receives column j of that block: out[j][e] = block[e][j].
// Vectors of __bf16 are only ever built or taken apart as whole registers
// (bit casts of integer vectors); element access on them is avoided.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_copy.h"  // chunk_swizzle and the tile-copy offsets (host-callable)

namespace blasst {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 16-byte global load (one global_load_dwordx4).
__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two fp32 -> two bf16 (round to nearest even), packed low|high into one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposed 8-byte LDS read (see the layout note at the top).
__device__ __forceinline__ u32x2 lds_read_tr16(const lds_char* p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    return __builtin_bit_cast(u32x2, r);
}

// Two transposed 8-byte reads joined into one 8 x bf16 MFMA operand (the
// shuffle lets the two results land in one register quad, with no moves).
__device__ __forceinline__ bf16x8 lds_read_tr16_pair(const lds_char* lo, const lds_char* hi) {
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lo);
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)hi);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// 16-byte HBM -> LDS copy (global_load_lds_dwordx4): lane l's 16 bytes land at
// lds_base + 16*l, lds_base being wave-uniform (it travels in M0).  Issued as
// inline asm so the compiler adds no wait of its own for the LDS bytes it cannot
// see; the caller waits with an explicit, counted s_waitcnt vmcnt.
// The compiler's hazard pass cannot see that the asm is an LDS-DMA load, so the
// wait states this family needs before it are in the asm itself: one after a
// scalar write of M0 (which the compiler emits right before the asm).
// STREAM sets the non-temporal cache policy (nt), for rows that one pass reads
// once and no other workgroup needs from L2 later: the decode kernels' V, and
// their K where no partner workgroup re-reads it (decode.hip says where).  A
// 134 MB decode pass runs 8% faster with it (a plain streaming read of that size
// runs 5.6-5.9 TB/s with ordinary loads and 6.1-6.5 TB/s with non-temporal
// ones).  The prefill tiles, which the query blocks of a kv head share in L2,
// keep the default policy (non-temporal, prefill ran 3% slower).
template <bool STREAM = false>
__device__ __forceinline__ void global_to_lds16(const void* gptr, uint32_t lds_base) {
    if constexpr (STREAM)
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr),
                     "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory");
    else
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr),
                     "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory");
}

// Same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset (the instruction's saddr form): one VGPR of address per lane.
// The base must be the same in every lane; readfirstlane states that to the
// compiler (it cannot always prove it) so the operand is an SGPR pair.  A VMEM
// instruction that reads an SGPR written by a VALU instruction (v_readfirstlane)
// needs five wait states in between, which the compiler cannot insert for an
// asm it does not look into; without them the copy can read a stale base (a
// wild address) wherever the compiler places the readfirstlane right before
// it, so the asm starts with them (they also cover the scalar write of M0).
// STREAM: the non-temporal cache policy, as for global_to_lds16.
template <bool STREAM = false>
__device__ __forceinline__ void global_to_lds16_sbase(const void* sbase, uint32_t voff, uint32_t lds_base) {
    const uint64_t p = (uint64_t)sbase;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const void* sp = (const void*)(((uint64_t)hi << 32) | lo);
    if constexpr (STREAM)
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sp),
                     "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory");
    else
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sp),
                     "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory");
}

__device__ __forceinline__ float wave_shfl_xor(float x, int mask) {
    return __shfl_xor(x, mask, 64);
}

// Cross-lane reductions on the VALU (no LDS round trip).  gfx950's
// v_permlane32_swap applied to (x, x) leaves x of lane (i & 31) in the first
// result and x of lane 32 + (i & 31) in the second; v_permlane16_swap does the
// same for the 16-lane rows of each half (rows 0/2 and 1/3).  Combining the two
// results reduces over lanes i and i ^ 32 (resp. i ^ 16) in every lane.  The
// DPP forms reduce within a 16-lane row: quad_perm [1,0,3,2] and [2,3,0,1]
// pair lanes i ^ 1 and i ^ 2, then row_half_mirror (i <-> 7 - i within 8
// lanes) and row_mirror (i <-> 15 - i) join the quads and the half rows.
// (Lane layouts verified on the device.)
__device__ __forceinline__ float wave_max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const uint32_t a = r[0], b = r[1];
    return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float wave_sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const uint32_t a = r[0], b = r[1];
    return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ float wave_max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const uint32_t a = r[0], b = r[1];
    return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float wave_sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const uint32_t a = r[0], b = r[1];
    return __uint_as_float(a) + __uint_as_float(b);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
// OR / max over the 16 lanes of each row (every lane gets its row's result)
__device__ __forceinline__ uint32_t row16_or(uint32_t x) {
    x |= dpp_u32<0xB1>(x);   // quad_perm [1,0,3,2]
    x |= dpp_u32<0x4E>(x);   // quad_perm [2,3,0,1]
    x |= dpp_u32<0x141>(x);  // row_half_mirror
    x |= dpp_u32<0x140>(x);  // row_mirror
    return x;
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(dpp_u32<0x141>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(dpp_u32<0x140>(__float_as_uint(x))));
    return x;
}

}  // namespace blasst
