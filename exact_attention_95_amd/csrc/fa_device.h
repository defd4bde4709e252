// Device-side building blocks shared by the forward kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4v __attribute__((vector_size(8)));
typedef int i32x2v __attribute__((vector_size(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Wave index as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Asynchronous 16-byte copy global -> LDS.  Lane i of the wave writes to
// lds_wave_base + 16 * i; lds_wave_base must be the same in every lane.
__device__ __forceinline__ void copy16_to_lds(const void *gsrc, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(gsrc, (FA_LDS void *)lds_wave_base, 16, 0, 0);
}

// Buffer resource for a byte range [base, base + bytes) (word 3 = 0x20000:
// 32-bit raw data format, no stride, no swizzle).  Loads past `bytes` return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Asynchronous 16-byte copy from a buffer (SGPR base + 32-bit per-lane byte
// offset) to LDS (buffer_load_dwordx4 ... lds); lane i writes to
// lds_wave_base + 16 * i.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, unsigned voff, void *lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void *)lds_wave_base, 16, voff, 0, 0, 0);
}

// Waits until every outstanding global load of this wave (including the
// direct-to-LDS copies) has completed.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposed 64-bit LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j supplies the address of 4 consecutive 16-bit elements; lane i
// receives element (i % 4) of the chunks addressed by lanes i/4, 4 + i/4,
// 8 + i/4 and 12 + i/4, in that order.
__device__ __forceinline__ i16x4 lds_read_tr16(const void *p) {
    i16x4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4v *)p);
    return __builtin_bit_cast(i16x4, r);
}

// Transposed 64-bit LDS read of 8-bit elements (ds_read_b64_tr_b8): within
// each group of 16 lanes, lane j supplies the address of 8 consecutive bytes;
// lane i receives byte (i % 8) of the chunks addressed by lanes
// i/8, 2 + i/8, ..., 14 + i/8, in that order.
__device__ __forceinline__ i32x2v lds_read_tr8(const void *p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2v *)p);
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC 2011): ten rounds of two 32x32->64-bit products
// with the multipliers 0xD2511F53 and 0xCD9E8D57, the words recombined as
// (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0), the key bumped by the Weyl
// constants 0x9E3779B9 and 0xBB67AE85 after each round.
__device__ __forceinline__ void philox4x32_10(unsigned c0, unsigned c1, unsigned c2, unsigned c3, unsigned k0,
                                              unsigned k1, unsigned (&out)[4]) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const unsigned hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
        const unsigned hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
        const unsigned n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

// Maps the hardware workgroup index to a logical one so that consecutive
// logical indices (the query blocks of one head) land on the same XCD:
// workgroups are dispatched to the 8 XCDs round-robin, and each XCD has its
// own L2, so a head's K/V tiles are then fetched from HBM once per XCD.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int per = n >> 3;
    if (bid < (per << 3)) return (bid & 7) * per + (bid >> 3);
    return bid;
}

}  // namespace fa
