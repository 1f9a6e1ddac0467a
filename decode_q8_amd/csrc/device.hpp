// Device-side helpers shared by the gfx950 kernels of libq8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace q8k {


typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// fp32 -> fp16 bits, round to nearest even, subnormals kept (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Component c (0..3) of a uint4, c known at compile time after unrolling.
__device__ __forceinline__ uint32_t word_of(const uint4 &v, int c) {
    return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// A 16-byte load with the non-temporal hint (global_load_dwordx4 ... nt), for
// data read once per call, the weight stream: its lines are then the first
// the caches give up, so they do not displace what many workgroups share
// (activations, step counters and flags).  Measured on the decode step: 318
// -> 306 us (m = 1), 637 -> 622 us (m = 8).  It lost where each 128-byte line
// is read by several load instructions of one lane or wave, since the line
// can then go between them: the row-layout weights (2x slower with it) and
// the weight quantizer's input (10%) keep plain loads.
__device__ __forceinline__ uint4 load_nt(const void *p) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The same hint as the cache-policy operand of __builtin_amdgcn_global_load_lds
// (global_load_lds_dwordx4 ... nt).
constexpr int CPOL_NT = 2;

// Index of this wave in its workgroup, as a wave-uniform (SGPR) value so that
// everything derived from it stays scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Maximum over each aligned group of 8 lanes, left in all 8: three DPP steps
// (swap neighbours, swap pairs, mirror the two halves of the 8 lanes), each a
// single v_max_f32 with a DPP source; the s_nop gives a DPP read the 2 wait
// states it needs after the VALU write of its source.  max is exact, so the
// order of the steps does not change the result.
__device__ __forceinline__ float max_over_8_lanes(float x) {
    asm("s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf"
        : "+v"(x));
    return x;
}

// Sum of the 8 block terms of one group, in the fixed tree order
// ((t0+t1)+(t2+t3))+((t4+t5)+(t6+t7)).
__device__ __forceinline__ float tree8(const float (&t)[8]) {
    return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

}  // namespace q8k
