// Device helpers shared by the gfx950 kernels of the paged-decode library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// streaming (non-temporal) 16-byte load
__device__ __forceinline__ uint4 load_nt(const void *p)
{
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Read-only plan data (page table, request and chunk arrays) through the
// scalar cache: the address is wave-uniform, and an address-space-4 (constant)
// pointer lets the compiler use a scalar load instead of a vector load plus
// readfirstlane.  Nothing in the kernels writes these arrays.
__device__ __forceinline__ int32_t ld_uniform(const int32_t *p)
{
    typedef const __attribute__((address_space(4))) int32_t constant_i32;
    return *(constant_i32 *)p;   // generic -> constant address space
}

// gfx950 permlane swaps.  After swap32(a, b) the lanes of the lower half
// hold (a of lane l, a of lane l + 32) and those of the upper half hold (b of
// lane l - 32, b of lane l): each half gets the (lower, upper) pair of one of
// the two values.  swap16 does the same for each pair of 16-lane rows (even
// row: the pair of a, odd row: the pair of b).  They are issued as inline
// assembly because the compiler's builtins for them hand back the first
// result in place of the second; the nop covers the wait states a permlane
// needs after a VALU write of its operands.
__device__ __forceinline__ void swap32(float &a, float &b)
{
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16(float &a, float &b)
{
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// max / sum over the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float group_max4(float x)
{
    float a = x, b = x;
    swap16(a, b);
    x = fmaxf(a, b);
    a = x;
    b = x;
    swap32(a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float group_sum4(float x)
{
    float a = x, b = x;
    swap16(a, b);
    x = a + b;
    a = x;
    b = x;
    swap32(a, b);
    return a + b;
}

}  // namespace pd
