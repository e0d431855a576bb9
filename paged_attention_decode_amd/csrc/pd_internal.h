// Internal declarations of the paged-decode library (not part of the C-ABI).
#pragma once

#include <cstdint>
#include <string>

#include "paged_decode.h"

#if defined(__HIPCC__)
#define PD_HD __host__ __device__ __forceinline__
#else
#define PD_HD inline
#endif

namespace pd {

// Invariant-integer division by d >= 1 for numerators below 2^32
// (Granlund & Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, the unsigned round-up method): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (t + ((n - t) >> s1)) >> s2 where t = mulhi(m, n), s1 = min(l, 1),
// s2 = max(l - 1, 0).  The page indirection splits a token slot into
// (page, entry) with it.
struct FastDiv {
    uint32_t d;
    uint32_t m;
    uint32_t s1;
    uint32_t s2;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    FastDiv f;
    f.d = d;
    f.m = uint32_t(m);
    f.s1 = l < 1 ? l : 1;
    f.s2 = l > 0 ? l - 1 : 0;
    return f;
}

PD_HD uint32_t mulhi32(uint32_t a, uint32_t b)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __umulhi(a, b);
#else
    return uint32_t((uint64_t(a) * uint64_t(b)) >> 32);
#endif
}

PD_HD uint32_t fastdiv_q(const FastDiv &f, uint32_t n)
{
    uint32_t t = mulhi32(f.m, n);
    return (t + ((n - t) >> f.s1)) >> f.s2;
}

// paged-MLA kernel (latent width 512, one KV head): query heads per
// workgroup for a group of num_qo_heads (or a negative code), and the
// workgroups resident at once on `device` (-1: current)
int mla_q_heads_per_wg(int32_t num_qo_heads);
int mla_resident_wgs(int32_t device, int32_t num_qo_heads);

// thread-local error message
void set_error(const std::string &msg);
int fail(int code, const std::string &msg);

}  // namespace pd
