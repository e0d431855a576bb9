// Cascade head stacking, for gfx950.
//
// Method: mlxcel cascade-attention doc, "head stacking": the shared span is
// attended once as a single request whose query heads are the members'
// heads stacked so that stacked head h0 = kv*(M*G) + m*G + g is query head
// kv*G + g of member m (a [M, Hkv, G, D] -> [Hkv, M, G, D] transpose); the
// partial kernel's rule "query head h reads KV head h / group" then reads KV
// head kv.  The level-0 partial rows go back through the inverse transpose
// into each member's merge group, next to that member's own level-1
// rows, so a single merge (the cascade doc's "one merge, pairing each
// member's states") finishes the step.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pd_internal.h"

namespace pd {
namespace {

// one thread per 16-byte vector of a head row
__global__ void __launch_bounds__(256) stack_q_kernel(const uint4 *__restrict__ q, int members,
                                                      int hkv, int g, int vecs_per_row,
                                                      uint4 *__restrict__ q0)
{
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = int64_t(members) * hkv * g * vecs_per_row;
    if (idx >= total) return;
    const int x = int(idx % vecs_per_row);
    int64_t rest = idx / vecs_per_row;            // source (m, kv, gi) in [M, Hkv, G] order
    const int gi = int(rest % g);
    rest /= g;
    const int kv = int(rest % hkv);
    const int m = int(rest / hkv);
    const int64_t h0 = (int64_t(kv) * members + m) * g + gi;
    q0[h0 * vecs_per_row + x] = q[idx];
}

// One thread per float of a destination row (and the LSE for x == 0).
// Threads [0, n0*M*Hq*D) un-stack the level-0 rows; the rest move the
// level-1 rows next to them.
__global__ void __launch_bounds__(256) gather_kernel(const float *__restrict__ v0,
                                                     const float *__restrict__ lse0, int n0,
                                                     const float *__restrict__ v1,
                                                     const float *__restrict__ lse1, int n1,
                                                     const int32_t *__restrict__ req1,
                                                     int members, int hkv, int g, int d,
                                                     float *__restrict__ v_dst,
                                                     float *__restrict__ lse_dst)
{
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int hq = hkv * g;
    const int64_t part0 = int64_t(n0) * members * hq * d;
    const int64_t total = part0 + int64_t(n1) * hq * d;
    if (idx >= total) return;
    if (idx < part0) {
        const int x = int(idx % d);
        int64_t rest = idx / d;                   // destination (i, m, kv, gi)
        const int gi = int(rest % g);
        rest /= g;
        const int kv = int(rest % hkv);
        rest /= hkv;
        const int m = int(rest % members);
        const int i = int(rest / members);
        const int64_t h0 = (int64_t(kv) * members + m) * g + gi;   // stacked head
        const int64_t src = int64_t(i) * members * hq + h0;        // row of [n0, M*Hq]
        // member m's group starts at m*n0 + (level-1 rows of members before m);
        // those rows number o1[m] = the count of level-1 chunks with req1 < m
        int lo = 0, hi = n1;                       // lower bound of m in sorted req1
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (req1[mid] < m) lo = mid + 1;
            else hi = mid;
        }
        const int64_t dst = (int64_t(m) * n0 + lo + i) * hq + int64_t(kv) * g + gi;
        v_dst[dst * d + x] = v0[src * d + x];
        if (x == 0) lse_dst[dst] = lse0[src];
    } else {
        const int64_t j = idx - part0;
        const int x = int(j % d);
        const int64_t rest = j / d;               // (n, h) of level 1
        const int h = int(rest % hq);
        const int n = int(rest / hq);
        const int64_t dst = (int64_t(req1[n] + 1) * n0 + n) * hq + h;
        v_dst[dst * d + x] = v1[rest * d + x];
        if (x == 0) lse_dst[dst] = lse1[rest];
    }
}

}  // namespace
}  // namespace pd

using namespace pd;

extern "C" int paged_cascade_stack_q(const void *q, int32_t dtype, int32_t members,
                                     int32_t num_qo_heads, int32_t num_kv_heads,
                                     int32_t head_dim, void *q0, void *stream)
{
    if (!q || !q0) return fail(PD_E_NULL, "paged_cascade_stack_q: null pointer");
    if (members < 1 || num_kv_heads < 1 || num_qo_heads % num_kv_heads != 0 || head_dim < 1)
        return fail(PD_E_ARG, "paged_cascade_stack_q: bad sizes");
    const int esz = dtype == PD_DTYPE_FP16 ? 2 : (dtype == PD_DTYPE_FP32 ? 4 : 0);
    if (!esz) return fail(PD_E_UNSUPPORTED, "paged_cascade_stack_q: dtype");
    if ((head_dim * esz) % 16 || (reinterpret_cast<uintptr_t>(q) & 15u) ||
        (reinterpret_cast<uintptr_t>(q0) & 15u))
        return fail(PD_E_UNSUPPORTED, "paged_cascade_stack_q: rows must be 16-byte multiples");
    const int vecs = head_dim * esz / 16;
    const int g = num_qo_heads / num_kv_heads;
    const int64_t total = int64_t(members) * num_qo_heads * vecs;
    hipLaunchKernelGGL(stack_q_kernel, dim3(uint32_t((total + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4 *>(q), members,
                       num_kv_heads, g, vecs, static_cast<uint4 *>(q0));
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string("paged_cascade_stack_q: ") + hipGetErrorString(err));
    return PD_OK;
}

extern "C" int paged_cascade_gather_states(const float *v0, const float *lse0, int32_t n0,
                                           const float *v1, const float *lse1, int32_t n1,
                                           const int32_t *req1, int32_t members,
                                           int32_t num_qo_heads, int32_t num_kv_heads,
                                           int32_t head_dim, float *v_dst, float *lse_dst,
                                           void *stream)
{
    if (!v_dst || !lse_dst || (n0 > 0 && (!v0 || !lse0)) || (n1 > 0 && (!v1 || !lse1 || !req1)))
        return fail(PD_E_NULL, "paged_cascade_gather_states: null pointer");
    if (n0 < 0 || n1 < 0 || members < 1 || num_kv_heads < 1 ||
        num_qo_heads % num_kv_heads != 0 || head_dim < 1)
        return fail(PD_E_ARG, "paged_cascade_gather_states: bad sizes");
    const int64_t total = (int64_t(n0) * members + n1) * num_qo_heads * head_dim;
    if (total == 0) return PD_OK;
    hipLaunchKernelGGL(gather_kernel, dim3(uint32_t((total + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), v0, lse0, n0, v1, lse1, n1, req1,
                       members, num_kv_heads, num_qo_heads / num_kv_heads, head_dim, v_dst,
                       lse_dst);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string("paged_cascade_gather_states: ") +
                                  hipGetErrorString(err));
    return PD_OK;
}
