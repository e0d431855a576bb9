// Cascade head stacking, for gfx950.
//
// Method: mlxcel cascade-attention doc, "head stacking": the shared span is
// attended once as a single request whose query heads are the members'
// heads stacked so that stacked head h0 = kv*(M*G) + m*G + g is query head
// kv*G + g of member m (a [M, Hkv, G, D] -> [Hkv, M, G, D] transpose); the
// partial kernel's rule "query head h reads KV head h / group" then reads KV
// head kv.  The level-0 partial rows go back through the inverse transpose
// into each member's merge group, next to that member's own level-1 rows
// (rows placed by the host layout; a non-member's group is its level-1 rows
// alone), so a single merge pairing each member's states finishes the step.
// The merge can also apply the inverse transpose itself and read the rows
// where the launches wrote them (paged_cascade_merge_states); the copy here
// serves other head sizes.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pd_internal.h"

namespace pd {
namespace {

// one thread per 16-byte vector of a head row
__global__ void __launch_bounds__(256) stack_q_kernel(const uint4 *__restrict__ q,
                                                      const int32_t *__restrict__ member_req,
                                                      int members, int hkv, int g,
                                                      int vecs_per_row, uint4 *__restrict__ q0)
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
    const int64_t req = member_req ? member_req[m] : m;
    const int64_t h0 = (int64_t(kv) * members + m) * g + gi;
    q0[h0 * vecs_per_row + x] = q[((req * hkv + kv) * g + gi) * vecs_per_row + x];
}

// One workgroup per destination row, 16-byte copies.  Workgroups
// [0, n0*M) un-stack level-0 rows: workgroup (i, m) copies row i of stacked
// heads h0 = kv*(M*G) + m*G + g into row dst0[m] + i, heads kv*G + g.  The
// rest move level-1 row n to row dst1[n].  The destinations come from the
// host layout, which puts each request's level-0 rows (members only) before
// its level-1 rows.
__global__ void __launch_bounds__(256) gather_kernel(const float4 *__restrict__ v0,
                                                     const float *__restrict__ lse0, int n0,
                                                     int members, const int32_t *__restrict__ dst0,
                                                     const float4 *__restrict__ v1,
                                                     const float *__restrict__ lse1,
                                                     const int32_t *__restrict__ dst1, int hkv,
                                                     int g, int d4, float4 *__restrict__ v_dst,
                                                     float *__restrict__ lse_dst)
{
    const int b = blockIdx.x;
    const int hq = hkv * g;
    const int row_vecs = hq * d4;                 // 16-byte vectors of one [Hq, D] row
    if (b < n0 * members) {
        const int i = b / members;
        const int m = b - i * members;
        const int64_t src_row = int64_t(i) * members * hq;       // row i of [n0, M*Hq]
        const int64_t dst_row = (int64_t(dst0[m]) + i) * hq;
        for (int t = threadIdx.x; t < row_vecs; t += blockDim.x) {
            const int h = t / d4;
            const int x = t - h * d4;
            const int kv = h / g;
            const int h0 = (kv * members + m) * g + (h - kv * g);
            v_dst[(dst_row + h) * d4 + x] = v0[(src_row + h0) * d4 + x];
            if (x == 0) lse_dst[dst_row + h] = lse0[src_row + h0];
        }
    } else {
        const int n = b - n0 * members;
        const int64_t dst_row = int64_t(dst1[n]) * hq;
        const int64_t src_row = int64_t(n) * hq;
        for (int t = threadIdx.x; t < row_vecs; t += blockDim.x)
            v_dst[dst_row * d4 + t] = v1[src_row * d4 + t];
        for (int h = threadIdx.x; h < hq; h += blockDim.x) lse_dst[dst_row + h] = lse1[src_row + h];
    }
}

}  // namespace
}  // namespace pd

using namespace pd;

extern "C" int paged_cascade_stack_q(const void *q, int32_t dtype, const int32_t *member_req,
                                     int32_t members, int32_t num_qo_heads,
                                     int32_t num_kv_heads, int32_t head_dim, void *q0,
                                     void *stream)
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
                       static_cast<hipStream_t>(stream), static_cast<const uint4 *>(q),
                       member_req, members, num_kv_heads, g, vecs, static_cast<uint4 *>(q0));
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string("paged_cascade_stack_q: ") + hipGetErrorString(err));
    return PD_OK;
}

extern "C" int paged_cascade_gather_states(const float *v0, const float *lse0, int32_t n0,
                                           int32_t members, const int32_t *dst0, const float *v1,
                                           const float *lse1, int32_t n1, const int32_t *dst1,
                                           int32_t num_qo_heads, int32_t num_kv_heads,
                                           int32_t head_dim, float *v_dst, float *lse_dst,
                                           void *stream)
{
    if (!v_dst || !lse_dst || (n0 > 0 && (!v0 || !lse0 || !dst0)) ||
        (n1 > 0 && (!v1 || !lse1 || !dst1)))
        return fail(PD_E_NULL, "paged_cascade_gather_states: null pointer");
    if (n0 < 0 || n1 < 0 || members < 1 || num_kv_heads < 1 ||
        num_qo_heads % num_kv_heads != 0 || head_dim < 1)
        return fail(PD_E_ARG, "paged_cascade_gather_states: bad sizes");
    if (head_dim % 4 || (reinterpret_cast<uintptr_t>(v_dst) & 15u) ||
        (n0 > 0 && (reinterpret_cast<uintptr_t>(v0) & 15u)) ||
        (n1 > 0 && (reinterpret_cast<uintptr_t>(v1) & 15u)))
        return fail(PD_E_UNSUPPORTED,
                    "paged_cascade_gather_states: head_dim % 4 and 16-byte aligned rows needed");
    const int64_t blocks = int64_t(n0) * members + n1;
    if (blocks == 0) return PD_OK;
    if (blocks > INT32_MAX) return fail(PD_E_ARG, "paged_cascade_gather_states: too many rows");
    hipLaunchKernelGGL(gather_kernel, dim3(uint32_t(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<const float4 *>(v0),
                       lse0, n0, members, dst0, reinterpret_cast<const float4 *>(v1), lse1, dst1,
                       num_kv_heads, num_qo_heads / num_kv_heads, head_dim / 4,
                       reinterpret_cast<float4 *>(v_dst), lse_dst);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string("paged_cascade_gather_states: ") +
                                  hipGetErrorString(err));
    return PD_OK;
}
