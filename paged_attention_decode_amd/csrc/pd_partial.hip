// Split-KV partial attention over a CSR page table, for gfx950.
//
// Method: mlxcel PR #984 "fused paged-attention decode v2" (kernel commit and
// PR body item 2) and issue #898 items 1-2: one workgroup owns one (chunk, KV
// head) pair, reads each K/V element of its chunk once for every query head
// of the GQA group, scores in base 2 (log2 e folded into the scale) and emits
// a partial normalized by its own softmax denominator plus its LSE in log2
// units.  Page indirection follows the sparse-paged-decode doc,
// "Indirection": visible token i of request r is entry (fpo_r + i) %
// page_size of page indices[indptr[r] + (fpo_r + i) / page_size].
//
// gfx950 mapping (not the pages' Metal/CUDA shape):
//  - a K or V row of one head is D * sizeof(T) bytes; L = row_bytes / 16
//    lanes load it with one dwordx4 each, so a 64-lane wave covers R = 64 / L
//    token rows per load instruction (L = 16, R = 4 for fp16 D = 128);
//  - q . k partial sums are reduced inside each L-lane row with DPP
//    (quad_perm, row_half_mirror, row_mirror), leaving every lane of the row
//    with the same score;
//  - each row keeps its own online-softmax state (m, l, acc) per query head
//    and updates it once per J tokens; rows are combined with lane shuffles
//    and the four waves through LDS at the end;
//  - the chunk's page ids are staged in LDS once, so the per-token page
//    lookup is an LDS read rather than a dependent global load; the K/V loads
//    of the next step are in flight while the current step computes.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPageWindow = 1024;   // page ids staged in LDS per round

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

union Row16 {
    uint4 u;
    half2_t h2[4];
    _Float16 h[8];
    float f[4];
};

struct PartialArgs {
    const void *q;
    const void *k;
    const void *v;
    int64_t page_stride, token_stride, head_stride;
    const int32_t *indices, *indptr, *lpl, *fpo, *req_idx, *tile_idx;
    int32_t num_kv_heads, num_qo_heads, page_size, pages_per_chunk;
    FastDiv fd;
    float scale_log2;
    float *v_out;
    float *lse_out;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the L consecutive lanes of a row; every lane of the row ends with
// the same bits (each step adds the same two operands on both partners).
template <int L>
__device__ __forceinline__ float row_sum(float x)
{
    static_assert(L == 8 || L == 16 || L == 32, "row width");
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp<0x141>(x);   // row_half_mirror: lane ^ 7 inside 8
    if constexpr (L >= 16) x += dpp<0x140>(x);   // row_mirror: lane ^ 15 inside 16
    if constexpr (L == 32) x += __shfl_xor(x, 16);
    return x;
}

template <typename T>
struct Vec;
template <>
struct Vec<_Float16> {
    static constexpr int N = 8;
};
template <>
struct Vec<float> {
    static constexpr int N = 4;
};

template <typename T>
__device__ __forceinline__ float dot_row(const Row16 &q, const Row16 &k)
{
    if constexpr (sizeof(T) == 2) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s = __builtin_amdgcn_fdot2(q.h2[i], k.h2[i], s, false);
        return s;
    } else {
        float s = q.f[0] * k.f[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) s = fmaf(q.f[i], k.f[i], s);
        return s;
    }
}

template <typename T>
__device__ __forceinline__ float elem(const Row16 &v, int e)
{
    if constexpr (sizeof(T) == 2) return float(v.h[e]);
    else return v.f[e];
}

template <typename T, int D, int G, int J>
__global__ void __launch_bounds__(kThreads) partial_kernel(PartialArgs a)
{
    constexpr int VEC = Vec<T>::N;
    constexpr int L = D / VEC;        // lanes per token row
    constexpr int R = 64 / L;         // token rows per wave
    constexpr int TPS = R * J;        // tokens per wave step
    static_assert(L * VEC == D && R * L == 64, "shape");

    __shared__ int32_t s_pid[kPageWindow];
    __shared__ float s_acc[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];

    const int wg = blockIdx.x;
    const int n = wg / a.num_kv_heads;
    const int kvh = wg - n * a.num_kv_heads;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int row = lane / L;
    const int li = lane % L;

    const int r = a.req_idx[n];
    const int t = a.tile_idx[n];
    const int pbeg = a.indptr[r];
    const int npages = a.indptr[r + 1] - pbeg;
    const int fpo = a.fpo[r];
    const int ps = a.page_size;
    const int64_t nr = npages > 0 ? int64_t(npages - 1) * ps + a.lpl[r] - fpo : 0;
    const int64_t span = int64_t(a.pages_per_chunk) * ps;
    const int64_t tb = max(int64_t(0), int64_t(t) * span - fpo);
    const int64_t te = min(nr, int64_t(t + 1) * span - fpo);
    const int cp0 = t * a.pages_per_chunk;
    const int cp1 = min(npages, cp0 + a.pages_per_chunk);

    const T *qp = static_cast<const T *>(a.q) +
                  (int64_t(r) * a.num_qo_heads + int64_t(kvh) * G) * D + li * VEC;
    Row16 qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h].u = *reinterpret_cast<const uint4 *>(qp + h * D);

    const T *kbase = static_cast<const T *>(a.k) + int64_t(kvh) * a.head_stride + li * VEC;
    const T *vbase = static_cast<const T *>(a.v) + int64_t(kvh) * a.head_stride + li * VEC;

    float m[G], l[G], acc[G][VEC];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
    }

    for (int wp0 = cp0; wp0 < cp1; wp0 += kPageWindow) {
        const int wp1 = min(cp1, wp0 + kPageWindow);
        __syncthreads();
        for (int i = tid; i < wp1 - wp0; i += kThreads) s_pid[i] = a.indices[pbeg + wp0 + i];
        __syncthreads();
        const int64_t wtb = max(tb, int64_t(wp0) * ps - fpo);
        const int64_t wte = min(te, int64_t(wp1) * ps - fpo);
        const int ntok = int(max(int64_t(0), wte - wtb));
        const int nsteps = (ntok + TPS - 1) / TPS;

        auto load = [&](int s, Row16 (&kr)[J], Row16 (&vr)[J]) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                int tok = s * TPS + j * R + row;          // offset inside the window range
                tok = min(tok, ntok - 1);                 // clamp: masked later
                const uint32_t slot = uint32_t(fpo + wtb + tok);
                const uint32_t pi = fastdiv_q(a.fd, slot);
                const uint32_t e = slot - pi * uint32_t(ps);
                const int64_t pid = s_pid[int(pi) - wp0];
                const int64_t off = pid * a.page_stride + int64_t(e) * a.token_stride;
                kr[j].u = *reinterpret_cast<const uint4 *>(kbase + off);
                vr[j].u = *reinterpret_cast<const uint4 *>(vbase + off);
            }
        };

        auto compute = [&](int s, const Row16 (&kr)[J], const Row16 (&vr)[J]) {
            float sc[J][G];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const bool valid = s * TPS + j * R + row < ntok;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float x = row_sum<L>(dot_row<T>(qv[h], kr[j])) * a.scale_log2;
                    sc[j][h] = valid ? x : -INFINITY;
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float mx = m[h];
#pragma unroll
                for (int j = 0; j < J; ++j) mx = fmaxf(mx, sc[j][h]);
                const float ms = mx == -INFINITY ? 0.f : mx;
                const float alpha = fast_exp2(m[h] - ms);
                float p[J];
                float psum = 0.f;
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    p[j] = fast_exp2(sc[j][h] - ms);
                    psum += p[j];
                }
                l[h] = fmaf(l[h], alpha, psum);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float x = acc[h][e] * alpha;
#pragma unroll
                    for (int j = 0; j < J; ++j) x = fmaf(p[j], elem<T>(vr[j], e), x);
                    acc[h][e] = x;
                }
                m[h] = mx;
            }
        };

        Row16 k0[J], v0[J], k1[J], v1[J];
        int s = wave;
        if (s < nsteps) load(s, k0, v0);
        while (s < nsteps) {
            const int s1 = s + kWaves;
            if (s1 < nsteps) load(s1, k1, v1);
            compute(s, k0, v0);
            if (s1 >= nsteps) break;
            const int s2 = s1 + kWaves;
            if (s2 < nsteps) load(s2, k0, v0);
            compute(s1, k1, v1);
            s = s2;
        }
    }

    // combine the R rows of each wave (lanes li, li + L, ... hold the same dims)
#pragma unroll
    for (int off = L; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(m[h], off);
            const float lo = __shfl_xor(l[h], off);
            const float mx = fmaxf(m[h], mo);
            const float ms = mx == -INFINITY ? 0.f : mx;
            const float a1 = fast_exp2(m[h] - ms);
            const float a2 = fast_exp2(mo - ms);
            l[h] = l[h] * a1 + lo * a2;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float ao = __shfl_xor(acc[h][e], off);
                acc[h][e] = acc[h][e] * a1 + ao * a2;
            }
            m[h] = mx;
        }
    }
    if (row == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) s_acc[wave][h][li * VEC + e] = acc[h][e];
            if (li == 0) {
                s_m[wave][h] = m[h];
                s_l[wave][h] = l[h];
            }
        }
    }
    __syncthreads();
    const int64_t out_head0 = int64_t(n) * a.num_qo_heads + int64_t(kvh) * G;
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D;
        const int d = idx - h * D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
        const float ms = mx == -INFINITY ? 0.f : mx;
        float lsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = fast_exp2(s_m[w][h] - ms);
            lsum = fmaf(s_l[w][h], sc, lsum);
            o = fmaf(s_acc[w][h][d], sc, o);
        }
        a.v_out[(out_head0 + h) * D + d] = lsum > 0.f ? o / lsum : 0.f;
        if (d == 0) a.lse_out[out_head0 + h] = mx == -INFINITY ? -INFINITY : mx + fast_log2(lsum);
    }
}

template <typename T, int D, int G>
constexpr int tokens_per_row_step()
{
    return G <= 4 ? 4 : (G <= 8 ? 2 : 1);
}

using KernelFn = void (*)(PartialArgs);

template <typename T, int D>
KernelFn pick_g(int g)
{
    switch (g) {
    case 1: return partial_kernel<T, D, 1, tokens_per_row_step<T, D, 1>()>;
    case 2: return partial_kernel<T, D, 2, tokens_per_row_step<T, D, 2>()>;
    case 4: return partial_kernel<T, D, 4, tokens_per_row_step<T, D, 4>()>;
    case 8: return partial_kernel<T, D, 8, tokens_per_row_step<T, D, 8>()>;
    case 12: return partial_kernel<T, D, 12, tokens_per_row_step<T, D, 12>()>;
    case 16: return partial_kernel<T, D, 16, tokens_per_row_step<T, D, 16>()>;
    default: return nullptr;
    }
}

KernelFn pick_kernel(int dtype, int d, int g)
{
    if (dtype == PD_DTYPE_FP16) {
        if (d == 64) return pick_g<_Float16, 64>(g);
        if (d == 128) return pick_g<_Float16, 128>(g);
    } else if (dtype == PD_DTYPE_FP32) {
        if (d == 64) return pick_g<float, 64>(g);
        if (d == 128) return pick_g<float, 128>(g);
    }
    return nullptr;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace pd

using namespace pd;

extern "C" int paged_decode_partial(const void *q, const void *k_pool, const void *v_pool,
                                    int64_t page_stride, int64_t token_stride,
                                    int64_t head_stride, int32_t dtype,
                                    const int32_t *indices, const int32_t *indptr,
                                    const int32_t *last_page_len,
                                    const int32_t *first_page_offset,
                                    const int32_t *request_indices,
                                    const int32_t *kv_tile_indices, int32_t num_chunks,
                                    int32_t pages_per_chunk, int32_t batch,
                                    int32_t num_qo_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t page_size, float sm_scale,
                                    float *v_partial, float *lse_partial, void *stream)
{
    if (!q || !k_pool || !v_pool || !indices || !indptr || !last_page_len ||
        !first_page_offset || !request_indices || !kv_tile_indices || !v_partial ||
        !lse_partial)
        return fail(PD_E_NULL, "paged_decode_partial: null pointer");
    if (num_chunks < 0 || batch < 1 || pages_per_chunk < 1 || page_size < 1 ||
        num_kv_heads < 1 || num_qo_heads < 1 || num_qo_heads % num_kv_heads != 0 ||
        page_stride < 0 || token_stride < 0 || head_stride < 0 || !std::isfinite(sm_scale))
        return fail(PD_E_ARG, "paged_decode_partial: bad sizes or strides");
    if (int64_t(num_chunks) > PD_MAX_CHUNKS)
        return fail(PD_E_ARG, "paged_decode_partial: more chunks than the launch bound");
    const int g = num_qo_heads / num_kv_heads;
    KernelFn fn = pick_kernel(dtype, head_dim, g);
    if (!fn)
        return fail(PD_E_UNSUPPORTED, "paged_decode_partial: no kernel for this (dtype, D, group)");
    const int64_t esz = dtype == PD_DTYPE_FP16 ? 2 : 4;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (page_stride * esz) % 16 || (token_stride * esz) % 16 || (head_stride * esz) % 16)
        return fail(PD_E_UNSUPPORTED, "paged_decode_partial: q/pools need 16-byte alignment");
    if (!aligned16(v_partial))
        return fail(PD_E_UNSUPPORTED, "paged_decode_partial: v_partial needs 16-byte alignment");
    if (num_chunks == 0) return PD_OK;

    PartialArgs a;
    a.q = q;
    a.k = k_pool;
    a.v = v_pool;
    a.page_stride = page_stride;
    a.token_stride = token_stride;
    a.head_stride = head_stride;
    a.indices = indices;
    a.indptr = indptr;
    a.lpl = last_page_len;
    a.fpo = first_page_offset;
    a.req_idx = request_indices;
    a.tile_idx = kv_tile_indices;
    a.num_kv_heads = num_kv_heads;
    a.num_qo_heads = num_qo_heads;
    a.page_size = page_size;
    a.pages_per_chunk = pages_per_chunk;
    a.fd = make_fastdiv(uint32_t(page_size));
    a.scale_log2 = float(double(sm_scale) * 1.4426950408889634074);   // log2(e)
    a.v_out = v_partial;
    a.lse_out = lse_partial;

    const dim3 grid(uint32_t(int64_t(num_chunks) * num_kv_heads));
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string("paged_decode_partial: launch failed: ") +
                                  hipGetErrorString(err));
    return PD_OK;
}

extern "C" int paged_decode_default_target_wgs(int32_t device, int32_t group_size,
                                               int32_t head_dim, int32_t dtype)
{
    KernelFn fn = pick_kernel(dtype, head_dim, group_size);
    if (!fn) return fail(PD_E_UNSUPPORTED, "paged_decode_default_target_wgs: unsupported shape");
    int dev = device;
    if (dev < 0 && hipGetDevice(&dev) != hipSuccess)
        return fail(PD_E_HIP, "paged_decode_default_target_wgs: no current device");
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(PD_E_HIP, "paged_decode_default_target_wgs: cannot query CU count");
    int per_cu = 0;
    int prev = -1;
    hipGetDevice(&prev);
    hipSetDevice(dev);
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void *>(fn), kThreads, 0);
    if (prev >= 0) hipSetDevice(prev);
    if (e != hipSuccess || per_cu < 1)
        return fail(PD_E_HIP, "paged_decode_default_target_wgs: occupancy query failed");
    return cus * per_cu;
}
