// HBM read-stream probe, for gfx950: reads a buffer once with 16-byte
// loads and folds what it read into one word per workgroup (so
// the loads cannot be dropped).  Timed next to the decode kernels, it gives
// the read rate this GPU actually reaches, against which the decode's
// achieved bandwidth is compared.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "pd_device.h"
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 8;

// Workgroup b reads the contiguous segment [b*per, (b+1)*per) of 16-byte
// units; each iteration its threads read kProbeUnroll consecutive 8 KB
// blocks (64 KB in flight per workgroup).
template <bool NT>
__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const uint4 *__restrict__ buf,
                                                                   int64_t n16,
                                                                   uint32_t *__restrict__ sink)
{
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t beg = int64_t(blockIdx.x) * per;
    const int64_t end = min(n16, beg + per);
    uint32_t acc = 0;
    int64_t i = beg + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < end; i += kProbeUnroll * kProbeThreads) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = NT ? load_nt(buf + i + u * kProbeThreads) : buf[i + u * kProbeThreads];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += kProbeThreads) {
        const uint4 v = NT ? load_nt(buf + i) : buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t s_acc[kProbeThreads / 64];
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int w = 0; w < kProbeThreads / 64; ++w) x ^= s_acc[w];
        sink[blockIdx.x] = x;
    }
}

}  // namespace
}  // namespace pd

using namespace pd;

extern "C" int paged_hbm_read_probe(const void *buf, int64_t bytes, int32_t num_wgs,
                                    int32_t nontemporal, uint32_t *sink, void *stream)
{
    if (!buf || !sink) return fail(PD_E_NULL, "paged_hbm_read_probe: null pointer");
    if (bytes < 16 || bytes % 16 || num_wgs < 1)
        return fail(PD_E_ARG, "paged_hbm_read_probe: bytes must be a positive multiple of 16 "
                              "and num_wgs >= 1");
    if (reinterpret_cast<uintptr_t>(buf) & 15u)
        return fail(PD_E_UNSUPPORTED, "paged_hbm_read_probe: buffer needs 16-byte alignment");
    hipLaunchKernelGGL(nontemporal ? read_probe_kernel<true> : read_probe_kernel<false>,
                       dim3(uint32_t(num_wgs)), dim3(kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4 *>(buf),
                       bytes / 16, sink);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string("paged_hbm_read_probe: launch failed: ") +
                                  hipGetErrorString(err));
    return PD_OK;
}
