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
// gfx950 mapping (not the pages' Metal/CUDA shape).  A K or V row of one head
// is D * sizeof(T) bytes; L = row_bytes / 16 lanes load it with one dwordx4
// each, so a 64-lane wave covers R = 64 / L token rows per load instruction.
// Two kernels share one epilogue:
//
//  * page kernel (rows of 256 B, i.e. L = 16: fp16 D = 128 or fp32 D = 64;
//    G in {4, 8, 16}; page_size a multiple of the 64/G slots of one step).
//    A wave step covers 64/G consecutive slots of ONE page, so the page id is
//    wave-uniform: it is read with readlane from a register holding the next
//    64 page ids of the chunk, and the load address is a scalar page base
//    plus a per-lane offset fixed for the whole kernel (no per-token division
//    or 64-bit multiply).  Each lane loads J = 16/G token
//    rows; the J*G = 16 partial dot products of a 16-lane row are
//    reduce-scattered with DPP so that lane i ends up owning the score of one
//    (token, head) pair; the softmax then runs once per score instead of on
//    all 16 lanes, and the probabilities reach the PV lanes by DPP
//    row_newbcast.  The running max is only raised when a block's max exceeds
//    it by more than 2^8 (probabilities stay <= 256 in between), so the
//    accumulator rescale is rare.  Slots outside the visible range (before
//    first_page_offset in the first page, from last_page_len on in the last)
//    get score -inf and V = 0, so whatever those entries hold is never used.
//
//  * token kernel (any D in {64, 128}, any G, any page_size): each lane
//    resolves its own token through a fast divide by page_size and the page
//    ids staged in LDS; partial dots are all-reduced inside the row with DPP.
//
// Epilogue: the R rows of a wave are combined (page kernel: a permlane
// reduce-scatter, after which each row holds a quarter of the heads; token
// kernel: lane shuffles), the waves that share a head through LDS, and the
// result is either written as the chunk's partial row, or -- in the fused
// mode -- written straight to the output when the request has one chunk, else
// written as a partial after which the last workgroup of the request (found
// with an agent-scope atomic counter that it resets to zero) merges the
// request's partial rows into the output.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <mutex>
#include <vector>

#include "pd_device.h"
#include "pd_internal.h"

namespace pd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPageWindow = 1024;     // token kernel: page ids staged in LDS per round
#ifndef PD_PIPELINE_DEPTH
#define PD_PIPELINE_DEPTH 2
#endif
constexpr int kDepth = PD_PIPELINE_DEPTH;   // page kernel: steps per wave in the load pipeline
// rounds of the load pipeline between the workgroup barriers that keep its
// waves (one per KV head) in lockstep, 0 for none.  Measured on MI355X with
// the MFMA kernel on the long-context geometry: every 2 or 3 rounds 63.96-
// 64.08 us, every round 64.19-64.26, every 4 rounds 64.10-64.23, never
// 65.47; G = 4 at page size 1 on the any-page kernel 68.07-68.14 against
// 68.47-68.70 every round.
#ifndef PD_LOCKSTEP_ROUNDS
#define PD_LOCKSTEP_ROUNDS 2
#endif
constexpr int kLockstep = PD_LOCKSTEP_ROUNDS;
constexpr float kLazyMargin = 8.0f;   // log2 units: p <= 2^8 between rescales
constexpr float kNoMax = -1e30f;      // finite "no score yet" running max
constexpr int kBufferWord3 = 0x00020000;   // gfx9 buffer descriptor dword 3 (32-bit data)
constexpr int kLoadNT = 2;                 // cache policy "nt": K/V rows are read exactly once

union Row16 {
    uint4 u;
    half2_t h2[4];
    _Float16 h[8];
    float f[4];
};

// Waits until every vector memory operation this thread issued, stores
// included, has completed (on gfx9 stores are counted by vmcnt).
__device__ __forceinline__ void wait_stores()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

struct PartialArgs {
    const void *q;
    const void *k;
    const void *v;
    int64_t page_stride, token_stride, head_stride;   // elements
    const int32_t *indices, *indptr, *lpl, *fpo, *req_idx, *tile_idx;
    int32_t num_kv_heads, num_qo_heads, page_size, pages_per_chunk;
    int32_t spp_log2;                                  // page kernel: steps per page = 2^spp_log2
    FastDiv fd;
    float scale_log2;
    float *v_out;        // partial rows [N, Hq, D]
    float *lse_out;      // [N, Hq]
    int32_t group;       // query heads per KV head of this launch (G = Hq / Hkv)
    // stacked launches (the cascade's shared level): the queries are read
    // where they lie in q [B, Hkv * q_group, D]; stacked head m*q_group + g
    // of KV head kv is query head kv*q_group + g of request q_members[m].
    // NULL: query head h of request r is row r*Hq + h.
    const int32_t *q_members;
    int32_t q_group;
    // fused mode
    float *o_final;      // [B, Hq, D]
    float *lse_final;    // [B, Hq]
    int32_t *counters;   // [B, Hkv], zero between launches
};

// Row of q (in D-element rows) holding query head h (0 <= h < G) of KV head
// kvh for request r of the launch.
__device__ __forceinline__ int64_t q_row(const PartialArgs &a, int r, int kvh, int G, int h)
{
    if (a.q_members) {
        const int m = h / a.q_group;
        const int g = h - m * a.q_group;
        return int64_t(a.q_members[m]) * (int64_t(a.num_kv_heads) * a.q_group) +
               int64_t(kvh) * a.q_group + g;
    }
    return int64_t(r) * a.num_qo_heads + int64_t(kvh) * G + h;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// DPP controls (gfx9 encoding)
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kRowHalfMirror = 0x141; // lane ^ 7 inside each 8 lanes
constexpr int kRowMirror = 0x140;     // lane ^ 15 inside each 16 lanes
constexpr int kRowRor4 = 0x124;       // lane (i + 4) mod 16 of the row
constexpr int kRowRor8 = 0x128;       // lane (i + 8) mod 16 of the row
template <int K>
__device__ __forceinline__ float row_bcast(float x)   // lane K of each 16-lane row
{
    return dpp<0x150 + K>(x);
}

// out[k] = lane k's x, in every lane of its 16-lane row (unused entries are
// dropped by the compiler)
__device__ __forceinline__ void row_bcast_all(float x, float (&out)[16])
{
    out[0] = row_bcast<0>(x);
    out[1] = row_bcast<1>(x);
    out[2] = row_bcast<2>(x);
    out[3] = row_bcast<3>(x);
    out[4] = row_bcast<4>(x);
    out[5] = row_bcast<5>(x);
    out[6] = row_bcast<6>(x);
    out[7] = row_bcast<7>(x);
    out[8] = row_bcast<8>(x);
    out[9] = row_bcast<9>(x);
    out[10] = row_bcast<10>(x);
    out[11] = row_bcast<11>(x);
    out[12] = row_bcast<12>(x);
    out[13] = row_bcast<13>(x);
    out[14] = row_bcast<14>(x);
    out[15] = row_bcast<15>(x);
}

// One level of the reduce-scatter combine of softmax states: the lane keeps
// state a (lower half / even row) or state b (upper half / odd row), merged
// with the same state of its partner lane.  Partners compute from the same
// (lower, upper) pair, so a state's two copies stay bit-identical.
template <bool HALVES, int VEC>
__device__ __forceinline__ void merge_level(float ma, float mb, float la, float lb,
                                            const float (&xa)[VEC], const float (&xb)[VEC],
                                            float &m, float &l, float (&x)[VEC])
{
    auto swap = [](float &u, float &v) {
        if constexpr (HALVES) swap32(u, v);
        else swap16(u, v);
    };
    swap(ma, mb);
    swap(la, lb);
    const float mx = fmaxf(ma, mb);
    const float s0 = fast_exp2(ma - mx);
    const float s1 = fast_exp2(mb - mx);
    m = mx;
    l = la * s0 + lb * s1;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        float u = xa[e], v = xb[e];
        swap(u, v);
        x[e] = u * s0 + v * s1;
    }
}

// Sum over the L consecutive lanes of a row; every lane of the row ends with
// the same bits (each step adds the same two operands on both partners).
template <int L>
__device__ __forceinline__ float row_sum(float x)
{
    static_assert(L == 8 || L == 16 || L == 32, "row width");
    x += dpp<kQuadXor1>(x);
    x += dpp<kQuadXor2>(x);
    x += dpp<kRowHalfMirror>(x);
    if constexpr (L >= 16) x += dpp<kRowMirror>(x);
    if constexpr (L == 32) x += __shfl_xor(x, 16);
    return x;
}

// Lane li of each 16-lane row holds x[0..15]; returns sum over the row's
// lanes of x[li].  Four halving steps; in each, the lane keeps the half of
// its values whose index bit matches its own lane bit and adds the partner's
// copy of that half (partners: lane ^ 8, lane ^ 7, lane ^ 2, lane ^ 1, which
// together span all 16 lanes).
__device__ __forceinline__ float reduce_scatter16(const float (&x)[16], int li)
{
    const bool b3 = li & 8, b2 = li & 4, b1 = li & 2, b0 = li & 1;
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float send = b3 ? x[k] : x[k + 8];
        const float keep = b3 ? x[k + 8] : x[k];
        y[k] = keep + dpp<kRowRor8>(send);
    }
    float z[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float send = b2 ? y[k] : y[k + 4];
        const float keep = b2 ? y[k + 4] : y[k];
        z[k] = keep + dpp<kRowHalfMirror>(send);
    }
    float w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float send = b1 ? z[k] : z[k + 2];
        const float keep = b1 ? z[k + 2] : z[k];
        w[k] = keep + dpp<kQuadXor2>(send);
    }
    const float send = b0 ? w[0] : w[1];
    const float keep = b0 ? w[1] : w[0];
    return keep + dpp<kQuadXor1>(send);
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

// Shared-memory image of the epilogue.
template <int G, int D>
struct EpilogueSmem {
    float acc[kWaves][G][D];
    float m[kWaves][G];
    float l[kWaves][G];
    int last;
};

// Combine the per-row states of the workgroup and store.  On entry every lane
// holds, for each head h of the group, the running max m[h] and denominator
// l[h] of its row (the same in all lanes of the row) and its VEC dims of the
// row's accumulator acc[h].
template <int G, int D, int L, bool FUSED>
__device__ __forceinline__ void epilogue(const PartialArgs &a, EpilogueSmem<G, D> &sm, float (&m)[G],
                                         float (&l)[G], float (&acc)[G][D / L], int n, int kvh,
                                         int r, int t, int npages)
{
    constexpr int VEC = D / L;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int row = lane / L;
    const int li = lane % L;
#pragma unroll
    for (int off = L; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(m[h], off);
            const float lo = __shfl_xor(l[h], off);
            const float mx = fmaxf(m[h], mo);
            const float a1 = fast_exp2(m[h] - mx);
            const float a2 = fast_exp2(mo - mx);
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
            for (int e = 0; e < VEC; ++e) sm.acc[wave][h][li * VEC + e] = acc[h][e];
            if (li == 0) {
                sm.m[wave][h] = m[h];
                sm.l[wave][h] = l[h];
            }
        }
    }
    __syncthreads();

    const int hq = a.num_qo_heads;
    const int64_t head0 = int64_t(kvh) * G;
    int ntiles = 1;
    if constexpr (FUSED) {
        const int c = a.pages_per_chunk;
        ntiles = npages > 0 ? (npages + c - 1) / c : 1;
    }
    // single-chunk requests in fused mode go straight to the output; a chunk
    // whose row another workgroup will merge is published with agent-scope
    // (cross-XCD coherent, "sc1") stores
    const bool direct = FUSED && ntiles == 1;
    const bool publish = FUSED && !direct;
    float *vdst = direct ? a.o_final + (int64_t(r) * hq + head0) * D
                         : a.v_out + (int64_t(n) * hq + head0) * D;
    float *ldst = direct ? a.lse_final + int64_t(r) * hq + head0 : a.lse_out + int64_t(n) * hq + head0;
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D;
        const int d = idx - h * D;
        float mx = sm.m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][h]);
        float lsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = fast_exp2(sm.m[w][h] - mx);
            lsum = fmaf(sm.l[w][h], sc, lsum);
            o = fmaf(sm.acc[w][h][d], sc, o);
        }
        const float ov = lsum > 0.f ? o / lsum : 0.f;
        const float lv = lsum > 0.f ? mx + fast_log2(lsum) : -INFINITY;
        if (publish) {
            __hip_atomic_store(vdst + int64_t(h) * D + d, ov, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (d == 0) __hip_atomic_store(ldst + h, lv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            vdst[int64_t(h) * D + d] = ov;
            if (d == 0) ldst[h] = lv;
        }
    }
    if constexpr (FUSED) {
        if (direct) return;
        // Every thread waits until its own coherent stores have completed
        // (vmcnt counts stores on gfx9), then the barrier, then one thread
        // counts the chunk.  A workgroup-scope fence would not do: on gfx950
        // it emits no vmcnt wait, so another wave's rows could still be in
        // flight when the count is added.  The workgroup that brings the
        // count to ntiles merges rows n - t .. n - t + ntiles - 1, reading
        // them with coherent loads, and resets the counter for the next
        // launch.
        //
        // Ordering: the rows and LSEs are written and read only with
        // agent-scope atomics, so no cache holds a stale copy; every
        // writer's stores have completed before the count is added, and the
        // merging workgroup's loads are issued after (and only because of)
        // the count it read.  The counter therefore needs no acquire or
        // release of its own, which on gfx950 would write back and
        // invalidate the whole L2 of the XCD.
        wait_stores();
        __syncthreads();
        int32_t *ctr = a.counters + int64_t(r) * a.num_kv_heads + kvh;
        if (tid == 0) {
            const int prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            sm.last = prev == ntiles - 1;
        }
        __syncthreads();
        if (!sm.last) return;
        const int64_t first = n - t;
        for (int idx = tid; idx < G * D; idx += kThreads) {
            const int h = idx / D;
            const int d = idx - h * D;
            const float *lrow = a.lse_out + first * hq + head0 + h;
            const float *vrow = a.v_out + (first * hq + head0 + h) * D + d;
            constexpr int U = 16;
            float mx = -INFINITY;
            for (int i0 = 0; i0 < ntiles; i0 += U) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = min(i0 + u, ntiles - 1);
                    mx = fmaxf(mx, __hip_atomic_load(lrow + int64_t(i) * hq, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
                }
            }
            float wsum = 0.f, o = 0.f;
            if (mx != -INFINITY) {
                for (int i0 = 0; i0 < ntiles; i0 += U) {
                    float x[U], vv[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int i = min(i0 + u, ntiles - 1);
                        x[u] = __hip_atomic_load(lrow + int64_t(i) * hq, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                        vv[u] = __hip_atomic_load(vrow + int64_t(i) * hq * D, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool live = i0 + u < ntiles && x[u] != -INFINITY;
                        const float w = live ? fast_exp2(x[u] - mx) : 0.f;
                        wsum += w;
                        o = live ? fmaf(w, vv[u], o) : o;
                    }
                }
            }
            a.o_final[(int64_t(r) * hq + head0 + h) * D + d] = wsum > 0.f ? o / wsum : 0.f;
            if (d == 0)
                a.lse_final[int64_t(r) * hq + head0 + h] = wsum > 0.f ? mx + fast_log2(wsum) : -INFINITY;
        }
        if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------- page kernel
// A workgroup holds HPW KV heads of one chunk with WPH waves per head (wave =
// hi * WPH + wp).  With HPW = 8, WPH = 1 the eight waves of a workgroup walk
// the same pages at the same time, each reading its head's rows, so every
// page of K and V is fetched as one 32 KB burst on one CU (DRAM rows are
// opened once per page instead of once per head).  Each wave is one (chunk,
// KV head) unit in the sense of the plan.
template <int G, int D, int HPW, int WPH>
struct PageSmem {
    float acc[WPH > 1 ? HPW * WPH : 1][G][WPH > 1 ? D : 1];
    float m[HPW * WPH][G];
    float l[HPW * WPH][G];
    int last;
};

template <typename T, int G, int HPW, int WPH, bool FUSED>
__global__ void __launch_bounds__(64 * HPW * WPH) partial_page_kernel(PartialArgs a)
{
    constexpr int NW = HPW * WPH;     // waves per workgroup
    constexpr int NT = 64 * NW;
    constexpr int VEC = Vec<T>::N;
    constexpr int L = 16;             // lanes per 256-byte row
    constexpr int R = 4;              // rows per wave
    constexpr int D = L * VEC;
    constexpr int J = 16 / G;         // token rows per lane per step
    constexpr int SPS = R * J;        // slots per step
    static_assert(J * G == 16 && J >= 1, "group");

    __shared__ PageSmem<G, D, HPW, WPH> sm;

    const int groups = a.num_kv_heads / HPW;
    const int wg = blockIdx.x;
    const int n = wg / groups;
    const int kvg = wg - n * groups;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
    const int hi = wave / WPH;
    const int wp = wave - hi * WPH;
    const int kvh = kvg * HPW + hi;
    const int lane = tid & 63;
    const int row = lane >> 4;
    const int li = lane & 15;

    const int r = ld_uniform(a.req_idx + n);
    const int t = ld_uniform(a.tile_idx + n);
    const int pbeg = ld_uniform(a.indptr + r);
    const int npages = ld_uniform(a.indptr + r + 1) - pbeg;
    const int fpo = ld_uniform(a.fpo + r);
    const int lpl = ld_uniform(a.lpl + r);
    const int ps = a.page_size;
    const int cp0 = t * a.pages_per_chunk;
    const int cp1 = min(npages, cp0 + a.pages_per_chunk);
    const int spp_log2 = a.spp_log2;

    // The page ids of the chunk are taken 64 at a time, one per lane of a
    // vector register (one load per wave; no LDS staging and no barrier), and
    // read out per step with readlane.  The load is bounded by a buffer
    // descriptor of the window's size: lanes past the window, and windows past
    // the chunk, read 0 and touch no memory, so the load is unconditional.
    auto load_ids = [&](int w0) -> int32_t {
        // (readfirstlane keeps the clamp scalar: as a VALU med3 the descriptor
        // would land in vector registers)
        const int cnt = __builtin_amdgcn_readfirstlane(max(0, min(cp1 - w0, 64)));
        const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t *>(a.indices) + pbeg + w0, 0, cnt * 4, kBufferWord3);
        return int32_t(__builtin_amdgcn_raw_buffer_load_b32(ri, lane * 4, 0, 0));
    };
    // issued before the query rows: loads complete in order, so the first K/V
    // loads then wait for the page ids alone
    int32_t idv = load_ids(cp0);

    Row16 qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
        qv[h].u = *reinterpret_cast<const uint4 *>(static_cast<const T *>(a.q) +
                                                   q_row(a, r, kvh, G, h) * D + li * VEC);

    constexpr int ESZ = sizeof(T);
    const char *kb = static_cast<const char *>(a.k) + int64_t(kvh) * a.head_stride * ESZ;
    const char *vb = static_cast<const char *>(a.v) + int64_t(kvh) * a.head_stride * ESZ;
    const int64_t page_bytes = a.page_stride * ESZ;
    const uint32_t step_bytes = uint32_t(a.token_stride * ESZ * SPS);
    // bytes of one page that this KV head's rows span: loads are buffer loads
    // bounded by it (an offset past it would read 0, never another page)
    const int32_t page_span = int32_t(int64_t(ps - 1) * a.token_stride * ESZ + D * ESZ);
    int32_t lane_off[J];
#pragma unroll
    for (int j = 0; j < J; ++j)
        lane_off[j] = int32_t((j * R + row) * a.token_stride * ESZ) + li * 16;

    float m_run = kNoMax;             // running max of head (li % G) of this row
    float l_part = 0.f;               // denominator share of this lane's (token, head)
    float acc[G][VEC];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;

    const int j_own = li / G;         // the token row this lane scores

    for (int wp0 = cp0; wp0 < cp1; wp0 += 64) {
        const int wcount = min(cp1 - wp0, 64);
        const int32_t idn = load_ids(wp0 + 64);    // the next window's ids, one window ahead
        const int nsteps = wcount << spp_log2;

        // Loads are issued unconditionally so that the wait before each
        // step's compute only covers that step's loads (a load under a
        // branch makes the wait count conservative, i.e. wait for all).  A
        // step past the end gets a zero-size buffer: its loads return zeros
        // and touch no memory.
        auto load = [&](int s, Row16 (&kr)[J], Row16 (&vr)[J]) {
            const bool live = s < nsteps;
            const int p = min(s >> spp_log2, wcount - 1);
            const int sub = s & ((1 << spp_log2) - 1);
            const int pid = __builtin_amdgcn_readlane(idv, p);
            const int64_t base = int64_t(pid) * page_bytes;
            const int32_t span = live ? page_span : 0;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(kb + base), 0, span, kBufferWord3);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(vb + base), 0, span, kBufferWord3);
            const int soff = int(sub * step_bytes);
#pragma unroll
            for (int j = 0; j < J; ++j) {
                kr[j].u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off[j], soff, kLoadNT));
                vr[j].u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off[j], soff, kLoadNT));
            }
        };

        auto compute = [&](int s, const Row16 (&kr)[J], Row16 (&vr)[J]) {
            const int p = wp0 + (s >> spp_log2);          // request-relative page
            const int sub = s & ((1 << spp_log2) - 1);
            float x[16];
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int h = 0; h < G; ++h) x[j * G + h] = dot_row<T>(qv[h], kr[j]);
            float sc = reduce_scatter16(x, li) * a.scale_log2;
            // slots outside the visible range: first page before fpo, last
            // page from lpl on
            const bool edge = (p == 0 && fpo > 0) || (p == npages - 1 && lpl < ps);
            if (edge) {
                const int lo = p == 0 ? fpo : 0;
                const int hi_slot = p == npages - 1 ? lpl : ps;
                const int slot_own = sub * SPS + j_own * R + row;
                sc = (slot_own >= lo && slot_own < hi_slot) ? sc : -INFINITY;
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const int slot = sub * SPS + j * R + row;
                    const bool ok = slot >= lo && slot < hi_slot;
                    vr[j].u.x = ok ? vr[j].u.x : 0u;
                    vr[j].u.y = ok ? vr[j].u.y : 0u;
                    vr[j].u.z = ok ? vr[j].u.z : 0u;
                    vr[j].u.w = ok ? vr[j].u.w : 0u;
                }
            }
            // block max over the J lanes that hold the same head
            float mb = sc;
            if constexpr (J >= 2) mb = fmaxf(mb, dpp<G == 8 ? kRowRor8 : kRowRor4>(mb));
            if constexpr (J == 4) mb = fmaxf(mb, dpp<kRowRor8>(mb));
            const bool need = mb > m_run + kLazyMargin;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float m_new = need ? mb : m_run;
                const float alpha = fast_exp2(m_run - m_new);
                l_part *= alpha;
                m_run = m_new;
                float ab[16];            // lane h of the row holds head h
                row_bcast_all(alpha, ab);
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[h][e] *= ab[h];
            }
            const float pl = fast_exp2(sc - m_run);
            l_part += pl;
            float pb[16];                // p of (token j, head h) is in lane j*G + h
            row_bcast_all(pl, pb);
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float y = acc[h][e];
#pragma unroll
                    for (int j = 0; j < J; ++j) y = fmaf(pb[j * G + h], elem<T>(vr[j], e), y);
                    acc[h][e] = y;
                }
        };

        // software pipeline: the loads of this wave's next kDepth-1 steps
        // are in flight while a step computes
        Row16 kbuf[kDepth][J], vbuf[kDepth][J];
        int s = wp;
#pragma unroll
        for (int d = 0; d < kDepth - 1; ++d) load(s + d * WPH, kbuf[d], vbuf[d]);
        // Every wave runs the same number of rounds (the step count is
        // uniform over the workgroup), so the waves can be held in lockstep
        // by a barrier every kLockstep rounds.  Without it the SIMD issues
        // the older of its two waves first: waves 0..3 end their pages long
        // before waves 4..7, and for the rest of the chunk the CU streams
        // with half its waves.  The barrier orders no memory, so it is the
        // bare instruction: the loads in flight stay in flight across it.
        const int rounds = (nsteps + WPH * kDepth - 1) / (WPH * kDepth);
        for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
            for (int u = 0; u < kDepth; ++u) {
                load(s + (kDepth - 1) * WPH, kbuf[(u + kDepth - 1) % kDepth],
                     vbuf[(u + kDepth - 1) % kDepth]);
                if (s < nsteps) compute(s, kbuf[u], vbuf[u]);
                s += WPH;
            }
            if constexpr (kLockstep > 0 && NW > 1) {
                constexpr int every = kLockstep > 0 ? kLockstep : 1;
                if (rd % every == every - 1) __builtin_amdgcn_s_barrier();
            }
        }
        idv = idn;
    }

    // per-row state for every head: head h lives in lanes li = h (mod G); the
    // J lanes of a head share m_run and split l
    float lsum = l_part;
    if constexpr (J >= 2) lsum += dpp<G == 8 ? kRowRor8 : kRowRor4>(lsum);
    if constexpr (J == 4) lsum += dpp<kRowRor8>(lsum);
    float m[G], l[G];
    {
        float tm[16], tl[16];
        row_bcast_all(m_run, tm);
        row_bcast_all(lsum, tl);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m[h] = tm[h];
            l[h] = tl[h];
        }
    }
    // Combine the four rows of the wave (same head, same dims in lanes li,
    // li + 16, li + 32, li + 48) as a reduce-scatter: the halves split the G
    // heads in two, then the row pairs split each half again, so row rho
    // ends with the combined state of heads rho * G/4 .. rho * G/4 + G/4 - 1.
    constexpr int G2 = G / 2, G4 = G / 4;
    float m1[G2], l1[G2], acc1[G2][VEC];
#pragma unroll
    for (int k = 0; k < G2; ++k)
        merge_level<true>(m[k], m[k + G2], l[k], l[k + G2], acc[k], acc[k + G2], m1[k], l1[k], acc1[k]);
    float m2[G4], l2[G4], acc2[G4][VEC];
#pragma unroll
    for (int k = 0; k < G4; ++k)
        merge_level<false>(m1[k], m1[k + G4], l1[k], l1[k + G4], acc1[k], acc1[k + G4], m2[k], l2[k],
                           acc2[k]);
    const int h_row = row * G4;       // first head of this row

    const int hq = a.num_qo_heads;
    int ntiles = 1;
    if constexpr (FUSED) {
        const int c = a.pages_per_chunk;
        ntiles = npages > 0 ? (npages + c - 1) / c : 1;
    }
    const bool direct = FUSED && ntiles == 1;
    const bool publish = FUSED && !direct;
    const int64_t head_lo = int64_t(kvg) * HPW * G;      // first query head of the workgroup
    float *vrow = direct ? a.o_final + int64_t(r) * hq * D : a.v_out + int64_t(n) * hq * D;
    float *lrow = direct ? a.lse_final + int64_t(r) * hq : a.lse_out + int64_t(n) * hq;
    auto put = [&](int64_t qh, int d, float ov, bool with_lse, float lv) {
        if (publish) {
            __hip_atomic_store(vrow + qh * D + d, ov, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (with_lse) __hip_atomic_store(lrow + qh, lv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            vrow[qh * D + d] = ov;
            if (with_lse) lrow[qh] = lv;
        }
    };

    if constexpr (WPH == 1) {
        // each wave owns its KV head; every row writes the heads it holds
#pragma unroll
        for (int k = 0; k < G4; ++k) {
            const float inv = l2[k] > 0.f ? 1.f / l2[k] : 0.f;
            const float lv = l2[k] > 0.f ? m2[k] + fast_log2(l2[k]) : -INFINITY;
            const int64_t qh = int64_t(kvh) * G + h_row + k;
#pragma unroll
            for (int e = 0; e < VEC; ++e) put(qh, li * VEC + e, acc2[k][e] * inv, e == 0 && li == 0, lv);
        }
    } else {
#pragma unroll
        for (int k = 0; k < G4; ++k) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) sm.acc[wave][h_row + k][li * VEC + e] = acc2[k][e];
            if (li == 0) {
                sm.m[wave][h_row + k] = m2[k];
                sm.l[wave][h_row + k] = l2[k];
            }
        }
        __syncthreads();
        for (int idx = tid; idx < HPW * G * D; idx += NT) {
            const int hh = idx / D;               // hi * G + h
            const int d = idx - hh * D;
            const int hw = hh / G;
            const int h = hh - hw * G;
            float mx = sm.m[hw * WPH][h];
#pragma unroll
            for (int w = 1; w < WPH; ++w) mx = fmaxf(mx, sm.m[hw * WPH + w][h]);
            float lsum2 = 0.f, o = 0.f;
#pragma unroll
            for (int w = 0; w < WPH; ++w) {
                const float sc = fast_exp2(sm.m[hw * WPH + w][h] - mx);
                lsum2 = fmaf(sm.l[hw * WPH + w][h], sc, lsum2);
                o = fmaf(sm.acc[hw * WPH + w][h][d], sc, o);
            }
            put(head_lo + hh, d, lsum2 > 0.f ? o / lsum2 : 0.f, d == 0,
                lsum2 > 0.f ? mx + fast_log2(lsum2) : -INFINITY);
        }
    }

    if constexpr (FUSED) {
        if (direct) return;
        // Every thread waits until its own coherent stores have completed,
        // then one thread counts the chunk.  The workgroup that brings the
        // count to ntiles merges rows n - t .. n - t + ntiles - 1 for its
        // heads, reading them with coherent loads, and resets the counter.
        // (The ordering argument is the one in epilogue(), above.)
        wait_stores();
        __syncthreads();
        int32_t *ctr = a.counters + int64_t(r) * a.num_kv_heads + kvg;
        if (tid == 0) {
            const int prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            sm.last = prev == ntiles - 1;
        }
        __syncthreads();
        if (!sm.last) return;
        const int64_t first = n - t;
        for (int idx = tid; idx < HPW * G * D; idx += NT) {
            const int64_t qh = head_lo + idx / D;
            const int d = idx % D;
            const float *lr = a.lse_out + first * hq + qh;
            const float *vr = a.v_out + (first * hq + qh) * D + d;
            constexpr int U = 16;
            float mx = -INFINITY;
            for (int i0 = 0; i0 < ntiles; i0 += U) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = min(i0 + u, ntiles - 1);
                    mx = fmaxf(mx, __hip_atomic_load(lr + int64_t(i) * hq, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
                }
            }
            float wsum = 0.f, o = 0.f;
            if (mx != -INFINITY) {
                for (int i0 = 0; i0 < ntiles; i0 += U) {
                    float x[U], vv[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int i = min(i0 + u, ntiles - 1);
                        x[u] = __hip_atomic_load(lr + int64_t(i) * hq, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                        vv[u] = __hip_atomic_load(vr + int64_t(i) * hq * D, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool live = i0 + u < ntiles && x[u] != -INFINITY;
                        const float w = live ? fast_exp2(x[u] - mx) : 0.f;
                        wsum += w;
                        o = live ? fmaf(w, vv[u], o) : o;
                    }
                }
            }
            a.o_final[(int64_t(r) * hq + qh) * D + d] = wsum > 0.f ? o / wsum : 0.f;
            if (d == 0)
                a.lse_final[int64_t(r) * hq + qh] = wsum > 0.f ? mx + fast_log2(wsum) : -INFINITY;
        }
        if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// --------------------------------------------------------------- token kernel
template <typename T, int D, int G, int J, bool FUSED>
__global__ void __launch_bounds__(kThreads) partial_token_kernel(PartialArgs a)
{
    constexpr int VEC = Vec<T>::N;
    constexpr int L = D / VEC;        // lanes per token row
    constexpr int R = 64 / L;         // token rows per wave
    constexpr int TPS = R * J;        // tokens per wave step
    static_assert(L * VEC == D && R * L == 64, "shape");

    __shared__ int32_t s_pid[kPageWindow];
    __shared__ EpilogueSmem<G, D> sm;

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

    Row16 qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
        qv[h].u = *reinterpret_cast<const uint4 *>(static_cast<const T *>(a.q) +
                                                   q_row(a, r, kvh, G, h) * D + li * VEC);

    const T *kbase = static_cast<const T *>(a.k) + int64_t(kvh) * a.head_stride + li * VEC;
    const T *vbase = static_cast<const T *>(a.v) + int64_t(kvh) * a.head_stride + li * VEC;

    float m[G], l[G], acc[G][VEC];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNoMax;
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
                kr[j].u = load_nt(kbase + off);
                vr[j].u = load_nt(vbase + off);
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
                const float alpha = fast_exp2(m[h] - mx);
                float p[J];
                float psum = 0.f;
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    p[j] = fast_exp2(sc[j][h] - mx);
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

        // loads issued unconditionally (rows past the end are clamped to the
        // last token) so that each wait covers only the step it feeds
        Row16 k0[J], v0[J], k1[J], v1[J];
        int s = wave;
        if (s < nsteps) load(s, k0, v0);
        while (s < nsteps) {
            const int s1 = s + kWaves;
            load(s1, k1, v1);
            compute(s, k0, v0);
            if (s1 >= nsteps) break;
            const int s2 = s1 + kWaves;
            load(s2, k0, v0);
            compute(s1, k1, v1);
            s = s2;
        }
    }
    epilogue<G, D, L, FUSED>(a, sm, m, l, acc, n, kvh, r, t, npages);
}

// ------------------------------------------------------------------- dispatch
using KernelFn = void (*)(PartialArgs);

template <int G>
constexpr int token_rows_per_step()
{
    return G <= 4 ? 4 : (G <= 8 ? 2 : 1);
}

// ----------------------------------------------------------------- MFMA kernel
// fp16 with head dim D in {64, 128}: the scores and the value sum as dense
// products on the matrix cores.  A tile of 16 tokens of one KV head against
// the group's queries is S^T [16 tokens x 16 heads] = K [16 x D] . Q^T
// [D x 16]: D/32 v_mfma_f32_16x16x32_f16.  The value sum is taken
// transposed, O^T [16 dims x 16 heads] += V^T [16 dims x 16 tokens] . P^T
// [16 tokens x 16 heads]: one v_mfma_f32_16x16x32_f16 per 16 dims, whose
// K = 32 holds each token twice -- once with p rounded to fp16, once with
// the rounding's remainder -- so that P enters the product with about 22
// bits, not fp16's 11 (the softmax weights stay fp32 arithmetic, as the
// fp16 path's products and sums are).  Groups under 16 heads are
// zero-padded 16-head tiles: the kernel streams K/V at the same rate.
//
// Lane layouts of the 16x16xK products (checked on gfx950): A [M x K] --
// lane l holds row l%16, k = (K/4)*(l/16) + e; B [K x N] -- lane l holds
// column l%16, the same k; C [M x N] -- lane l holds column l%16, rows
// 4*(l/16) + i.  With S^T in C layout, lane l holds head l%16 for tokens
// 4*(l/16) + i: that is P^T's B layout for the value product, and O^T's C
// layout puts the same head in lane l.  So a lane owns one head's running
// max and sum and D/4 of its output dims, and a rescale is a per-lane
// scalar.
//
// K and V are loaded by rows: each load instruction reads whole rows of
// 2*D bytes (D/8 lanes of 16 bytes per row: 4 rows at D = 128, 8 at
// D = 64), and the rows go to the wave's LDS tiles.  K's A operand (lane l:
// token l%16, 16 bytes at dims 8*(l/16) + 32*kc) is read back with
// ds_read_b128.  Loading it straight into the operand layout reads 16 rows
// x 64 bytes per instruction, twice the cache lines per request: measured
// on MI355X at D = 128 and G = 8 that took the long-context partial from
// 65.6 to 67.1 us, and the any-page variant at page size 1 from 68.7 to
// 72.5 us.  V^T's A operand (4 tokens of one dim per lane) is read from the
// V tile with the gfx950 transpose read ds_read_b64_tr_b16: in each 16-lane
// group, lanes 4r..4r+3 name 4 consecutive halves each (together row r of a
// 4 x 16 tile) and lane c receives column c.  Each wave has its own LDS
// tiles, rows padded by 16 bytes against bank conflicts.
template <int D>
struct MfmaShape {
    static_assert(D == 64 || D == 128, "MFMA kernels: head dim 64 or 128");
    static constexpr int KC = D / 32;            // K-steps of the score product
    static constexpr int DT = D / 16;            // 16-dim tiles of the value product
    static constexpr int RB = 2 * D + 16;        // LDS bytes per tile row
    static constexpr int LPR = D / 8;            // lanes per row of a row load
    static constexpr int RPI = 64 / LPR;         // rows per load instruction
    static constexpr int NJ = 16 / RPI;          // load instructions per 16-row tile
    static constexpr int TILE_BYTES = 32 * RB;   // per wave: V tile, then K tile
};

// Q^T as the B operand of the score product: lane l holds head 16*ht + l%16
// (zero past G) at dims 32*kc + 8*(l/16) .. + 7
template <int D, int HT>
__device__ __forceinline__ void mfma_load_q(const PartialArgs &a, int r, int kvh, int G,
                                            int lane, half8_t (&qb)[HT][MfmaShape<D>::KC])
{
    const int grp = lane >> 4;
    const int col = lane & 15;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = ht * 16 + col;
        const _Float16 *qp = static_cast<const _Float16 *>(a.q) +
                             q_row(a, r, kvh, G, min(h, G - 1)) * D + 8 * grp;
#pragma unroll
        for (int kc = 0; kc < MfmaShape<D>::KC; ++kc) {
            const uint4 u = *reinterpret_cast<const uint4 *>(qp + 32 * kc);
            qb[ht][kc] = h < G ? __builtin_bit_cast(half8_t, u) : half8_t{};
        }
    }
}

// One 16-token tile of one KV head.  kr / vr: the tile's K and V rows as
// loaded (load j, lane l: row l/(D/8) + (64/(D/8))*j, bytes 16*(l%(D/8))).
// vis(i) says whether tile token i is visible; it is asked only on an edge
// tile.  Hidden tokens get zero V rows (whatever they hold never reaches the
// sum) and -inf scores.
template <int D, int HT, typename Vis>
__device__ __forceinline__ void mfma_tile(const uint4 (&kr)[MfmaShape<D>::NJ],
                                          const uint4 (&vr)[MfmaShape<D>::NJ], bool edge,
                                          Vis vis, char *vt, float scale_log2,
                                          const half8_t (&qb)[HT][MfmaShape<D>::KC],
                                          float (&m_run)[HT], float (&l_part)[HT],
                                          float4_t (&acc)[HT][MfmaShape<D>::DT], int lane)
{
    using S = MfmaShape<D>;
    const int grp = lane >> 4;
    const int col = lane & 15;
    const int lrow = lane / S::LPR;
    const int lpc = lane % S::LPR;
    char *kt = vt + 16 * S::RB;
#pragma unroll
    for (int j = 0; j < S::NJ; ++j) {
        const int row = lrow + S::RPI * j;
        uint4 v = vr[j];
        if (edge) {
            const bool ok = vis(row);
            v.x = ok ? v.x : 0u;
            v.y = ok ? v.y : 0u;
            v.z = ok ? v.z : 0u;
            v.w = ok ? v.w : 0u;
        }
        *reinterpret_cast<uint4 *>(vt + row * S::RB + 16 * lpc) = v;
        *reinterpret_cast<uint4 *>(kt + row * S::RB + 16 * lpc) = kr[j];
    }
    // the rows written above are read back below by the same wave: LDS
    // operations of a wave complete in order, so only the compiler must keep
    // them in order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    uint4 kf[S::KC];
#pragma unroll
    for (int kc = 0; kc < S::KC; ++kc)
        kf[kc] = *reinterpret_cast<const uint4 *>(kt + col * S::RB + 16 * grp + 64 * kc);
    // scores S^T = K . Q^T, per 16-head tile
    float4_t sc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        sc[ht] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < S::KC; ++kc)
            sc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, kf[kc]),
                                                            qb[ht][kc], sc[ht], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // V^T, 16 dims at a time: row 4*(l/16) + (l%16)/4, halves 16*dt + 4*(l%4)
    typedef __attribute__((address_space(3))) short4_t lds_short4;
    const int tr_off = (4 * grp + (col >> 2)) * S::RB + 8 * (lane & 3);
    half4_t vtr[S::DT];
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
        vtr[dt] = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                  (lds_short4 *)(vt + tr_off + 32 * dt)));
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        float x[4];
        float mb = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = sc[ht][i] * scale_log2;
            if (edge) v = vis(4 * grp + i) ? v : -INFINITY;
            x[i] = v;
            mb = fmaxf(mb, v);
        }
        mb = group_max4(mb);                       // over the tile's 16 tokens
        const bool need = mb > m_run[ht] + kLazyMargin;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float m_new = need ? mb : m_run[ht];
            const float alpha = fast_exp2(m_run[ht] - m_new);
            m_run[ht] = m_new;
            l_part[ht] *= alpha;
#pragma unroll
            for (int dt = 0; dt < S::DT; ++dt) acc[ht][dt] *= alpha;
        }
        // P^T in two fp16 parts: k = 8*(l/16) + e holds, for token
        // 4*(l/16) + e%4, p rounded to fp16 (e < 4) or the remainder
        // p - that, rounded to fp16 (e >= 4); the A operand repeats the
        // token's V^T for both.  The product then carries p to about 22
        // bits, the sum takes p itself, and the K = 32 product takes as
        // long as the K = 16 one it replaces.
        half8_t pb;
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(x[i] - m_run[ht]);
            const _Float16 ph = _Float16(p);
            pb[i] = ph;
            pb[4 + i] = _Float16(p - float(ph));
            ls += p;
        }
        l_part[ht] += ls;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) {
            const half8_t va = __builtin_shufflevector(vtr[dt], vtr[dt], 0, 1, 2, 3, 0, 1, 2, 3);
            acc[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, acc[ht][dt], 0, 0, 0);
        }
    }
}

// per head: the sum over the four 16-lane groups; each group holds 4 of
// every 16 dims, so the accumulators need no combine
template <int D, int HT>
__device__ __forceinline__ void mfma_epilogue(const PartialArgs &a, int n, int kvh, int G,
                                              int lane, const float (&m_run)[HT],
                                              const float (&l_part)[HT],
                                              const float4_t (&acc)[HT][MfmaShape<D>::DT])
{
    const int grp = lane >> 4;
    const int col = lane & 15;
    const int hq = a.num_qo_heads;
    float *vrow = a.v_out + int64_t(n) * hq * D;
    float *lrow = a.lse_out + int64_t(n) * hq;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const float l = group_sum4(l_part[ht]);
        const int h = ht * 16 + col;
        if (h >= G) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int64_t qh = int64_t(kvh) * G + h;
#pragma unroll
        for (int dt = 0; dt < MfmaShape<D>::DT; ++dt) {
            const float4_t o = acc[ht][dt] * inv;
            *reinterpret_cast<float4 *>(vrow + qh * D + 16 * dt + 4 * grp) =
                make_float4(o[0], o[1], o[2], o[3]);
        }
        if (grp == 0) lrow[qh] = l > 0.f ? m_run[ht] + fast_log2(l) : -INFINITY;
    }
}

// The page-tiled kernel: a step is a 16-token tile of one page.  The group
// size G = a.group is a run-time value up to 16 * HT (heads past G are zero
// columns of the 16-head tiles), so one instantiation serves every group of
// its tile count, and a pair launch can run two tables of different groups.
template <int D, int HT, int HPW>
__device__ __forceinline__ void mfma_body(const PartialArgs &a, int wg,
                                          char (&s_v)[HPW][MfmaShape<D>::TILE_BYTES])
{
    using S = MfmaShape<D>;
    constexpr int ESZ = 2;
    const int G = a.group;

    const int groups = a.num_kv_heads / HPW;
    const int n = wg / groups;
    const int kvg = wg - n * groups;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kvh = kvg * HPW + wave;
    const int lane = tid & 63;

    const int r = ld_uniform(a.req_idx + n);
    const int t = ld_uniform(a.tile_idx + n);
    const int pbeg = ld_uniform(a.indptr + r);
    const int npages = ld_uniform(a.indptr + r + 1) - pbeg;
    const int fpo = ld_uniform(a.fpo + r);
    const int lpl = ld_uniform(a.lpl + r);
    const int ps = a.page_size;
    const int cp0 = t * a.pages_per_chunk;
    const int cp1 = min(npages, cp0 + a.pages_per_chunk);
    const int spp_log2 = a.spp_log2;    // 16-token tiles per page = 2^spp_log2

    auto load_ids = [&](int w0) -> int32_t {
        const int cnt = __builtin_amdgcn_readfirstlane(max(0, min(cp1 - w0, 64)));
        const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t *>(a.indices) + pbeg + w0, 0, cnt * 4, kBufferWord3);
        return int32_t(__builtin_amdgcn_raw_buffer_load_b32(ri, lane * 4, 0, 0));
    };
    int32_t idv = load_ids(cp0);

    half8_t qb[HT][S::KC];
    mfma_load_q<D, HT>(a, r, kvh, G, lane, qb);

    const char *kb = static_cast<const char *>(a.k) + int64_t(kvh) * a.head_stride * ESZ;
    const char *vb = static_cast<const char *>(a.v) + int64_t(kvh) * a.head_stride * ESZ;
    const int64_t page_bytes = a.page_stride * ESZ;
    const int32_t tsb = int32_t(a.token_stride * ESZ);
    const uint32_t tile_bytes = uint32_t(tsb) * 16u;
    const int32_t page_span = int32_t(int64_t(ps - 1) * a.token_stride * ESZ + D * ESZ);
    // load j, lane l: row l/(D/8) + (64/(D/8))*j at bytes 16*(l%(D/8))
    const int32_t row_off = (lane / S::LPR) * tsb + 16 * (lane % S::LPR);

    // per 16-head tile: the lane's head's running max and its share of the sum
    float m_run[HT], l_part[HT];
    float4_t acc[HT][S::DT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        m_run[ht] = kNoMax;
        l_part[ht] = 0.f;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) acc[ht][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    char *vt = s_v[wave];

    for (int wp0 = cp0; wp0 < cp1; wp0 += 64) {
        const int wcount = min(cp1 - wp0, 64);
        const int32_t idn = load_ids(wp0 + 64);    // the next window's ids, one window ahead
        const int nsteps = wcount << spp_log2;

        auto load = [&](int s, uint4 (&kr)[S::NJ], uint4 (&vr)[S::NJ]) {
            const bool live = s < nsteps;
            const int p = min(s >> spp_log2, wcount - 1);
            const int sub = s & ((1 << spp_log2) - 1);
            const int pid = __builtin_amdgcn_readlane(idv, p);
            const int64_t base = int64_t(pid) * page_bytes;
            const int32_t span = live ? page_span : 0;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(kb + base), 0, span, kBufferWord3);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(vb + base), 0, span, kBufferWord3);
            const int soff = int(sub * tile_bytes);
#pragma unroll
            for (int j = 0; j < S::NJ; ++j) {
                const int32_t off = row_off + S::RPI * j * tsb;
                kr[j] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, soff, kLoadNT));
                vr[j] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, soff, kLoadNT));
            }
        };

        auto compute = [&](int s, const uint4 (&kr)[S::NJ], const uint4 (&vr)[S::NJ]) {
            const int p = wp0 + (s >> spp_log2);          // request-relative page
            const int slot0 = (s & ((1 << spp_log2) - 1)) * 16;
            const bool edge = (p == 0 && fpo > 0) || (p == npages - 1 && lpl < ps);
            const int lo = p == 0 ? fpo : 0;
            const int hi_slot = p == npages - 1 ? lpl : ps;
            auto vis = [&](int i) {
                const int slot = slot0 + i;
                return slot >= lo && slot < hi_slot;
            };
            mfma_tile<D, HT>(kr, vr, edge, vis, vt, a.scale_log2, qb, m_run, l_part, acc, lane);
        };

        uint4 kbuf[kDepth][S::NJ], vbuf[kDepth][S::NJ];
        int s = 0;
#pragma unroll
        for (int d = 0; d < kDepth - 1; ++d) load(s + d, kbuf[d], vbuf[d]);
        const int rounds = (nsteps + kDepth - 1) / kDepth;
        for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
            for (int u = 0; u < kDepth; ++u) {
                load(s + kDepth - 1, kbuf[(u + kDepth - 1) % kDepth], vbuf[(u + kDepth - 1) % kDepth]);
                if (s < nsteps) compute(s, kbuf[u], vbuf[u]);
                ++s;
            }
            if constexpr (kLockstep > 0 && HPW > 1) {
                constexpr int every = kLockstep > 0 ? kLockstep : 1;
                if (rd % every == every - 1) __builtin_amdgcn_s_barrier();
            }
        }
        idv = idn;
    }
    mfma_epilogue<D, HT>(a, n, kvh, G, lane, m_run, l_part, acc);
}

template <int D, int HT, int HPW>
__global__ void __launch_bounds__(64 * HPW) partial_mfma_kernel(PartialArgs a)
{
    __shared__ __align__(16) char s_v[HPW][MfmaShape<D>::TILE_BYTES];
    mfma_body<D, HT, HPW>(a, blockIdx.x, s_v);
}

// Several tables in one grid: workgroups [wg_end[i-1], wg_end[i]) work on
// table i's chunks.  The cascade runs every launch of its shared level
// (stacked heads) and its per-request level this way, so that no level's
// grid alone has to fill the GPU.  The tables share the pools, strides, KV
// heads and page size; each has its own page table, plan, queries, group
// and outputs.  The table is picked by a workgroup-uniform index into the
// kernel arguments, so the body is compiled once.
constexpr int kMaxTables = 8;
struct PartialTables {
    PartialArgs t[kMaxTables];
    int32_t wg_end[kMaxTables];
    int32_t count;
};

template <int D, int HT, int HPW>
__global__ void __launch_bounds__(64 * HPW) partial_mfma_multi_kernel(PartialTables tabs)
{
    __shared__ __align__(16) char s_v[HPW][MfmaShape<D>::TILE_BYTES];
    const int wg = blockIdx.x;
    int i = 0;
    while (i < tabs.count - 1 && wg >= tabs.wg_end[i]) ++i;
    const int base = i > 0 ? tabs.wg_end[i - 1] : 0;
    mfma_body<D, HT, HPW>(tabs.t[i], wg - base, s_v);
}

// ----------------------------------------------------- MFMA kernel, any page
// The MFMA kernel above reads a 16-token tile from one page.  This variant
// serves page sizes it cannot (page size 1 -- token-sparse selections --
// and sizes that are not a power-of-two multiple of 16): the tile's 16
// tokens may lie on 16 pages.  Each wave keeps the byte offsets of 64
// consecutive tokens of its chunk in a register (lane t: token w0 + t,
// from the page id and in-page slot of the PR #984 page-table walk,
// fast-divided by the page size) and gathers a tile's offsets from it with
// ds_bpermute: lane l loads the K and V rows of the tokens the page variant's
// row loads give it (l/(D/8) + (64/(D/8))*j), one gathered offset per load.
// The tile's products, softmax and the epilogue are the page variant's.
// Tokens past the chunk take the last token's offset (valid rows) and are
// masked: -inf scores, zero V rows.
template <int D, int HT, int HPW>
__device__ __forceinline__ void mfma_tok_body(const PartialArgs &a, int wg,
                                              char (&s_v)[HPW][MfmaShape<D>::TILE_BYTES])
{
    using S = MfmaShape<D>;
    constexpr int ESZ = 2;
    const int G = a.group;

    const int groups = a.num_kv_heads / HPW;
    const int n = wg / groups;
    const int kvg = wg - n * groups;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kvh = kvg * HPW + wave;
    const int lane = tid & 63;
    const int lrow = lane / S::LPR;
    const int lpc = lane % S::LPR;

    const int r = ld_uniform(a.req_idx + n);
    const int t = ld_uniform(a.tile_idx + n);
    const int pbeg = ld_uniform(a.indptr + r);
    const int npages = ld_uniform(a.indptr + r + 1) - pbeg;
    const int fpo = ld_uniform(a.fpo + r);
    const int lpl = ld_uniform(a.lpl + r);
    const int ps = a.page_size;
    // the chunk's visible tokens, request-relative: pages [t*c, (t+1)*c)
    const int64_t n_r = npages > 0 ? int64_t(npages - 1) * ps + lpl - fpo : 0;
    const int64_t span = int64_t(a.pages_per_chunk) * ps;
    const int64_t tok0 = max(int64_t(0), int64_t(t) * span - fpo);
    const int64_t tok1 = min(n_r, int64_t(t + 1) * span - fpo);
    const int ntok = tok1 > tok0 ? int(tok1 - tok0) : 0;

    const int64_t page_bytes = a.page_stride * ESZ;
    const int64_t tsb = a.token_stride * ESZ;
    // page id and in-page slot of chunk token w0 + lane (clamped to the last)
    auto load_pid = [&](int w0, uint32_t &slot_e) -> int32_t {
        const int tk = min(w0 + lane, max(ntok - 1, 0));
        const uint32_t slot = uint32_t(fpo + tok0 + tk);
        const uint32_t pi = fastdiv_q(a.fd, slot);
        slot_e = slot - pi * uint32_t(ps);
        return a.indices[pbeg + min(int(pi), npages - 1)];
    };

    half8_t qb[HT][S::KC];
    mfma_load_q<D, HT>(a, r, kvh, G, lane, qb);

    const char *kb = static_cast<const char *>(a.k) + int64_t(kvh) * a.head_stride * ESZ;
    const char *vb = static_cast<const char *>(a.v) + int64_t(kvh) * a.head_stride * ESZ;

    float m_run[HT], l_part[HT];
    float4_t acc[HT][S::DT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        m_run[ht] = kNoMax;
        l_part[ht] = 0.f;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) acc[ht][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    char *vt = s_v[wave];

    // row offsets of the load cursor's 64-token window, split for ds_bpermute;
    // the page ids of the window after it are loaded one window ahead
    const int nsteps = (ntok + 15) / 16;
    int32_t off_lo = 0, off_hi = 0;
    uint32_t e_next = 0;
    int32_t pid_next = 0;
    auto set_window = [&](int32_t pid, uint32_t e) {
        const int64_t off = int64_t(pid) * page_bytes + int64_t(e) * tsb;
        off_lo = int32_t(uint32_t(uint64_t(off)));
        off_hi = int32_t(uint32_t(uint64_t(off) >> 32));
    };
    if (ntok > 0) {
        uint32_t e0;
        const int32_t pid0 = load_pid(0, e0);
        set_window(pid0, e0);
        pid_next = load_pid(64, e_next);
    }
    auto gather = [&](int src) -> int64_t {         // offset of window token src
        const uint32_t lo = uint32_t(__builtin_amdgcn_ds_bpermute(4 * src, off_lo));
        const uint32_t hi = uint32_t(__builtin_amdgcn_ds_bpermute(4 * src, off_hi));
        return int64_t((uint64_t(hi) << 32) | lo);
    };

    // loads run in step order, so the cursor moves to window s/4 at the
    // first step of it; steps past the chunk reload the last one
    auto load = [&](int s, uint4 (&kr)[S::NJ], uint4 (&vr)[S::NJ]) {
        if (s < nsteps && s > 0 && (s & 3) == 0) {
            set_window(pid_next, e_next);
            // unconditional (clamped to the last token): a conditional load
            // would be merged through a register copy that waits for it
            pid_next = load_pid(16 * s + 64, e_next);
        }
        const int sl = (min(s, nsteps - 1) & 3) * 16;
        // K and V rows of tokens lrow + RPI*j, whole rows per load
#pragma unroll
        for (int j = 0; j < S::NJ; ++j) {
            const int64_t o = gather(sl + lrow + S::RPI * j) + 16 * lpc;
            kr[j] = load_nt(kb + o);
            vr[j] = load_nt(vb + o);
        }
    };

    auto compute = [&](int s, const uint4 (&kr)[S::NJ], const uint4 (&vr)[S::NJ]) {
        const int tt0 = 16 * s;                     // chunk token of the tile's first row
        const bool edge = tt0 + 16 > ntok;
        auto vis = [&](int i) { return tt0 + i < ntok; };
        mfma_tile<D, HT>(kr, vr, edge, vis, vt, a.scale_log2, qb, m_run, l_part, acc, lane);
    };

    uint4 kbuf[kDepth][S::NJ], vbuf[kDepth][S::NJ];
    int s = 0;
    if (nsteps > 0) {
#pragma unroll
        for (int d = 0; d < kDepth - 1; ++d) load(s + d, kbuf[d], vbuf[d]);
    }
    const int rounds = (nsteps + kDepth - 1) / kDepth;
    for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
            load(s + kDepth - 1, kbuf[(u + kDepth - 1) % kDepth], vbuf[(u + kDepth - 1) % kDepth]);
            if (s < nsteps) compute(s, kbuf[u], vbuf[u]);
            ++s;
        }
        // the workgroup's KV heads share every token's row of the pool: in
        // lockstep their loads of a step meet in the same DRAM pages (every
        // wave of the workgroup has the same chunk, so the same round count)
        if constexpr (kLockstep > 0 && HPW > 1) {
            constexpr int every = kLockstep > 0 ? kLockstep : 1;
            if (rd % every == every - 1) __builtin_amdgcn_s_barrier();
        }
    }
    mfma_epilogue<D, HT>(a, n, kvh, G, lane, m_run, l_part, acc);
}
template <int D, int HT, int HPW>
__global__ void __launch_bounds__(64 * HPW) partial_mfma_tok_kernel(PartialArgs a)
{
    __shared__ __align__(16) char s_v[HPW][MfmaShape<D>::TILE_BYTES];
    mfma_tok_body<D, HT, HPW>(a, blockIdx.x, s_v);
}

template <typename T, int D, bool FUSED>
KernelFn pick_token(int g)
{
    switch (g) {
    case 1: return partial_token_kernel<T, D, 1, token_rows_per_step<1>(), FUSED>;
    case 2: return partial_token_kernel<T, D, 2, token_rows_per_step<2>(), FUSED>;
    case 4: return partial_token_kernel<T, D, 4, token_rows_per_step<4>(), FUSED>;
    case 8: return partial_token_kernel<T, D, 8, token_rows_per_step<8>(), FUSED>;
    case 12: return partial_token_kernel<T, D, 12, token_rows_per_step<12>(), FUSED>;
    case 16: return partial_token_kernel<T, D, 16, token_rows_per_step<16>(), FUSED>;
    default: return nullptr;
    }
}

// KV heads per workgroup of the page kernel: every head of the chunk (up to
// 8), one wave each; a group of fewer heads gets more waves per head so the
// workgroup still has 4 to 8 waves.
#ifndef PD_PAGE_HPW_MAX
#define PD_PAGE_HPW_MAX 8
#endif
int page_heads_per_wg(int hkv, int g)
{
    // G = 16 needs more than 256 VGPRs per lane: at most 4 waves per group
    const int cap = g >= 16 ? (PD_PAGE_HPW_MAX < 4 ? PD_PAGE_HPW_MAX : 4) : PD_PAGE_HPW_MAX;
    for (int h = cap; h > 1; h >>= 1)
        if (hkv % h == 0) return h;
    return 1;
}

template <typename T, int G, bool FUSED>
KernelFn pick_page_shape(int hpw)
{
    switch (hpw) {
    case 8:
        if constexpr (G < 16) return partial_page_kernel<T, G, 8, 1, FUSED>;
        else return nullptr;
    case 4: return partial_page_kernel<T, G, 4, 1, FUSED>;
    case 2: return partial_page_kernel<T, G, 2, 2, FUSED>;
    default: return partial_page_kernel<T, G, 1, 4, FUSED>;
    }
}

int page_threads(int hpw) { return hpw >= 4 ? 64 * hpw : 256; }

template <typename T, bool FUSED>
KernelFn pick_page(int g, int hpw)
{
    switch (g) {
    case 4: return pick_page_shape<T, 4, FUSED>(hpw);
    case 8: return pick_page_shape<T, 8, FUSED>(hpw);
    case 16: return pick_page_shape<T, 16, FUSED>(hpw);
    default: return nullptr;
    }
}

struct Choice {
    KernelFn fn;
    int spp_log2;
    int heads_per_wg;   // KV heads one workgroup covers
    int threads;
    int kind;           // 0 token kernel, 1 page kernel, 2 MFMA kernel, 3 MFMA kernel, any page
};

template <int D, int HT>
KernelFn pick_mfma_shape(int hpw)
{
    switch (hpw) {
    case 8: return partial_mfma_kernel<D, HT, 8>;
    case 4: return partial_mfma_kernel<D, HT, 4>;
    case 2: return partial_mfma_kernel<D, HT, 2>;
    default: return partial_mfma_kernel<D, HT, 1>;
    }
}

template <int D, int HT>
KernelFn pick_mfma_tok_shape(int hpw)
{
    switch (hpw) {
    case 8: return partial_mfma_tok_kernel<D, HT, 8>;
    case 4: return partial_mfma_tok_kernel<D, HT, 4>;
    case 2: return partial_mfma_tok_kernel<D, HT, 2>;
    default: return partial_mfma_tok_kernel<D, HT, 1>;
    }
}

// 16-head tiles per wave for a group size, 0 for a group the MFMA kernels
// do not take
int mfma_head_tiles(int g)
{
    switch (g) {
    case 1:
    case 2:
    case 4:
    case 8:
    case 12:
    case 16: return 1;
    case 24:
    case 32: return 2;
    default: return 0;
    }
}

// the page-tiled (any_page false) or any-page MFMA kernel for (D, G, width)
KernelFn pick_mfma(int d, int g, int hpw, bool any_page)
{
    const int ht = mfma_head_tiles(g);
    if (ht == 0 || (d != 64 && d != 128)) return nullptr;
    if (any_page) {
        if (d == 64) return ht == 1 ? pick_mfma_tok_shape<64, 1>(hpw) : pick_mfma_tok_shape<64, 2>(hpw);
        return ht == 1 ? pick_mfma_tok_shape<128, 1>(hpw) : pick_mfma_tok_shape<128, 2>(hpw);
    }
    if (d == 64) return ht == 1 ? pick_mfma_shape<64, 1>(hpw) : pick_mfma_shape<64, 2>(hpw);
    return ht == 1 ? pick_mfma_shape<128, 1>(hpw) : pick_mfma_shape<128, 2>(hpw);
}

// KV heads per MFMA workgroup: the largest power of two up to 8 that divides
// the KV head count, or up to 2 for chunks shorter than kNarrowChunkTokens.
// Short chunks are latency-bound: spread over more, narrower workgroups they
// reach more CUs.  Measured on MI355X, long-context geometry (8 KV heads)
// with chunks forced to c pages of 16 tokens, partial kernel: c = 4 87.6 ->
// 79.6 us, c = 8 82.5 -> 74.1, c = 13 70.7 -> 69.2 with 2 heads per
// workgroup instead of 8, but c = 16 69.2 -> 72.7 and the default c = 26
// 64.1 -> 65.0; the batched workload's 48-token chunks: step 13.9 -> 13.4 us
// and the shared-prefix batch's flat decode (160-token chunks) 32.0 -> 27.0 us
// (graph-replayed).  4 heads per workgroup measured between the two or worse.
constexpr int64_t kNarrowChunkTokens = 224;
int mfma_heads_per_wg(int hkv, int64_t chunk_tokens = 0)
{
    const int cap = chunk_tokens > 0 && chunk_tokens < kNarrowChunkTokens ? 2 : 8;
    for (int h = cap; h > 1; h >>= 1)
        if (hkv % h == 0) return h;
    return 1;
}

// In the two-launch mode, fp16 with D = 64 or 128 runs on the MFMA kernels
// for every group they take (1, 2, 4, 8, 12, 16, 24, 32; groups under 16 as
// zero-padded 16-head tiles): the page-tiled one at page sizes that are a
// power-of-two multiple of 16, the any-page one at every other.  The page
// kernel takes 256-byte rows, G in {4, 8, 16} and page sizes that are a
// power-of-two multiple of its 64/G slots per step, for the shapes off the
// MFMA kernels (fp32 with D = 64, the fused launch, the VALU-only choice).
// Every other shape takes the token kernel.  The page-tiled kernels need
// 32-bit in-page offsets.
Choice pick(int dtype, int d, int g, int page_size, int64_t token_stride, bool fused,
            bool allow_page = true, int hkv = 1, bool allow_mfma = true,
            int64_t chunk_tokens = 0)
{
    Choice c{nullptr, 0, 1, kThreads, 0};
    const int esz = dtype == PD_DTYPE_FP16 ? 2 : 4;
    const bool mfma_ok = allow_page && allow_mfma && !fused && dtype == PD_DTYPE_FP16 &&
                         (d == 64 || d == 128) && mfma_head_tiles(g) > 0;
    if (mfma_ok && page_size % 16 == 0 &&
        token_stride * esz * page_size < (int64_t(1) << 31)) {
        const int tiles = page_size / 16;
        if ((tiles & (tiles - 1)) == 0) {
            int lg = 0;
            while ((1 << lg) < tiles) ++lg;
            const int hpw = mfma_heads_per_wg(hkv, chunk_tokens);
            c.fn = pick_mfma(d, g, hpw, false);
            c.spp_log2 = lg;
            c.heads_per_wg = hpw;
            c.threads = 64 * hpw;
            c.kind = 2;
            return c;
        }
    }
    const bool row256 = (dtype == PD_DTYPE_FP16 && d == 128) || (dtype == PD_DTYPE_FP32 && d == 64);
    if (allow_page && row256 && (g == 4 || g == 8 || g == 16) && !mfma_ok) {
        const int sps = 64 / g;
        if (page_size % sps == 0) {
            const int spp = page_size / sps;
            if ((spp & (spp - 1)) == 0 && token_stride * esz * page_size < (int64_t(1) << 31)) {
                int lg = 0;
                while ((1 << lg) < spp) ++lg;
                c.spp_log2 = lg;
                const int hpw = page_heads_per_wg(hkv, g);
                c.heads_per_wg = hpw;
                c.threads = page_threads(hpw);
                c.kind = 1;
                if (dtype == PD_DTYPE_FP16) c.fn = fused ? pick_page<_Float16, true>(g, hpw) : pick_page<_Float16, false>(g, hpw);
                else c.fn = fused ? pick_page<float, true>(g, hpw) : pick_page<float, false>(g, hpw);
                return c;
            }
        }
    }
    if (mfma_ok) {
        const int hpw = mfma_heads_per_wg(hkv, chunk_tokens);
        c.fn = pick_mfma(d, g, hpw, true);
        c.heads_per_wg = hpw;
        c.threads = 64 * hpw;
        c.kind = 3;
        return c;
    }
    if (dtype == PD_DTYPE_FP16) {
        if (d == 64) c.fn = fused ? pick_token<_Float16, 64, true>(g) : pick_token<_Float16, 64, false>(g);
        if (d == 128) c.fn = fused ? pick_token<_Float16, 128, true>(g) : pick_token<_Float16, 128, false>(g);
    } else if (dtype == PD_DTYPE_FP32) {
        if (d == 64) c.fn = fused ? pick_token<float, 64, true>(g) : pick_token<float, 64, false>(g);
        if (d == 128) c.fn = fused ? pick_token<float, 128, true>(g) : pick_token<float, 128, false>(g);
    }
    return c;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_and_fill(PartialArgs &a, const void *q, const void *k_pool, const void *v_pool,
                   int64_t page_stride, int64_t token_stride, int64_t head_stride, int32_t dtype,
                   const int32_t *indices, const int32_t *indptr, const int32_t *last_page_len,
                   const int32_t *first_page_offset, const int32_t *request_indices,
                   const int32_t *kv_tile_indices, int32_t num_chunks, int32_t pages_per_chunk,
                   int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t page_size, float sm_scale, float *v_partial, float *lse_partial,
                   const char *who)
{
    (void)head_dim;   // the kernel choice checks it
    if (!q || !k_pool || !v_pool || !indices || !indptr || !last_page_len ||
        !first_page_offset || !request_indices || !kv_tile_indices || !v_partial ||
        !lse_partial)
        return fail(PD_E_NULL, std::string(who) + ": null pointer");
    if (num_chunks < 0 || batch < 1 || pages_per_chunk < 1 || page_size < 1 ||
        num_kv_heads < 1 || num_qo_heads < 1 || num_qo_heads % num_kv_heads != 0 ||
        page_stride < 0 || token_stride < 0 || head_stride < 0 || !std::isfinite(sm_scale))
        return fail(PD_E_ARG, std::string(who) + ": bad sizes or strides");
    if (int64_t(num_chunks) > PD_MAX_CHUNKS)
        return fail(PD_E_ARG, std::string(who) + ": more chunks than the launch bound");
    if (dtype != PD_DTYPE_FP16 && dtype != PD_DTYPE_FP32)
        return fail(PD_E_UNSUPPORTED, std::string(who) + ": dtype");
    const int64_t esz = dtype == PD_DTYPE_FP16 ? 2 : 4;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (page_stride * esz) % 16 || (token_stride * esz) % 16 || (head_stride * esz) % 16)
        return fail(PD_E_UNSUPPORTED, std::string(who) + ": q/pools need 16-byte alignment");
    if (!aligned16(v_partial))
        return fail(PD_E_UNSUPPORTED, std::string(who) + ": v_partial needs 16-byte alignment");
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
    a.spp_log2 = 0;
    a.fd = make_fastdiv(uint32_t(page_size));
    a.scale_log2 = float(double(sm_scale) * 1.4426950408889634074);   // log2(e)
    a.group = num_qo_heads / num_kv_heads;
    a.q_members = nullptr;
    a.q_group = 0;
    a.v_out = v_partial;
    a.lse_out = lse_partial;
    a.o_final = nullptr;
    a.lse_final = nullptr;
    a.counters = nullptr;
    return PD_OK;
}

int launch(const Choice &c, const PartialArgs &a, int32_t num_chunks, void *stream,
           const char *who)
{
    PartialArgs b = a;
    b.spp_log2 = c.spp_log2;
    const dim3 grid(uint32_t(int64_t(num_chunks) * (a.num_kv_heads / c.heads_per_wg)));
    hipLaunchKernelGGL(c.fn, grid, dim3(c.threads), 0, static_cast<hipStream_t>(stream), b);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string(who) + ": launch failed: " + hipGetErrorString(err));
    return PD_OK;
}

// kernel choice hook: 0 default, 1 every shape to the token kernel, 2 no MFMA kernel
int g_force_token_kernel = 0;
int g_no_mfma = 0;

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
    PartialArgs a;
    const char *who = "paged_decode_partial";
    int rc = check_and_fill(a, q, k_pool, v_pool, page_stride, token_stride, head_stride, dtype,
                            indices, indptr, last_page_len, first_page_offset, request_indices,
                            kv_tile_indices, num_chunks, pages_per_chunk, batch, num_qo_heads,
                            num_kv_heads, head_dim, page_size, sm_scale, v_partial, lse_partial,
                            who);
    if (rc) return rc;
    const Choice c = pick(dtype, head_dim, num_qo_heads / num_kv_heads, page_size, token_stride,
                          false, !g_force_token_kernel, num_kv_heads, !g_no_mfma,
                          int64_t(pages_per_chunk) * page_size);
    if (!c.fn) return fail(PD_E_UNSUPPORTED, "paged_decode_partial: no kernel for this (dtype, D, group)");
    if (num_chunks == 0) return PD_OK;
    return launch(c, a, num_chunks, stream, who);
}

extern "C" int paged_decode_fused(const void *q, const void *k_pool, const void *v_pool,
                                  int64_t page_stride, int64_t token_stride, int64_t head_stride,
                                  int32_t dtype, const int32_t *indices, const int32_t *indptr,
                                  const int32_t *last_page_len, const int32_t *first_page_offset,
                                  const int32_t *request_indices, const int32_t *kv_tile_indices,
                                  int32_t num_chunks, int32_t pages_per_chunk, int32_t batch,
                                  int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t page_size, float sm_scale, float *v_partial,
                                  float *lse_partial, int32_t *counters, float *out,
                                  float *lse_out, void *stream)
{
    PartialArgs a;
    const char *who = "paged_decode_fused";
    int rc = check_and_fill(a, q, k_pool, v_pool, page_stride, token_stride, head_stride, dtype,
                            indices, indptr, last_page_len, first_page_offset, request_indices,
                            kv_tile_indices, num_chunks, pages_per_chunk, batch, num_qo_heads,
                            num_kv_heads, head_dim, page_size, sm_scale, v_partial, lse_partial,
                            who);
    if (rc) return rc;
    if (!counters || !out || !lse_out) return fail(PD_E_NULL, "paged_decode_fused: null pointer");
    if (num_chunks < batch)
        return fail(PD_E_ARG, "paged_decode_fused: fewer chunks than requests");
    const Choice c = pick(dtype, head_dim, num_qo_heads / num_kv_heads, page_size, token_stride,
                          true, !g_force_token_kernel, num_kv_heads);
    if (!c.fn) return fail(PD_E_UNSUPPORTED, "paged_decode_fused: no kernel for this (dtype, D, group)");
    a.o_final = out;
    a.lse_final = lse_out;
    a.counters = counters;
    return launch(c, a, num_chunks, stream, who);
}

// ------------------------------------------------------------ cascade partial
namespace pd {
namespace {

using MultiFn = void (*)(PartialTables);

template <int D, int HT>
MultiFn pick_mfma_multi_shape(int hpw)
{
    switch (hpw) {
    case 8: return partial_mfma_multi_kernel<D, HT, 8>;
    case 4: return partial_mfma_multi_kernel<D, HT, 4>;
    case 2: return partial_mfma_multi_kernel<D, HT, 2>;
    default: return partial_mfma_multi_kernel<D, HT, 1>;
    }
}

MultiFn pick_mfma_multi(int d, int ht, int hpw)
{
    if (d == 64) return ht == 1 ? pick_mfma_multi_shape<64, 1>(hpw) : pick_mfma_multi_shape<64, 2>(hpw);
    return ht == 1 ? pick_mfma_multi_shape<128, 1>(hpw) : pick_mfma_multi_shape<128, 2>(hpw);
}

int check_level(const paged_cascade_level *lv, const char *who)
{
    if (!lv->indices || !lv->indptr || !lv->last_page_len || !lv->first_page_offset ||
        !lv->request_indices || !lv->kv_tile_indices || !lv->v_partial || !lv->lse_partial)
        return fail(PD_E_NULL, std::string(who) + ": null pointer in a level");
    if (lv->batch < 1 || lv->num_chunks < 0 || lv->pages_per_chunk < 1)
        return fail(PD_E_ARG, std::string(who) + ": bad level sizes");
    return PD_OK;
}

}  // namespace
}  // namespace pd

extern "C" int paged_cascade_partial(const void *q, int32_t batch, const int32_t *member_req,
                                     int32_t members, int32_t members_per_launch,
                                     const void *k_pool, const void *v_pool, int64_t page_stride,
                                     int64_t token_stride, int64_t head_stride, int32_t dtype,
                                     int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t page_size, float sm_scale,
                                     const paged_cascade_level *level0,
                                     const paged_cascade_level *level1,
                                     int32_t heads_per_workgroup, void *stream)
{
    const char *who = "paged_cascade_partial";
    if (!q || !member_req || !level0) return fail(PD_E_NULL, std::string(who) + ": null pointer");
    if (batch < 1 || members < 1 || members > batch || members_per_launch < 1 ||
        num_kv_heads < 1 || num_qo_heads < 1 || num_qo_heads % num_kv_heads != 0 ||
        int64_t(members_per_launch) * num_qo_heads > (1 << 20))
        return fail(PD_E_ARG, std::string(who) + ": bad sizes");
    if (heads_per_workgroup != 0 &&
        ((heads_per_workgroup & (heads_per_workgroup - 1)) != 0 || heads_per_workgroup > 8 ||
         heads_per_workgroup < 1 || num_kv_heads % heads_per_workgroup != 0))
        return fail(PD_E_ARG, std::string(who) + ": heads_per_workgroup must be 0 or a power of "
                                                 "two up to 8 dividing num_kv_heads");
    const int g = num_qo_heads / num_kv_heads;
    const int launches0 = (members + members_per_launch - 1) / members_per_launch;
    // every table: level-0 launch j stacks members [j*per, min(M, (j+1)*per)),
    // level 1 (if given) comes last
    const int ntab = launches0 + (level1 ? 1 : 0);
    std::vector<PartialArgs> args(ntab);
    std::vector<Choice> choice(ntab);
    std::vector<int32_t> chunks(ntab);
    bool all_mfma = g <= 16;
    for (int j = 0; j < ntab; ++j) {
        const bool is0 = j < launches0;
        const paged_cascade_level *lv = is0 ? &level0[j] : level1;
        int rc = check_level(lv, who);
        if (rc) return rc;
        if (!is0 && lv->batch != batch)
            return fail(PD_E_ARG, std::string(who) + ": level 1 must hold every request");
        const int sj = is0 ? std::min(members_per_launch, members - j * members_per_launch) : 1;
        const int gj = is0 ? sj * g : g;
        rc = check_and_fill(args[j], q, k_pool, v_pool, page_stride, token_stride, head_stride,
                            dtype, lv->indices, lv->indptr, lv->last_page_len,
                            lv->first_page_offset, lv->request_indices, lv->kv_tile_indices,
                            lv->num_chunks, lv->pages_per_chunk, lv->batch, gj * num_kv_heads,
                            num_kv_heads, head_dim, page_size, sm_scale, lv->v_partial,
                            lv->lse_partial, who);
        if (rc) return rc;
        if (is0) {
            args[j].q_members = member_req + int64_t(j) * members_per_launch;
            args[j].q_group = g;
        }
        choice[j] = pick(dtype, head_dim, gj, page_size, token_stride, false,
                         !g_force_token_kernel, num_kv_heads, !g_no_mfma,
                         int64_t(lv->pages_per_chunk) * page_size);
        if (!choice[j].fn)
            return fail(PD_E_UNSUPPORTED, std::string(who) + ": no kernel for stacked group " +
                                              std::to_string(gj));
        chunks[j] = lv->num_chunks;
        if (is0 && choice[j].kind != 2) all_mfma = false;
    }
    if (!all_mfma) {
        // one launch per table, each on the kernel paged_decode_partial picks
        for (int j = 0; j < ntab; ++j) {
            if (chunks[j] == 0) continue;
            const int rc = launch(choice[j], args[j], chunks[j], stream, who);
            if (rc) return rc;
        }
        return PD_OK;
    }
    // every stacked launch runs on the MFMA kernel: the tables share grids of
    // up to kMaxTables tables, the per-request level on the same kernel with
    // its group as a run-time value.  Default width: one KV head per
    // workgroup: the shared level has few chunks, so narrow workgroups spread
    // it over many CUs.  In sweeps on MI355X (4 to 16 members, 8K to 32K
    // shared tokens) at the same chunking, one head per workgroup was as fast
    // as two or faster (up to 5%), and eight up to 2x slower.
    const int hpw = heads_per_workgroup ? heads_per_workgroup : 1;
    int ht = 1;
    for (int j = 0; j < ntab; ++j)
        if (args[j].group > 16) ht = 2;
    const MultiFn fn = pick_mfma_multi(head_dim, ht, hpw);
    const int groups = num_kv_heads / hpw;
    int j = 0;
    while (j < ntab) {
        PartialTables tabs;
        tabs.count = 0;
        int64_t wgs = 0;
        for (; j < ntab && tabs.count < kMaxTables; ++j) {
            if (chunks[j] == 0) continue;
            PartialArgs b = args[j];
            b.spp_log2 = choice[0].spp_log2;   // one page size: tiles per page alike
            wgs += int64_t(chunks[j]) * groups;
            tabs.t[tabs.count] = b;
            tabs.wg_end[tabs.count] = int32_t(wgs);
            ++tabs.count;
        }
        if (tabs.count == 0) break;
        if (wgs > int64_t(INT32_MAX)) return fail(PD_E_ARG, std::string(who) + ": grid too large");
        hipLaunchKernelGGL(fn, dim3(uint32_t(wgs)), dim3(64 * hpw), 0,
                           static_cast<hipStream_t>(stream), tabs);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return fail(PD_E_HIP, std::string(who) + ": launch failed: " + hipGetErrorString(err));
    }
    return PD_OK;
}

// ------------------------------------------------------ no-allocation entry
// paged_decode_fused_noalloc keeps the fused launch's workspace -- the
// partial rows, their LSEs and the arrival counters -- in this array instead
// of caller-owned buffers.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` only names the symbol:
// kernels get the device address that hipGetSymbolAddress returns for the
// current device.
constexpr int64_t kScratchBytes = int64_t(16) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace pd {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
int scratch_base(char **base, const char *who)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(PD_E_HIP, std::string(who) + ": no current device");
    if (dev >= kMaxDevices)
        return fail(PD_E_UNSUPPORTED, std::string(who) + ": device index beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(PD_E_HIP, std::string(who) + ": cannot resolve the scratch array: " +
                                      hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<char *>(ptr);
    }
    *base = g_scratch_ptr[dev];
    return PD_OK;
}

__global__ void __launch_bounds__(256) zero_i32_kernel(int32_t *p, int32_t n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

int64_t round_up256(int64_t x) { return (x + 255) & ~int64_t(255); }

}  // namespace
}  // namespace pd

extern "C" int paged_decode_fused_noalloc(const void *q, const void *k_pool, const void *v_pool,
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
                                          float *out, float *lse_out, void *stream)
{
    const char *who = "paged_decode_fused_noalloc";
    if (num_chunks < 0 || batch < 1 || num_qo_heads < 1 || num_kv_heads < 1 || head_dim < 1)
        return fail(PD_E_ARG, std::string(who) + ": bad sizes");
    // workspace layout in the scratch array: partial rows [N, Hq, D], their
    // LSEs [N, Hq], counters [B, Hkv], each at a 256-byte boundary
    const int64_t lse_off = round_up256(int64_t(num_chunks) * num_qo_heads * head_dim * 4);
    const int64_t ctr_off = round_up256(lse_off + int64_t(num_chunks) * num_qo_heads * 4);
    const int64_t need = ctr_off + int64_t(batch) * num_kv_heads * 4;
    if (need > kScratchBytes)
        return fail(PD_E_CAPACITY,
                    std::string(who) + ": the workspace needs " + std::to_string(need) +
                        " bytes, more than the library's " + std::to_string(kScratchBytes) +
                        "-byte scratch array (use paged_decode_fused with caller-owned buffers)");
    char *base = nullptr;
    int rc = scratch_base(&base, who);
    if (rc) return rc;
    float *v_partial = reinterpret_cast<float *>(base);
    float *lse_partial = reinterpret_cast<float *>(base + lse_off);
    int32_t *counters = reinterpret_cast<int32_t *>(base + ctr_off);
    PartialArgs a;
    rc = check_and_fill(a, q, k_pool, v_pool, page_stride, token_stride, head_stride, dtype,
                        indices, indptr, last_page_len, first_page_offset, request_indices,
                        kv_tile_indices, num_chunks, pages_per_chunk, batch, num_qo_heads,
                        num_kv_heads, head_dim, page_size, sm_scale, v_partial, lse_partial, who);
    if (rc) return rc;
    if (!out || !lse_out) return fail(PD_E_NULL, std::string(who) + ": null pointer");
    if (num_chunks < batch) return fail(PD_E_ARG, std::string(who) + ": fewer chunks than requests");
    const Choice c = pick(dtype, head_dim, num_qo_heads / num_kv_heads, page_size, token_stride,
                          true, !g_force_token_kernel, num_kv_heads);
    if (!c.fn) return fail(PD_E_UNSUPPORTED, std::string(who) + ": no kernel for this (dtype, D, group)");
    // the counters start at zero on every call, whatever an earlier call left
    // (a fill kernel, not a memset: the call may be captured in a HIP graph)
    const int32_t nctr = batch * num_kv_heads;
    hipLaunchKernelGGL(zero_i32_kernel, dim3(uint32_t((nctr + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), counters, nctr);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string(who) + ": launch failed: " + hipGetErrorString(err));
    a.o_final = out;
    a.lse_final = lse_out;
    a.counters = counters;
    return launch(c, a, num_chunks, stream, who);
}

extern "C" int paged_decode_set_kernel_choice(int32_t choice)
{
    if (choice < 0 || choice > 2) return fail(PD_E_ARG, "paged_decode_set_kernel_choice: 0, 1 or 2");
    g_force_token_kernel = choice == 1;
    g_no_mfma = choice == 2;
    return PD_OK;
}

extern "C" int paged_decode_kernel_kind(int32_t dtype, int32_t head_dim, int32_t group_size,
                                        int32_t page_size, int64_t token_stride)
{
    const Choice c = pick(dtype, head_dim, group_size, page_size, token_stride, false,
                          !g_force_token_kernel, 1, !g_no_mfma);
    if (!c.fn) return fail(PD_E_UNSUPPORTED, "paged_decode_kernel_kind: unsupported shape");
    return c.kind;   // 0 token kernel, 1 page kernel, 2 MFMA kernel
}

extern "C" int paged_decode_default_target_wgs(int32_t device, int32_t group_size,
                                               int32_t head_dim, int32_t dtype,
                                               int32_t num_kv_heads)
{
    if (num_kv_heads < 1)
        return fail(PD_E_ARG, "paged_decode_default_target_wgs: num_kv_heads must be >= 1");
    if (head_dim == 512) {   // the paged-MLA kernel: one unit per workgroup
        if (num_kv_heads != 1 || dtype != PD_DTYPE_FP16)
            return fail(PD_E_UNSUPPORTED,
                        "paged_decode_default_target_wgs: paged MLA needs fp16 and one KV head");
        return mla_resident_wgs(device, group_size);
    }
    const Choice c = pick(dtype, head_dim, group_size, 16, int64_t(num_kv_heads) * head_dim,
                          false, !g_force_token_kernel, num_kv_heads, !g_no_mfma);
    if (!c.fn) return fail(PD_E_UNSUPPORTED, "paged_decode_default_target_wgs: unsupported shape");
    int dev = device;
    if (dev < 0 && hipGetDevice(&dev) != hipSuccess)
        return fail(PD_E_HIP, "paged_decode_default_target_wgs: no current device");
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(PD_E_HIP, "paged_decode_default_target_wgs: cannot query CU count");
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev && hipSetDevice(dev) != hipSuccess)
        return fail(PD_E_HIP, "paged_decode_default_target_wgs: cannot select device");
    int per_cu = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void *>(c.fn), c.threads, 0);
    if (prev >= 0 && prev != dev && hipSetDevice(prev) != hipSuccess)
        return fail(PD_E_HIP, "paged_decode_default_target_wgs: cannot restore device");
    if (e != hipSuccess || per_cu < 1)
        return fail(PD_E_HIP, "paged_decode_default_target_wgs: occupancy query failed");
    // resident (chunk, KV head) units: a workgroup of the page kernel holds
    // heads_per_wg of them
    return cus * per_cu * c.heads_per_wg;
}
