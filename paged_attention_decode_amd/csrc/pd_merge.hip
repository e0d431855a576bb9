// Variable-length merge of (V, LSE) attention states, for gfx950.
//
// Method: mlxcel PR #984 body item 3 and issue #898 item 3; the algebra is
// the cascade-attention doc's "Softmax states compose": for rows i of a
// group, m = max lse_i, w_i = 2^(lse_i - m), V = sum w_i V_i / sum w_i, and
// the group's LSE is m + log2(sum w_i) (base 2).  A row with lse = -inf is an
// empty chunk and carries no weight; a group without a finite row gives
// zeros and -inf rather than NaN.
//
// One thread owns four consecutive dims of one (output row, head) and walks
// the group's rows once for the max and once for the weighted sum; the lse
// values it reads are shared by the D/4 threads of the head and come from
// cache.  No LDS and no barrier, so any grouping works (the cascade's
// gathered layout reuses it with its own o_indptr).  The slice kernel below
// also reads a cascade step's groups in place: each member's stacked
// level-0 rows followed by its own level-1 rows.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pd_internal.h"

namespace pd {
namespace {

template <int W>
struct VecF;
template <>
struct VecF<4> {
    using type = float4;
};
template <>
struct VecF<1> {
    using type = float;
};

__device__ __forceinline__ void fma_into(float4 &acc, float w, const float4 &v)
{
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
}
__device__ __forceinline__ void fma_into(float &acc, float w, const float &v) { acc = fmaf(w, v, acc); }
__device__ __forceinline__ void fma_live(float4 &acc, bool live, float w, const float4 &v)
{
    acc.x = live ? fmaf(w, v.x, acc.x) : acc.x;
    acc.y = live ? fmaf(w, v.y, acc.y) : acc.y;
    acc.z = live ? fmaf(w, v.z, acc.z) : acc.z;
    acc.w = live ? fmaf(w, v.w, acc.w) : acc.w;
}
__device__ __forceinline__ void fma_live(float &acc, bool live, float w, const float &v)
{
    acc = live ? fmaf(w, v, acc) : acc;
}
__device__ __forceinline__ float4 scaled(const float4 &v, float s)
{
    return make_float4(v.x * s, v.y * s, v.z * s, v.w * s);
}
__device__ __forceinline__ float scaled(const float &v, float s) { return v * s; }
template <typename V>
__device__ __forceinline__ V filled(float x);
template <>
__device__ __forceinline__ float4 filled<float4>(float x) { return make_float4(x, x, x, x); }
template <>
__device__ __forceinline__ float filled<float>(float x) { return x; }

// Rows are visited kUnroll at a time with no branch in the loop body, so the
// loads of several rows are in flight together: the merge runs right after
// the partial kernel and is bound by load latency, not bandwidth.
constexpr int kUnroll = 8;

template <int W>
__global__ void __launch_bounds__(256) merge_kernel(const float *__restrict__ v_in,
                                                    const float *__restrict__ lse_in,
                                                    const int32_t *__restrict__ o_indptr,
                                                    int32_t num_out, int32_t num_heads,
                                                    int32_t head_dim, float *__restrict__ v_out,
                                                    float *__restrict__ lse_out)
{
    using V = typename VecF<W>::type;
    const int per_head = head_dim / W;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = int64_t(num_out) * num_heads * per_head;
    if (idx >= total) return;
    const int dv = int(idx % per_head);
    const int64_t oh = idx / per_head;
    const int h = int(oh % num_heads);
    const int64_t o = oh / num_heads;
    const int b = o_indptr[o];
    const int e = o_indptr[o + 1];

    float m = -INFINITY;
    bool nan_seen = false;
    for (int i0 = b; i0 < e; i0 += kUnroll) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = min(i0 + u, e - 1);
            const float x = lse_in[int64_t(i) * num_heads + h];
            nan_seen |= x != x;
            m = fmaxf(m, x);
        }
    }
    V *dst = reinterpret_cast<V *>(v_out + oh * head_dim) + dv;
    if (nan_seen || m == -INFINITY) {
        const float fill = nan_seen ? NAN : 0.f;
        *dst = filled<V>(fill);
        if (dv == 0) lse_out[oh] = nan_seen ? NAN : -INFINITY;
        return;
    }
    float wsum = 0.f;
    V acc = filled<V>(0.f);
    for (int i0 = b; i0 < e; i0 += kUnroll) {
        float x[kUnroll];
        V vi[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = min(i0 + u, e - 1);
            x[u] = lse_in[int64_t(i) * num_heads + h];
            vi[u] = reinterpret_cast<const V *>(v_in + (int64_t(i) * num_heads + h) * head_dim)[dv];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            // a row past the group end or with lse = -inf (empty chunk) has no
            // weight, and its V (possibly not finite) is never multiplied in
            const bool live = i0 + u < e && x[u] != -INFINITY;
            const float w = live ? __builtin_amdgcn_exp2f(x[u] - m) : 0.f;
            wsum += w;
            fma_live(acc, live, w, vi[u]);
        }
    }
    *dst = scaled(acc, 1.f / wsum);
    if (dv == 0) lse_out[oh] = m + __builtin_amdgcn_logf(wsum);
}

// One workgroup per (output row, head, dim slice) for heads whose D is a
// multiple of 32: a slice is DL float4 dim lanes (DL = 8, 32 dims, for heads up
// to 128 wide; DL = 32, 128 dims, for wider heads such as 512-wide latent
// rows), and the 256 threads are 256 / DL row lanes x DL dim lanes (lane =
// DL * row lane + dim lane within each wave).  Row lane k merges rows k, k +
// 256 / DL, ... of the group into a partial state (max, weight sum, weighted
// V) with the loads of up to UNROLL rows in flight.  The row states of a
// wave are combined by a butterfly of lane swaps (xor DL ... 32), the 4 wave
// states through LDS.  Slicing the dims spreads one (row, head) over several
// CUs; the merge runs right after the partial kernel and is bound by load
// latency, not bandwidth.
// 512-wide rows (the paged MLA latent): 256-dim slices, one row lane per
// wave.  Measured on MI355X with 128 heads: 7.1 us against 8.7 us for
// 128-dim slices at 8 rows x 16 partials, the same 7.3-7.4 us at 4 x 32.
#ifndef PD_MERGE_WIDE_DL
#define PD_MERGE_WIDE_DL 64
#endif
#ifndef PD_MERGE_WIDE_UNROLL
#define PD_MERGE_WIDE_UNROLL 4
#endif
constexpr int kWideDL = PD_MERGE_WIDE_DL;     // dim lanes per slice for 512-wide rows
constexpr int kWideUnroll = PD_MERGE_WIDE_UNROLL;
// Other widths divisible by 32: 32-dim slices.  The merge is bound by its
// fixed latency chain (row bounds, one round of loads, the combine), not by
// its slice shape: at 4 rows x 79 partials, 32 heads of 128 dims, 32-, 64-
// and 128-dim slices of four waves all took 3.5-4.1 us of GPU time.  The flat
// merge takes each slice in one wave (merge_wave_kernel below): without the
// cross-wave LDS combine and its barrier the long-context step went from
// 69.2 to 68.6-68.8 us on MI355X with 8 row lanes x 10 rows in flight; 16 x 5,
// 4 x 20 and 8 x 16 measured no better.  The cascade merge takes the same
// one-wave slices with 11 rows in flight per row lane (its launcher gives the
// measurements).
constexpr int kNarrowDL = 8;          // float4 dim lanes per slice, other widths
constexpr int kWaveUnroll = 10;       // one-wave kernel: rows in flight per row lane
constexpr int kCascadeWaveUnroll = 11;    // the same, for the cascade merge

// State of a partial merge: running max m (NaN once a NaN lse was seen),
// weight sum w relative to m, weighted sum a relative to m.
template <typename V>
struct MState {
    float m, w;
    V a;
};

// Combine two states; m = -inf means "no finite row yet", NaN propagates.
template <typename V>
__device__ __forceinline__ MState<V> combine(const MState<V> &x, const MState<V> &y)
{
    MState<V> r;
    if (x.m != x.m || y.m != y.m) {
        r.m = NAN;
        r.w = 0.f;
        r.a = filled<V>(0.f);
        return r;
    }
    r.m = fmaxf(x.m, y.m);
    if (r.m == -INFINITY) {
        r.w = 0.f;
        r.a = filled<V>(0.f);
        return r;
    }
    const float sx = x.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x.m - r.m);
    const float sy = y.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(y.m - r.m);
    r.w = fmaf(x.w, sx, y.w * sy);
    r.a = scaled(y.a, sy);
    fma_into(r.a, sx, x.a);
    return r;
}

__device__ __forceinline__ float4 shfl_xor4(const float4 &v, int mask)
{
    return make_float4(__shfl_xor(v.x, mask), __shfl_xor(v.y, mask), __shfl_xor(v.z, mask),
                       __shfl_xor(v.w, mask));
}

// Where the rows of a merge group live.  bind(o, h, H, D) gives the group of
// output row o, head h as rows [b, e) with lse(i) and v(i) (a pointer to row
// i's head-h vector of D floats).
//
// FlatRows: the rows o_indptr[o] .. o_indptr[o+1] of v_in [N, H, D] and
// lse_in [N, H].
struct FlatRows {
    const float *v_in, *lse_in;
    const int32_t *o_indptr;
    struct Group {
        int b, e, h;
        const float *v_in, *lse_in;
        int32_t num_heads, head_dim;
        __device__ float lse(int i) const { return lse_in[int64_t(i) * num_heads + h]; }
        __device__ const float *v(int i) const
        {
            return v_in + (int64_t(i) * num_heads + h) * head_dim;
        }
    };
    __device__ Group bind(int64_t o, int h, int32_t num_heads, int32_t head_dim) const
    {
        return Group{o_indptr[o], o_indptr[o + 1], h, v_in, lse_in, num_heads, head_dim};
    }
};

// CascadeRows: a cascade step's groups read in place.  Output row r's group
// is its level-0 rows (a member of a stacked launch; none otherwise)
// followed by its own level-1 rows o_indptr1[r] .. o_indptr1[r+1] of v1 [n1,
// Hq, D].  The level-0 launches' rows sit one after another in v0 as [D]
// vectors: launch j, stacking S members, holds rows [first_j, first_j +
// n0*S*Hq), chunk i's stacked head h0 at first_j + i*S*Hq + h0, and member
// position p's head h = kv*G + g is stacked head kv*S*G + p*G + g.  l0_desc
// [batch, 3] = (first_j, S, p) per request, p = -1 for a non-member.
struct CascadeRows {
    const float *v0, *lse0, *v1, *lse1;
    const int32_t *l0_desc, *o_indptr1;
    int32_t n0, group_size;
    struct Group {
        int b, e, n0r;
        int64_t row0, step0, row1;      // level 0: row0 + i*step0; level 1: row1 + i*Hq
        const float *v0, *lse0, *v1, *lse1;
        int32_t num_heads, head_dim;
        __device__ int64_t row(int i) const
        {
            return i < n0r ? row0 + int64_t(i) * step0 : row1 + int64_t(i) * num_heads;
        }
        __device__ float lse(int i) const { return (i < n0r ? lse0 : lse1)[row(i)]; }
        __device__ const float *v(int i) const { return (i < n0r ? v0 : v1) + row(i) * head_dim; }
    };
    __device__ Group bind(int64_t r, int h, int32_t num_heads, int32_t head_dim) const
    {
        const int first = l0_desc[3 * r];
        const int stack = l0_desc[3 * r + 1];
        const int pos = l0_desc[3 * r + 2];
        const int o1b = o_indptr1[r];
        const int own = o_indptr1[r + 1] - o1b;
        const int n0r = pos >= 0 ? n0 : 0;
        const int kv = h / group_size;
        const int g = h - kv * group_size;
        Group q;
        q.b = 0;
        q.e = n0r + own;
        q.n0r = n0r;
        q.row0 = int64_t(first) + (int64_t(kv) * stack + pos) * group_size + g;
        q.step0 = int64_t(stack) * num_heads;
        q.row1 = (int64_t(o1b) - n0r) * num_heads + h;
        q.v0 = v0;
        q.lse0 = lse0;
        q.v1 = v1;
        q.lse1 = lse1;
        q.num_heads = num_heads;
        q.head_dim = head_dim;
        return q;
    }
};

template <int DL, int UNROLL, typename Rows>
__global__ void __launch_bounds__(256) merge_slice_kernel(const Rows rows, int32_t num_heads,
                                                          int32_t head_dim,
                                                          float *__restrict__ v_out,
                                                          float *__restrict__ lse_out)
{
    using V = float4;
    constexpr int SPLIT = 256 / DL;              // row lanes
    __shared__ MState<V> s_st[4][DL];
    const int slices = head_dim / (4 * DL);      // a multiple of 4 * DL, checked by the launcher
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int dl_i = lane & (DL - 1);
    const int k = wave * (64 / DL) + lane / DL;  // row lane
    const int64_t ohs = blockIdx.x;              // (o * num_heads + h) * slices + slice
    const int64_t oh = ohs / slices;
    const int dv = int(ohs - oh * slices) * DL + dl_i;
    const int h = int(oh % num_heads);
    const int64_t o = oh / num_heads;
    const typename Rows::Group grp = rows.bind(o, h, num_heads, head_dim);
    const int b = grp.b;
    const int e = grp.e;

    MState<V> st;
    st.m = -INFINITY;
    st.w = 0.f;
    st.a = filled<V>(0.f);
    bool nan_seen = false;
    for (int i0 = b + k; i0 < e; i0 += SPLIT * UNROLL) {
        float x[UNROLL];
        V vi[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int i = min(i0 + u * SPLIT, e - 1);
            x[u] = grp.lse(i);
            vi[u] = reinterpret_cast<const V *>(grp.v(i))[dv];
        }
        float mb = st.m;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            nan_seen |= x[u] != x[u];
            mb = fmaxf(mb, x[u]);
        }
        if (mb == -INFINITY) continue;              // nothing finite yet
        const float sc = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - mb);
        st.w *= sc;
        st.a = scaled(st.a, sc);
        st.m = mb;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            // a row past the group end or with lse = -inf (empty chunk) has no
            // weight, and its V (possibly not finite) is never multiplied in
            const bool live = i0 + u * SPLIT < e && x[u] != -INFINITY;
            const float w = live ? __builtin_amdgcn_exp2f(x[u] - st.m) : 0.f;
            st.w += w;
            fma_live(st.a, live, w, vi[u]);
        }
    }
    if (nan_seen) st.m = NAN;
    // the row lanes of the wave: lanes dl_i, dl_i + DL, ...
#pragma unroll
    for (int mask = DL; mask < 64; mask <<= 1) {
        MState<V> y;
        y.m = __shfl_xor(st.m, mask);
        y.w = __shfl_xor(st.w, mask);
        y.a = shfl_xor4(st.a, mask);
        st = combine(st, y);
    }
    if (lane < DL) s_st[wave][lane] = st;
    __syncthreads();
    if (tid >= DL) return;
    st = s_st[0][tid];
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) st = combine(st, s_st[wv][tid]);
    V *dst = reinterpret_cast<V *>(v_out + oh * head_dim) + dv;
    const bool lse_lane = dv == 0;
    if (st.m != st.m || st.m == -INFINITY) {
        const bool nan = st.m != st.m;
        *dst = filled<V>(nan ? NAN : 0.f);
        if (lse_lane) lse_out[oh] = nan ? NAN : -INFINITY;
        return;
    }
    *dst = scaled(st.a, 1.f / st.w);
    if (lse_lane) lse_out[oh] = st.m + __builtin_amdgcn_logf(st.w);
}

// One wave per (output row, head, 4*DL-dim slice): DL float4 dim lanes x
// 64/DL row lanes (lane = DL * row lane + dim lane).  Row lane k merges rows
// k, k + 64/DL, ... with UNROLL rows' loads in flight, and the row lanes'
// states are combined by the butterfly alone: no LDS and no barrier.
template <int DL, int UNROLL, typename Rows>
__global__ void __launch_bounds__(64) merge_wave_kernel(const Rows rows, int32_t num_heads,
                                                        int32_t head_dim,
                                                        float *__restrict__ v_out,
                                                        float *__restrict__ lse_out)
{
    using V = float4;
    constexpr int SPLIT = 64 / DL;               // row lanes
    const int slices = head_dim / (4 * DL);      // a multiple of 4 * DL, checked by the launcher
    const int lane = threadIdx.x;
    const int dl_i = lane & (DL - 1);
    const int k = lane / DL;                     // row lane
    const int64_t ohs = blockIdx.x;              // (o * num_heads + h) * slices + slice
    const int64_t oh = ohs / slices;
    const int dv = int(ohs - oh * slices) * DL + dl_i;
    const int h = int(oh % num_heads);
    const int64_t o = oh / num_heads;
    const typename Rows::Group grp = rows.bind(o, h, num_heads, head_dim);
    const int b = grp.b;
    const int e = grp.e;

    MState<V> st;
    st.m = -INFINITY;
    st.w = 0.f;
    st.a = filled<V>(0.f);
    bool nan_seen = false;
    for (int i0 = b + k; i0 < e; i0 += SPLIT * UNROLL) {
        float x[UNROLL];
        V vi[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int i = min(i0 + u * SPLIT, e - 1);
            x[u] = grp.lse(i);
            vi[u] = reinterpret_cast<const V *>(grp.v(i))[dv];
        }
        float mb = st.m;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            nan_seen |= x[u] != x[u];
            mb = fmaxf(mb, x[u]);
        }
        if (mb == -INFINITY) continue;              // nothing finite yet
        const float sc = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - mb);
        st.w *= sc;
        st.a = scaled(st.a, sc);
        st.m = mb;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            // a row past the group end or with lse = -inf (empty chunk) has no
            // weight, and its V (possibly not finite) is never multiplied in
            const bool live = i0 + u * SPLIT < e && x[u] != -INFINITY;
            const float w = live ? __builtin_amdgcn_exp2f(x[u] - st.m) : 0.f;
            st.w += w;
            fma_live(st.a, live, w, vi[u]);
        }
    }
    if (nan_seen) st.m = NAN;
#pragma unroll
    for (int mask = DL; mask < 64; mask <<= 1) {
        MState<V> y;
        y.m = __shfl_xor(st.m, mask);
        y.w = __shfl_xor(st.w, mask);
        y.a = shfl_xor4(st.a, mask);
        st = combine(st, y);
    }
    if (lane >= DL) return;
    V *dst = reinterpret_cast<V *>(v_out + oh * head_dim) + dv;
    const bool lse_lane = dv == 0;
    if (st.m != st.m || st.m == -INFINITY) {
        const bool nan = st.m != st.m;
        *dst = filled<V>(nan ? NAN : 0.f);
        if (lse_lane) lse_out[oh] = nan ? NAN : -INFINITY;
        return;
    }
    *dst = scaled(st.a, 1.f / st.w);
    if (lse_lane) lse_out[oh] = st.m + __builtin_amdgcn_logf(st.w);
}

// One workgroup per (output row, head), for any other head size: its 256
// threads are `split` row lanes x D/W dim lanes; row lane k merges rows k,
// k + split, ... of the group and the split states are combined through LDS.
template <int W>
__global__ void __launch_bounds__(256) merge_split_kernel(const float *__restrict__ v_in,
                                                          const float *__restrict__ lse_in,
                                                          const int32_t *__restrict__ o_indptr,
                                                          int32_t num_heads, int32_t head_dim,
                                                          float *__restrict__ v_out,
                                                          float *__restrict__ lse_out)
{
    using V = typename VecF<W>::type;
    __shared__ float s_m[256];
    __shared__ float s_w[256];
    __shared__ V s_acc[256];
    const int per_head = head_dim / W;           // <= 256, checked by the launcher
    const int split = 256 / per_head;
    const int tid = threadIdx.x;
    const int k = tid / per_head;                // row lane
    const int dv = tid - k * per_head;
    const int64_t oh = blockIdx.x;               // o * num_heads + h
    const int h = int(oh % num_heads);
    const int64_t o = oh / num_heads;
    const int b = o_indptr[o];
    const int e = o_indptr[o + 1];
    const bool active = k < split;

    float m = -INFINITY;
    bool nan_seen = false;
    float wsum = 0.f;
    V acc = filled<V>(0.f);
    if (active) {
        for (int i0 = b + k; i0 < e; i0 += split * kUnroll) {
            float x[kUnroll];
            V vi[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = min(i0 + u * split, e - 1);
                x[u] = lse_in[int64_t(i) * num_heads + h];
                vi[u] = reinterpret_cast<const V *>(v_in + (int64_t(i) * num_heads + h) * head_dim)[dv];
            }
            float mb = m;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                nan_seen |= x[u] != x[u];
                mb = fmaxf(mb, x[u]);
            }
            if (mb == -INFINITY) continue;              // nothing finite yet
            const float sc = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mb);
            wsum *= sc;
            acc = scaled(acc, sc);
            m = mb;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const bool live = i0 + u * split < e && x[u] != -INFINITY;
                const float w = live ? __builtin_amdgcn_exp2f(x[u] - m) : 0.f;
                wsum += w;
                fma_live(acc, live, w, vi[u]);
            }
        }
    }
    s_m[tid] = nan_seen ? NAN : m;
    s_w[tid] = wsum;
    s_acc[tid] = acc;
    __syncthreads();
    if (k != 0) return;
    float mx = -INFINITY;
    bool any_nan = false;
    for (int j = 0; j < split; ++j) {
        const float mj = s_m[j * per_head + dv];
        any_nan |= mj != mj;
        mx = fmaxf(mx, mj);
    }
    V *dst = reinterpret_cast<V *>(v_out + oh * head_dim) + dv;
    if (any_nan || mx == -INFINITY) {
        *dst = filled<V>(any_nan ? NAN : 0.f);
        if (dv == 0) lse_out[oh] = any_nan ? NAN : -INFINITY;
        return;
    }
    float wt = 0.f;
    V o_acc = filled<V>(0.f);
    for (int j = 0; j < split; ++j) {
        const float mj = s_m[j * per_head + dv];
        const float sc = mj == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mj - mx);
        wt = fmaf(s_w[j * per_head + dv], sc, wt);
        fma_into(o_acc, sc, s_acc[j * per_head + dv]);
    }
    *dst = scaled(o_acc, 1.f / wt);
    if (dv == 0) lse_out[oh] = mx + __builtin_amdgcn_logf(wt);
}

}  // namespace
}  // namespace pd

using namespace pd;

extern "C" int paged_merge_states(const float *v_in, const float *lse_in,
                                  const int32_t *o_indptr, int32_t num_out_rows,
                                  int32_t num_heads, int32_t head_dim, float *v_out,
                                  float *lse_out, void *stream)
{
    if (!o_indptr || !v_out || !lse_out || (!v_in && num_out_rows > 0) ||
        (!lse_in && num_out_rows > 0))
        return fail(PD_E_NULL, "paged_merge_states: null pointer");
    if (num_out_rows < 0 || num_heads < 1 || head_dim < 1)
        return fail(PD_E_ARG, "paged_merge_states: bad sizes");
    if (num_out_rows == 0) return PD_OK;
    const bool vec4 = head_dim % 4 == 0 &&
                      ((reinterpret_cast<uintptr_t>(v_in) | reinterpret_cast<uintptr_t>(v_out)) & 15u) == 0;
    const int w = vec4 ? 4 : 1;
    const int64_t total = int64_t(num_out_rows) * num_heads * (head_dim / w);
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return fail(PD_E_ARG, "paged_merge_states: too large");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const FlatRows rows{v_in, lse_in, o_indptr};
    if (vec4 && head_dim % 512 == 0) {
        // wide heads: one workgroup per (output row, head, 4*kWideDL-dim slice)
        const int64_t nblk = int64_t(num_out_rows) * num_heads * (head_dim / (4 * kWideDL));
        if (nblk > 0x7fffffff) return fail(PD_E_ARG, "paged_merge_states: too large");
        hipLaunchKernelGGL((merge_slice_kernel<kWideDL, kWideUnroll, FlatRows>),
                           dim3(uint32_t(nblk)), dim3(256), 0, s, rows, num_heads, head_dim,
                           v_out, lse_out);
    } else if (vec4 && head_dim % (4 * kNarrowDL) == 0) {
        // one workgroup per (output row, head, 4*kNarrowDL-dim slice)
        const int64_t nblk = int64_t(num_out_rows) * num_heads * (head_dim / (4 * kNarrowDL));
        if (nblk > 0x7fffffff) return fail(PD_E_ARG, "paged_merge_states: too large");
        hipLaunchKernelGGL((merge_wave_kernel<kNarrowDL, kWaveUnroll, FlatRows>),
                           dim3(uint32_t(nblk)), dim3(64), 0, s, rows, num_heads, head_dim,
                           v_out, lse_out);
    } else if (head_dim / w <= 256) {
        // one workgroup per (output row, head), rows split across lanes
        const int64_t nblk = int64_t(num_out_rows) * num_heads;
        if (nblk > 0x7fffffff) return fail(PD_E_ARG, "paged_merge_states: too large");
        if (vec4)
            hipLaunchKernelGGL(merge_split_kernel<4>, dim3(uint32_t(nblk)), dim3(256), 0, s, v_in,
                               lse_in, o_indptr, num_heads, head_dim, v_out, lse_out);
        else
            hipLaunchKernelGGL(merge_split_kernel<1>, dim3(uint32_t(nblk)), dim3(256), 0, s, v_in,
                               lse_in, o_indptr, num_heads, head_dim, v_out, lse_out);
    } else if (vec4)
        hipLaunchKernelGGL(merge_kernel<4>, dim3(uint32_t(blocks)), dim3(256), 0, s, v_in, lse_in,
                           o_indptr, num_out_rows, num_heads, head_dim, v_out, lse_out);
    else
        hipLaunchKernelGGL(merge_kernel<1>, dim3(uint32_t(blocks)), dim3(256), 0, s, v_in, lse_in,
                           o_indptr, num_out_rows, num_heads, head_dim, v_out, lse_out);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string("paged_merge_states: launch failed: ") +
                                  hipGetErrorString(err));
    return PD_OK;
}

extern "C" int paged_cascade_merge_states(const float *v0, const float *lse0, int32_t n0,
                                          const int32_t *l0_desc, const float *v1,
                                          const float *lse1, const int32_t *o_indptr1,
                                          int32_t batch, int32_t num_qo_heads,
                                          int32_t num_kv_heads, int32_t head_dim, float *v_out,
                                          float *lse_out, void *stream)
{
    if (!v0 || !lse0 || !l0_desc || !v1 || !lse1 || !o_indptr1 || !v_out || !lse_out)
        return fail(PD_E_NULL, "paged_cascade_merge_states: null pointer");
    if (batch < 1 || n0 < 1 || num_qo_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
        num_qo_heads % num_kv_heads)
        return fail(PD_E_ARG, "paged_cascade_merge_states: bad sizes");
    if (head_dim % (4 * kNarrowDL) ||
        ((reinterpret_cast<uintptr_t>(v0) | reinterpret_cast<uintptr_t>(v1) |
          reinterpret_cast<uintptr_t>(v_out)) & 15u))
        return fail(PD_E_UNSUPPORTED, "paged_cascade_merge_states: head_dim must be a multiple "
                                      "of 32 and the V buffers 16-byte aligned");
    const CascadeRows rows{v0, lse0, v1, lse1, l0_desc, o_indptr1, n0,
                           num_qo_heads / num_kv_heads};
    hipStream_t s = static_cast<hipStream_t>(stream);
    // 32-dim slices of one wave, 8 row lanes with 11 rows in flight each (88
    // rows per pass).  The shared level's plan gives a group 64 level-0 rows
    // plus the request's own level-1 rows, about 81 at 4 members x 8192
    // shared tokens.  Measured on MI355X against four-wave slices (4 rows in
    // flight per lane): step 18.4-18.6 against 19.0-19.1 us there, 34.1-34.2
    // against 34.7 us at 4 x 32768 and 44.3 against 45.1 us at 16 x 8192;
    // 10 rows in flight (two passes for 81 rows) 19.7 us, 12 rows 18.6 us.
    // Under an earlier plan of about 300 rows per group the four-wave kernel
    // was the faster one.
    const bool wide = head_dim % (4 * kWideDL) == 0;
    const int64_t nblk =
        int64_t(batch) * num_qo_heads * (head_dim / (4 * (wide ? kWideDL : kNarrowDL)));
    if (nblk > 0x7fffffff) return fail(PD_E_ARG, "paged_cascade_merge_states: too large");
    if (wide)
        hipLaunchKernelGGL((merge_slice_kernel<kWideDL, kWideUnroll, CascadeRows>),
                           dim3(uint32_t(nblk)), dim3(256), 0, s, rows, num_qo_heads, head_dim,
                           v_out, lse_out);
    else
        hipLaunchKernelGGL((merge_wave_kernel<kNarrowDL, kCascadeWaveUnroll, CascadeRows>),
                           dim3(uint32_t(nblk)), dim3(64), 0, s, rows, num_qo_heads, head_dim,
                           v_out, lse_out);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string("paged_cascade_merge_states: launch failed: ") +
                                  hipGetErrorString(err));
    return PD_OK;
}
