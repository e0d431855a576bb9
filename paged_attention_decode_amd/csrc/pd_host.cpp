// Host side of the paged-decode library: CSR validation and construction,
// the split-KV plan, and small shared helpers.  Nothing here touches a GPU
// except paged_decode_default_target_wgs (in pd_partial.hip).
//
// Method: mlxcel PR #984 "fused paged-attention decode v2" -- the commit
// adding cache::paged_csr (CSR view, first_page_offset, geometry identity,
// exactly-full last page, retired pages dropped) and the commit adding the
// plan (binary search for the largest pages-per-chunk whose workgroup count
// reaches the device target, the 65535 launch floor, one chunk at least per
// request, request-major emission, write-O-directly when no request splits).

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>

#include "pd_internal.h"

namespace pd {

static thread_local std::string g_error;

void set_error(const std::string &msg) { g_error = msg; }

int fail(int code, const std::string &msg)
{
    g_error = msg;
    return code;
}

static std::string fmt(const char *f, long long a = 0, long long b = 0, long long c = 0)
{
    char buf[256];
    std::snprintf(buf, sizeof(buf), f, a, b, c);
    return std::string(buf);
}

}  // namespace pd

using namespace pd;

extern "C" const char *pd_last_error(void) { return g_error.c_str(); }

extern "C" const char *pd_version(void) { return "paged_decode 0.1 (gfx950)"; }

extern "C" int csr_validate(int32_t batch, int32_t page_size, int32_t num_pool_pages,
                            const int32_t *indptr, const int32_t *indices,
                            const int32_t *last_page_len, const int32_t *first_page_offset,
                            const int32_t *seq_lens, int32_t *bad_request)
{
    if (bad_request) *bad_request = -1;
    if (!indptr || !last_page_len || !first_page_offset)
        return fail(PD_E_NULL, "csr_validate: null array");
    if (batch < 0 || page_size < 1 || num_pool_pages < 0)
        return fail(PD_E_ARG, fmt("csr_validate: bad sizes batch=%lld page_size=%lld pool=%lld",
                                  batch, page_size, num_pool_pages));
    if (indptr[0] != 0) return fail(PD_E_INDPTR, "csr_validate: indptr[0] != 0");
    for (int32_t r = 0; r < batch; ++r) {
        if (indptr[r + 1] < indptr[r]) {
            if (bad_request) *bad_request = r;
            return fail(PD_E_INDPTR, fmt("csr_validate: indptr decreases at request %lld", r));
        }
    }
    if (indptr[batch] > 0 && !indices) return fail(PD_E_NULL, "csr_validate: null indices");
    for (int32_t r = 0; r < batch; ++r) {
        const int64_t pages = int64_t(indptr[r + 1]) - indptr[r];
        const int32_t lpl = last_page_len[r], fpo = first_page_offset[r];
        for (int32_t i = indptr[r]; i < indptr[r + 1]; ++i) {
            if (indices[i] < 0 || indices[i] >= num_pool_pages) {
                if (bad_request) *bad_request = r;
                return fail(PD_E_INDEX_RANGE,
                            fmt("csr_validate: request %lld page id %lld outside the pool of %lld",
                                r, indices[i], num_pool_pages));
            }
        }
        if (pages == 0) {
            if (lpl != 0) {
                if (bad_request) *bad_request = r;
                return fail(PD_E_LAST_PAGE_LEN,
                            fmt("csr_validate: request %lld has no pages but last_page_len %lld", r, lpl));
            }
            if (fpo != 0) {
                if (bad_request) *bad_request = r;
                return fail(PD_E_FIRST_PAGE_OFFSET,
                            fmt("csr_validate: request %lld has no pages but first_page_offset %lld", r, fpo));
            }
        } else {
            if (lpl < 1 || lpl > page_size) {
                if (bad_request) *bad_request = r;
                return fail(PD_E_LAST_PAGE_LEN,
                            fmt("csr_validate: request %lld last_page_len %lld outside [1, %lld]",
                                r, lpl, page_size));
            }
            if (fpo < 0 || fpo >= page_size || (pages == 1 && fpo >= lpl)) {
                if (bad_request) *bad_request = r;
                return fail(PD_E_FIRST_PAGE_OFFSET,
                            fmt("csr_validate: request %lld first_page_offset %lld invalid (lpl %lld)",
                                r, fpo, lpl));
            }
        }
        if (seq_lens) {
            const int64_t n = pages ? (pages - 1) * page_size + lpl - fpo : 0;
            if (n != seq_lens[r]) {
                if (bad_request) *bad_request = r;
                return fail(PD_E_GEOMETRY,
                            fmt("csr_validate: request %lld geometry gives %lld tokens, seq_len %lld",
                                r, n, seq_lens[r]));
            }
        }
    }
    return PD_OK;
}

extern "C" int paged_csr_build(int32_t batch, int32_t page_size, int32_t num_pool_pages,
                               const int32_t *bt_offsets, const int32_t *block_tables,
                               const int32_t *logical_start, const int32_t *written_len,
                               int32_t capacity, int32_t *indptr, int32_t *indices,
                               int32_t *last_page_len, int32_t *first_page_offset,
                               int32_t *seq_lens, int32_t *rope_offsets)
{
    if (!bt_offsets || !logical_start || !written_len || !indptr || !last_page_len ||
        !first_page_offset || !seq_lens || !rope_offsets)
        return fail(PD_E_NULL, "paged_csr_build: null array");
    if (batch < 0 || page_size < 1 || capacity < 0)
        return fail(PD_E_ARG, "paged_csr_build: bad sizes");
    int64_t nnz = 0;
    indptr[0] = 0;
    for (int32_t r = 0; r < batch; ++r) {
        const int64_t ls = logical_start[r], wl = written_len[r];
        const int64_t nblocks = int64_t(bt_offsets[r + 1]) - bt_offsets[r];
        if (ls < 0 || wl < ls || nblocks < 0)
            return fail(PD_E_ARG, fmt("paged_csr_build: request %lld start %lld > length %lld",
                                      r, ls, wl));
        rope_offsets[r] = int32_t(wl);
        seq_lens[r] = int32_t(wl - ls);
        if (wl == ls) {  // nothing visible: no pages at all
            last_page_len[r] = 0;
            first_page_offset[r] = 0;
            indptr[r + 1] = int32_t(nnz);
            continue;
        }
        const int64_t first_block = ls / page_size;      // blocks before it are retired
        const int64_t last_block = (wl - 1) / page_size;
        if (last_block >= nblocks)
            return fail(PD_E_ARG, fmt("paged_csr_build: request %lld needs %lld blocks, has %lld",
                                      r, last_block + 1, nblocks));
        first_page_offset[r] = int32_t(ls - first_block * page_size);
        last_page_len[r] = int32_t(wl - last_block * page_size);   // in [1, page_size]
        if (nnz + (last_block - first_block + 1) > capacity)
            return fail(PD_E_CAPACITY, "paged_csr_build: indices capacity too small");
        if (!indices) return fail(PD_E_NULL, "paged_csr_build: null indices");
        for (int64_t b = first_block; b <= last_block; ++b) {
            const int32_t page = block_tables[bt_offsets[r] + b];
            if (page < 0 || page >= num_pool_pages)
                return fail(PD_E_INDEX_RANGE,
                            fmt("paged_csr_build: request %lld block %lld maps to page %lld",
                                r, b, page));
            indices[nnz++] = page;
        }
        indptr[r + 1] = int32_t(nnz);
    }
    return csr_validate(batch, page_size, num_pool_pages, indptr, indices, last_page_len,
                        first_page_offset, seq_lens, nullptr);
}

namespace {

// Smallest chunk, in token slots (pages x page_size), that the device-default
// target lets the plan choose.  Calibrated on MI355X by timing every
// power-of-two pages-per-chunk (bench.py --sweep-chunks, HIP-graph replay):
// page_size-1 tables (token-sparse selections) were fastest at 16-32 slots
// per chunk and 3-5x slower at the 2-4 slots the occupancy target alone gave;
// paged pools (16-token pages) were unaffected.
constexpr int64_t kMinChunkTokens = 32;

// latent width of the paged-MLA kernel: a plan or shape query with this head
// dim is for that kernel
constexpr int32_t kMlaDim = 512;

int64_t chunks_at(int32_t batch, const int32_t *indptr, int64_t c)
{
    int64_t total = 0;
    for (int32_t r = 0; r < batch; ++r) {
        const int64_t pages = int64_t(indptr[r + 1]) - indptr[r];
        total += std::max<int64_t>(1, (pages + c - 1) / c);
    }
    return total;
}

// the plan rule: largest c in [c_min, c_max] with chunks(c) * wg_per_chunk >=
// target, else c_min
int64_t plan_c(int32_t batch, const int32_t *indptr, int64_t wg_per_chunk, int64_t target,
               int64_t cmin, int64_t cmax)
{
    if (chunks_at(batch, indptr, cmin) * wg_per_chunk < target) return cmin;
    int64_t lo = cmin, hi = cmax;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (chunks_at(batch, indptr, mid) * wg_per_chunk >= target) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

int64_t cmin_of(int32_t batch, const int32_t *indptr, int64_t cmax)
{
    int64_t lo = 1, hi = cmax;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (chunks_at(batch, indptr, mid) <= PD_MAX_CHUNKS) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

// Largest target t <= slots whose plan uses at most `slots` units (units(t)
// is non-decreasing in t); `slots` itself when even t = 1 overflows.
int64_t fit_target(int32_t batch, const int32_t *indptr, int64_t wg_per_chunk, int64_t slots)
{
    int64_t cmax = 1;
    for (int32_t r = 0; r < batch; ++r) cmax = std::max<int64_t>(cmax, int64_t(indptr[r + 1]) - indptr[r]);
    const int64_t cmin = cmin_of(batch, indptr, cmax);
    auto units = [&](int64_t t) {
        return chunks_at(batch, indptr, plan_c(batch, indptr, wg_per_chunk, t, cmin, cmax)) *
               wg_per_chunk;
    };
    if (units(1) > slots) return slots;
    int64_t lo = 1, hi = slots;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (units(mid) <= slots) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

}  // namespace

extern "C" int paged_decode_q_heads_per_wg(int32_t group_size, int32_t head_dim, int32_t dtype)
{
    if (head_dim == kMlaDim) {   // the paged-MLA kernel: q groups of up to 64 heads
        if (dtype != PD_DTYPE_FP16)
            return fail(PD_E_UNSUPPORTED, "paged MLA decode: fp16 only");
        return mla_q_heads_per_wg(group_size);
    }
    // G = 24 and 32 only on the MFMA kernel: fp16, head dim 128
    const bool g_ok = group_size == 1 || group_size == 2 || group_size == 4 ||
                      group_size == 8 || group_size == 12 || group_size == 16 ||
                      ((group_size == 24 || group_size == 32) && dtype == PD_DTYPE_FP16 &&
                       head_dim == 128);
    const bool d_ok = head_dim == 64 || head_dim == 128;
    const bool t_ok = dtype == PD_DTYPE_FP16 || dtype == PD_DTYPE_FP32;
    if (!g_ok || !d_ok || !t_ok)
        return fail(PD_E_UNSUPPORTED,
                    fmt("no partial kernel for group %lld, head_dim %lld, dtype %lld",
                        group_size, head_dim, dtype));
    return group_size;
}

extern "C" int paged_decode_plan(int32_t batch, const int32_t *indptr,
                                 int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t dtype, int32_t page_size, int32_t target_wgs,
                                 int32_t fixed_pages_per_chunk,
                                 int32_t capacity, int32_t *request_indices,
                                 int32_t *kv_tile_indices, int32_t *o_indptr,
                                 paged_decode_plan_info *info)
{
    if (!indptr || !o_indptr || !info) return fail(PD_E_NULL, "paged_decode_plan: null argument");
    if (batch < 1 || num_kv_heads < 1 || num_qo_heads < 1 || head_dim < 1 || page_size < 1 ||
        num_qo_heads % num_kv_heads != 0)
        return fail(PD_E_ARG, fmt("paged_decode_plan: bad sizes batch=%lld Hq=%lld Hkv=%lld",
                                  batch, num_qo_heads, num_kv_heads) +
                                  fmt(" page_size=%lld", page_size));
    if ((request_indices == nullptr) != (kv_tile_indices == nullptr))
        return fail(PD_E_NULL, "paged_decode_plan: pass both chunk arrays or neither");
    if (indptr[0] != 0) return fail(PD_E_INDPTR, "paged_decode_plan: indptr[0] != 0");
    int64_t cmax = 1;
    for (int32_t r = 0; r < batch; ++r) {
        const int64_t pages = int64_t(indptr[r + 1]) - indptr[r];
        if (pages < 0) return fail(PD_E_INDPTR, "paged_decode_plan: indptr decreases");
        cmax = std::max(cmax, pages);
    }
    // a workgroup serves every query head of its KV head, except on the
    // paged-MLA kernel (head_dim 512, one KV head): q groups of 64 heads
    int64_t q_groups = 1;
    if (head_dim == kMlaDim) {
        if (num_kv_heads != 1)
            return fail(PD_E_UNSUPPORTED, "paged_decode_plan: head_dim 512 (paged MLA) needs one KV head");
        const int qh = mla_q_heads_per_wg(num_qo_heads);
        if (qh < 0) return qh;
        q_groups = (num_qo_heads + qh - 1) / qh;
    }
    const int64_t wg_per_chunk = int64_t(num_kv_heads) * q_groups;
    if (chunks_at(batch, indptr, cmax) > PD_MAX_CHUNKS)
        return fail(PD_E_INFEASIBLE,
                    fmt("paged_decode_plan: %lld requests exceed the %lld-chunk launch bound",
                        batch, PD_MAX_CHUNKS));
    int64_t target = target_wgs;
    if (target <= 0 && fixed_pages_per_chunk <= 0) {
        // device default: the units the device holds resident at once, and
        // within that the largest target whose plan still fits one round
        // (the plan rule rounds the count up past its target, which would
        // leave a few workgroups for a second, nearly empty round)
        const int slots = paged_decode_default_target_wgs(-1, num_qo_heads / num_kv_heads,
                                                          head_dim, dtype, num_kv_heads);
        if (slots <= 0) return slots < 0 ? slots : fail(PD_E_ARG, "paged_decode_plan: no device target");
        target = fit_target(batch, indptr, wg_per_chunk, slots);
        // ... but no target whose chunks hold fewer than kMinChunkTokens
        // token slots: below that a unit's fixed cost (the dependent loads
        // that start it, the G*(D+1)*4-byte partial it writes and the merge
        // reads back) outweighs the K/V it streams.  The plan takes the
        // largest c whose unit count reaches the target, so a target of
        // units(c_lo) gives c >= c_lo.
        const int64_t c_lo = std::min<int64_t>(
            cmax, std::max<int64_t>(1, (kMinChunkTokens + page_size - 1) / page_size));
        target = std::min<int64_t>(target, chunks_at(batch, indptr, c_lo) * wg_per_chunk);
    }
    if (target <= 0) target = 1;
    int64_t c;
    if (fixed_pages_per_chunk > 0) {
        c = fixed_pages_per_chunk;
        if (chunks_at(batch, indptr, c) > PD_MAX_CHUNKS)
            return fail(PD_E_INFEASIBLE,
                        fmt("paged_decode_plan: %lld pages per chunk gives more than %lld chunks",
                            c, PD_MAX_CHUNKS));
    } else {
        c = plan_c(batch, indptr, wg_per_chunk, target, cmin_of(batch, indptr, cmax), cmax);
    }
    const int64_t n = chunks_at(batch, indptr, c);
    info->pages_per_chunk = int32_t(c);
    info->num_chunks = int32_t(n);
    info->num_wgs = int32_t(n * wg_per_chunk);
    info->q_groups = int32_t(q_groups);
    info->needs_merge = n != batch;
    info->target_wgs = int32_t(target);
    info->workspace_bytes = n * int64_t(num_qo_heads) * (int64_t(head_dim) + 1) * 4;
    int32_t k = 0;
    o_indptr[0] = 0;
    for (int32_t r = 0; r < batch; ++r) {
        const int64_t pages = int64_t(indptr[r + 1]) - indptr[r];
        const int64_t tiles = std::max<int64_t>(1, (pages + c - 1) / c);
        if (request_indices) {
            if (k + tiles > capacity)
                return fail(PD_E_CAPACITY,
                            fmt("paged_decode_plan: %lld chunks exceed capacity %lld", n, capacity));
            for (int64_t t = 0; t < tiles; ++t) {
                request_indices[k + t] = r;
                kv_tile_indices[k + t] = int32_t(t);
            }
        }
        k += int32_t(tiles);
        o_indptr[r + 1] = k;
    }
    return PD_OK;
}

extern "C" int paged_fastdiv_eval(int32_t d, const uint32_t *n, int64_t count, uint32_t *q,
                                  uint32_t *r)
{
    if (d < 1) return fail(PD_E_ARG, "paged_fastdiv_eval: divisor must be >= 1");
    if (count > 0 && (!n || !q || !r)) return fail(PD_E_NULL, "paged_fastdiv_eval: null array");
    const FastDiv f = make_fastdiv(uint32_t(d));
    for (int64_t i = 0; i < count; ++i) {
        if (n[i] >= (uint32_t(1) << 31))
            return fail(PD_E_ARG, "paged_fastdiv_eval: numerator >= 2^31");
        q[i] = fastdiv_q(f, n[i]);
        r[i] = n[i] - q[i] * f.d;
    }
    return PD_OK;
}
