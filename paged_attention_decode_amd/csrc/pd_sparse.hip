// Selection of KV blocks -> page table rows, for gfx950.
//
// Method: mlxcel docs, "Sparse paged decode": a sparse-attention model picks
// blocks of C positions per (request, KV head); the page table can either
// name those blocks directly (block-granular pages: page_size = C, valid when
// the pool rows are blocks, i.e. row of block j of request r = base(r)/C + j)
// or name every selected position (token-exact pages: page_size = 1), which
// needs an expansion of block ids into token rows in one pass over the
// selection.  The selection itself is a device value; the table's shape
// (how many rows each request holds) follows from the selection size alone,
// so nothing is read back.
//
// A block-granular table may also name each block by s = C / P pages of P
// rows (P dividing C): the rows read are the same whole blocks, the table
// holds s entries per block instead of C, and the plan can cut a selection
// into chunks smaller than a block.  P = C is the doc's one page per block,
// P = 1 the token-exact table.
//
// paged_sparse_csr builds that shape on the host; paged_sparse_expand_blocks
// writes the row ids on the device: selected block j of request r, span s
// (pages per block: C for token rows, 1 for one page per block) becomes rows
// base[r] + id * s + t, t < s, except that the request's last listed block
// contributes only final_rows[r] rows (the pages that hold the partially
// written final block's positions).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "pd_internal.h"

namespace pd {
namespace {

// one thread per output row
__global__ void __launch_bounds__(256) expand_kernel(const int32_t *__restrict__ block_ids,
                                                     int32_t num_requests, int32_t blocks,
                                                     const int32_t *__restrict__ base,
                                                     int32_t span,
                                                     const int32_t *__restrict__ final_rows,
                                                     const int32_t *__restrict__ out_indptr,
                                                     int32_t num_blocks,
                                                     int32_t *__restrict__ rows)
{
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;   // (r, j, t)
    const int64_t per_req = int64_t(blocks) * span;
    if (idx >= per_req * num_requests) return;
    const int r = int(idx / per_req);
    const int64_t rest = idx - r * per_req;
    const int j = int(rest / span);
    const int t = int(rest - int64_t(j) * span);
    if (j == blocks - 1 && t >= final_rows[r]) return;   // past the final block's pages
    // an id outside [0, num_blocks) is clamped: the rows stay inside the
    // request's region, so the decode that reads them never leaves the pool
    const int id = min(max(block_ids[int64_t(r) * blocks + j], 0), num_blocks - 1);
    rows[out_indptr[r] + int64_t(j) * span + t] = base[r] + id * span + t;
}

}  // namespace
}  // namespace pd

using namespace pd;

extern "C" int paged_sparse_csr(int32_t num_requests, int32_t blocks_per_request,
                                int32_t block_size, int32_t page_size, const int32_t *tail,
                                int32_t *indptr, int32_t *last_page_len,
                                int32_t *first_page_offset)
{
    if (!tail || !indptr || !last_page_len || !first_page_offset)
        return fail(PD_E_NULL, "paged_sparse_csr: null pointer");
    if (num_requests < 1 || blocks_per_request < 1 || block_size < 1)
        return fail(PD_E_ARG, "paged_sparse_csr: bad sizes");
    if (page_size < 1 || block_size % page_size != 0)
        return fail(PD_E_ARG, "paged_sparse_csr: page_size must divide block_size");
    const int64_t per_block = block_size / page_size;
    indptr[0] = 0;
    for (int32_t r = 0; r < num_requests; ++r) {
        if (tail[r] < 1 || tail[r] > block_size)
            return fail(PD_E_ARG, "paged_sparse_csr: tail must be in [1, block_size]");
        const int64_t final_pages = (tail[r] + page_size - 1) / page_size;
        const int64_t pages = int64_t(blocks_per_request - 1) * per_block + final_pages;
        if (indptr[r] + pages > INT32_MAX) return fail(PD_E_ARG, "paged_sparse_csr: too many rows");
        indptr[r + 1] = int32_t(indptr[r] + pages);
        last_page_len[r] = int32_t(tail[r] - (final_pages - 1) * page_size);
        first_page_offset[r] = 0;
    }
    return PD_OK;
}

extern "C" int paged_sparse_expand_blocks(const int32_t *block_ids, int32_t num_requests,
                                          int32_t blocks_per_request, const int32_t *base,
                                          int32_t span, const int32_t *final_rows,
                                          const int32_t *out_indptr, int32_t num_blocks,
                                          int32_t *rows, void *stream)
{
    if (!block_ids || !base || !final_rows || !out_indptr || !rows)
        return fail(PD_E_NULL, "paged_sparse_expand_blocks: null pointer");
    if (num_requests < 1 || blocks_per_request < 1 || span < 1 || num_blocks < 1)
        return fail(PD_E_ARG, "paged_sparse_expand_blocks: bad sizes");
    const int64_t total = int64_t(num_requests) * blocks_per_request * span;
    if ((total + 255) / 256 > INT32_MAX)
        return fail(PD_E_ARG, "paged_sparse_expand_blocks: selection too large");
    hipLaunchKernelGGL(expand_kernel, dim3(uint32_t((total + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), block_ids, num_requests,
                       blocks_per_request, base, span, final_rows, out_indptr, num_blocks,
                       rows);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PD_E_HIP, std::string("paged_sparse_expand_blocks: ") + hipGetErrorString(err));
    return PD_OK;
}
