/*
 * paged_decode.h -- C-ABI of the MI355X (gfx950) paged-attention decode
 * library: a CSR page table, a split-KV partial-attention kernel, a
 * variable-length merge of (V, LSE) states, and the host plan that sizes the
 * split.  Method: the mlxcel pages "fused paged-attention decode v2"
 * (PR #984), "sparse paged decode" and "cascade attention".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Status: 0 on success, a negative PD_E_* code on failure.  A failing call
 *    writes nothing to its outputs and launches nothing; pd_last_error()
 *    returns a thread-local message for the last failure on this thread.
 *  - HOST pointers are ordinary CPU memory, read or written before the call
 *    returns.  DEVICE pointers are HIP device memory owned by the caller; the
 *    library never allocates, frees or synchronizes, and launches only on the
 *    caller's stream (a hipStream_t passed as void*; NULL = the null stream).
 *    Kernel faults are asynchronous: they surface at the caller's next
 *    synchronization of that stream.
 *  - All integer arrays are int32, all sizes are in elements.
 *  - LSE values are base-2 log-sum-exp ("log2 units"); multiply by ln 2 for
 *    the natural-log value.
 *  - Inputs are read-only; outputs must not alias inputs.
 *  - Thread safety: no global mutable state apart from the per-thread error
 *    message and a per-device property cache filled on first use.
 */
#ifndef PAGED_DECODE_H
#define PAGED_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PD_OK = 0,
    PD_E_NULL = -1,              /* a required pointer is NULL */
    PD_E_ARG = -2,               /* a size or count is out of range */
    PD_E_INDPTR = -3,            /* indptr does not start at 0, decreases, or disagrees with nnz */
    PD_E_INDEX_RANGE = -4,       /* a page id is outside [0, num_pool_pages) */
    PD_E_LAST_PAGE_LEN = -5,     /* last_page_len outside its range for the request */
    PD_E_FIRST_PAGE_OFFSET = -6, /* first_page_offset outside its range */
    PD_E_GEOMETRY = -7,          /* (pages-1)*page_size + lpl - fpo != seq_len */
    PD_E_CAPACITY = -8,          /* an output array is too small */
    PD_E_INFEASIBLE = -9,        /* no chunk size keeps the launch within its bound */
    PD_E_UNSUPPORTED = -10,      /* a shape, dtype or alignment with no compiled kernel */
    PD_E_HIP = -11               /* the HIP runtime reported an error at launch */
};

enum { PD_DTYPE_FP16 = 0, PD_DTYPE_FP32 = 1 };

/* Largest number of chunks a plan may emit (the pages' grid-z launch bound). */
#define PD_MAX_CHUNKS 65535

/* Message for the last failure on the calling thread ("" if none). */
const char *pd_last_error(void);

/* ------------------------------------------------------------------------
 * csr_validate -- PR #984, commit "cache::paged_csr" and PR body item 1.
 *
 * Checks a CSR page table before it reaches a kernel, because every way it
 * can be inconsistent is an out-of-bounds read inside the kernel.  Request r
 * owns pages indices[indptr[r] .. indptr[r+1]); its first visible token sits
 * at entry first_page_offset[r] of its first page and its last page holds
 * last_page_len[r] valid entries.  Rules (all HOST arrays):
 *   indptr[0] == 0, non-decreasing;
 *   every page id in [0, num_pool_pages);
 *   a request with no pages has last_page_len == first_page_offset == 0
 *   (empty or fully trimmed);
 *   otherwise 1 <= last_page_len <= page_size (an exactly-full last page is
 *   page_size, never 0), 0 <= first_page_offset < page_size, and for a
 *   one-page request first_page_offset < last_page_len (retired pages are
 *   dropped, so a page with no visible token never appears);
 *   if seq_lens != NULL: (pages-1)*page_size + last_page_len -
 *   first_page_offset == seq_lens[r] (0 for no pages).
 * Returns the code of the first violation; *bad_request (nullable) receives
 * the request it was found in (-1 when not request-specific).
 * ---------------------------------------------------------------------- */
int csr_validate(int32_t batch, int32_t page_size, int32_t num_pool_pages,
                 const int32_t *indptr, const int32_t *indices,
                 const int32_t *last_page_len, const int32_t *first_page_offset,
                 const int32_t *seq_lens, int32_t *bad_request);

/* ------------------------------------------------------------------------
 * paged_csr_build -- PR #984, commit "cache::paged_csr" (the builder).
 *
 * Builds the CSR view from per-request block tables: block_tables[
 * bt_offsets[r] + b] is the pool page of logical block b of request r (-1 for
 * a released page); tokens [logical_start[r], written_len[r]) are visible.
 * Fully retired pages are dropped, first_page_offset = logical_start mod
 * page_size, last_page_len in [1, page_size], seq_lens = written_len -
 * logical_start, rope_offsets = written_len (the absolute next position).
 * A request with nothing visible gets no pages and lpl = fpo = 0.  All HOST;
 * `indices` has room for `capacity` ids.  The result is validated before
 * returning (PD_E_INDEX_RANGE if a visible block is released or beyond
 * num_pool_pages).
 * ---------------------------------------------------------------------- */
int paged_csr_build(int32_t batch, int32_t page_size, int32_t num_pool_pages,
                    const int32_t *bt_offsets, const int32_t *block_tables,
                    const int32_t *logical_start, const int32_t *written_len,
                    int32_t capacity, int32_t *indptr, int32_t *indices,
                    int32_t *last_page_len, int32_t *first_page_offset,
                    int32_t *seq_lens, int32_t *rope_offsets);

/* ------------------------------------------------------------------------
 * paged_decode_plan -- PR #984 body item 4 and commit "plan + launch";
 * issue #898 "four composable pieces" item 4.
 *
 * Chooses pages_per_chunk c and emits the flat chunk list.  With P_r =
 * indptr[r+1]-indptr[r] pages, chunks(c) = sum_r max(1, ceil(P_r / c)); each
 * chunk is launched as num_kv_heads * q_groups workgroups.  c lies in
 * [c_min, c_max], c_max = max(1, max_r P_r), c_min the smallest c with
 * chunks(c) <= PD_MAX_CHUNKS (PD_E_INFEASIBLE if even c_max exceeds it).  The
 * plan takes the largest c in that range whose workgroup count reaches
 * target_wgs (binary search: chunks(c) is non-increasing), or c_min when
 * none does.  fixed_pages_per_chunk > 0 pins c instead (e.g. 1 to force every
 * request through the merge).  The count is in (chunk, KV head) units, the
 * pages' CTAs: a workgroup of the token kernel is one unit, a wave of the
 * page kernel is one unit.  target_wgs <= 0 fits the device: with S =
 * paged_decode_default_target_wgs() units resident at once on the current
 * device, the target is the largest t <= S whose plan has at most S units,
 * lowered if needed to the unit count at c_lo = min(c_max, ceil(32 /
 * page_size)) so that chunks hold at least 32 token slots (the pages leave
 * the target uncalibrated; this floor is this library's calibration on
 * MI355X).  The target used is reported in info->target_wgs; `dtype`
 * (PD_DTYPE_*) selects the kernel whose occupancy defines S, and page_size
 * (>= 1) sets the floor; neither is used otherwise.  head_dim 512 plans the
 * paged-MLA kernel (paged_mla_decode_partial; num_kv_heads must be 1): its
 * workgroups own (chunk, q group) units of up to 64 query heads, so a chunk
 * is ceil(Hq / 64) units (q_groups), as the pages' (chunk, KV head, q-head
 * group) ownership allows.
 *
 * Outputs (HOST): request_indices[n] / kv_tile_indices[n] for n < N, in
 * request order (chunk t of request r covers its pages [t*c, (t+1)*c));
 * o_indptr[B+1] groups each request's chunks for the merge.  Pass NULL for
 * request_indices / kv_tile_indices to query only `info` (sizes); otherwise
 * they must hold `capacity` >= N entries (indptr[B] + batch always suffices).
 * info->needs_merge is 0 when every request has exactly one chunk: then the
 * partial output, in request order, already is the answer.
 * info->workspace_bytes = N*Hq*(D+1)*4, the fp32 partial V and LSE.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t pages_per_chunk;
    int32_t num_chunks;
    int32_t num_wgs;          /* (chunk, KV head) units: num_chunks * num_kv_heads * q_groups */
    int32_t q_groups;         /* 1: a workgroup owns every query head of its KV head */
    int32_t needs_merge;
    int32_t target_wgs;       /* the target actually used */
    int64_t workspace_bytes;
} paged_decode_plan_info;

int paged_decode_plan(int32_t batch, const int32_t *indptr,
                      int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t dtype, int32_t page_size, int32_t target_wgs,
                      int32_t fixed_pages_per_chunk,
                      int32_t capacity, int32_t *request_indices,
                      int32_t *kv_tile_indices, int32_t *o_indptr,
                      paged_decode_plan_info *info);

/* ------------------------------------------------------------------------
 * paged_decode_partial -- PR #984 kernel commit and body item 2; issue #898
 * items 1 and 2; sparse-paged-decode doc "Indirection".
 *
 * One unit per (chunk n, KV head g): it attends the G = Hq/Hkv query heads
 * of KV head g of request r = request_indices[n] over that chunk's visible
 * tokens, reading every K and V row once for all G heads.  A unit is one
 * wave (or a few, for small head counts); a workgroup takes 1 to 8 KV heads
 * of one chunk.  Visible
 * token i of request r lives in page indices[indptr[r] + (fpo_r + i) /
 * page_size] at entry (fpo_r + i) % page_size; the chunk t =
 * kv_tile_indices[n] covers tokens [max(0, t*c*ps - fpo_r), min(n_r,
 * (t+1)*c*ps - fpo_r)).  Scores are q.k * sm_scale (sm_scale in natural
 * units, e.g. 1/sqrt(D)), evaluated in base 2; the output row is normalized
 * by its own softmax denominator and its LSE is in log2 units.  A chunk with
 * no visible token writes zeros and -inf.
 *
 * Layouts (DEVICE): q [batch, Hq, D] contiguous; k_pool and v_pool share
 * element strides: element d of token entry e of page p, KV head g is at
 * p*page_stride + e*token_stride + g*head_stride + d (D contiguous); this
 * covers the [pages, page_size, Hkv, D] pool and the page_size=1 view of a
 * dense [B, H, Cap, D] allocation.  q and the pools share `dtype`
 * (PD_DTYPE_FP16 or PD_DTYPE_FP32) and must be 16-byte aligned, strides
 * multiples of 16 bytes.  indices/indptr/last_page_len/first_page_offset
 * are the (validated) CSR; request_indices/kv_tile_indices the plan's.
 * Outputs: v_partial [num_chunks, Hq, D] fp32 and lse_partial [num_chunks,
 * Hq] fp32.  Supported: D in {64, 128} with G in {1, 2, 4, 8, 12, 16};
 * and G in {24, 32} for fp16, at any page size (the MFMA kernels;
 * paged_decode_kernel_kind() tells which kernel serves a shape).
 * Other shapes return PD_E_UNSUPPORTED before any launch.
 * ---------------------------------------------------------------------- */
int paged_decode_partial(const void *q, const void *k_pool, const void *v_pool,
                         int64_t page_stride, int64_t token_stride, int64_t head_stride,
                         int32_t dtype,
                         const int32_t *indices, const int32_t *indptr,
                         const int32_t *last_page_len, const int32_t *first_page_offset,
                         const int32_t *request_indices, const int32_t *kv_tile_indices,
                         int32_t num_chunks, int32_t pages_per_chunk, int32_t batch,
                         int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, float sm_scale,
                         float *v_partial, float *lse_partial, void *stream);

/* ------------------------------------------------------------------------
 * paged_decode_fused -- the partial and the merge in one launch (PR #984 body
 * item 5 "write O directly" for single-chunk requests; issue #898 items 2-3).
 *
 * Same inputs as paged_decode_partial; the fused launch runs the page and
 * token kernels only, so G in {24, 32} returns PD_E_UNSUPPORTED here.  A
 * request with one chunk writes its
 * result straight to out[r] / lse_out[r].  A request with several chunks
 * writes its partial rows to v_partial / lse_partial (as paged_decode_partial
 * would), then the last of its workgroups to finish -- counted per (request,
 * KV head) in `counters` with agent-scope atomics -- merges them into out[r]
 * exactly as paged_merge_states does and sets its counter back to zero.
 * DEVICE: counters int32 [batch * num_kv_heads], all zero before the first
 * call (zero them once; every completed launch leaves them zero again; after
 * an aborted launch zero them again); out [batch, Hq, D] fp32, lse_out
 * [batch, Hq] fp32 (log2).  request_indices must list every request's chunks
 * contiguously with tiles 0..k-1 in order (the plan's layout).  Launches that
 * share a counters buffer must not overlap in time.
 * ---------------------------------------------------------------------- */
int paged_decode_fused(const void *q, const void *k_pool, const void *v_pool,
                       int64_t page_stride, int64_t token_stride, int64_t head_stride,
                       int32_t dtype,
                       const int32_t *indices, const int32_t *indptr,
                       const int32_t *last_page_len, const int32_t *first_page_offset,
                       const int32_t *request_indices, const int32_t *kv_tile_indices,
                       int32_t num_chunks, int32_t pages_per_chunk, int32_t batch,
                       int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t page_size, float sm_scale,
                       float *v_partial, float *lse_partial, int32_t *counters,
                       float *out, float *lse_out, void *stream);

/* ------------------------------------------------------------------------
 * paged_decode_fused_noalloc -- paged_decode_fused for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Same arguments, semantics and outputs as paged_decode_fused, without the
 * v_partial, lse_partial and counters buffers: the library keeps that
 * workspace in a file-scope device array of 16 MiB (one copy per GPU, held
 * until the process ends).  The call allocates nothing and frees nothing.
 * The workspace needs N*Hq*D*4 + N*Hq*4 + B*Hkv*4 bytes (each part rounded
 * up to 256); a plan that needs more returns PD_E_CAPACITY before any launch
 * (use paged_decode_fused with caller-owned buffers then).  Each call first
 * zeroes the counters on the caller's stream with a small kernel, so it does
 * not depend on what an earlier call left.  All calls on one GPU share the
 * array: calls that overlap in time on one GPU (two streams, two threads)
 * race and give wrong results; calls on one stream are ordered and safe.
 * ---------------------------------------------------------------------- */
int paged_decode_fused_noalloc(const void *q, const void *k_pool, const void *v_pool,
                               int64_t page_stride, int64_t token_stride, int64_t head_stride,
                               int32_t dtype,
                               const int32_t *indices, const int32_t *indptr,
                               const int32_t *last_page_len, const int32_t *first_page_offset,
                               const int32_t *request_indices, const int32_t *kv_tile_indices,
                               int32_t num_chunks, int32_t pages_per_chunk, int32_t batch,
                               int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t page_size, float sm_scale, float *out, float *lse_out,
                               void *stream);

/* ------------------------------------------------------------------------
 * paged_merge_states -- PR #984 body item 3; issue #898 item 3;
 * cascade-attention doc "Softmax states compose".
 *
 * For output row o and head h, combines input rows i in [o_indptr[o],
 * o_indptr[o+1]): m = max_i lse_in[i,h] over finite values, w_i = 2^(lse_i -
 * m), v_out[o,h,:] = sum_i w_i v_in[i,h,:] / sum_i w_i, lse_out[o,h] = m +
 * log2(sum_i w_i).  Rows with lse = -inf carry no weight; a group with no
 * finite row (or no row) gives zeros and -inf.  A NaN lse propagates.
 * DEVICE: v_in [N, H, D] fp32 (each row already normalized), lse_in [N, H]
 * fp32, o_indptr [num_out_rows+1] int32 (non-decreasing, o_indptr[M] <= N),
 * v_out [M, H, D], lse_out [M, H].  Any D >= 1.
 * ---------------------------------------------------------------------- */
int paged_merge_states(const float *v_in, const float *lse_in, const int32_t *o_indptr,
                       int32_t num_out_rows, int32_t num_heads, int32_t head_dim,
                       float *v_out, float *lse_out, void *stream);

/* ------------------------------------------------------------------------
 * Cascade decode -- mlxcel cascade-attention doc.
 *
 * A page span shared by several requests is attended once (level 0) instead
 * of once per request; every request's own pages are attended per request
 * (level 1); one merge finishes the step.
 *
 * paged_cascade_detect (HOST arrays; the doc's detection section): page i
 *   of two requests is shared when both hold the same pool row there
 *   (positional comparison of `indices`).  Candidates are the requests with
 *   at least one page and first_page_offset 0, grouped by their first page.
 *   A group's span is the number of leading positions on which all members
 *   agree, capped at (pages - 1) of every member (the last page may be
 *   partial, level 0's pages are full).  Groups with fewer than min_members
 *   members or a span below min_shared_pages are dropped; of the rest, the
 *   one with the largest span * (members - 1) wins (ties: the group whose
 *   first member comes first).  Out: member_req[0 .. *num_members) the
 *   members in ascending request order (room for `batch`), *shared_pages the
 *   span; *num_members = *shared_pages = 0 when nothing qualifies.
 *   min_shared_pages >= 1 and min_members >= 2 (the doc's defaults: 16, 2).
 *
 * paged_cascade_split (HOST): the two levels' page tables.  Level 0 is one
 *   request of `shared_pages` full pages: indices0 [shared_pages] (its
 *   indptr is {0, shared_pages}, last_page_len {page_size},
 *   first_page_offset {0}).  Level 1 keeps every request: a member keeps the
 *   pages after the span (first_page_offset 0), a non-member its whole list;
 *   indptr1 [batch+1], indices1 [indptr[batch] - num_members*shared_pages],
 *   last_page_len1 / first_page_offset1 [batch].  PD_E_ARG if member_req is
 *   not ascending, or a member starts mid-page, holds no page after the
 *   span, or does not hold the span.
 *
 * paged_cascade_layout (HOST): the merge input's row layout.  Request r's
 *   group is [o_indptr[r], o_indptr[r+1]): first its level0_rows level-0
 *   rows when it is a member, then its level-1 rows (o_indptr1 = the level-1
 *   plan's o_indptr).  Out: dst0 [num_members] (first row of member m's
 *   level-0 rows), dst1 [o_indptr1[batch]] (row of level-1 chunk n),
 *   o_indptr [batch+1].
 *
 * paged_cascade_stack_q (DEVICE): q [B, Hq, D] -> q0 [1, members*Hq, D];
 *   stacked head h0 = kv*(members*G) + m*G + g holds query head kv*G + g of
 *   request member_req[m] (member_req: DEVICE [members], or NULL for
 *   members 0..members-1), so the kernel's head-to-KV-head rule
 *   h0 / (members*G) reads KV head kv (the doc's head stacking; stacking
 *   member-major instead reads the wrong KV heads).
 *
 * paged_cascade_gather_states (DEVICE): the merge input.  Level-0 row i
 *   (v0 [n0, members*Hq, D], lse0 [n0, members*Hq]) is un-stacked into row
 *   dst0[m] + i for every member m; level-1 row n (v1 [n1, Hq, D], lse1
 *   [n1, Hq]) goes to row dst1[n].  v_dst / lse_dst [rows, Hq, D] / [rows,
 *   Hq] fp32 with rows = o_indptr[batch] of the layout.  dst0, dst1: DEVICE
 *   copies of the layout's arrays.  head_dim % 4 == 0 and 16-byte aligned buffers
 *   (PD_E_UNSUPPORTED otherwise).
 *
 * paged_cascade_merge_layout (HOST): where the level-0 rows of each request
 *   sit when the stacked launches write one buffer, launch after launch.
 *   Members are stacked members_per_launch at a time in member_req order, so
 *   launch j stacks S_j = min(members_per_launch, num_members - j *
 *   members_per_launch) members and holds level0_rows x S_j*Hq rows of D
 *   floats ([level0_rows, S_j*Hq, D], the partial kernel's output for that
 *   launch), starting at row j * members_per_launch * level0_rows * Hq.
 *   Out: l0_desc [batch, 3] int32 = (that first row, S_j, the request's
 *   position in its launch) for a member, (0, 0, -1) for a non-member.
 *   PD_E_ARG if member_req is not ascending within [0, batch) or the rows
 *   exceed int32.
 *
 * paged_cascade_merge_states (DEVICE, caller's stream): the cascade's
 *   merge, read in place (the same algebra as paged_merge_states).  Output
 *   row r, head h = kv*G + g merges, in this order, the request's level-0
 *   rows i < n0 (members only: row first + i*S*Hq + kv*S*G + p*G + g of v0 /
 *   lse0, with (first, S, p) = l0_desc[r]) and its level-1 rows
 *   o_indptr1[r] .. o_indptr1[r+1] of v1 [n1, Hq, D] / lse1 [n1, Hq].  This
 *   is paged_cascade_gather_states followed by paged_merge_states without
 *   the intermediate copy.  l0_desc, o_indptr1: DEVICE.  v_out [batch, Hq,
 *   D], lse_out [batch, Hq] fp32 (log2), not aliasing the inputs.
 *   head_dim % 32 == 0 and 16-byte aligned V buffers, else
 *   PD_E_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
/* ------------------------------------------------------------------------
 * paged_cascade_partial -- the cascade step's partial work (cascade-attention
 * doc, head stacking; the partial itself is paged_decode_partial's).
 *
 * Level 0 attends the shared span once for all `members` requests with
 * their query heads stacked, in L = ceil(members / members_per_launch)
 * tables: table j stacks members [j*per, min(members, (j+1)*per)) (per =
 * members_per_launch; S_j of them), and its stacked head h0 = kv*(S_j*G) +
 * m*G + g is query head kv*G + g of request member_req[j*per + m], read
 * straight from q [batch, Hq, D] (no stacked copy of q is made).  Table j's
 * rows are [level0[j].num_chunks, S_j*Hq, D], exactly what
 * paged_decode_partial would write for those stacked queries.  Level 1
 * (nullable) is the per-request level: every request's own pages, queries q
 * as they are, rows [level1->num_chunks, Hq, D].  Each table brings its
 * validated page table and its plan (paged_decode_plan with num_qo_heads =
 * S_j*Hq for level 0).  When every stacked group runs on the MFMA kernel
 * (fp16, head_dim 128, S_j*G in {8, 12, 16, 24, 32}, page_size a
 * power-of-two multiple of 16) and G <= 16, all tables run in one grid
 * (up to 8 tables per launch), workgroups [W_{i-1}, W_i) on table i, so
 * that no level's grid has to fill the GPU alone; otherwise each table is
 * one launch of the kernel paged_decode_partial would pick.
 * heads_per_workgroup: KV heads per workgroup of the one-grid form (1, 2, 4
 * or 8 dividing num_kv_heads), or 0 for one:
 * the shared level has few chunks, and narrow workgroups spread it over
 * more CUs.
 * DEVICE: q, pools (strides, dtype and alignment as paged_decode_partial),
 * member_req [members] (requests in [0, batch)), and every pointer inside
 * the level structs.  HOST: the structs themselves (level0 is an array of
 * L), read before the call returns.
 * ---------------------------------------------------------------------- */
typedef struct {
    const int32_t *indices, *indptr, *last_page_len, *first_page_offset;
    const int32_t *request_indices, *kv_tile_indices;
    int32_t batch;            /* requests of this table's page table */
    int32_t num_chunks, pages_per_chunk;
    float *v_partial;         /* [num_chunks, heads, D] fp32 */
    float *lse_partial;       /* [num_chunks, heads] fp32, log2 */
} paged_cascade_level;

int paged_cascade_partial(const void *q, int32_t batch, const int32_t *member_req,
                          int32_t members, int32_t members_per_launch, const void *k_pool,
                          const void *v_pool, int64_t page_stride, int64_t token_stride,
                          int64_t head_stride, int32_t dtype, int32_t num_qo_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                          float sm_scale, const paged_cascade_level *level0,
                          const paged_cascade_level *level1, int32_t heads_per_workgroup,
                          void *stream);

int paged_cascade_detect(int32_t batch, const int32_t *indptr, const int32_t *indices,
                         const int32_t *first_page_offset, int32_t min_shared_pages,
                         int32_t min_members, int32_t *member_req, int32_t *num_members,
                         int32_t *shared_pages);

int paged_cascade_split(int32_t batch, int32_t page_size, const int32_t *indptr,
                        const int32_t *indices, const int32_t *last_page_len,
                        const int32_t *first_page_offset, const int32_t *member_req,
                        int32_t num_members, int32_t shared_pages, int32_t *indices0,
                        int32_t *indptr1, int32_t *indices1, int32_t *last_page_len1,
                        int32_t *first_page_offset1);

int paged_cascade_layout(int32_t batch, const int32_t *member_req, int32_t num_members,
                         int32_t level0_rows, const int32_t *o_indptr1, int32_t *dst0,
                         int32_t *dst1, int32_t *o_indptr);

int paged_cascade_stack_q(const void *q, int32_t dtype, const int32_t *member_req,
                          int32_t members, int32_t num_qo_heads, int32_t num_kv_heads,
                          int32_t head_dim, void *q0, void *stream);

int paged_cascade_gather_states(const float *v0, const float *lse0, int32_t n0,
                                int32_t members, const int32_t *dst0, const float *v1,
                                const float *lse1, int32_t n1, const int32_t *dst1,
                                int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                float *v_dst, float *lse_dst, void *stream);

int paged_cascade_merge_layout(int32_t batch, const int32_t *member_req, int32_t num_members,
                               int32_t members_per_launch, int32_t level0_rows,
                               int32_t num_qo_heads, int32_t *l0_desc);

int paged_cascade_merge_states(const float *v0, const float *lse0, int32_t n0,
                               const int32_t *l0_desc, const float *v1, const float *lse1,
                               const int32_t *o_indptr1, int32_t batch, int32_t num_qo_heads,
                               int32_t num_kv_heads, int32_t head_dim, float *v_out,
                               float *lse_out, void *stream);

/* ------------------------------------------------------------------------
 * Block selections -- mlxcel "Sparse paged decode" doc (the two page-table
 * granularities and the block-to-token expansion).
 *
 * A sparse-attention model selects, per request (one per (sequence, KV head)
 * after folding), blocks_per_request blocks of block_size positions; the
 * request's last listed block is its final, partially written block and holds
 * tail[r] in [1, block_size] positions.
 *
 * paged_sparse_csr (HOST): the page table's shape, which needs no selection
 *   values.  The table names every selected block by s = block_size /
 *   page_size pages of page_size rows (page_size must divide block_size):
 *   page_size = block_size is the doc's block-granular table (one page per
 *   block), page_size = 1 the token-exact one, and sizes between read the
 *   same whole blocks while letting the plan cut chunks smaller than a block.
 *   Request r holds (blocks-1)*s + ceil(tail[r] / page_size) pages, the last
 *   holding tail[r] - (that count - 1)*page_size positions (last_page_len).
 *   first_page_offset 0.  Out: indptr [R+1], last_page_len [R],
 *   first_page_offset [R].  A page_size that does not divide block_size, or a
 *   tail outside [1, block_size], returns PD_E_ARG.
 *
 * paged_sparse_expand_blocks (DEVICE arrays, caller's stream): one pass over
 *   the selection.  Block j of request r (block_ids [R, blocks], int32)
 *   becomes rows base[r] + id*span + t for t < span, written from
 *   rows[out_indptr[r] + j*span]; the last block writes only final_rows[r]
 *   rows.  span = block_size / page_size (pages per block) over a pool read
 *   in pages of page_size rows, whose page of block j, piece t, of request r
 *   is base[r] + j*span + t; final_rows[r] = ceil(tail[r] / page_size).
 *   Block ids must lie in [0, num_blocks); an id outside is clamped into it,
 *   so the rows never leave the request's region of the pool.
 *   base, final_rows [R]; out_indptr [R+1] (the table's indptr); rows
 *   [out_indptr[R]].
 * ---------------------------------------------------------------------- */
int paged_sparse_csr(int32_t num_requests, int32_t blocks_per_request, int32_t block_size,
                     int32_t page_size, const int32_t *tail, int32_t *indptr,
                     int32_t *last_page_len, int32_t *first_page_offset);

int paged_sparse_expand_blocks(const int32_t *block_ids, int32_t num_requests,
                               int32_t blocks_per_request, const int32_t *base, int32_t span,
                               const int32_t *final_rows, const int32_t *out_indptr,
                               int32_t num_blocks, int32_t *rows, void *stream);

/* ------------------------------------------------------------------------
 * paged_mla_decode_partial -- sparse-paged-decode doc, the DSA section (the
 * recommended kernel generalization: a row stride plus a second key stream,
 * as paged-MLA kernels take a latent and a rope part).
 *
 * The decode-v2 partial with one KV head and two key streams: for visible
 * token t of request r (page table as in paged_decode_partial) and query head
 * h, score = sm_scale * (q[r,h,:] . k[t][0:dim]) + sm_scale * (q_extra[r,h,:]
 * . k_extra[t][0:extra_dim]), evaluated in base 2; the values are the latent
 * rows k[t][0:dim] themselves (the latent serves as key and value, the
 * output projection is applied by the caller).  Output rows are normalized
 * per chunk with log2 LSEs, exactly like paged_decode_partial, so
 * paged_merge_states (head_dim = dim) finishes split requests.
 *
 * Layouts (DEVICE): q [batch, Hq, dim] and q_extra [batch, Hq, extra_dim]
 * contiguous fp16; k_pool element (page p, entry e, d) at p*k_page_stride +
 * e*k_token_stride + d, the row holding at least `dim` elements (e.g. the
 * latent followed by an indexer key: a row stride of 640 for dim 512);
 * k_extra_pool likewise with x_page_stride / x_token_stride.  Both pools are
 * addressed through the same indices: page_size 1 views of dense [B, Cap,
 * row] allocations and [pages, page_size, row] pools both fit.  Pointers
 * 16-byte aligned, strides multiples of 8 elements.  The plan comes from
 * paged_decode_plan(head_dim = dim, num_kv_heads = 1).  Outputs: v_partial
 * [num_chunks, Hq, dim] fp32, lse_partial [num_chunks, Hq] fp32; an empty
 * chunk writes zeros and -inf.
 *
 * Supported: dtype PD_DTYPE_FP16, dim 512, extra_dim 64, Hq in {16, 32, 64,
 * 128}; anything else returns PD_E_UNSUPPORTED before any launch.  Launch
 * errors return PD_E_HIP; device faults surface at the next synchronization.
 * ---------------------------------------------------------------------- */
int paged_mla_decode_partial(const void *q, const void *q_extra, const void *k_pool,
                             const void *k_extra_pool, int64_t k_page_stride,
                             int64_t k_token_stride, int64_t x_page_stride,
                             int64_t x_token_stride, int32_t dim, int32_t extra_dim,
                             int32_t dtype, const int32_t *indices, const int32_t *indptr,
                             const int32_t *last_page_len, const int32_t *first_page_offset,
                             const int32_t *request_indices, const int32_t *kv_tile_indices,
                             int32_t num_chunks, int32_t pages_per_chunk, int32_t batch,
                             int32_t num_qo_heads, int32_t page_size, float sm_scale,
                             float *v_partial, float *lse_partial, void *stream);

/* ------------------------------------------------------------------------
 * Helpers shared by the plan and the launcher, so the two cannot drift
 * (PR #984 kernel commit: the query-heads-per-workgroup and wave-count
 * helpers exported next to the kernels).
 * ---------------------------------------------------------------------- */
/* Query heads one workgroup serves for group size G and head dim D (G: one
 * workgroup per KV head; head_dim 512, the paged-MLA kernel: min(G, 64)), or
 * a negative code if unsupported. */
int paged_decode_q_heads_per_wg(int32_t group_size, int32_t head_dim, int32_t dtype);

/* (chunk, KV head) units the device holds resident at once for this shape:
 * compute units x resident partial-kernel workgroups per CU (HIP occupancy
 * query) x units per workgroup, on `device` (-1: the current device).
 * head_dim 512 with one KV head counts paged-MLA workgroups.  Returns the
 * count, or a negative code. */
int paged_decode_default_target_wgs(int32_t device, int32_t group_size, int32_t head_dim,
                                    int32_t dtype, int32_t num_kv_heads);

/* Which partial kernel paged_decode_partial launches for a shape:
 * 2 = MFMA kernel (fp16, head_dim 64 or 128, group 1, 2, 4, 8, 12, 16, 24
 *     or 32, page_size a power-of-two multiple of 16, in-page offsets below
 *     2^31 bytes);
 * 3 = any-page MFMA kernel (the same dtype, head_dim and groups at every
 *     other page size: a 16-token tile may span 16 pages);
 * 1 = page kernel (256-byte K/V rows, group 4, 8 or 16, page_size a
 *     power-of-two multiple of the 64/group slots of one step), for the
 *     shapes the MFMA kernels do not take (fp32 with head_dim 64, or fp16
 *     with paged_decode_set_kernel_choice(2));
 * 0 = token kernel (every other supported shape);
 * negative = unsupported (PD_E_UNSUPPORTED).
 * The answer follows paged_decode_set_kernel_choice().  Host only: no device
 * is touched. */
int paged_decode_kernel_kind(int32_t dtype, int32_t head_dim, int32_t group_size,
                             int32_t page_size, int64_t token_stride);

/* Testing hook: 1 routes every later launch in this process to the token
 * kernel, 2 keeps every launch off the MFMA kernel (page or token kernel),
 * 0 restores the normal choice; so every kernel can be checked on the same
 * shapes.  Other values return PD_E_ARG.  Not thread-safe with concurrent
 * launches. */
int paged_decode_set_kernel_choice(int32_t force_token_kernel);

/* Host evaluation of the kernels' invariant-integer division by d
 * (Granlund & Montgomery 1994): q[i] = n[i] / d, r[i] = n[i] % d, for
 * n[i] < 2^31.  For testing the division on the CPU. */
int paged_fastdiv_eval(int32_t d, const uint32_t *n, int64_t count, uint32_t *q,
                       uint32_t *r);

/* Measurement helper: reads `bytes` (a positive multiple of 16) of the
 * DEVICE buffer `buf` (16-byte aligned) once with 16-byte loads
 * (non-temporal if `nontemporal`), in `num_wgs` workgroups of 512 threads
 * each streaming one contiguous segment, and writes one word per workgroup
 * to the DEVICE array sink [num_wgs] (so the loads cannot be dropped).  Timed
 * back to back over buffers larger than the last-level cache, it gives the
 * HBM read rate the GPU actually reaches -- the ceiling against which the
 * decode kernels' achieved bandwidth is compared. */
int paged_hbm_read_probe(const void *buf, int64_t bytes, int32_t num_wgs, int32_t nontemporal,
                         uint32_t *sink, void *stream);

/* Library version string. */
const char *pd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_DECODE_H */
