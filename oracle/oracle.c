/*
 * f64 CPU oracle for fused paged-attention decode v2.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * tests, the smoke check and the benchmark's CPU-baseline leg compare the HIP
 * library against.  It shares no source, header, table or helper with that
 * library and must never be called from the product path.
 *
 * Everything here is the plain definition, written out in the most direct
 * way: tokens are gathered one by one through the page table, attention is a
 * naive two-pass softmax in double precision with natural exp/log, and the
 * plan is a linear scan over every chunk size.  Sources (the mlxcel pages):
 *
 *   - PR #984 "fused paged-attention decode v2", commit "cache::paged_csr":
 *     the CSR page table (indices / indptr / last_page_len plus
 *     first_page_offset), the geometry identity
 *     (pages-1)*page_size + last_page_len - first_page_offset == seq_len,
 *     exactly-full last pages, retired pages dropped.
 *   - sparse-paged-decode doc, "Indirection": visible token i of request r
 *     lives in page indices[indptr[r] + (first_page_offset[r]+i)/page_size]
 *     at entry (first_page_offset[r]+i) % page_size.
 *   - issue #898 "four composable pieces" item 3 and the cascade-attention
 *     doc "Softmax states compose": the merge of normalized partial states
 *     with base-2 log-sum-exp weights.
 *   - PR #984 body, "What changed" items 3 and 4: an empty partial has
 *     lse = -inf and contributes nothing; a group with no finite partial
 *     gives zeros and -inf; the plan takes the largest pages-per-chunk whose
 *     workgroup count still reaches the target, never emits more than 65535
 *     chunks, gives every request at least one chunk, and emits chunks in
 *     request order.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD (-1)
#define ORC_NOMEM (-2)

/* ------------------------------------------------------------------ */
/* Exact widening of IEEE-754 binary16 to double (from the format's     */
/* definition: 1 sign bit, 5 exponent bits with bias 15, 10 fraction).  */
/* ------------------------------------------------------------------ */
static double half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), expo - 25);  /* (1 + frac/1024) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

double orc_half_to_double(uint16_t h) { return half_to_double(h); }

/* element e of an array of the given dtype (0 = fp16, 1 = fp32), as double */
static double elem(const void *base, int dtype, int64_t e)
{
    if (dtype == 0)
        return half_to_double(((const uint16_t *)base)[e]);
    return (double)((const float *)base)[e];
}

/* ------------------------------------------------------------------ */
/* O5: CSR page table from block tables, by enumerating every visible  */
/* token and recording which page and entry it lands in.               */
/* ------------------------------------------------------------------ */
int orc_csr_from_block_tables(int32_t batch, int32_t page_size,
                              const int32_t *bt_offsets, /* [B+1] into bt */
                              const int32_t *bt,          /* logical block -> page, -1 = released */
                              const int32_t *logical_start, const int32_t *written_len,
                              int32_t capacity,
                              int32_t *indptr, int32_t *indices,
                              int32_t *last_page_len, int32_t *first_page_offset,
                              int32_t *seq_lens, int32_t *rope_offsets)
{
    if (batch < 0 || page_size < 1) return ORC_BAD;
    int32_t nnz = 0;
    indptr[0] = 0;
    for (int32_t r = 0; r < batch; ++r) {
        int32_t ls = logical_start[r], wl = written_len[r];
        int32_t nblocks = bt_offsets[r + 1] - bt_offsets[r];
        if (ls < 0 || wl < ls) return ORC_BAD;
        int32_t count = 0, prev_block = -1, first_entry = 0, last_entry = 0;
        for (int32_t pos = ls; pos < wl; ++pos) {
            int32_t block = pos / page_size, entry = pos % page_size;
            if (block >= nblocks) return ORC_BAD;
            if (block != prev_block) {            /* the token opens a new page */
                int32_t page = bt[bt_offsets[r] + block];
                if (page < 0) return ORC_BAD;     /* a visible token in a released page */
                if (nnz >= capacity) return ORC_BAD;
                indices[nnz++] = page;
                prev_block = block;
            }
            if (count == 0) first_entry = entry;
            last_entry = entry;
            ++count;
        }
        indptr[r + 1] = nnz;
        seq_lens[r] = count;
        rope_offsets[r] = wl;
        first_page_offset[r] = count ? first_entry : 0;
        last_page_len[r] = count ? last_entry + 1 : 0;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* O1 / O2: attention of query head h of request r over its visible    */
/* tokens [tok_begin, tok_end), gathered one by one.                   */
/* ------------------------------------------------------------------ */
typedef struct {
    int32_t batch, hq, hkv, d, page_size, dtype;
    const int32_t *indptr, *indices, *lpl, *fpo;
    const void *q, *k, *v;
    int64_t page_stride, token_stride, head_stride;
    double sm_scale;
    /* partial mode */
    int32_t num_chunks, pages_per_chunk;
    const int32_t *request_indices, *kv_tile_indices;
    double *out, *lse2;
    int32_t num_units, nthreads, status;
} job_t;

static int64_t visible_tokens(const job_t *j, int32_t r)
{
    int64_t pages = j->indptr[r + 1] - j->indptr[r];
    if (pages == 0) return 0;
    return (pages - 1) * j->page_size + j->lpl[r] - j->fpo[r];
}

static int attend(const job_t *j, int32_t r, int32_t h, int64_t tok_begin, int64_t tok_end,
                  double *o, double *lse2)
{
    const int32_t d = j->d;
    const int32_t group = j->hq / j->hkv;
    const int32_t kvh = h / group;              /* query head h reads KV head h / group */
    const int64_t n = tok_end > tok_begin ? tok_end - tok_begin : 0;
    for (int32_t e = 0; e < d; ++e) o[e] = 0.0;
    if (n == 0) {
        *lse2 = -INFINITY;
        return ORC_OK;
    }
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    int64_t *rowbase = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!s || !rowbase) { free(s); free(rowbase); return ORC_NOMEM; }
    const int64_t qbase = ((int64_t)r * j->hq + h) * d;
    for (int64_t i = 0; i < n; ++i) {
        int64_t slot = j->fpo[r] + tok_begin + i;
        int64_t page_iter = slot / j->page_size;
        int64_t entry = slot % j->page_size;
        int64_t page = j->indices[j->indptr[r] + page_iter];
        int64_t base = page * j->page_stride + entry * j->token_stride + kvh * j->head_stride;
        rowbase[i] = base;
        double dot = 0.0;
        for (int32_t e = 0; e < d; ++e)
            dot += elem(j->q, j->dtype, qbase + e) * elem(j->k, j->dtype, base + e);
        s[i] = j->sm_scale * dot;
    }
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i) if (s[i] > m) m = s[i];
    double z = 0.0;
    for (int64_t i = 0; i < n; ++i) z += exp(s[i] - m);
    for (int64_t i = 0; i < n; ++i) {
        double w = exp(s[i] - m) / z;
        for (int32_t e = 0; e < d; ++e) o[e] += w * elem(j->v, j->dtype, rowbase[i] + e);
    }
    *lse2 = (m + log(z)) / log(2.0);
    free(s);
    free(rowbase);
    return ORC_OK;
}

static void *worker(void *arg)
{
    job_t *j = (job_t *)((void **)arg)[0];
    int32_t tid = (int32_t)(intptr_t)((void **)arg)[1];
    for (int32_t u = tid; u < j->num_units; u += j->nthreads) {
        int32_t row = u / j->hq, h = u % j->hq;
        int32_t r;
        int64_t tb, te;
        if (j->request_indices) {               /* partial: one chunk of pages */
            r = j->request_indices[row];
            int64_t t = j->kv_tile_indices[row];
            int64_t n_r = visible_tokens(j, r);
            int64_t span = (int64_t)j->pages_per_chunk * j->page_size;
            tb = t * span - j->fpo[r];
            te = (t + 1) * span - j->fpo[r];
            if (tb < 0) tb = 0;
            if (te > n_r) te = n_r;
        } else {                                /* whole request */
            r = row;
            tb = 0;
            te = visible_tokens(j, r);
        }
        int rc = attend(j, r, h, tb, te, j->out + (int64_t)u * j->d, j->lse2 + u);
        if (rc != ORC_OK) j->status = rc;
    }
    return NULL;
}

static int run(job_t *j, int32_t rows)
{
    if (j->hkv < 1 || j->hq % j->hkv != 0 || j->d < 1 || j->page_size < 1) return ORC_BAD;
    j->num_units = rows * j->hq;
    j->status = ORC_OK;
    int32_t nt = j->nthreads < 1 ? 1 : j->nthreads;
    if (nt > 256) nt = 256;
    j->nthreads = nt;
    pthread_t th[256];
    void *args[256][2];
    for (int32_t t = 0; t < nt; ++t) {
        args[t][0] = j;
        args[t][1] = (void *)(intptr_t)t;
        if (nt == 1) worker(args[t]);
        else pthread_create(&th[t], NULL, worker, args[t]);
    }
    if (nt > 1)
        for (int32_t t = 0; t < nt; ++t) pthread_join(th[t], NULL);
    return j->status;
}

/* O1: attention of every (request, query head) over all its visible tokens. */
int orc_attention(int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t page_size, int32_t dtype,
                  const int32_t *indptr, const int32_t *indices,
                  const int32_t *last_page_len, const int32_t *first_page_offset,
                  const void *q, const void *k_pool, const void *v_pool,
                  int64_t page_stride, int64_t token_stride, int64_t head_stride,
                  double sm_scale, double *out, double *lse2, int32_t nthreads)
{
    job_t j;
    memset(&j, 0, sizeof(j));
    j.batch = batch; j.hq = num_qo_heads; j.hkv = num_kv_heads; j.d = head_dim;
    j.page_size = page_size; j.dtype = dtype;
    j.indptr = indptr; j.indices = indices; j.lpl = last_page_len; j.fpo = first_page_offset;
    j.q = q; j.k = k_pool; j.v = v_pool;
    j.page_stride = page_stride; j.token_stride = token_stride; j.head_stride = head_stride;
    j.sm_scale = sm_scale; j.out = out; j.lse2 = lse2; j.nthreads = nthreads;
    return run(&j, batch);
}

/* O2: attention restricted to each chunk's token range.  Chunk n covers
 * pages [t*c, (t+1)*c) of request r = request_indices[n], t =
 * kv_tile_indices[n]; with the first page's offset that is visible tokens
 * [max(0, t*c*ps - fpo), min(n_r, (t+1)*c*ps - fpo)). */
int orc_partial(int32_t num_chunks, const int32_t *request_indices,
                const int32_t *kv_tile_indices, int32_t pages_per_chunk,
                int32_t num_qo_heads, int32_t num_kv_heads,
                int32_t head_dim, int32_t page_size, int32_t dtype,
                const int32_t *indptr, const int32_t *indices,
                const int32_t *last_page_len, const int32_t *first_page_offset,
                const void *q, const void *k_pool, const void *v_pool,
                int64_t page_stride, int64_t token_stride, int64_t head_stride,
                double sm_scale, double *out, double *lse2, int32_t nthreads)
{
    if (pages_per_chunk < 1) return ORC_BAD;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.hq = num_qo_heads; j.hkv = num_kv_heads; j.d = head_dim;
    j.page_size = page_size; j.dtype = dtype;
    j.indptr = indptr; j.indices = indices; j.lpl = last_page_len; j.fpo = first_page_offset;
    j.q = q; j.k = k_pool; j.v = v_pool;
    j.page_stride = page_stride; j.token_stride = token_stride; j.head_stride = head_stride;
    j.sm_scale = sm_scale; j.out = out; j.lse2 = lse2; j.nthreads = nthreads;
    j.num_chunks = num_chunks; j.pages_per_chunk = pages_per_chunk;
    j.request_indices = request_indices; j.kv_tile_indices = kv_tile_indices;
    return run(&j, num_chunks);
}

/* ------------------------------------------------------------------ */
/* O3: merge of normalized partial states.  For output row o and head  */
/* h the rows [o_indptr[o], o_indptr[o+1]) are combined with weights   */
/* 2^(lse_i - m), m the largest finite lse; rows with lse = -inf carry  */
/* no weight; with no finite row the result is 0 and -inf.              */
/* ------------------------------------------------------------------ */
int orc_merge(int32_t num_out, int32_t num_heads, int32_t head_dim,
              const double *v_in, const double *lse_in, const int32_t *o_indptr,
              double *v_out, double *lse_out)
{
    for (int32_t o = 0; o < num_out; ++o) {
        int32_t b = o_indptr[o], e = o_indptr[o + 1];
        if (e < b) return ORC_BAD;
        for (int32_t h = 0; h < num_heads; ++h) {
            double *vo = v_out + ((int64_t)o * num_heads + h) * head_dim;
            double m = -INFINITY;
            int nan_seen = 0;
            for (int32_t i = b; i < e; ++i) {
                double l = lse_in[(int64_t)i * num_heads + h];
                if (isnan(l)) nan_seen = 1;
                else if (l > m) m = l;
            }
            for (int32_t x = 0; x < head_dim; ++x) vo[x] = 0.0;
            if (nan_seen) {
                for (int32_t x = 0; x < head_dim; ++x) vo[x] = NAN;
                lse_out[(int64_t)o * num_heads + h] = NAN;
                continue;
            }
            if (m == -INFINITY) {
                lse_out[(int64_t)o * num_heads + h] = -INFINITY;
                continue;
            }
            double wsum = 0.0;
            for (int32_t i = b; i < e; ++i) {
                double l = lse_in[(int64_t)i * num_heads + h];
                if (l == -INFINITY) continue;
                double w = pow(2.0, l - m);
                wsum += w;
                const double *vi = v_in + ((int64_t)i * num_heads + h) * head_dim;
                for (int32_t x = 0; x < head_dim; ++x) vo[x] += w * vi[x];
            }
            for (int32_t x = 0; x < head_dim; ++x) vo[x] /= wsum;
            lse_out[(int64_t)o * num_heads + h] = m + log2(wsum);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* O4: plan by exhaustive scan over every pages-per-chunk value c.     */
/* chunks(c) = sum over requests of max(1, ceil(pages_r / c)).  A c is */
/* launchable when chunks(c) <= max_chunks.  Among launchable c, take  */
/* the largest whose workgroup count chunks(c) * wg_per_chunk reaches   */
/* the target; if none reaches it, the launchable c with the most      */
/* chunks (the smallest).  c ranges over 1 .. max(1, max_r pages_r):   */
/* beyond that chunks(c) no longer changes.                            */
/* ------------------------------------------------------------------ */
static int64_t chunks_for(int32_t batch, const int32_t *indptr, int64_t c)
{
    int64_t total = 0;
    for (int32_t r = 0; r < batch; ++r) {
        int64_t pages = indptr[r + 1] - indptr[r];
        int64_t k = (pages + c - 1) / c;
        total += k < 1 ? 1 : k;
    }
    return total;
}

int orc_plan(int32_t batch, const int32_t *indptr, int64_t wg_per_chunk, int64_t target,
             int32_t fixed_pages_per_chunk, int64_t max_chunks,
             int32_t *pages_per_chunk, int32_t *num_chunks,
             int32_t *request_indices, int32_t *kv_tile_indices, int32_t *o_indptr,
             int32_t capacity)
{
    if (batch < 1) return ORC_BAD;
    int64_t cmax = 1;
    for (int32_t r = 0; r < batch; ++r) {
        int64_t pages = indptr[r + 1] - indptr[r];
        if (pages < 0) return ORC_BAD;
        if (pages > cmax) cmax = pages;
    }
    int64_t best = -1, smallest_ok = -1;
    if (fixed_pages_per_chunk > 0) {
        if (chunks_for(batch, indptr, fixed_pages_per_chunk) > max_chunks) return ORC_BAD;
        best = fixed_pages_per_chunk;
    } else {
        for (int64_t c = 1; c <= cmax; ++c) {
            int64_t n = chunks_for(batch, indptr, c);
            if (n > max_chunks) continue;
            if (smallest_ok < 0) smallest_ok = c;
            if (n * wg_per_chunk >= target) best = c;   /* keep the largest */
        }
        if (smallest_ok < 0) return ORC_BAD;            /* nothing launchable */
        if (best < 0) best = smallest_ok;
    }
    int64_t n = chunks_for(batch, indptr, best);
    if (n > capacity) return ORC_BAD;
    int32_t k = 0;
    o_indptr[0] = 0;
    for (int32_t r = 0; r < batch; ++r) {
        int64_t pages = indptr[r + 1] - indptr[r];
        int64_t tiles = (pages + best - 1) / best;
        if (tiles < 1) tiles = 1;
        for (int64_t t = 0; t < tiles; ++t) {
            request_indices[k] = r;
            kv_tile_indices[k] = (int32_t)t;
            ++k;
        }
        o_indptr[r + 1] = k;
    }
    *pages_per_chunk = (int32_t)best;
    *num_chunks = k;
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Cascade detection (cascade-attention doc, the detection section),   */
/* by brute force.  Candidates: requests with at least one page whose   */
/* window starts on a page boundary.  For every candidate a that is the */
/* first candidate (lowest request index) holding its first page, the   */
/* group is every candidate holding that same first page; its span is   */
/* the number of leading positions s for which every member still has  */
/* a page after position s (s < pages - 1) and holds at position s the  */
/* same pool row as a.  Groups below min_members members or below       */
/* min_shared pages are dropped; the largest span * (members - 1) wins, */
/* the earlier leader on ties.  Nothing qualifying: 0 members, 0 span.  */
/* ------------------------------------------------------------------ */
static int cascade_candidate(const int32_t *indptr, const int32_t *fpo, int32_t r)
{
    return indptr[r + 1] - indptr[r] >= 1 && fpo[r] == 0;
}

int orc_cascade_detect(int32_t batch, const int32_t *indptr, const int32_t *indices,
                       const int32_t *first_page_offset, int32_t min_shared_pages,
                       int32_t min_members, int32_t *member_req, int32_t *num_members,
                       int32_t *shared_pages)
{
    int64_t best_score = -1;
    int32_t best_leader = -1, best_span = 0;
    *num_members = 0;
    *shared_pages = 0;
    for (int32_t a = 0; a < batch; ++a) {
        if (!cascade_candidate(indptr, first_page_offset, a)) continue;
        const int32_t first = indices[indptr[a]];
        int leads = 1;
        for (int32_t b = 0; b < a; ++b)
            if (cascade_candidate(indptr, first_page_offset, b) && indices[indptr[b]] == first)
                leads = 0;
        if (!leads) continue;
        int32_t count = 0;
        for (int32_t b = a; b < batch; ++b)
            if (cascade_candidate(indptr, first_page_offset, b) && indices[indptr[b]] == first)
                ++count;
        int32_t span = 0;
        for (;;) {
            int all = 1;
            for (int32_t b = a; b < batch && all; ++b) {
                if (!cascade_candidate(indptr, first_page_offset, b) || indices[indptr[b]] != first)
                    continue;
                if (span >= indptr[b + 1] - indptr[b] - 1) all = 0;
                else if (indices[indptr[b] + span] != indices[indptr[a] + span]) all = 0;
            }
            if (!all) break;
            ++span;
        }
        if (count < min_members || span < min_shared_pages) continue;
        const int64_t score = (int64_t)span * (count - 1);
        if (score > best_score) {
            best_score = score;
            best_leader = a;
            best_span = span;
        }
    }
    if (best_leader < 0) return ORC_OK;
    const int32_t first = indices[indptr[best_leader]];
    for (int32_t b = best_leader; b < batch; ++b)
        if (cascade_candidate(indptr, first_page_offset, b) && indices[indptr[b]] == first)
            member_req[(*num_members)++] = b;
    *shared_pages = best_span;
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* O8: decode with a second key stream (sparse-paged-decode doc, the   */
/* DSA section: the score of a visible token t is                      */
/*   sm_scale * (q . k[t][0:Dim]) + sm_scale * (q_extra . k_extra[t]), */
/* with k read from rows of RowStride >= Dim elements and k_extra from */
/* a pool of its own with the same page table).  One KV head.  The     */
/* values are the first Dim elements of the k rows (the latent rows    */
/* serve as keys and values).  Chunk mode restricts each (chunk, head) */
/* to its chunk's token range, as orc_partial does.                    */
/* ------------------------------------------------------------------ */
typedef struct {
    int32_t hq, dim, extra_dim, page_size;
    const int32_t *indptr, *indices, *lpl, *fpo;
    const uint16_t *q, *q_extra, *k, *k_extra;          /* fp16 bit patterns */
    int64_t k_page_stride, k_token_stride, x_page_stride, x_token_stride;
    double sm_scale;
    int32_t pages_per_chunk;
    const int32_t *request_indices, *kv_tile_indices;
    double *out, *lse2;
    int32_t num_units, nthreads, status;
} mla_job_t;

static int64_t mla_visible(const mla_job_t *j, int32_t r)
{
    int64_t pages = j->indptr[r + 1] - j->indptr[r];
    if (pages == 0) return 0;
    return (pages - 1) * j->page_size + j->lpl[r] - j->fpo[r];
}

static int mla_attend(const mla_job_t *j, int32_t r, int32_t h, int64_t tb, int64_t te,
                      double *o, double *lse2)
{
    const int64_t n = te > tb ? te - tb : 0;
    for (int32_t e = 0; e < j->dim; ++e) o[e] = 0.0;
    if (n == 0) {
        *lse2 = -INFINITY;
        return ORC_OK;
    }
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    int64_t *kb = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!s || !kb) { free(s); free(kb); return ORC_NOMEM; }
    const int64_t qb = ((int64_t)r * j->hq + h) * j->dim;
    const int64_t xb = ((int64_t)r * j->hq + h) * j->extra_dim;
    for (int64_t i = 0; i < n; ++i) {
        int64_t slot = j->fpo[r] + tb + i;
        int64_t page = j->indices[j->indptr[r] + slot / j->page_size];
        int64_t entry = slot % j->page_size;
        int64_t krow = page * j->k_page_stride + entry * j->k_token_stride;
        int64_t xrow = page * j->x_page_stride + entry * j->x_token_stride;
        kb[i] = krow;
        double dot = 0.0, dot_x = 0.0;
        for (int32_t e = 0; e < j->dim; ++e)
            dot += half_to_double(j->q[qb + e]) * half_to_double(j->k[krow + e]);
        for (int32_t e = 0; e < j->extra_dim; ++e)
            dot_x += half_to_double(j->q_extra[xb + e]) * half_to_double(j->k_extra[xrow + e]);
        s[i] = j->sm_scale * dot + j->sm_scale * dot_x;
    }
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i) if (s[i] > m) m = s[i];
    double z = 0.0;
    for (int64_t i = 0; i < n; ++i) z += exp(s[i] - m);
    for (int64_t i = 0; i < n; ++i) {
        double w = exp(s[i] - m) / z;
        for (int32_t e = 0; e < j->dim; ++e) o[e] += w * half_to_double(j->k[kb[i] + e]);
    }
    *lse2 = (m + log(z)) / log(2.0);
    free(s);
    free(kb);
    return ORC_OK;
}

static void *mla_worker(void *arg)
{
    mla_job_t *j = (mla_job_t *)((void **)arg)[0];
    int32_t tid = (int32_t)(intptr_t)((void **)arg)[1];
    for (int32_t u = tid; u < j->num_units; u += j->nthreads) {
        int32_t row = u / j->hq, h = u % j->hq, r;
        int64_t tb, te;
        if (j->request_indices) {
            r = j->request_indices[row];
            int64_t t = j->kv_tile_indices[row];
            int64_t span = (int64_t)j->pages_per_chunk * j->page_size;
            tb = t * span - j->fpo[r];
            te = (t + 1) * span - j->fpo[r];
            if (tb < 0) tb = 0;
            if (te > mla_visible(j, r)) te = mla_visible(j, r);
        } else {
            r = row;
            tb = 0;
            te = mla_visible(j, r);
        }
        int rc = mla_attend(j, r, h, tb, te, j->out + (int64_t)u * j->dim, j->lse2 + u);
        if (rc != ORC_OK) j->status = rc;
    }
    return NULL;
}

/* rows = batch (whole requests) or num_chunks (chunk mode, request_indices
 * non-NULL).  q [B, Hq, Dim], q_extra [B, Hq, ExtraDim]; k element (page,
 * entry, e) at page*k_page_stride + entry*k_token_stride + e, likewise
 * k_extra with its own strides.  out [rows, Hq, Dim], lse2 [rows, Hq]. */
int orc_attention_mla(int32_t rows, int32_t num_qo_heads, int32_t dim, int32_t extra_dim,
                      int32_t page_size, const int32_t *indptr, const int32_t *indices,
                      const int32_t *last_page_len, const int32_t *first_page_offset,
                      const uint16_t *q, const uint16_t *q_extra, const uint16_t *k_pool,
                      const uint16_t *k_extra_pool, int64_t k_page_stride,
                      int64_t k_token_stride, int64_t x_page_stride, int64_t x_token_stride,
                      double sm_scale, const int32_t *request_indices,
                      const int32_t *kv_tile_indices, int32_t pages_per_chunk,
                      double *out, double *lse2, int32_t nthreads)
{
    if (rows < 0 || num_qo_heads < 1 || dim < 1 || extra_dim < 0 || page_size < 1)
        return ORC_BAD;
    mla_job_t j;
    memset(&j, 0, sizeof(j));
    j.hq = num_qo_heads; j.dim = dim; j.extra_dim = extra_dim; j.page_size = page_size;
    j.indptr = indptr; j.indices = indices; j.lpl = last_page_len; j.fpo = first_page_offset;
    j.q = q; j.q_extra = q_extra; j.k = k_pool; j.k_extra = k_extra_pool;
    j.k_page_stride = k_page_stride; j.k_token_stride = k_token_stride;
    j.x_page_stride = x_page_stride; j.x_token_stride = x_token_stride;
    j.sm_scale = sm_scale; j.pages_per_chunk = pages_per_chunk;
    j.request_indices = request_indices; j.kv_tile_indices = kv_tile_indices;
    j.out = out; j.lse2 = lse2;
    j.num_units = rows * num_qo_heads;
    j.status = ORC_OK;
    int32_t nt = nthreads < 1 ? 1 : (nthreads > 256 ? 256 : nthreads);
    j.nthreads = nt;
    pthread_t th[256];
    void *args[256][2];
    for (int32_t t = 0; t < nt; ++t) {
        args[t][0] = &j;
        args[t][1] = (void *)(intptr_t)t;
        if (nt == 1) mla_worker(args[t]);
        else pthread_create(&th[t], NULL, mla_worker, args[t]);
    }
    if (nt > 1)
        for (int32_t t = 0; t < nt; ++t) pthread_join(th[t], NULL);
    return j.status;
}
