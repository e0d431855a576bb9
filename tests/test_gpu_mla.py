"""GPU parity of the paged-MLA / DSA decode (second key stream) against the
f64 oracle (needs an MI355X).

Every partial row and every final output is compared element by element
(fp16 pools, fp32 accumulation: max |diff| <= 2e-3 on outputs, <= 1e-3 on
log2 LSEs; -inf LSEs must match exactly); plans are the library's and are
checked against the oracle's exhaustive plan.  Unused pages, unselected rows
and the indexer-key columns of every row are NaN in the poisoned cases, so a
read outside the page table or past the latent shows up as NaN.  At full size
the oracle computes a sample of query heads.
"""
import os
import sys

import numpy as np
import pytest

from paged_attention_decode_amd import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from paged_attention_decode_amd import binding as B  # noqa: E402
from paged_attention_decode_amd import decode as PD  # noqa: E402

NTHREADS = min(16, os.cpu_count() or 1)
DEV = torch.device("cuda:0")
TOL_V, TOL_L = 2e-3, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check(got_v, got_l, ref_v, ref_l, what):
    got_v = np.asarray(got_v, np.float64)
    got_l = np.asarray(got_l, np.float64)
    assert got_v.shape == ref_v.shape and got_l.shape == ref_l.shape, what
    assert np.all(np.isfinite(got_v)), what + ": non-finite output"
    inf_ref = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), inf_ref), what + ": -inf LSE pattern differs"
    dv = float(np.max(np.abs(got_v - ref_v))) if got_v.size else 0.0
    fin = ~inf_ref
    dl = float(np.max(np.abs(got_l[fin] - ref_l[fin]))) if fin.any() else 0.0
    say("  %s: max|dv|=%.3g max|dlse|=%.3g" % (what, dv, dl))
    assert dv <= TOL_V, "%s: max |dv| %.3g" % (what, dv)
    assert dl <= TOL_L, "%s: max |dlse| %.3g" % (what, dl)


def run_mla(orc, w, *, fixed=0, target=0, heads=None, partial_rows=True):
    """Decode w on the GPU and compare with the oracle (all heads, or the
    given sample of query heads)."""
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                            w.k_pool.shape[0])
    dec = PD.MlaDecode(csr, page_size=w.page_size, num_pool_pages=w.k_pool.shape[0],
                       num_qo_heads=w.num_qo_heads, dim=w.dim, extra_dim=w.extra_dim,
                       target_wgs=target, fixed_pages_per_chunk=fixed)
    say("case %s B=%d Hq=%d ps=%d plan=%s" % (w.name, w.batch, w.num_qo_heads, w.page_size,
                                              dec.plan_summary()))
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                     w.page_size)
    for key in ("indptr", "indices", "last_page_len", "first_page_offset"):
        assert np.array_equal(np.asarray(csr[key]), ocsr[key]), key
    ref_plan = orc.plan(ocsr["indptr"], dec.info.q_groups, dec.info.target_wgs,
                        fixed_pages_per_chunk=fixed)
    assert dec.info.pages_per_chunk == ref_plan["pages_per_chunk"]
    assert np.array_equal(dec.request_indices, ref_plan["request_indices"])
    assert np.array_equal(dec.o_indptr, ref_plan["o_indptr"])
    q, qx = to_dev(w.q), to_dev(w.q_extra)
    k, kx = to_dev(w.k_pool), to_dev(w.k_extra_pool)
    for _ in range(2):                      # a second step reuses the buffers
        out, lse = dec.run(q, qx, k, kx, w.sm_scale)
    torch.cuda.synchronize()
    sel = np.arange(w.num_qo_heads) if heads is None else np.asarray(heads)
    qs = np.ascontiguousarray(w.q[:, sel])
    qxs = np.ascontiguousarray(w.q_extra[:, sel])
    ref_v, ref_l = orc.attention_mla(qs, qxs, w.k_pool, w.k_extra_pool, ocsr, w.page_size,
                                     w.sm_scale, nthreads=NTHREADS)
    check(out.cpu().numpy()[:, sel], lse.cpu().numpy()[:, sel], ref_v, ref_l, "output")
    if partial_rows and dec.info.needs_merge:
        pv, pl = orc.attention_mla(qs, qxs, w.k_pool, w.k_extra_pool, ocsr, w.page_size,
                                   w.sm_scale, chunks=(dec.request_indices, dec.kv_tile_indices,
                                                       dec.info.pages_per_chunk),
                                   nthreads=NTHREADS)
        check(dec.v_partial.cpu().numpy()[:, sel], dec.lse_partial.cpu().numpy()[:, sel],
              pv, pl, "partial rows")
    return dec


def test_mla_peaked_scores(orc):
    """Queries and rope queries scaled by 8: a few tokens carry most of each
    head's weight, where rounding the probabilities to fp16 for the value
    product would cost the most.  The kernel carries them as an fp16 part
    plus an fp16 remainder; partial rows must stay within a quarter of the
    fp16 tolerance."""
    w = workloads.mla_paged("mla_peaked", seed=321, logical_start=[0, 5], written_len=[900, 700],
                            num_qo_heads=128, page_size=16)
    w.q[:] = (w.q.astype(np.float32) * 8).astype(np.float16)
    w.q_extra[:] = (w.q_extra.astype(np.float32) * 8).astype(np.float16)
    dec = run_mla(orc, w, fixed=4)
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len, 16)
    pv, pl = orc.attention_mla(w.q, w.q_extra, w.k_pool, w.k_extra_pool, ocsr, 16, w.sm_scale,
                               chunks=(dec.request_indices, dec.kv_tile_indices,
                                       dec.info.pages_per_chunk), nthreads=NTHREADS)
    dv = float(np.max(np.abs(dec.v_partial.cpu().numpy() - pv)))
    fin = np.isfinite(pl)
    dl = float(np.max(np.abs(dec.lse_partial.cpu().numpy()[fin] - pl[fin])))
    say("  peaked scores: partial rows max|dv|=%.3g max|dlse|=%.3g" % (dv, dl))
    assert dv <= TOL_V / 4 and dl <= TOL_L / 4


@pytest.mark.parametrize("hq", [64, 128])
def test_mla_scores_ramp_rescale_every_tile(orc, hq):
    """Rope keys rewritten so that head 0's scores rise by 0.6 log2 units per
    token (K_extra[t] = lambda_t * q_extra / |q_extra|; the latent rows, which
    are also the values, stay N(0,1)): its running max passes the lazy-rescale
    margin on every 32-token tile, so the accumulators are rescaled every
    time, over about 540 log2 units; the other heads see the same keys at
    random angles.  Outputs and every partial row against the oracle."""
    w = workloads.mla_paged("mla_ramp", seed=331, logical_start=[0, 5], written_len=[900, 700],
                            num_qo_heads=hq, page_size=16)
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len, 16)
    scale_log2 = w.sm_scale / np.log(2.0)
    kx = w.k_extra_pool.astype(np.float32)
    for r in range(w.batch):
        n = int(ocsr["seq_lens"][r])
        slots = ocsr["first_page_offset"][r] + np.arange(n)
        pages = ocsr["indices"][ocsr["indptr"][r] + slots // 16]
        qx = w.q_extra[r, 0].astype(np.float64)
        lam = 0.6 * np.arange(n) / (scale_log2 * np.linalg.norm(qx))
        row = (lam[:, None] * (qx / np.linalg.norm(qx))[None, :]).astype(np.float32)
        assert np.abs(row).max() < 6e4                       # inside the fp16 range
        kx[pages, slots % 16] = row
    w.k_extra_pool[:] = kx.astype(np.float16)
    run_mla(orc, w, fixed=4)


@pytest.mark.parametrize("hq", [16, 32, 64, 128])
@pytest.mark.parametrize("ps", [1, 16, 64, 128])
def test_mla_ragged_poisoned(orc, hq, ps):
    """Ragged batch: an empty request, windows starting mid-page, an exactly
    full last page, a single token; unused pages and indexer columns NaN;
    chunks of one page (every request split) and the default plan."""
    lens = [(0, 700), (13, 300), (0, 0), (0, 64 * 5), (37, 38)]
    w = workloads.mla_paged("mla_ragged", seed=100 + hq + ps,
                            logical_start=[a for a, _ in lens],
                            written_len=[b for _, b in lens], num_qo_heads=hq, page_size=ps,
                            poison_unused=True, poison_indexer=True)
    run_mla(orc, w, fixed=max(1, 48 // ps))
    run_mla(orc, w)


def test_dsa_selection_poisoned(orc):
    """DSA decode: top-k positions of a dense latent cache read as
    page_size-1 rows; every unselected row and the indexer columns NaN."""
    w = workloads.dsa_sparse_fp16(batch=3, capacity=8192, kv_len=8000, topk=1000,
                                  poison_unselected=True)
    run_mla(orc, w)
    run_mla(orc, w, fixed=64)


def test_mla_paged_full_size_sampled_heads(orc):
    """The benchmark geometry (4 requests x 32768 tokens, 128 heads, pages of
    64) in the launch configuration the benchmark times; the oracle computes
    heads from both q groups and every 16-head wave."""
    w = workloads.mla_paged_fp16()
    run_mla(orc, w, heads=[0, 21, 47, 63, 64, 90, 111, 127], partial_rows=False)


def test_dsa_full_size_sampled_heads(orc):
    w = workloads.dsa_sparse_fp16()
    run_mla(orc, w, heads=[0, 17, 50, 63, 64, 99, 127])


def test_mla_graph_replay_matches_eager(orc):
    """The MLA step captured in a HIP graph and replayed equals the eager
    step, replay after replay, with new queries written in between."""
    w = workloads.dsa_sparse_fp16(batch=2, capacity=4096, kv_len=4000, topk=512)
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                            w.k_pool.shape[0])
    dec = PD.MlaDecode(csr, page_size=1, num_pool_pages=w.k_pool.shape[0],
                       num_qo_heads=w.num_qo_heads)
    assert dec.info.needs_merge
    k, kx = to_dev(w.k_pool), to_dev(w.k_extra_pool)
    qs = [(w.q, w.q_extra),
          (workloads._normal(np.random.default_rng(5), w.q.shape, workloads.FP16),
           workloads._normal(np.random.default_rng(6), w.q_extra.shape, workloads.FP16))]
    qb, qxb = to_dev(w.q), to_dev(w.q_extra)
    eager = []
    for a, b in qs:
        qb.copy_(to_dev(a))
        qxb.copy_(to_dev(b))
        out, lse = dec.run(qb, qxb, k, kx, w.sm_scale)
        torch.cuda.synchronize()
        eager.append((out.cpu().numpy().copy(), lse.cpu().numpy().copy()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dec.run(qb, qxb, k, kx, w.sm_scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_g, lse_g = dec.run(qb, qxb, k, kx, w.sm_scale)
    torch.cuda.synchronize()
    for rep in range(4):
        a, b = qs[rep % 2]
        qb.copy_(to_dev(a))
        qxb.copy_(to_dev(b))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ev, el = eager[rep % 2]
        np.testing.assert_allclose(out_g.cpu().numpy(), ev, rtol=0, atol=1e-6)
        np.testing.assert_allclose(lse_g.cpu().numpy(), el, rtol=0, atol=1e-6)


def test_mla_autotune_times_every_candidate_and_stays_exact(orc):
    """Chunk-size autotune of the MLA decode on a DSA selection: every
    power-of-two candidate and the default plan's choice are timed, the
    fastest is kept, and its output matches the oracle."""
    w = workloads.dsa_sparse_fp16(batch=2, capacity=4096, kv_len=4000, topk=512)
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                            w.k_pool.shape[0])
    q, qx = to_dev(w.q), to_dev(w.q_extra)
    k, kx = to_dev(w.k_pool), to_dev(w.k_extra_pool)
    dec, table = PD.autotune_mla(csr, q, qx, k, kx, w.sm_scale, page_size=w.page_size,
                                 num_pool_pages=w.k_pool.shape[0],
                                 num_qo_heads=w.num_qo_heads, n=30)
    say("  autotune table: %s" % table)
    cs = [row["pages_per_chunk"] for row in table]
    assert cs == sorted(set(cs)) and {1, 2, 4, 256, 512} <= set(cs)
    fastest = min(table, key=lambda row: row["step_us"])
    assert dec.info.pages_per_chunk == fastest["pages_per_chunk"]
    out, lse = dec.run(q, qx, k, kx, w.sm_scale)
    torch.cuda.synchronize()
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                     w.page_size)
    ref_v, ref_l = orc.attention_mla(w.q, w.q_extra, w.k_pool, w.k_extra_pool, ocsr,
                                     w.page_size, w.sm_scale, nthreads=NTHREADS)
    check(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, "autotuned")


def test_mla_strided_pools(orc):
    """Pools that are views of wider allocations: each page holds one padding
    row, latent rows are 1024 halves apart and rope rows 96 apart, and every
    element outside the views is NaN -- the kernel must address rows by the
    caller's strides alone."""
    w = workloads.mla_paged("mla_strided", seed=321, logical_start=[0, 5, 0, 40],
                            written_len=[500, 260, 1, 41], num_qo_heads=64, page_size=16,
                            poison_unused=True, poison_indexer=True)
    pages, ps = w.k_pool.shape[0], w.page_size
    kw = np.full((pages, ps + 1, 1024), np.nan, np.float16)
    kw[:, :ps, :w.k_pool.shape[2]] = w.k_pool
    xw = np.full((pages, ps + 1, 96), np.nan, np.float16)
    xw[:, :ps, :w.extra_dim] = w.k_extra_pool
    k = to_dev(kw)[:, :ps, :w.k_pool.shape[2]]
    kx = to_dev(xw)[:, :ps, :w.extra_dim]
    assert k.stride() == ((ps + 1) * 1024, 1024, 1) and kx.stride() == ((ps + 1) * 96, 96, 1)
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, ps, pages)
    for fixed in (0, 2):
        dec = PD.MlaDecode(csr, page_size=ps, num_pool_pages=pages, num_qo_heads=w.num_qo_heads,
                           fixed_pages_per_chunk=fixed)
        out, lse = dec.run(to_dev(w.q), to_dev(w.q_extra), k, kx, w.sm_scale)
        torch.cuda.synchronize()
        ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len, ps)
        ref_v, ref_l = orc.attention_mla(w.q, w.q_extra, w.k_pool, w.k_extra_pool, ocsr, ps,
                                         w.sm_scale, nthreads=NTHREADS)
        check(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, "strided c=%d" % fixed)
