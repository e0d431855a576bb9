"""GPU parity of the HIP path against the f64 oracle (needs an MI355X).

Every case feeds the same seeded inputs to both sides.  The HIP side builds
its page table and plan with the library; the oracle builds its own page table
by token enumeration and its own plan by exhaustive scan, and the two plans
must agree bit-exactly before any output is compared.  Final outputs and
every partial row are compared element by element:
  fp32 pools: max |diff| <= 1e-5 (outputs and log2 LSE);
  fp16 pools: max |diff| <= 2e-3 on outputs, <= 1e-3 on log2 LSE;
and -inf LSEs (empty chunks, empty requests) must match exactly.
Unused pool rows are NaN in the random cases, so a read outside the page
table shows up as NaN.
"""
import dataclasses
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tol(dtype):
    return (1e-5, 1e-5) if dtype == workloads.FP32 else (2e-3, 1e-3)


def check_close(got_v, got_l, ref_v, ref_l, dtype, what):
    tv, tl = tol(dtype)
    got_v = np.asarray(got_v, np.float64)
    got_l = np.asarray(got_l, np.float64)
    assert got_v.shape == ref_v.shape and got_l.shape == ref_l.shape, what
    assert np.all(np.isfinite(got_v)), what + ": non-finite output"
    dv = np.max(np.abs(got_v - ref_v)) if got_v.size else 0.0
    inf_ref = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), inf_ref), what + ": -inf LSE pattern differs"
    fin = ~inf_ref
    dl = np.max(np.abs(got_l[fin] - ref_l[fin])) if fin.any() else 0.0
    say("  %s: max|dv|=%.3g max|dlse|=%.3g" % (what, dv, dl))
    assert dv <= tv, "%s: max |dv| %.3g > %.3g" % (what, dv, tv)
    # the kernels store LSEs in fp32: one fp32 unit in the last place of the
    # reference (at most |lse| * 2^-23) is added to the bound, which only
    # matters where |lse| is in the hundreds (one ulp is 6.1e-5 at 737)
    over = np.abs(got_l[fin] - ref_l[fin]) - (tl + np.abs(ref_l[fin]) * 2.0 ** -23)
    assert not fin.any() or over.max() <= 0, "%s: max |dlse| %.3g > %.3g + 1 fp32 ulp" % (
        what, dl, tl)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


_WORKLOADS = {}


def cached(name, **kw):
    """Large workloads are generated once per session (tests only read them)."""
    key = (name, tuple(sorted(kw.items())))
    if key not in _WORKLOADS:
        _WORKLOADS[key] = getattr(workloads, name)(**kw)
    return _WORKLOADS[key]


# "auto" takes the default kernel (the MFMA kernels where they apply in the
# two-launch mode), "valu" every shape off the MFMA kernels, "token" every
# shape on the token kernel
MODES = [("auto", False), ("auto", True), ("token", False), ("token", True), ("valu", False)]
MODE_IDS = ["page-2launch", "page-fused", "token-2launch", "token-fused", "valu-2launch"]
CHOICE = {"auto": 0, "token": 1, "valu": 2}
KIND = {0: "token", 1: "page", 2: "mfma", 3: "mfma-any-page"}


@pytest.fixture(params=MODES, ids=MODE_IDS)
def mode(request):
    kernel, fused = request.param
    B.paged_decode_set_kernel_choice(CHOICE[kernel])
    yield dict(fused=fused, kernel=kernel)
    B.paged_decode_set_kernel_choice(0)


def run_flat(orc, w, target=0, fixed=0, check_partials=True, stream=None, fused=False,
             repeat=1):
    """HIP flat decode of workload w vs the oracle; returns the decoder."""
    say("case %s dtype=%s B=%d Hq=%d Hkv=%d D=%d ps=%d target=%d fixed=%d fused=%s" % (
        w.name, w.dtype, w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
        target, fixed, fused))
    pool_pages = w.k_pool.shape[0]
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                            pool_pages)
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                     w.page_size)
    for k in ocsr:
        assert np.array_equal(csr[k], ocsr[k]), k
    dec = PD.PagedDecode(csr, page_size=w.page_size, num_pool_pages=pool_pages,
                         num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                         head_dim=w.head_dim, target_wgs=target, fixed_pages_per_chunk=fixed,
                         fused=fused,
                         dtype=torch.float32 if w.dtype == workloads.FP32 else torch.float16)
    info = dec.info
    kind = B.paged_decode_kernel_kind(B.PD_DTYPE_FP16 if w.dtype == workloads.FP16 else
                                      B.PD_DTYPE_FP32, w.head_dim,
                                      w.num_qo_heads // w.num_kv_heads, w.page_size,
                                      w.k_pool.shape[2] * w.head_dim)
    say("  plan", dec.plan_summary(), "kernel", "fused-" if fused else "", KIND[kind])
    oplan = orc.plan(ocsr["indptr"], w.num_kv_heads, info.target_wgs,
                     fixed_pages_per_chunk=fixed)
    assert oplan["pages_per_chunk"] == info.pages_per_chunk
    assert np.array_equal(oplan["request_indices"], dec.request_indices)
    assert np.array_equal(oplan["kv_tile_indices"], dec.kv_tile_indices)
    assert np.array_equal(oplan["o_indptr"], dec.o_indptr)
    q, k, v = to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool)
    ref_v, ref_l = orc.attention(w.q, w.k_pool, w.v_pool, ocsr, w.page_size, w.sm_scale,
                                 nthreads=NTHREADS)
    for it in range(repeat):
        if stream is not None:
            with torch.cuda.stream(stream):
                out, lse = dec.run(q, k, v, w.sm_scale)
            stream.synchronize()
        else:
            out, lse = dec.run(q, k, v, w.sm_scale)
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype,
                    "final (call %d)" % it)
        if fused:
            assert int(dec.counters.abs().sum()) == 0, "fused launch left a counter non-zero"
    if check_partials and not fused:
        pv, pl = orc.partial(w.q, w.k_pool, w.v_pool, ocsr, w.page_size, w.sm_scale,
                             oplan["request_indices"], oplan["kv_tile_indices"],
                             oplan["pages_per_chunk"], nthreads=NTHREADS)
        check_close(dec.v_partial.cpu().numpy(), dec.lse_partial.cpu().numpy(), pv, pl,
                    w.dtype, "partials")
        # the merge on the GPU's own partial rows, against the oracle merge of
        # those same rows: isolates the merge kernel's error
        if info.needs_merge:
            mv, ml = orc.merge(dec.v_partial.cpu().numpy().astype(np.float64),
                               dec.lse_partial.cpu().numpy().astype(np.float64), dec.o_indptr)
            check_close(out.cpu().numpy(), lse.cpu().numpy(), mv, ml, workloads.FP32,
                        "merge-of-gpu-partials")
    return dec


# ---------------------------------------------------------------- configs

def test_tiny_fp32_single_merge_of_four(orc, mode):
    w = workloads.tiny_fp32()
    dec = run_flat(orc, w, target=8, fused=mode["fused"])
    assert dec.info.pages_per_chunk == 10 and dec.info.num_chunks == 4
    assert list(dec.o_indptr) == [0, 4] and dec.info.needs_merge
    dec = run_flat(orc, w, target=8, fixed=8, fused=mode["fused"])
    assert dec.info.num_chunks == 4


def test_tiny_fp32_poisoned_pool(orc, mode):
    run_flat(orc, workloads.tiny_fp32(poison_unused=True), target=8, fused=mode["fused"],
             repeat=2)


@pytest.mark.parametrize("target", [0, 64, 1024])
def test_batched_fp16(orc, target, mode):
    w = cached("batched_fp16", poison_unused=True)
    assert w.written_len[0] % w.page_size == 0          # an exactly-full last page
    run_flat(orc, w, target=target, fused=mode["fused"], repeat=2)


@pytest.mark.parametrize("target", [0, 1024, 1])
def test_long_context_fp16_full_size(orc, target, mode):
    """Full size; target 1 gives 2048-page chunks (32 windows of 64 page ids in the page kernel)."""
    w = cached("long_context_fp16", poison_unused=True)
    dec = run_flat(orc, w, target=target, fused=mode["fused"], repeat=2)
    if target == 1:       # one 2048-page chunk per request: written directly
        assert dec.info.pages_per_chunk == 2048 and not dec.info.needs_merge
    else:
        assert dec.info.needs_merge


_LIMIT = {}


@pytest.mark.parametrize("page_size,pages,chunks", [(1, 65535, 65535), (1, 65536, 32768),
                                                    (16, 65535, 65535)],
                         ids=["ps1-65535", "ps1-65536", "ps16-65535"])
def test_plan_at_the_chunk_limit(orc, page_size, pages, chunks, mode):
    """The largest grid a plan may launch: 65535 pages split one page per
    chunk give exactly PD_MAX_CHUNKS chunks (every partial row compared, and
    one merge of 65535 rows), at page size 1 (the token kernel) and at page
    size 16 (the page kernel, 1M tokens); one page more forces two pages per
    chunk."""
    key = (page_size, pages)
    if key not in _LIMIT:
        _LIMIT[key] = workloads.generic(
            "chunk_limit_ps%d_%d" % key, seed=71, dtype=workloads.FP16, page_size=page_size,
            num_qo_heads=4, num_kv_heads=1, head_dim=128, logical_start=[0],
            written_len=[pages * page_size], pool_slack=1.25, poison_unused=True)
    dec = run_flat(orc, _LIMIT[key], target=10 ** 9, fused=mode["fused"])
    assert dec.info.num_chunks == chunks and dec.info.needs_merge


def test_token_sparse_page_size_one(orc):
    s = workloads.token_sparse_fp16()
    hkv, cap, d = s.k_dense.shape[1], s.k_dense.shape[2], s.k_dense.shape[3]
    hq = s.q.shape[1]
    say("case token_sparse Hq=%d Hkv=%d cap=%d topk=%d" % (hq, hkv, cap, len(s.positions[0])))
    kd, vd = to_dev(s.k_dense), to_dev(s.v_dense)
    kp, vp = PD.sparse_pool_view(kd, vd)
    qf = PD.sparse_fold_query(to_dev(s.q), hkv)
    tables = PD.sparse_block_tables(s.positions, cap)
    lens = [len(p) for p in s.positions]
    csr = B.paged_csr_build(tables, [0] * hkv, lens, 1, kp.shape[0])
    dec = PD.PagedDecode(csr, page_size=1, num_pool_pages=kp.shape[0], num_qo_heads=hq // hkv,
                         num_kv_heads=1, head_dim=d)
    say("  plan", dec.plan_summary())
    out, lse = dec.run(qf, kp, vp, s.sm_scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy().reshape(1, hq, d)
    lse = lse.cpu().numpy().reshape(1, hq)
    # oracle: the same selection gathered straight from the dense allocation
    ref_v = np.zeros((1, hq, d))
    ref_l = np.zeros((1, hq))
    g = hq // hkv
    for i in range(hq):
        h = i // g
        kr = s.k_dense[0, h, s.positions[h]]
        vr = s.v_dense[0, h, s.positions[h]]
        ref_v[0, i], ref_l[0, i] = orc.attention_dense_f64(s.q[0, i, 0], kr, vr, s.sm_scale)
    check_close(out, lse, ref_v, ref_l, workloads.FP16, "sparse final")
    # every partial row, against the oracle's partial over the folded table
    # (its own CSR by token enumeration and its own plan by exhaustive scan)
    fw = workloads.folded_sparse(s)
    ocsr = orc.csr_from_block_tables(fw.block_tables, fw.logical_start, fw.written_len, 1)
    oplan = orc.plan(ocsr["indptr"], 1, dec.info.target_wgs)
    assert oplan["pages_per_chunk"] == dec.info.pages_per_chunk
    assert np.array_equal(oplan["request_indices"], dec.request_indices)
    assert np.array_equal(oplan["kv_tile_indices"], dec.kv_tile_indices)
    pv, pl = orc.partial(fw.q, fw.k_pool, fw.v_pool, ocsr, 1, fw.sm_scale,
                         oplan["request_indices"], oplan["kv_tile_indices"],
                         oplan["pages_per_chunk"], nthreads=NTHREADS)
    check_close(dec.v_partial.cpu().numpy(), dec.lse_partial.cpu().numpy(), pv, pl,
                workloads.FP16, "sparse partials")


def test_sparse_expand_blocks_exact():
    """Block ids -> rows at every page size dividing the block (token rows,
    sub-block pages, one page per block), against the definition: block j's
    pages id*span + t, the final block only the pages that hold its written
    positions; ids outside [0, num_blocks) are clamped into the request's
    region."""
    rng = np.random.Generator(np.random.PCG64(90))
    r, blocks, c, nb = 5, 7, 16, 40
    ids = rng.integers(-3, nb + 3, size=(r, blocks)).astype(np.int32)
    tail = rng.integers(1, c + 1, size=r).astype(np.int32)
    base = (np.arange(r) * 1000).astype(np.int32)
    for ps in (1, 2, 4, 8, 16):
        span = c // ps
        final = (tail + ps - 1) // ps
        csr = B.paged_sparse_csr(blocks, c, tail, ps)
        ip = csr["indptr"]
        rows = torch.full((int(ip[-1]),), -1, dtype=torch.int32, device=DEV)
        B.paged_sparse_expand_blocks(to_dev(ids), r, blocks, to_dev(base), span, to_dev(final),
                                     to_dev(ip), nb, rows)
        torch.cuda.synchronize()
        want = []
        for i in range(r):
            for j in range(blocks):
                cid = min(max(int(ids[i, j]), 0), nb - 1)
                # pages of this block that hold selected positions
                n = span if j < blocks - 1 else -(-int(tail[i]) // ps)
                want.extend(int(base[i]) + cid * span + t for t in range(n))
        assert rows.cpu().numpy().tolist() == want, ps


def _block_sparse_reference(orc, w):
    b, hkv, cap, d = w.k_dense.shape
    hq = w.q.shape[1]
    g = hq // hkv
    ref_v = np.zeros((b, hq, d))
    ref_l = np.zeros((b, hq))
    for s in range(b):
        for i in range(hq):
            h = i // g
            pos = orc.block_positions(w.block_ids[s * hkv + h], w.block_size, w.kv_len[s])
            ref_v[s, i], ref_l[s, i] = orc.attention_dense_f64(
                w.q[s, i], w.k_dense[s, h, pos], w.v_dense[s, h, pos], w.sm_scale)
    return ref_v, ref_l


@pytest.mark.parametrize("token_exact,page_size", [(False, 0), (False, -1), (False, 32),
                                                   (False, 8), (True, 0)],
                         ids=["block-granular", "one-page-per-block", "32-row-pages",
                              "8-row-pages", "token-exact"])
@pytest.mark.parametrize("geom", [dict(), dict(seed=8, hq=16, hkv=4, cap=8192, block_size=64,
                                                blocks=9, kv_len=8192),
                                  dict(seed=9, hq=8, hkv=2, cap=4096, block_size=64,
                                       blocks=5, kv_len=4000 - 21)],
                         ids=["minimax-like", "g4-full-final-block", "g4-mid-page-final"])
def test_block_sparse_decode(orc, token_exact, page_size, geom):
    """The selection read through each page-table granularity (one-token
    pages, pages of 8 to 32 rows, one page per block, and the default 16-row
    pages) matches attention over the selected positions of the dense
    allocation; the positions past the live length are NaN, so reading past
    the final block's written positions would show."""
    w = workloads.block_sparse_fp16(**geom)
    b, hkv, cap, d = w.k_dense.shape
    ps = w.block_size if page_size == -1 else page_size
    dec = PD.BlockSparseDecode(to_dev(w.k_dense), to_dev(w.v_dense), num_qo_heads=w.q.shape[1],
                               block_size=w.block_size, blocks_per_request=w.block_ids.shape[1],
                               kv_len=w.kv_len, token_exact=token_exact, page_size=ps)
    say("case block_sparse %s exact=%s plan=%s" % (geom, token_exact, dec.plan_summary()))
    ids = to_dev(w.block_ids)
    for it in range(2):
        out, lse = dec.run(to_dev(w.q), ids, w.sm_scale)
        torch.cuda.synchronize()
    ref_v, ref_l = _block_sparse_reference(orc, w)
    check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, workloads.FP16,
                "block sparse")


@pytest.mark.parametrize("kind", ["flat", "block-sparse", "cascade"])
def test_decode_step_replayed_from_hip_graph(orc, kind):
    """A decode step captured in a HIP graph (partial + merge; for the block
    selection also the row expansion; for the cascade the head stacking,
    both levels and the in-place merge) and replayed: every
    replay equals the eager step on the same inputs, with eager work and
    synchronization between replays and a new query written into the
    captured buffer."""
    if kind == "flat":
        w = cached("batched_fp16", poison_unused=True)
        csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                                w.k_pool.shape[0])
        dec = PD.PagedDecode(csr, page_size=w.page_size, num_pool_pages=w.k_pool.shape[0],
                             num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                             head_dim=w.head_dim)
        assert dec.info.needs_merge
        k, v = to_dev(w.k_pool), to_dev(w.v_pool)
        qs = [w.q, workloads._normal(np.random.default_rng(3), w.q.shape, workloads.FP16)]
        step = lambda qb: dec.run(qb, k, v, w.sm_scale)   # noqa: E731
    elif kind == "cascade":
        w = workloads.cascade_fp16(seed=7, members=5, prefix_tokens=2048, suffix_lo=100,
                                   suffix_hi=900, poison_unused=True)
        dec = _cascade(w)
        assert dec.active and dec.rows0 is not None
        k, v = to_dev(w.k_pool), to_dev(w.v_pool)
        qs = [w.q, workloads._normal(np.random.default_rng(5), w.q.shape, workloads.FP16)]
        step = lambda qb: dec.run(qb, k, v, w.sm_scale)   # noqa: E731
    else:
        w = workloads.block_sparse_fp16(seed=8, hq=16, hkv=4, cap=8192, block_size=64,
                                        blocks=9, kv_len=8000)
        dec = PD.BlockSparseDecode(to_dev(w.k_dense), to_dev(w.v_dense),
                                   num_qo_heads=w.q.shape[1], block_size=w.block_size,
                                   blocks_per_request=w.block_ids.shape[1], kv_len=w.kv_len,
                                   token_exact=True)
        ids = to_dev(w.block_ids)
        qs = [w.q, workloads._normal(np.random.default_rng(4), w.q.shape, workloads.FP16)]
        step = lambda qb: dec.run(qb, ids, w.sm_scale)   # noqa: E731
    qbuf = to_dev(qs[0])
    eager = []
    for qh in qs:
        qbuf.copy_(to_dev(qh))
        out, lse = step(qbuf)
        torch.cuda.synchronize()
        eager.append((out.cpu().numpy().copy(), lse.cpu().numpy().copy()))
    qbuf.copy_(to_dev(qs[0]))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(qbuf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_g, lse_g = step(qbuf)
    torch.cuda.synchronize()
    for rep in range(6):
        which = rep % 2
        qbuf.copy_(to_dev(qs[which]))
        torch.cuda.synchronize()
        _ = (qbuf.float() * 2).sum().item()          # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        ev, el = eager[which]
        got_v, got_l = out_g.cpu().numpy(), lse_g.cpu().numpy()
        say("  graph %s replay %d: max|dv|=%.3g" % (kind, rep, np.max(np.abs(got_v - ev))))
        np.testing.assert_allclose(got_v, ev, rtol=0, atol=1e-6)
        np.testing.assert_allclose(got_l, el, rtol=0, atol=1e-6)


def test_autotune_times_every_candidate_and_stays_exact(orc):
    """Chunk-size autotune on the token-sparse selection (page_size 1): every
    power-of-two candidate and the default plan's choice are timed, the
    fastest is kept, and its output matches the oracle."""
    w = workloads.folded_sparse(workloads.token_sparse_fp16())
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                            w.k_pool.shape[0])
    k, v, q = to_dev(w.k_pool), to_dev(w.v_pool), to_dev(w.q)
    dec, table = PD.autotune(csr, q, k, v, w.sm_scale, page_size=w.page_size,
                             num_pool_pages=w.k_pool.shape[0], num_qo_heads=w.num_qo_heads,
                             num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, n=60)
    say("  autotune table: %s" % table)
    cs = [row["pages_per_chunk"] for row in table]
    assert cs == sorted(set(cs)) and {1, 2, 4, 1024, 2048} <= set(cs) and 32 in cs
    fastest = min(table, key=lambda row: row["step_us"])
    assert dec.info.pages_per_chunk == fastest["pages_per_chunk"]
    out, lse = dec.run(q, k, v, w.sm_scale)
    torch.cuda.synchronize()
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                     w.page_size)
    ref_v, ref_l = orc.attention(w.q, w.k_pool, w.v_pool, ocsr, w.page_size, w.sm_scale,
                                 nthreads=NTHREADS)
    check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype, "autotuned")


def _cascade(w, **kw):
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                            w.k_pool.shape[0])
    return PD.CascadeDecode(csr, page_size=w.page_size, num_pool_pages=w.k_pool.shape[0],
                            num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                            head_dim=w.head_dim, **kw)


def _check_cascade_partials(orc, w, cas):
    """Every level-0 row (per launch, on the stacked queries) and every
    level-1 row of a cascade step against the oracle's partial over the two
    levels' page tables, which the test builds from the oracle's own CSR:
    level 0 is one request holding the first shared_pages pages of the first
    member; level 1 keeps each member's pages after them and every other
    request's whole list.  Stacked head kv*(S*G) + m*G + g of a launch is
    query head kv*G + g of its m-th member (cascade doc, head stacking)."""
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                     w.page_size)
    ip, ix = ocsr["indptr"], ocsr["indices"]
    sp, members = cas.shared_pages, [int(m) for m in cas.member_req]
    ps, hq, hkv, d = w.page_size, w.num_qo_heads, w.num_kv_heads, w.head_dim
    g = hq // hkv
    csr0 = dict(indptr=np.array([0, sp], np.int32),
                indices=ix[ip[members[0]]:ip[members[0]] + sp].copy(),
                last_page_len=np.array([ps], np.int32),
                first_page_offset=np.array([0], np.int32))
    ind1, ip1 = [], [0]
    for r in range(w.batch):
        pages = ix[ip[r]:ip[r + 1]]
        if r in members:
            assert np.array_equal(pages[:sp], csr0["indices"])
            pages = pages[sp:]
        ind1.append(pages)
        ip1.append(ip1[-1] + len(pages))
    csr1 = dict(indptr=np.array(ip1, np.int32), indices=np.concatenate(ind1).astype(np.int32),
                last_page_len=ocsr["last_page_len"], first_page_offset=ocsr["first_page_offset"])
    for j, (lv, sub) in enumerate(zip(cas.level0, cas.subgroups)):
        n_m = len(sub)
        q0 = np.zeros((1, n_m * hq, d), w.q.dtype)
        for kv in range(hkv):
            for m, req in enumerate(sub):
                q0[0, kv * n_m * g + m * g:kv * n_m * g + (m + 1) * g] = \
                    w.q[req, kv * g:(kv + 1) * g]
        assert np.all(lv.request_indices == 0)
        pv, pl = orc.partial(q0, w.k_pool, w.v_pool, csr0, ps, w.sm_scale, lv.request_indices,
                             lv.kv_tile_indices, lv.info.pages_per_chunk, nthreads=NTHREADS)
        check_close(lv.v_partial.cpu().numpy(), lv.lse_partial.cpu().numpy(), pv, pl, w.dtype,
                    "level-0 partials, launch %d (%d members, stacked G=%d)" % (j, n_m, n_m * g))
    l1 = cas.level1
    oplan = orc.plan(csr1["indptr"], hkv, l1.info.target_wgs,
                     fixed_pages_per_chunk=l1.fixed_pages_per_chunk)
    assert np.array_equal(oplan["request_indices"], l1.request_indices)
    assert np.array_equal(oplan["kv_tile_indices"], l1.kv_tile_indices)
    pv, pl = orc.partial(w.q, w.k_pool, w.v_pool, csr1, ps, w.sm_scale, l1.request_indices,
                         l1.kv_tile_indices, l1.info.pages_per_chunk, nthreads=NTHREADS)
    check_close(l1.v_partial.cpu().numpy(), l1.lse_partial.cpu().numpy(), pv, pl, w.dtype,
                "level-1 partials")


def _oracle_flat(orc, w):
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                     w.page_size)
    return orc.attention(w.q, w.k_pool, w.v_pool, ocsr, w.page_size, w.sm_scale,
                         nthreads=NTHREADS)


@pytest.mark.parametrize("in_place", [True, False], ids=["in-place-merge", "gathered-merge"])
def test_cascade_matches_flat_and_oracle(orc, in_place):
    w = workloads.cascade_fp16(poison_unused=True)
    flat = run_flat(orc, w, target=0, check_partials=False)
    sp = w.extra["shared_pages"]
    cas = _cascade(w, merge_in_place=in_place)
    assert (cas.rows0 is not None) == in_place
    say("case cascade members=%d shared_pages=%d suffix=%s plan=%s" % (
        w.batch, sp, list(w.extra["suffix_tokens"]), cas.plan_summary()))
    # detection finds the whole batch sharing the 8192-token prefix
    assert cas.active and list(cas.member_req) == list(range(w.batch))
    assert cas.shared_pages == sp and len(cas.subgroups) == 1
    q, k, v = to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool)
    out, lse = cas.run(q, k, v, w.sm_scale)
    torch.cuda.synchronize()
    ref_v, ref_l = _oracle_flat(orc, w)
    check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype, "cascade")
    _check_cascade_partials(orc, w, cas)
    fo, fl = flat.run(q, k, v, w.sm_scale)
    torch.cuda.synchronize()
    check_close(out.cpu().numpy(), lse.cpu().numpy(), fo.cpu().numpy().astype(np.float64),
                fl.cpu().numpy().astype(np.float64), w.dtype, "cascade-vs-flat")


@pytest.mark.parametrize("pair,hpw,fixed0,fixed1", [
    (True, 0, 0, 0), (True, 8, 0, 0), (True, 4, 0, 0), (True, 2, 0, 0), (True, 1, 0, 0),
    (True, 0, 8, 1), (True, 4, 2, 4), (False, 0, 0, 0)],
    ids=["pair-auto", "pair-hpw8", "pair-hpw4", "pair-hpw2", "pair-hpw1", "pair-c8-c1",
         "pair-hpw4-c2-c4", "level1-separate"])
def test_cascade_pair_launch_shapes(orc, pair, hpw, fixed0, fixed1):
    """The shared level (stacked G0 = 16, queries read through the member
    list) and the per-request level (G = 4) in one MFMA grid, at every
    workgroup width and several chunkings, and with level 1 launched on its
    own: outputs and every partial row of both levels against the oracle."""
    w = cached("cascade_fp16", poison_unused=True)
    cas = _cascade(w, pair_launch=pair, heads_per_workgroup=hpw, fixed_pages_level0=fixed0,
                   fixed_pages_level1=fixed1)
    say("case cascade pair=%s hpw=%d plan=%s" % (pair, hpw, cas.plan_summary()))
    assert cas.active and len(cas.subgroups) == 1
    if fixed0:
        assert cas.level0[0].info.pages_per_chunk == fixed0
    q, k, v = to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool)
    for it in range(2):
        out, lse = cas.run(q, k, v, w.sm_scale)
        torch.cuda.synchronize()
    ref_v, ref_l = _oracle_flat(orc, w)
    check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype, "cascade")
    _check_cascade_partials(orc, w, cas)


@pytest.mark.parametrize("choice", [1, 2], ids=["token-kernel", "valu-kernels"])
def test_cascade_stacked_queries_off_the_mfma_kernel(orc, choice):
    """The stacked level's queries read through the member list on the page
    and token kernels (two launches), against the oracle."""
    B.paged_decode_set_kernel_choice(choice)
    try:
        w = _mixed_batch(91, 4, hq=32)
        cas = _cascade(w, min_shared_pages=16)
        say("case cascade kernel-choice=%d plan=%s" % (choice, cas.plan_summary()))
        q, k, v = to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool)
        out, lse = cas.run(q, k, v, w.sm_scale)
        torch.cuda.synchronize()
        ref_v, ref_l = _oracle_flat(orc, w)
        check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype, "cascade")
        _check_cascade_partials(orc, w, cas)
    finally:
        B.paged_decode_set_kernel_choice(0)


@pytest.mark.parametrize("ps", [5, 48, 1])
def test_cascade_on_the_any_page_mfma_kernel(orc, ps):
    """Page sizes the page-tiled MFMA kernel cannot take: the stacked level's
    groups (S*G from 8 to 16 here) run on the any-page MFMA kernel, one launch
    per table, reading the members' queries through the member list; the
    per-request level (G = 4) runs on the page or token kernel.  The output
    and every partial row of both levels against the oracle."""
    w = _mixed_batch(95 + ps, 4, hq=32, ps=ps, prefix_pages=max(40, 640 // ps))
    assert B.paged_decode_kernel_kind(B.PD_DTYPE_FP16, 128, 16, ps, 8 * 128) == 3
    cas = _cascade(w, min_shared_pages=16)
    say("case cascade any-page ps=%d plan=%s" % (ps, cas.plan_summary()))
    assert cas.plan_summary()["cascade"]
    q, k, v = to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool)
    out, lse = cas.run(q, k, v, w.sm_scale)
    torch.cuda.synchronize()
    ref_v, ref_l = _oracle_flat(orc, w)
    check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype, "cascade")
    _check_cascade_partials(orc, w, cas)


def _mixed_batch(seed, members, hq=32, hkv=8, prefix_pages=40, ps=16):
    """A batch in which `members` requests share a prefix of pages, one more
    request holds the same pages but starts mid-page (so detection leaves it
    out), and two unrelated requests hold their own pages."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n_other = 3
    suf = rng.integers(1, 9, size=members + n_other)
    live = prefix_pages + int(suf.sum()) + 2 * prefix_pages
    pool = 2 * live
    perm = rng.permutation(pool).astype(np.int32)
    prefix = perm[:prefix_pages]
    pos = prefix_pages
    tables, ls, wl = [], [], []
    for i in range(members + 1):
        tail = perm[pos:pos + suf[i]]
        pos += suf[i]
        tables.append(np.concatenate([prefix, tail]))
        n_tok = (prefix_pages + suf[i] - 1) * ps + int(rng.integers(1, ps + 1))
        start = 5 if i == members else 0                  # the mid-page window
        ls.append(start)
        wl.append(n_tok)
    for i in range(2):
        own = perm[pos:pos + prefix_pages]
        pos += prefix_pages
        tables.append(own)
        ls.append(0)
        wl.append(prefix_pages * ps - 3)
    q = rng.standard_normal((len(tables), hq, 128), dtype=np.float32).astype(np.float16)
    k = rng.standard_normal((pool, ps, hkv, 128), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((pool, ps, hkv, 128), dtype=np.float32).astype(np.float16)
    w = workloads.Workload(name="mixed_cascade", dtype=workloads.FP16, page_size=ps,
                           num_qo_heads=hq, num_kv_heads=hkv, head_dim=128,
                           sm_scale=1.0 / np.sqrt(128), q=q, k_pool=k, v_pool=v,
                           block_tables=tables, logical_start=np.array(ls, np.int32),
                           written_len=np.array(wl, np.int32))
    return workloads.poison_invisible(w)


@pytest.mark.parametrize("in_place", [True, False], ids=["in-place-merge", "gathered-merge"])
@pytest.mark.parametrize("members,hq", [(3, 32), (6, 32), (5, 16), (9, 32), (2, 64), (3, 64),
                                        (2, 128)])
def test_cascade_mixed_batch_and_subgroups(orc, members, hq, in_place):
    """Members, a mid-page window over the same pages, and unrelated requests in
    one batch.  Stacked groups of 12 and 24 query heads per KV head run on the
    MFMA kernel; 9 members at G = 4 split into launches of 6 + 3 members (24 + 12
    heads), 5 members at G = 2 into 4 + 1 (8 + 2).  At G = 8 and 16 the level-1
    group runs on the one-grid MFMA kernel too (2 or 3 members stack 16, 24 or
    32 heads).  Every level-0 and level-1 partial row is checked as well as the
    outputs."""
    w = _mixed_batch(80 + members, members, hq=hq)
    cas = _cascade(w, min_shared_pages=16, merge_in_place=in_place)
    say("case mixed cascade members=%d hq=%d plan=%s" % (members, hq, cas.plan_summary()))
    assert cas.active and list(cas.member_req) == list(range(members))
    assert cas.shared_pages == 40
    g = hq // w.num_kv_heads
    assert all(sub.size * g <= 32 for sub in cas.subgroups)
    q, k, v = to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool)
    out, lse = cas.run(q, k, v, w.sm_scale)
    torch.cuda.synchronize()
    ref_v, ref_l = _oracle_flat(orc, w)
    check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype, "mixed cascade")
    _check_cascade_partials(orc, w, cas)


@pytest.mark.parametrize("members,hq,d", [(9, 32, 128), (5, 16, 128), (4, 32, 64)])
def test_cascade_in_place_merge_equals_gathered_merge(orc, members, hq, d):
    """The merge that reads the stacked level-0 rows in place and the merge
    of the gathered copy see the same rows (several stacked launches
    included): they agree to rounding (the in-place merge folds a group in
    load batches of 11 rows per row lane, the flat merge in batches of 10),
    and both match the oracle.  A row read from the wrong place would differ at the scale of the
    values themselves."""
    w = workloads.cascade_fp16(seed=90 + members, members=members, prefix_tokens=1024,
                               suffix_lo=16, suffix_hi=400, hq=hq, hkv=hq // 4, d=d,
                               poison_unused=True)
    a = _cascade(w, merge_in_place=True)
    b = _cascade(w, merge_in_place=False)
    say("case cascade in-place vs gathered members=%d hq=%d d=%d plan=%s"
        % (members, hq, d, a.plan_summary()))
    assert a.active and a.rows0 is not None and b.rows0 is None
    q, k, v = to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool)
    oa, la = (t.clone() for t in a.run(q, k, v, w.sm_scale))
    ob, lb = b.run(q, k, v, w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(torch.isneginf(la), torch.isneginf(lb))
    dv = float((oa - ob).abs().max())
    dl = float((la - lb)[torch.isfinite(la)].abs().max())
    say("  in-place vs gathered: max|dv|=%.3g max|dlse|=%.3g" % (dv, dl))
    # a few fp32 ulps (the LSEs are O(10) in log2 units)
    lmax = float(la[torch.isfinite(la)].abs().max())
    assert dv <= 1e-6 and dl <= 1e-6 * max(1.0, lmax)
    ref_v, ref_l = _oracle_flat(orc, w)
    check_close(oa.cpu().numpy(), la.cpu().numpy(), ref_v, ref_l, w.dtype, "in-place cascade")


@pytest.mark.parametrize("d,n0,counts", [(128, 7, (2, 0, 1, 4, 3)), (512, 7, (2, 0, 1, 4, 3)),
                                         (64, 7, (2, 0, 1, 4, 3)),
                                         (128, 150, (2, 0, 61, 97, 3)),
                                         (64, 88, (0, 0, 1, 130, 89))])
def test_cascade_merge_states_against_oracle(orc, d, n0, counts):
    """The in-place cascade merge on synthetic states: members 0, 2, 3 of 5
    requests stacked two per launch (launches of 2 and 1 members), empty
    chunks (lse = -inf, V never read), a member with one own row, and a
    non-member with none (zeros, -inf).  The expected groups are gathered on
    the host from the stacking rule and merged by the oracle.  The long cases
    (groups of up to 247 rows) take the one-wave merge through several
    88-row load passes; one group ends one row past a pass (88 + 1), one
    non-member group is exactly 89 rows."""
    rng = np.random.default_rng(95 + d + n0)
    batch, hkv, g, per = 5, 2, 4, 2
    hq = hkv * g
    members = np.array([0, 2, 3], np.int32)
    counts = np.array(counts)
    o1 = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n1 = int(o1[-1])
    rows0 = n0 * members.size * hq
    v0 = rng.standard_normal((rows0, d)).astype(np.float32)
    l0 = (rng.standard_normal(rows0) * 6).astype(np.float32)
    v1 = rng.standard_normal((n1, hq, d)).astype(np.float32)
    l1 = (rng.standard_normal((n1, hq)) * 6).astype(np.float32)
    l0[rng.random(rows0) < 0.2] = -np.inf
    l1[rng.random((n1, hq)) < 0.2] = -np.inf
    v0[np.isneginf(l0)] = 1e30
    v1[np.isneginf(l1)] = 1e30
    desc = B.paged_cascade_merge_layout(batch, members, per, n0, hq)
    # host gather from the stacking rule: launch j holds members j*per ..,
    # [n0, S*Hq] rows, stacked head kv*S*G + p*G + g
    gv, gl, oi = [], [], [0]
    for r in range(batch):
        if r in members:
            m = int(np.where(members == r)[0][0])
            j0 = (m // per) * per
            s_ = min(per, members.size - j0)
            p = m - j0
            first = j0 * n0 * hq
            for i in range(n0):
                idx = [first + i * s_ * hq + (h // g) * s_ * g + p * g + h % g for h in range(hq)]
                gv.append(v0[idx])
                gl.append(l0[idx])
        for n in range(o1[r], o1[r + 1]):
            gv.append(v1[n])
            gl.append(l1[n])
        oi.append(len(gv))
    rv, rl = orc.merge(np.array(gv, np.float64), np.array(gl, np.float64), oi)
    dev = torch.device("cuda")
    out = torch.empty((batch, hq, d), dtype=torch.float32, device=dev)
    lo = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    B.paged_cascade_merge_states(torch.from_numpy(v0).to(dev), torch.from_numpy(l0).to(dev), n0,
                                 torch.from_numpy(desc).to(dev), torch.from_numpy(v1).to(dev),
                                 torch.from_numpy(l1).to(dev), torch.from_numpy(o1).to(dev),
                                 batch, hq, hkv, d, out, lo)
    torch.cuda.synchronize()
    check_close(out.cpu().numpy(), lo.cpu().numpy(), rv, rl, workloads.FP32,
                "cascade merge d=%d" % d)
    assert np.all(out[1].cpu().numpy() == 0) and np.all(np.isneginf(lo[1].cpu().numpy()))


def test_cascade_merge_states_rejects_bad_arguments():
    dev = torch.device("cuda")
    v = torch.zeros((4, 8, 80), dtype=torch.float32, device=dev)
    lse = torch.zeros((4, 8), dtype=torch.float32, device=dev)
    desc = torch.tensor([[0, 0, -1]] * 2, dtype=torch.int32, device=dev)
    oi = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)
    out = torch.zeros((2, 8, 80), dtype=torch.float32, device=dev)
    lo = torch.zeros((2, 8), dtype=torch.float32, device=dev)
    with pytest.raises(B.PagedDecodeError) as e:      # 80 is not a multiple of 32
        B.paged_cascade_merge_states(v, lse, 1, desc, v, lse, oi, 2, 8, 2, 80, out, lo)
    assert e.value.name == "PD_E_UNSUPPORTED"
    with pytest.raises(B.PagedDecodeError) as e:      # 8 query heads over 3 KV heads
        B.paged_cascade_merge_states(v, lse, 1, desc, v, lse, oi, 2, 8, 3, 64, out, lo)
    assert e.value.name == "PD_E_ARG"


def test_cascade_fp32_pools(orc):
    """The cascade on fp32 pools (head dim 64; the stacked level 0 splits into
    launches the fp32 kernels support), merged in place, against the oracle
    at the fp32 tolerance."""
    w16 = workloads.cascade_fp16(seed=12, members=3, prefix_tokens=1024, suffix_lo=40,
                                 suffix_hi=300, hq=8, hkv=2, d=64, poison_unused=True)
    w = dataclasses.replace(w16, dtype=workloads.FP32, q=w16.q.astype(np.float32),
                            k_pool=w16.k_pool.astype(np.float32),
                            v_pool=w16.v_pool.astype(np.float32))
    cas = _cascade(w, dtype=torch.float32)
    say("case cascade fp32 plan=%s" % cas.plan_summary())
    assert cas.active and cas.rows0 is not None
    q, k, v = to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool)
    out, lse = cas.run(q, k, v, w.sm_scale)
    torch.cuda.synchronize()
    ref_v, ref_l = _oracle_flat(orc, w)
    check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype, "fp32 cascade")


def test_cascade_without_sharing_is_flat(orc):
    w = workloads.batched_fp16(poison_unused=True)
    cas = _cascade(w)
    assert not cas.active
    q, k, v = to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool)
    out, lse = cas.run(q, k, v, w.sm_scale)
    torch.cuda.synchronize()
    ref_v, ref_l = _oracle_flat(orc, w)
    check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype, "no-share cascade")


def test_cascade_member_major_stacking_is_wrong(orc):
    """Negative control: stacking heads member-major (a plain reshape) launches
    fine and reads the wrong KV heads, so it must not match."""
    w = workloads.cascade_fp16(seed=6, prefix_tokens=1024, suffix_lo=64, suffix_hi=128)
    cas = _cascade(w, merge_in_place=False)
    assert cas.active and len(cas.subgroups) == 1 and cas.v_cat is not None
    q, k, v = to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool)
    good, _ = cas.run(q, k, v, w.sm_scale)
    good = good.cpu().numpy().copy()
    wrong_q0 = q.reshape(1, -1, w.head_dim).contiguous()        # member-major
    cas.level0[0].partial(wrong_q0, k, v, w.sm_scale)
    cas.level1.partial(q, k, v, w.sm_scale)
    B.paged_cascade_gather_states(cas.level0[0].v_partial, cas.level0[0].lse_partial, cas.n0,
                                  cas.member_req.size, cas.d_dst0[0], cas.level1.v_partial,
                                  cas.level1.lse_partial, cas.n1, cas.d_dst1, w.num_qo_heads,
                                  w.num_kv_heads, w.head_dim, cas.v_cat, cas.lse_cat)
    B.paged_merge_states(cas.v_cat, cas.lse_cat, cas.d_oindptr, w.batch, w.num_qo_heads,
                         w.head_dim, cas.out, cas.lse)
    torch.cuda.synchronize()
    bad = cas.out.cpu().numpy()
    assert np.max(np.abs(bad - good)) > 0.05


# ------------------------------------------------------- invariance / edges

@pytest.mark.parametrize("fixed", [1, 2, 4, 8, 0])
def test_chunk_size_invariance(orc, fixed, mode):
    w = workloads.random_geometry(40, batch=5, page_size=16, max_len=3000, num_qo_heads=16,
                                  num_kv_heads=4)
    run_flat(orc, w, target=256, fixed=fixed, fused=mode["fused"])


@pytest.mark.parametrize("seed,ps", [(50, 1), (51, 3), (52, 16), (53, 64), (54, 7), (55, 32),
                                     (56, 4)])
def test_ragged_force_merge(orc, seed, ps, mode):
    """pages_per_chunk = 1: every request through the merge, maximally ragged."""
    w = workloads.random_geometry(seed, batch=7, page_size=ps, max_len=700, num_qo_heads=8,
                                  num_kv_heads=2, p_empty=0.2, p_trim=0.5)
    run_flat(orc, w, fixed=1, fused=mode["fused"], repeat=2)


@pytest.mark.parametrize("fixed", [0, 1])
def test_many_requests(orc, fixed):
    """3000 requests in one batch (mostly one or two pages, some empty, some
    trimmed, a few long): the plan arrays, chunk lists and merge groups at
    scale; pinned one-page chunks give 10k+ chunks."""
    rng = np.random.default_rng(77)
    b = 3000
    wl = rng.integers(0, 40, size=b)                      # 0 to 3 pages of 16
    wl[rng.choice(b, size=12, replace=False)] = rng.integers(500, 3000, size=12)
    ls = np.where(rng.random(b) < 0.3, (wl * rng.random(b)).astype(np.int64), 0)
    w = workloads.generic("many_requests", seed=78, dtype=workloads.FP16, page_size=16,
                          num_qo_heads=8, num_kv_heads=2, head_dim=128, logical_start=ls,
                          written_len=wl, poison_unused=True)
    dec = run_flat(orc, w, fixed=fixed, check_partials=False)
    assert dec.batch == b
    if fixed:
        assert dec.info.num_chunks > 3000


@pytest.mark.parametrize("g", [4, 8, 16])
@pytest.mark.parametrize("ps", [4, 16, 64])
def test_page_kernel_shapes_ragged(orc, g, ps, mode):
    """Ragged windows over the page kernel's group sizes and page sizes."""
    w = workloads.random_geometry(100 + g + ps, batch=5, page_size=ps, max_len=1500,
                                  num_qo_heads=2 * g, num_kv_heads=2, p_empty=0.15,
                                  p_trim=0.5)
    run_flat(orc, w, target=48, fused=mode["fused"])


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("g", [1, 2, 8, 12, 16, 24, 32])
@pytest.mark.parametrize("ps,hkv", [(16, 8), (32, 2), (64, 1)])
def test_mfma_kernel_ragged(orc, g, ps, hkv, d):
    """The MFMA kernel over ragged windows, mid-page starts, partial last
    pages, empty requests and NaN-poisoned pools, at each group size, head
    dim and workgroup shape (8, 2 or 1 KV heads per workgroup)."""
    w = workloads.random_geometry(300 + g + ps + d, batch=6, page_size=ps, max_len=2500,
                                  num_qo_heads=g * hkv, num_kv_heads=hkv, head_dim=d,
                                  p_empty=0.15, p_trim=0.5)
    assert B.paged_decode_kernel_kind(B.PD_DTYPE_FP16, d, g, ps, hkv * d) == 2
    for target, fixed in ((0, 0), (64, 0), (0, 1)):
        run_flat(orc, w, target=target, fixed=fixed)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("g", [1, 4, 8, 12, 24, 32])
@pytest.mark.parametrize("ps,hkv", [(1, 2), (3, 8), (48, 1), (4, 4)])
def test_mfma_any_page_kernel_ragged(orc, g, ps, hkv, d):
    """The any-page MFMA kernel, at page sizes the page-tiled one cannot take
    (a 16-token tile spread over 16, 6 or 4 pages; three tiles per page),
    over ragged windows, mid-page starts, partial last pages, empty requests
    and NaN-poisoned pools; 2, 8, 1 and 4 KV heads per workgroup; chunks from
    one page (down to a single token) to the whole request, and 37 pages,
    whose chunks start at every offset within the kernel's 64-token
    windows."""
    w = workloads.random_geometry(760 + g + ps + d, batch=6, page_size=ps, max_len=2500,
                                  num_qo_heads=g * hkv, num_kv_heads=hkv, head_dim=d,
                                  p_empty=0.15, p_trim=0.5)
    assert B.paged_decode_kernel_kind(B.PD_DTYPE_FP16, d, g, ps, hkv * d) == 3
    for target, fixed in ((0, 0), (64, 0), (0, 1), (0, 37)):
        run_flat(orc, w, target=target, fixed=fixed)


@pytest.mark.parametrize("g,ps,choice", [(12, 1, 0), (16, 5, 0), (8, 16, 0), (4, 16, 2), (2, 3, 0),
                                         (2, 3, 2)])
def test_pool_pages_past_4gib(orc, g, ps, choice):
    """Every visible page lies past byte 2^32 of the K and V pools (the
    pools are 5 GiB, NaN everywhere but the copied pages): each kernel forms
    64-bit page offsets (any-page MFMA at page sizes 1, 3 and 5, page-tiled
    MFMA, the page kernel, and the token kernel with the MFMA kernels switched
    off).  A truncated offset reads NaN."""
    hkv, d = 2, 128
    w = workloads.random_geometry(780 + g + ps, batch=4, page_size=ps, max_len=1200,
                                  num_qo_heads=g * hkv, num_kv_heads=hkv, p_empty=0.0,
                                  p_trim=0.5)
    pages = w.k_pool.shape[0]
    page_bytes = ps * hkv * d * 2
    shift = -(-(5 << 30) // page_bytes) - pages
    assert shift * page_bytes > (1 << 32)
    tables = [np.where(t >= 0, t + shift, -1).astype(np.int32) for t in w.block_tables]
    csr = B.paged_csr_build(tables, w.logical_start, w.written_len, ps, shift + pages)
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len, ps)
    ref_v, ref_l = orc.attention(w.q, w.k_pool, w.v_pool, ocsr, ps, w.sm_scale,
                                 nthreads=NTHREADS)
    kbig = vbig = None
    B.paged_decode_set_kernel_choice(choice)
    try:
        kind = B.paged_decode_kernel_kind(B.PD_DTYPE_FP16, d, g, ps, hkv * d)
        say("case past-4GiB g=%d ps=%d kernel %s shift=%d pages" % (g, ps, KIND[kind], shift))
        dec = PD.PagedDecode(csr, page_size=ps, num_pool_pages=shift + pages,
                             num_qo_heads=g * hkv, num_kv_heads=hkv, head_dim=d, target_wgs=64)
        kbig = torch.full((shift + pages, ps, hkv, d), float("nan"), dtype=torch.float16,
                          device=DEV)
        vbig = torch.full_like(kbig, float("nan"))
        kbig[shift:] = to_dev(w.k_pool)
        vbig[shift:] = to_dev(w.v_pool)
        out, lse = dec.run(to_dev(w.q), kbig, vbig, w.sm_scale)
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype, "past 4 GiB")
    finally:
        B.paged_decode_set_kernel_choice(0)
        kbig = vbig = None
        torch.cuda.empty_cache()


@pytest.mark.parametrize("g", [8, 16, 32])
@pytest.mark.parametrize("ps", [16, 1])
@pytest.mark.parametrize("d", [128, 64])
def test_mfma_kernel_peaked_scores(orc, g, ps, d):
    """Queries scaled by 8: natural-unit scores have a standard deviation of
    about 8, so a few tokens carry most of each head's weight -- the case in
    which rounding the probabilities to fp16 for the value product costs the
    most (up to 2^-11 of a weight).  The MFMA kernel carries P as an fp16
    part plus an fp16 remainder, so its error stays far inside the fp16
    tolerance; the bound asserted here is a quarter of it.  Page size 16
    runs the page-tiled MFMA kernel, page size 1 the any-page one."""
    w = workloads.random_geometry(700 + g + d, batch=4, page_size=ps, max_len=3000,
                                  num_qo_heads=g * 8, num_kv_heads=8, head_dim=d, p_empty=0.0,
                                  p_trim=0.5)
    w.q[:] = (w.q.astype(np.float32) * 8).astype(np.float16)
    assert B.paged_decode_kernel_kind(B.PD_DTYPE_FP16, d, g, ps, 8 * d) == (
        2 if ps == 16 else 3)
    dec = run_flat(orc, w, target=0, fixed=4 * 16 // ps)
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len, ps)
    pv, pl = orc.partial(w.q, w.k_pool, w.v_pool, ocsr, ps, w.sm_scale, dec.request_indices,
                         dec.kv_tile_indices, dec.info.pages_per_chunk, nthreads=NTHREADS)
    dv = float(np.max(np.abs(dec.v_partial.cpu().numpy() - pv)))
    fin = np.isfinite(pl)
    dl = float(np.max(np.abs(dec.lse_partial.cpu().numpy()[fin] - pl[fin])))
    say("  peaked scores G=%d: partial rows max|dv|=%.3g max|dlse|=%.3g" % (g, dv, dl))
    assert dv <= 5e-4 and dl <= 2.5e-4


def ramp_keys(orc, w, slope_log2):
    """Rewrites the visible K rows of workload w so that the scores of the
    first query head of every KV head rise by slope_log2 (log2 units) per
    token: K[t] = lambda_t * q / |q|.  Every step of every chunk then raises
    that head's running max past the lazy-rescale margin, so the rescale path
    runs on every step, over a score range of hundreds of log2 units."""
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                     w.page_size)
    g = w.num_qo_heads // w.num_kv_heads
    scale_log2 = w.sm_scale / np.log(2.0)
    k = w.k_pool.astype(np.float32)
    for r in range(w.batch):
        n = int(ocsr["seq_lens"][r])
        slots = ocsr["first_page_offset"][r] + np.arange(n)
        pages = ocsr["indices"][ocsr["indptr"][r] + slots // w.page_size]
        entries = slots % w.page_size
        for kvh in range(w.num_kv_heads):
            q = w.q[r, kvh * g].astype(np.float64)
            u = q / np.linalg.norm(q)
            lam = slope_log2 * np.arange(n) / (scale_log2 * np.linalg.norm(q))
            row = (lam[:, None] * u[None, :]).astype(np.float32)
            assert np.abs(row).max(initial=0.0) < 6e4          # inside the fp16 range
            k[pages, entries, kvh] = row
    w.k_pool[:] = k.astype(w.k_pool.dtype)


@pytest.mark.parametrize("g", [4, 16])
@pytest.mark.parametrize("ps", [16, 5])
@pytest.mark.parametrize("d", [128, 64])
def test_scores_ramp_rescale_every_step(orc, g, ps, d, mode):
    """Scores that rise by 0.6 log2 units per token for one head of every KV
    head (and fall or wander for the others): the running max grows past the
    lazy margin on every step and the accumulators are rescaled each time,
    over a score range of about 900 log2 units.  Every kernel mode, every
    partial row and the merge against the oracle at the usual tolerances."""
    w = workloads.random_geometry(730 + g + ps + d, batch=3, page_size=ps, max_len=1500,
                                  num_qo_heads=g * 4, num_kv_heads=4, head_dim=d, p_empty=0.0,
                                  p_trim=0.5)
    ramp_keys(orc, w, 0.6)
    run_flat(orc, w, target=0, fixed=16 * 16 // ps, fused=mode["fused"])


def test_kernel_choice():
    kk = B.paged_decode_kernel_kind
    assert kk(B.PD_DTYPE_FP16, 128, 4, 16, 1024) == 2    # fp16, D = 128: MFMA for every G
    assert kk(B.PD_DTYPE_FP16, 128, 8, 16, 1024) == 2
    assert kk(B.PD_DTYPE_FP16, 128, 12, 32, 1024) == 2
    assert kk(B.PD_DTYPE_FP16, 128, 16, 16, 1024) == 2
    assert kk(B.PD_DTYPE_FP16, 128, 32, 64, 1024) == 2
    assert kk(B.PD_DTYPE_FP16, 128, 16, 4, 1024) == 3    # page smaller than an MFMA tile
    assert kk(B.PD_DTYPE_FP16, 128, 8, 48, 1024) == 3    # 3 MFMA tiles per page
    assert kk(B.PD_DTYPE_FP16, 128, 32, 1, 128) == 3     # G = 32 at page size 1
    assert kk(B.PD_DTYPE_FP16, 128, 8, 16, 1 << 27) == 3  # in-page offsets past 2^31 bytes
    assert kk(B.PD_DTYPE_FP16, 64, 8, 1, 128) == 3       # D = 64 on the MFMA kernels too
    assert kk(B.PD_DTYPE_FP16, 64, 32, 16, 512) == 2
    assert kk(B.PD_DTYPE_FP32, 128, 8, 1, 128) == 0      # fp16 only
    assert kk(B.PD_DTYPE_FP32, 64, 16, 16, 128) == 1
    assert kk(B.PD_DTYPE_FP32, 64, 4, 16, 128) == 1
    B.paged_decode_set_kernel_choice(2)
    try:
        assert kk(B.PD_DTYPE_FP16, 128, 4, 16, 1024) == 1
        assert kk(B.PD_DTYPE_FP16, 128, 8, 16, 1024) == 1
        assert kk(B.PD_DTYPE_FP16, 128, 12, 16, 1024) == 0
        assert kk(B.PD_DTYPE_FP16, 128, 16, 4, 1024) == 1
        assert kk(B.PD_DTYPE_FP16, 128, 12, 1, 128) == 0
        assert kk(B.PD_DTYPE_FP16, 128, 1, 16, 1024) == 0
        assert kk(B.PD_DTYPE_FP16, 128, 4, 1, 128) == 0
        assert kk(B.PD_DTYPE_FP16, 64, 4, 16, 512) == 0
        with pytest.raises(B.PagedDecodeError):            # G = 32 needs an MFMA kernel
            kk(B.PD_DTYPE_FP16, 128, 32, 1, 128)
    finally:
        B.paged_decode_set_kernel_choice(0)
    assert kk(B.PD_DTYPE_FP16, 128, 4, 8, 1024) == 3     # page smaller than a step
    assert kk(B.PD_DTYPE_FP16, 128, 12, 1, 128) == 3     # token-sparse page_size 1
    assert kk(B.PD_DTYPE_FP16, 128, 1, 16, 1024) == 2    # G = 1 and 2: padded MFMA tiles
    assert kk(B.PD_DTYPE_FP16, 128, 2, 1, 128) == 3
    assert kk(B.PD_DTYPE_FP16, 128, 4, 1, 128) == 3
    assert kk(B.PD_DTYPE_FP16, 128, 4, 16, 1 << 27) == 3  # in-page offsets past 2^31 bytes
    assert kk(B.PD_DTYPE_FP16, 64, 4, 16, 512) == 2      # 128-byte rows
    assert kk(B.PD_DTYPE_FP16, 64, 1, 1, 64) == 3
    assert kk(B.PD_DTYPE_FP32, 128, 1, 16, 1024) == 0
    assert kk(B.PD_DTYPE_FP16, 128, 4, 48, 1024) == 3    # 3 steps per page


def test_empty_requests_do_not_poison_neighbours(orc):
    w = workloads.generic("empty-mix", seed=60, dtype=workloads.FP16, page_size=16,
                          num_qo_heads=8, num_kv_heads=2, head_dim=128,
                          logical_start=[0, 0, 40, 100, 0], written_len=[300, 0, 40, 777, 5],
                          poison_unused=True)
    for fixed in (0, 1, 3):
        dec = run_flat(orc, w, target=64, fixed=fixed)
        out = dec.out.cpu().numpy()
        lse = dec.lse.cpu().numpy()
        for r in (1, 2):
            assert np.all(out[r] == 0) and np.all(np.isneginf(lse[r]))


def test_reverse_order_pages(orc):
    w = workloads.generic("reverse", seed=61, dtype=workloads.FP16, page_size=16,
                          num_qo_heads=32, num_kv_heads=8, head_dim=128,
                          logical_start=[0, 9, 0], written_len=[2000, 1500, 33],
                          poison_unused=True, reverse_pages=True)
    run_flat(orc, w, target=128)


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(orc, seed):
    """Shapes drawn at random over every axis the kernel choice looks at:
    dtype, head dim, group (1 to 32), KV heads (odd counts included, which
    give one KV head per workgroup), page size (1 to 64, powers of two and
    not), chunk size (the plan's, one page, three pages) and ragged windows
    -- each against the oracle, every partial row included."""
    rng = np.random.Generator(np.random.PCG64(900 + seed))
    dtype = workloads.FP32 if rng.random() < 0.25 else workloads.FP16
    d = int(rng.choice([64, 128]))
    groups = [1, 2, 4, 8, 12, 16] + ([24, 32] if dtype == workloads.FP16 else [])
    g = int(rng.choice(groups))
    hkv = int(rng.choice([1, 2, 3, 5, 6, 8]))
    ps = int(rng.choice([1, 2, 3, 5, 8, 16, 32, 48, 64]))
    fixed = int(rng.choice([0, 1, 3]))
    w = workloads.random_geometry(910 + seed, batch=int(rng.integers(1, 6)), page_size=ps,
                                  max_len=int(rng.integers(1, 1500)), dtype=dtype,
                                  num_qo_heads=g * hkv, num_kv_heads=hkv, head_dim=d,
                                  p_empty=0.1, p_trim=0.5)
    run_flat(orc, w, target=0, fixed=fixed)


def test_windows_start_mid_page_single_page(orc):
    # one-page windows whose first entry is not 0, plus a page-crossing window
    w = workloads.generic("midpage", seed=62, dtype=workloads.FP32, page_size=16,
                          num_qo_heads=4, num_kv_heads=1, head_dim=64,
                          logical_start=[3, 17, 30, 0], written_len=[9, 31, 34, 16],
                          poison_unused=True)
    run_flat(orc, w, fixed=1)
    run_flat(orc, w, target=1)


def test_many_pages_per_chunk_cross_lds_window(orc):
    """A chunk with more page ids than one LDS staging round (page_size 1)."""
    w = workloads.generic("long-ps1", seed=63, dtype=workloads.FP16, page_size=1,
                          num_qo_heads=4, num_kv_heads=1, head_dim=128,
                          logical_start=[0, 500], written_len=[3000, 2600], poison_unused=True)
    run_flat(orc, w, target=1)


@pytest.mark.parametrize("dtype", [workloads.FP16, workloads.FP32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8, 12, 16, 32])
def test_group_and_head_dim_variants(orc, dtype, d, g):
    if g == 32 and dtype != workloads.FP16:
        pytest.skip("G = 32 runs on the MFMA kernels only (fp16)")
    hkv = 2
    w = workloads.random_geometry(70 + g + d, batch=3, page_size=16, max_len=900, dtype=dtype,
                                  num_qo_heads=g * hkv, num_kv_heads=hkv, head_dim=d)
    run_flat(orc, w, target=32)


def test_runs_on_a_side_stream(orc):
    s = torch.cuda.Stream()
    run_flat(orc, workloads.batched_fp16(), target=256, stream=s)


def test_strided_pool_with_padding(orc):
    """Pool rows padded in the page and head axes (non-contiguous strides)."""
    w = workloads.generic("strided", seed=64, dtype=workloads.FP16, page_size=8,
                          num_qo_heads=8, num_kv_heads=2, head_dim=64,
                          logical_start=[0, 5], written_len=[100, 77])
    pages = w.k_pool.shape[0]
    kbig = np.full((pages, 9, 3, 64), np.nan, np.float16)
    vbig = np.full((pages, 9, 3, 64), np.nan, np.float16)
    kbig[:, :8, :2] = w.k_pool
    vbig[:, :8, :2] = w.v_pool
    kd, vd = to_dev(kbig)[:, :8, :2], to_dev(vbig)[:, :8, :2]
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, 8, pages)
    dec = PD.PagedDecode(csr, page_size=8, num_pool_pages=pages, num_qo_heads=8,
                         num_kv_heads=2, head_dim=64, target_wgs=8)
    out, lse = dec.run(to_dev(w.q), kd, vd, w.sm_scale)
    torch.cuda.synchronize()
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len, 8)
    ref_v, ref_l = orc.attention(w.q, w.k_pool, w.v_pool, ocsr, 8, w.sm_scale)
    check_close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, w.dtype, "strided")


# ------------------------------------------------------------ merge kernel

def _merge_gpu(v, l, oi):
    m = len(oi) - 1
    h, d = l.shape[1], v.shape[2]
    vo = torch.empty((m, h, d), dtype=torch.float32, device=DEV)
    lo = torch.empty((m, h), dtype=torch.float32, device=DEV)
    B.paged_merge_states(to_dev(v.astype(np.float32)), to_dev(l.astype(np.float32)),
                         to_dev(np.asarray(oi, np.int32)), m, h, d, vo, lo)
    torch.cuda.synchronize()
    return vo.cpu().numpy(), lo.cpu().numpy()


@pytest.mark.parametrize("d", [128, 64, 5])
def test_merge_kernel_against_oracle(orc, d):
    rng = np.random.default_rng(80 + d)
    n, h = 60, 6
    v = rng.standard_normal((n, h, d)).astype(np.float32)
    l = (rng.standard_normal((n, h)) * 8).astype(np.float32)
    l[rng.random((n, h)) < 0.2] = -np.inf
    v[np.isneginf(l)] = 1e30                   # never read: carries no weight
    l[10:14] = -np.inf                         # a group with no finite row
    oi = [0, 1, 5, 5, 10, 14, 20, 33, 34, 60]  # includes an empty group
    gv, gl = _merge_gpu(v, l, oi)
    rv, rl = orc.merge(v.astype(np.float64), l.astype(np.float64), oi)
    check_close(gv, gl, rv, rl, workloads.FP32, "merge d=%d" % d)
    assert np.all(gv[4] == 0) and np.all(np.isneginf(gl[4]))
    assert np.all(gv[2] == 0) and np.all(np.isneginf(gl[2]))


@pytest.mark.parametrize("d", [512, 96, 128])
def test_merge_kernel_long_groups(orc, d):
    """Groups longer than one load round of the row lanes (up to 300 rows),
    head dims split into 16, 3 and 4 dim slices, and -inf rows spread over
    every round."""
    rng = np.random.default_rng(95 + d)
    sizes = [300, 1, 129, 128, 33, 0, 257]
    oi = np.concatenate([[0], np.cumsum(sizes)]).tolist()
    n, h = oi[-1], 3
    v = rng.standard_normal((n, h, d)).astype(np.float32)
    l = (rng.standard_normal((n, h)) * 12).astype(np.float32)
    l[rng.random((n, h)) < 0.3] = -np.inf
    v[np.isneginf(l)] = 1e30                   # never read: carries no weight
    gv, gl = _merge_gpu(v, l, oi)
    rv, rl = orc.merge(v.astype(np.float64), l.astype(np.float64), oi)
    check_close(gv, gl, rv, rl, workloads.FP32, "long merge d=%d" % d)


def test_merge_kernel_regrouping(orc):
    rng = np.random.default_rng(90)
    n, h, d = 16, 4, 128
    v = rng.standard_normal((n, h, d)).astype(np.float32)
    l = (rng.standard_normal((n, h)) * 5).astype(np.float32)
    whole_v, whole_l = _merge_gpu(v, l, [0, n])
    pv, pl = _merge_gpu(v, l, [0, 3, 4, 9, 16])
    gv, gl = _merge_gpu(pv, pl, [0, 4])
    check_close(gv, gl, whole_v.astype(np.float64), whole_l.astype(np.float64),
                workloads.FP32, "regrouped merge")


def test_merge_kernel_nan_propagates(orc):
    v = np.ones((2, 1, 4), np.float32)
    l = np.array([[0.0], [np.nan]], np.float32)
    gv, gl = _merge_gpu(v, l, [0, 2])
    assert np.all(np.isnan(gv)) and np.isnan(gl[0, 0])


def test_default_target_is_cu_multiple():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for g, hkv in ((4, 8), (4, 2), (8, 8), (16, 8), (12, 1)):
        t = B.paged_decode_default_target_wgs(0, g, 128, B.PD_DTYPE_FP16, hkv)
        assert t >= cus and t % cus == 0, (g, hkv, t)


@pytest.mark.parametrize("name", ["long_context_fp16", "batched_fp16", "tiny_fp32",
                                  "token_sparse_fp16"])
def test_default_target_fits_one_round(orc, name):
    """Default plan: the largest target whose unit count fits the resident
    capacity S, lowered to the unit count of 32-slot chunks when the fit
    would cut chunks smaller; checked against the oracle's exhaustive
    plans."""
    if name == "token_sparse_fp16":
        w = workloads.folded_sparse(workloads.token_sparse_fp16())
    else:
        w = cached(name)
    csr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                    w.page_size)
    g = w.num_qo_heads // w.num_kv_heads
    dt = B.PD_DTYPE_FP16 if w.dtype == workloads.FP16 else B.PD_DTYPE_FP32
    slots = B.paged_decode_default_target_wgs(0, g, w.head_dim, dt, w.num_kv_heads)
    info, _, _, _ = B.paged_decode_plan(csr["indptr"], w.num_qo_heads, w.num_kv_heads,
                                        w.head_dim, 0, 0, sizes_only=True, dtype=dt,
                                        page_size=w.page_size)
    units = lambda t: orc.plan(csr["indptr"], w.num_kv_heads, t)["num_chunks"] * w.num_kv_heads
    best = max([t for t in range(1, slots + 1) if units(t) <= slots] or [slots])
    cmax = max(1, int(np.max(np.diff(csr["indptr"]))))
    c_lo = min(cmax, -(-32 // w.page_size))
    floor_units = orc.plan(csr["indptr"], w.num_kv_heads, 1,
                           fixed_pages_per_chunk=c_lo)["num_chunks"] * w.num_kv_heads
    assert info.target_wgs == min(best, floor_units)
    assert info.pages_per_chunk >= c_lo
    ref = orc.plan(csr["indptr"], w.num_kv_heads, info.target_wgs)
    assert info.pages_per_chunk == ref["pages_per_chunk"]
    assert info.num_wgs <= slots or units(1) > slots
    if name == "token_sparse_fp16":
        assert info.pages_per_chunk == 32          # page_size 1: the floor binds
    if name == "long_context_fp16":
        assert info.pages_per_chunk == 26          # the fit binds
