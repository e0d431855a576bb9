"""GPU test of paged_decode_fused_noalloc: the fused decode with its
workspace (partial rows, LSEs, arrival counters) in the library's own device
array, for callers that cannot allocate.  Its output must match
paged_decode_fused with caller-owned buffers on the same inputs, to the fp16 /
fp32 tolerances, over two calls in a row whose second is smaller -- the array
keeps the first call's contents, which the second must neither read nor
depend on -- and through a HIP graph replay.  Both are also checked against
the f64 oracle.
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

DEV = torch.device("cuda:0")
NTHREADS = min(16, os.cpu_count() or 1)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tol(w):
    return (1e-5, 1e-5) if w.dtype == workloads.FP32 else (2e-3, 1e-3)


def _close(got_v, got_l, ref_v, ref_l, tv, tl, what):
    got_v = np.asarray(got_v, np.float64)
    got_l = np.asarray(got_l, np.float64)
    ref_v = np.asarray(ref_v, np.float64)
    ref_l = np.asarray(ref_l, np.float64)
    assert np.all(np.isfinite(got_v)), what
    inf = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), inf), what
    dv = float(np.max(np.abs(got_v - ref_v)))
    dl = float(np.max(np.abs(got_l[~inf] - ref_l[~inf]))) if (~inf).any() else 0.0
    say("  %s: max|dv|=%.3g max|dlse|=%.3g" % (what, dv, dl))
    assert dv <= tv and dl <= tl, what


def _noalloc(dec, q, k, v, sm_scale, out, lse):
    ps_, ts_, hs_ = PD.pool_strides(k, v)
    B.paged_decode_fused_noalloc(q, k, v, ps_, ts_, hs_, PD._pd_dtype(q), dec.d_indices,
                                 dec.d_indptr, dec.d_lpl, dec.d_fpo, dec.d_req, dec.d_tile,
                                 dec.info.num_chunks, dec.info.pages_per_chunk, dec.batch,
                                 dec.num_qo_heads, dec.num_kv_heads, dec.head_dim,
                                 dec.page_size, sm_scale, out, lse)


def _case(orc, w, target=0, fixed=0):
    say("case %s B=%d Hq=%d Hkv=%d D=%d ps=%d dtype=%s" % (
        w.name, w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, w.dtype))
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                            w.k_pool.shape[0])
    dt = torch.float32 if w.dtype == workloads.FP32 else torch.float16
    dec = PD.PagedDecode(csr, page_size=w.page_size, num_pool_pages=w.k_pool.shape[0],
                         num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                         head_dim=w.head_dim, target_wgs=target, fixed_pages_per_chunk=fixed,
                         fused=True, dtype=dt, device=DEV)
    say("  plan", dec.plan_summary())
    q = torch.from_numpy(w.q).to(DEV)
    k = torch.from_numpy(w.k_pool).to(DEV)
    v = torch.from_numpy(w.v_pool).to(DEV)
    ocsr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                     w.page_size)
    ref_v, ref_l = orc.attention(w.q, w.k_pool, w.v_pool, ocsr, w.page_size, w.sm_scale,
                                 nthreads=NTHREADS)
    return dec, q, k, v, ref_v, ref_l


def test_noalloc_matches_fused_two_calls_second_smaller(orc):
    big = workloads.random_geometry(901, batch=6, page_size=16, max_len=6000,
                                    num_qo_heads=32, num_kv_heads=8, p_empty=0.15, p_trim=0.5)
    small = workloads.tiny_fp32()
    results = []
    for w, target, fixed in ((big, 0, 2), (small, 8, 0)):
        dec, q, k, v, ref_v, ref_l = _case(orc, w, target, fixed)
        assert dec.info.needs_merge
        tv, tl = _tol(w)
        # the fused entry point with caller-owned buffers
        out_f, lse_f = dec.run(q, k, v, w.sm_scale)
        torch.cuda.synchronize()
        out_f, lse_f = out_f.cpu().numpy(), lse_f.cpu().numpy()
        # the no-allocation variant, into fresh outputs pre-filled with NaN
        out = torch.full((dec.batch, dec.num_qo_heads, dec.head_dim), float("nan"),
                         device=DEV)
        lse = torch.full((dec.batch, dec.num_qo_heads), float("nan"), device=DEV)
        _noalloc(dec, q, k, v, w.sm_scale, out, lse)
        torch.cuda.synchronize()
        _close(out.cpu().numpy(), lse.cpu().numpy(), out_f, lse_f, tv, tl,
               "%s noalloc vs fused" % w.name)
        _close(out.cpu().numpy(), lse.cpu().numpy(), ref_v, ref_l, tv, tl,
               "%s noalloc vs oracle" % w.name)
        same = np.array_equal(out.cpu().numpy(), out_f)
        say("  bit-identical to the fused entry point: %s" % same)
        results.append(same)


def test_noalloc_replayed_from_hip_graph(orc):
    """The call captured in a HIP graph (its counter reset is a kernel, not a
    memset node) and replayed several times with new queries, with eager
    work and synchronizations between replays; every replay against the
    fused entry point's eager result."""
    w = workloads.random_geometry(902, batch=4, page_size=16, max_len=4000,
                                  num_qo_heads=32, num_kv_heads=8, p_empty=0.0, p_trim=0.3)
    dec, q, k, v, _, _ = _case(orc, w, 0, 3)
    tv, tl = _tol(w)
    out = torch.zeros((dec.batch, dec.num_qo_heads, dec.head_dim), device=DEV)
    lse = torch.zeros((dec.batch, dec.num_qo_heads), device=DEV)
    qg = q.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _noalloc(dec, qg, k, v, w.sm_scale, out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _noalloc(dec, qg, k, v, w.sm_scale, out, lse)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(5)
    for it in range(4):
        qn = torch.randn(q.shape, generator=gen).to(torch.float16).to(DEV)
        qg.copy_(qn)
        g.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = dec.run(qn, k, v, w.sm_scale)
        torch.cuda.synchronize()
        _close(out.cpu().numpy(), lse.cpu().numpy(), ref_o.cpu().numpy(),
               ref_l.cpu().numpy(), tv, tl, "graph replay %d" % it)
