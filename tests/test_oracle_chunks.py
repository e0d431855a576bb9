"""CPU pins for the oracle's chunk -> token-range mapping (no GPU).

The partial oracle (``partial``) and the chunk mode of ``attention_mla``
restrict attention to the tokens of one chunk.  Split invariance and the sum
of the per-chunk counts cannot see how the chunks cut a request -- cutting by
tokens instead of pages, or dropping the first_page_offset shift, still tiles
[0, n_r).  These tests read every chunk's exact token range off the oracle
and compare it with ranges worked by hand from the page rule
(``tests/golden/chunk_ranges.json``, PR #984 body items 2 and 4 and the
"plan + launch" commit; sparse paged decode doc, "Indirection"):

- q = 0 makes every weight equal, so 2^LSE2 is the chunk's token count;
- V rows carry the token's own number (hi*64 + lo in two columns, exact in
  fp16 and fp32), so the output is the mean token number (tb + te - 1) / 2;
- every slot outside the visible tokens holds NaN, so a chunk that reads one
  returns NaN.

Count and mean together fix [tb, te) exactly.  The last test is the O7 pin
for the token-sparse folding (sparse paged decode doc, "ContiguousCacheLayout"):
attention over the folded page_size-1 table equals attention over the
selected positions of the dense allocation.
"""
import json
import math
import os

import numpy as np
import pytest

from paged_attention_decode_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "chunk_ranges.json")))


def _layout(case, seed, width, dtype, heads=1):
    """A pool [pages, ps, heads * width] whose visible slot of token i of
    request r holds (i // 64, i % 64, r) in columns 0..2 of each head's
    width (the rest 1.0), every other slot NaN; returns (pool, csr,
    request_indices, kv_tile_indices, ranges)."""
    ps, c = case["page_size"], case["pages_per_chunk"]
    reqs = case["requests"]
    total = sum(q["pages"] for q in reqs)
    rng = np.random.default_rng(seed)
    pool_pages = 2 * total + 3
    perm = rng.permutation(pool_pages).astype(np.int32)
    pool = np.full((pool_pages, ps, heads, width), np.nan, dtype)
    indptr, indices, lpl, fpo = [0], [], [], []
    ri, ti, ranges = [], [], []
    pos = 0
    for r, q in enumerate(reqs):
        pages = perm[pos:pos + q["pages"]]
        pos += q["pages"]
        indices += pages.tolist()
        indptr.append(indptr[-1] + q["pages"])
        lpl.append(q["lpl"])
        fpo.append(q["fpo"])
        n = (q["pages"] - 1) * ps + q["lpl"] - q["fpo"] if q["pages"] else 0
        for i in range(n):
            slot = q["fpo"] + i
            row = pool[pages[slot // ps], slot % ps]
            row[:] = 1.0
            row[:, 0], row[:, 1], row[:, 2] = i // 64, i % 64, r
        nchunks = max(1, -(-q["pages"] // c))
        assert len(q["ranges"]) == nchunks, case["name"]
        for t in range(nchunks):
            ri.append(r)
            ti.append(t)
            ranges.append((r, *q["ranges"][t]))
    csr = dict(indptr=np.array(indptr, np.int32), indices=np.array(indices, np.int32),
               last_page_len=np.array(lpl, np.int32), first_page_offset=np.array(fpo, np.int32))
    return (pool.reshape(pool_pages, ps, heads * width), csr, np.array(ri, np.int32),
            np.array(ti, np.int32), ranges)


def _check_ranges(out, lse, ranges, name):
    for row, (r, tb, te) in enumerate(ranges):
        n = te - tb
        if n == 0:
            assert np.all(lse[row] == -np.inf), (name, row)
            assert np.all(out[row] == 0.0), (name, row)
            continue
        assert np.all(np.isfinite(out[row])), (name, row, "read a slot outside the chunk")
        np.testing.assert_allclose(np.exp2(lse[row]), n, rtol=1e-12, err_msg=name)
        mean_tok = 64.0 * out[row, :, 0] + out[row, :, 1]
        np.testing.assert_allclose(mean_tok, (tb + te - 1) / 2.0, rtol=0, atol=1e-9,
                                   err_msg="%s chunk %d" % (name, row))
        np.testing.assert_allclose(out[row, :, 2], r, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=lambda c: c["name"])
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_partial_chunk_ranges_golden(orc, case, dtype):
    hkv, hq, d = 2, 4, 8
    pool, csr, ri, ti, ranges = _layout(case, 1, d, dtype, heads=hkv)
    ps = case["page_size"]
    k = pool.reshape(pool.shape[0], ps, hkv, d)
    v = k.copy()
    q = np.zeros((len(case["requests"]), hq, d), dtype)
    out, lse = orc.partial(q, k, v, csr, ps, 1.0 / math.sqrt(d), ri, ti,
                           case["pages_per_chunk"])
    _check_ranges(out, lse, ranges, case["name"])


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=lambda c: c["name"])
def test_mla_chunk_ranges_golden(orc, case):
    dim, ex, hq = 16, 8, 4
    ps = case["page_size"]
    lat, csr, ri, ti, ranges = _layout(case, 2, dim + 8, np.float16)
    xp = np.where(np.isnan(lat[:, :, :ex]), np.float16(np.nan), np.float16(0.5))
    q = np.zeros((len(case["requests"]), hq, dim), np.float16)
    qx = np.zeros((len(case["requests"]), hq, ex), np.float16)
    out, lse = orc.attention_mla(q, qx, lat, np.ascontiguousarray(xp), csr, ps, 0.1,
                                 chunks=(ri, ti, case["pages_per_chunk"]))
    _check_ranges(out, lse, ranges, case["name"])


def test_chunk_ranges_follow_the_plan(orc):
    """The plan's chunk list for the hand-worked ragged case (fixed c = 3) is
    the request-major enumeration the golden ranges assume."""
    case = next(c for c in GOLDEN["cases"] if c["name"] == "ragged_ps4_c3")
    _, csr, ri, ti, _ = _layout(case, 3, 4, np.float32)
    p = orc.plan(csr["indptr"], 1, 1, fixed_pages_per_chunk=3)
    assert p["request_indices"].tolist() == ri.tolist()
    assert p["kv_tile_indices"].tolist() == ti.tolist()


def test_token_sparse_folding_two_legs(orc):
    """O7: the selection read through the folded page_size-1 table (one
    request per KV head, query head i under request i // G) equals attention
    over the same positions gathered from the dense [1, Hkv, Cap, D]
    allocation; mapping query heads to KV heads any other way differs."""
    s = workloads.token_sparse_fp16(seed=21, cap=512, topk=40, hq=6, hkv=2, d=16)
    w = workloads.folded_sparse(s)
    csr = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len, 1)
    out, lse = orc.attention(w.q, w.k_pool, w.v_pool, csr, 1, w.sm_scale)
    _, hkv, cap, d = s.k_dense.shape
    hq = s.q.shape[1]
    g = hq // hkv
    k = s.k_dense.astype(np.float64)
    v = s.v_dense.astype(np.float64)
    qd = s.q.astype(np.float64)
    for i in range(hq):
        pos = s.positions[i // g]
        ref, lref = orc.attention_dense_f64(qd[0, i, 0], k[0, i // g, pos], v[0, i // g, pos],
                                            s.sm_scale)
        np.testing.assert_allclose(out[i // g, i % g], ref, rtol=0, atol=1e-12)
        assert abs(lse[i // g, i % g] - lref) < 1e-12
    # negative control: query head i under KV head i % Hkv reads other rows
    i = 1
    wrong, _ = orc.attention_dense_f64(qd[0, i, 0], k[0, i % hkv, s.positions[i % hkv]],
                                       v[0, i % hkv, s.positions[i % hkv]], s.sm_scale)
    assert np.max(np.abs(out[i // g, i % g] - wrong)) > 1e-3
