"""CPU pins for the oracle's attention, partial and merge (no GPU).

Pins, each chosen so that a plausible mistake in the oracle fails one of them:
- fp16 widening: exhaustive over all 65536 bit patterns against numpy.
- Closed forms: q = 0 gives the mean of V and LSE2 = log2 n; identical keys
  give the mean of V and LSE2 = s*log2(e) + log2 n; one visible token gives
  that token's V; constant V gives that V.
- Library special case: torch's scaled_dot_product_attention in float64 on
  K/V gathered through the block tables (not the CSR), per query head with
  KV head h // G.
- Relabelling pool rows (and the block tables with them) is bit-identical.
- Split invariance: merging the partials of any chunk size reproduces the
  whole-range attention (exact in real arithmetic).
- Merge algebra: identity on one row, -inf rows ignored, all -inf gives
  0 / -inf, equal LSEs give the mean and LSE + log2 n, regrouping and
  reordering do not change the result.
- Cascade identity: prefix + suffix merged equals the flat attention.
"""
import math

import numpy as np
import pytest

from paged_attention_decode_amd import workloads

LOG2E = 1.0 / math.log(2.0)


def test_half_widening_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _visible_rows(w, r, pool):
    """Rows of request r, gathered through its block table (not the CSR)."""
    ps = w.page_size
    rows = []
    for pos in range(int(w.logical_start[r]), int(w.written_len[r])):
        rows.append(pool[w.block_tables[r][pos // ps], pos % ps])
    return np.array(rows).reshape(-1, pool.shape[2], pool.shape[3])


def _csr(orc, w):
    return orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len, w.page_size)


def _geom(seed, dtype=workloads.FP32, hq=8, hkv=2, d=16, ps=4, b=5, max_len=60):
    return workloads.random_geometry(seed, batch=b, page_size=ps, max_len=max_len,
                                     dtype=dtype, num_qo_heads=hq, num_kv_heads=hkv,
                                     head_dim=d, poison_unused=True)


def test_closed_form_zero_query(orc):
    w = _geom(1)
    w.q[:] = 0
    out, lse = orc.attention(w.q, w.k_pool, w.v_pool, _csr(orc, w), w.page_size, w.sm_scale)
    g = w.num_qo_heads // w.num_kv_heads
    for r in range(w.batch):
        rows = _visible_rows(w, r, w.v_pool.astype(np.float64))
        n = rows.shape[0]
        for h in range(w.num_qo_heads):
            if n == 0:
                assert lse[r, h] == -np.inf and np.all(out[r, h] == 0)
                continue
            np.testing.assert_allclose(out[r, h], rows[:, h // g].mean(0), rtol=0, atol=1e-12)
            assert abs(lse[r, h] - math.log2(n)) < 1e-12


def test_closed_form_identical_keys_and_single_token(orc):
    w = _geom(2, ps=8)
    krow = np.random.default_rng(0).standard_normal(w.k_pool.shape[2:]).astype(w.k_pool.dtype)
    w.k_pool[:] = krow          # every key identical (per KV head)
    out, lse = orc.attention(w.q, w.k_pool, w.v_pool, _csr(orc, w), w.page_size, w.sm_scale)
    g = w.num_qo_heads // w.num_kv_heads
    for r in range(w.batch):
        rows = _visible_rows(w, r, w.v_pool.astype(np.float64))
        n = rows.shape[0]
        for h in range(w.num_qo_heads):
            if n == 0:
                continue
            s = w.sm_scale * float(np.dot(w.q[r, h].astype(np.float64),
                                          krow[h // g].astype(np.float64)))
            np.testing.assert_allclose(out[r, h], rows[:, h // g].mean(0), rtol=0, atol=1e-12)
            assert abs(lse[r, h] - (s * LOG2E + math.log2(n))) < 1e-11
    # n = 1: the output is that token's V, LSE2 = s0 * log2(e)
    w1 = workloads.generic("one", seed=3, dtype=workloads.FP32, page_size=4, num_qo_heads=4,
                           num_kv_heads=1, head_dim=8, logical_start=[5], written_len=[6])
    out, lse = orc.attention(w1.q, w1.k_pool, w1.v_pool, _csr(orc, w1), 4, w1.sm_scale)
    page = w1.block_tables[0][1]
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], w1.v_pool[page, 1, 0].astype(np.float64))
        s0 = w1.sm_scale * float(np.dot(w1.q[0, h].astype(np.float64),
                                        w1.k_pool[page, 1, 0].astype(np.float64)))
        assert abs(lse[0, h] - s0 * LOG2E) < 1e-12


def test_closed_form_constant_values(orc):
    w = _geom(4, dtype=workloads.FP16)
    w.v_pool[:] = np.float16(0.75)
    out, lse = orc.attention(w.q, w.k_pool, w.v_pool, _csr(orc, w), w.page_size, w.sm_scale)
    for r in range(w.batch):
        if w.written_len[r] > w.logical_start[r]:
            np.testing.assert_allclose(out[r], 0.75, rtol=0, atol=1e-13)


@pytest.mark.parametrize("dtype", [workloads.FP32, workloads.FP16])
def test_matches_torch_sdpa_float64(orc, dtype):
    torch = pytest.importorskip("torch")
    w = _geom(5, dtype=dtype, hq=12, hkv=3, d=32, ps=8, b=4, max_len=80)
    out, lse = orc.attention(w.q, w.k_pool, w.v_pool, _csr(orc, w), w.page_size, w.sm_scale)
    g = w.num_qo_heads // w.num_kv_heads
    for r in range(w.batch):
        k = _visible_rows(w, r, w.k_pool.astype(np.float64))
        v = _visible_rows(w, r, w.v_pool.astype(np.float64))
        if k.shape[0] == 0:
            continue
        for h in range(w.num_qo_heads):
            qt = torch.from_numpy(w.q[r, h].astype(np.float64)).view(1, 1, 1, -1)
            kt = torch.from_numpy(np.ascontiguousarray(k[:, h // g])).view(1, 1, k.shape[0], -1)
            vt = torch.from_numpy(np.ascontiguousarray(v[:, h // g])).view(1, 1, k.shape[0], -1)
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=w.sm_scale)
            np.testing.assert_allclose(out[r, h], ref.view(-1).numpy(), rtol=0, atol=1e-12)
            lref = torch.logsumexp(w.sm_scale * (kt.view(k.shape[0], -1) @ qt.view(-1)), 0)
            assert abs(lse[r, h] - float(lref) * LOG2E) < 1e-12


def test_relabel_invariance_bit_identical(orc):
    w = _geom(6, ps=4)
    out, lse = orc.attention(w.q, w.k_pool, w.v_pool, _csr(orc, w), w.page_size, w.sm_scale)
    perm = np.random.default_rng(0).permutation(w.k_pool.shape[0])
    inv = np.argsort(perm)
    k2, v2 = w.k_pool[perm], w.v_pool[perm]   # new row j holds old row perm[j]
    tables = [np.where(t >= 0, inv[np.maximum(t, 0)], -1).astype(np.int32) for t in w.block_tables]
    csr2 = orc.csr_from_block_tables(tables, w.logical_start, w.written_len, w.page_size)
    out2, lse2 = orc.attention(w.q, k2, v2, csr2, w.page_size, w.sm_scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_gqa_head_mapping_negative_control(orc):
    # KV head 1 holds different values from KV head 0: query heads 0..G-1 must
    # follow head 0 only
    w = workloads.generic("gqa", seed=8, dtype=workloads.FP32, page_size=4, num_qo_heads=4,
                          num_kv_heads=2, head_dim=8, logical_start=[0], written_len=[10])
    w.v_pool[:, :, 0, :] = 1.0
    w.v_pool[:, :, 1, :] = -1.0
    out, _ = orc.attention(w.q, w.k_pool, w.v_pool, _csr(orc, w), 4, w.sm_scale)
    np.testing.assert_allclose(out[0, :2], 1.0, atol=1e-14)
    np.testing.assert_allclose(out[0, 2:], -1.0, atol=1e-14)


@pytest.mark.parametrize("seed", [10, 11, 12])
def test_split_invariance_over_chunk_sizes(orc, seed):
    w = _geom(seed, ps=4, b=6, max_len=90)
    csr = _csr(orc, w)
    full, lfull = orc.attention(w.q, w.k_pool, w.v_pool, csr, w.page_size, w.sm_scale)
    pages = np.diff(csr["indptr"])
    for c in [1, 2, 3, 5, max(1, int(pages.max()))]:
        p = orc.plan(csr["indptr"], w.num_kv_heads, 1, fixed_pages_per_chunk=c)
        v, l = orc.partial(w.q, w.k_pool, w.v_pool, csr, w.page_size, w.sm_scale,
                           p["request_indices"], p["kv_tile_indices"], c)
        mo, ml = orc.merge(v, l, p["o_indptr"])
        np.testing.assert_allclose(mo, full, rtol=0, atol=1e-12)
        fin = np.isfinite(lfull)
        assert np.array_equal(fin, np.isfinite(ml))
        np.testing.assert_allclose(ml[fin], lfull[fin], rtol=0, atol=1e-12)
        # chunk token ranges tile the visible range exactly: the token counts
        # implied by each chunk's LSE under q = 0 add up to n_r
    wz = _geom(seed, ps=4, b=6, max_len=90)
    wz.q[:] = 0
    csrz = _csr(orc, wz)
    p = orc.plan(csrz["indptr"], wz.num_kv_heads, 1, fixed_pages_per_chunk=2)
    _, l = orc.partial(wz.q, wz.k_pool, wz.v_pool, csrz, 4, wz.sm_scale,
                       p["request_indices"], p["kv_tile_indices"], 2)
    counts = np.where(np.isfinite(l[:, 0]), np.exp2(l[:, 0]), 0.0)
    for r in range(wz.batch):
        a, b = p["o_indptr"][r], p["o_indptr"][r + 1]
        assert round(counts[a:b].sum()) == wz.written_len[r] - wz.logical_start[r]


def test_merge_algebra(orc):
    rng = np.random.default_rng(3)
    h, d = 3, 5
    v = rng.standard_normal((1, h, d))
    l = rng.standard_normal((1, h)) * 4
    mo, ml = orc.merge(v, l, [0, 1])
    np.testing.assert_allclose(mo, v, atol=1e-15)
    np.testing.assert_allclose(ml, l, atol=1e-15)
    # -inf rows carry no weight whatever their V
    v2 = np.concatenate([v, np.full((2, h, d), 1e30)])
    l2 = np.concatenate([l, np.full((2, h), -np.inf)])
    mo, ml = orc.merge(v2, l2, [0, 3])
    np.testing.assert_allclose(mo[0], v[0], atol=1e-15)
    np.testing.assert_allclose(ml[0], l[0], atol=1e-15)
    # all -inf (and the empty group) -> zeros, -inf, never NaN
    mo, ml = orc.merge(v2[1:], l2[1:], [0, 2, 2])
    assert np.all(mo == 0) and np.all(ml == -np.inf)
    # equal LSEs: arithmetic mean, LSE + log2 n
    v3 = rng.standard_normal((4, h, d))
    l3 = np.full((4, h), 2.5)
    mo, ml = orc.merge(v3, l3, [0, 4])
    np.testing.assert_allclose(mo[0], v3.mean(0), atol=1e-14)
    np.testing.assert_allclose(ml[0], 2.5 + 2.0, atol=1e-14)
    # two rows: weights 2^l / (2^la + 2^lb), by direct evaluation at a point
    va, vb = np.ones((1, 1, 1)), 3 * np.ones((1, 1, 1))
    mo, ml = orc.merge(np.concatenate([va, vb]), np.array([[0.0], [1.0]]), [0, 2])
    assert abs(mo[0, 0, 0] - (1 * 1 + 3 * 2) / 3) < 1e-15 and abs(ml[0, 0] - math.log2(3)) < 1e-15


def test_merge_regrouping_and_order(orc):
    rng = np.random.default_rng(5)
    n, h, d = 9, 2, 4
    v = rng.standard_normal((n, h, d))
    l = rng.standard_normal((n, h)) * 6
    l[3, 1] = -np.inf
    whole_v, whole_l = orc.merge(v, l, [0, n])
    for _ in range(20):
        perm = rng.permutation(n)
        cuts = np.sort(rng.choice(np.arange(1, n), size=rng.integers(1, 5), replace=False))
        oi = np.concatenate([[0], cuts, [n]])
        pv, pl = orc.merge(v[perm], l[perm], oi)
        gv, gl = orc.merge(pv, pl, [0, len(oi) - 1])
        np.testing.assert_allclose(gv, whole_v, atol=1e-13)
        np.testing.assert_allclose(gl, whole_l, atol=1e-13)


def test_cascade_identity(orc):
    """Prefix states and suffix states merged per member equal the flat
    attention over the whole page list."""
    w = workloads.cascade_fp16(seed=9, members=3, prefix_tokens=64, suffix_lo=5,
                               suffix_hi=40, hq=8, hkv=2, d=16, ps=16)
    ps = w.page_size
    csr = _csr(orc, w)
    flat, lflat = orc.attention(w.q, w.k_pool, w.v_pool, csr, ps, w.sm_scale)
    sp = w.extra["shared_pages"]
    pre = [t[:sp] for t in w.block_tables]
    suf = [t[sp:] for t in w.block_tables]
    cpre = orc.csr_from_block_tables(pre, [0] * 3, [sp * ps] * 3, ps)
    csuf = orc.csr_from_block_tables(suf, [0] * 3, w.extra["suffix_tokens"], ps)
    a, la = orc.attention(w.q, w.k_pool, w.v_pool, cpre, ps, w.sm_scale)
    b, lb = orc.attention(w.q, w.k_pool, w.v_pool, csuf, ps, w.sm_scale)
    v = np.stack([a, b], 1).reshape(6, 8, 16)
    l = np.stack([la, lb], 1).reshape(6, 8)
    mo, ml = orc.merge(v, l, [0, 2, 4, 6])
    np.testing.assert_allclose(mo, flat, atol=1e-12)
    np.testing.assert_allclose(ml, lflat, atol=1e-12)
