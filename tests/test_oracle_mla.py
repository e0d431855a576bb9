"""CPU pins for the oracle's decode with a second key stream (attention_mla).

The method (sparse-paged-decode doc, DSA section) scores a token with
scale * (q . k[0:Dim]) + scale * (q_extra . k_extra) and, with the latent as
values, reaches exactly plain attention over concatenated rows -- the doc
calls folding the positional term into the dot product "numerically exact".
Pins, each independent of attention_mla's own code:
- concatenation identity: plain attention (the flat oracle, itself pinned in
  test_oracle_attention.py) over rows concat(latent, rope) with values
  concat(latent, 0) and queries concat(q, q_extra) gives the same output and
  LSE;
- torch's scaled_dot_product_attention in float64 over the gathered rows;
- closed forms: both queries zero gives the mean latent row and LSE2 = log2 n;
  a zero q_extra makes the result independent of the rope keys (bit-exact);
- split invariance: merging the chunk-mode rows of any chunk size gives the
  whole-request result;
- the row columns past Dim (the indexer key) are never read: NaN there leaves
  the output finite and unchanged.
"""
import math

import numpy as np
import pytest

from paged_attention_decode_amd import workloads

LOG2E = 1.0 / math.log(2.0)


def _small(seed=1, **kw):
    geom = dict(seed=seed, logical_start=[0, 5, 0, 3], written_len=[100, 77, 0, 3],
                num_qo_heads=4, page_size=8, dim=32, extra_dim=8, row_stride=48)
    geom.update(kw)
    return workloads.mla_paged("tiny_mla", **geom)


def _csr(orc, w):
    return orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                     w.page_size)


def test_concatenation_identity_against_flat_oracle(orc):
    w = _small()
    csr = _csr(orc, w)
    out, lse = orc.attention_mla(w.q, w.q_extra, w.k_pool, w.k_extra_pool, csr, w.page_size,
                                 w.sm_scale)
    lat = w.k_pool[:, :, :w.dim]
    kcat = np.concatenate([lat, w.k_extra_pool], axis=2)[:, :, None, :]
    vcat = np.concatenate([lat, np.zeros_like(w.k_extra_pool)], axis=2)[:, :, None, :]
    qcat = np.concatenate([w.q, w.q_extra], axis=2)
    # plain attention: every query head reads the single KV head
    ref_v, ref_l = orc.attention(qcat, np.ascontiguousarray(kcat), np.ascontiguousarray(vcat),
                                 csr, w.page_size, w.sm_scale)
    np.testing.assert_allclose(out, ref_v[:, :, :w.dim], rtol=0, atol=1e-12)
    assert np.all(ref_v[:, :, w.dim:] == 0)
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], ref_l[fin], rtol=0, atol=1e-12)
    assert np.all(np.isneginf(lse[2]))              # the empty request


def test_matches_torch_sdpa_float64(orc):
    torch = pytest.importorskip("torch")
    w = _small(seed=2)
    csr = _csr(orc, w)
    out, lse = orc.attention_mla(w.q, w.q_extra, w.k_pool, w.k_extra_pool, csr, w.page_size,
                                 w.sm_scale)
    ps = w.page_size
    for r in range(w.batch):
        t = w.block_tables[r]
        pos = np.arange(int(w.logical_start[r]), int(w.written_len[r]))
        if pos.size == 0:
            continue
        pages, ents = t[pos // ps], pos % ps
        lat = w.k_pool[pages, ents, :w.dim].astype(np.float64)
        rope = w.k_extra_pool[pages, ents].astype(np.float64)
        k = torch.from_numpy(np.concatenate([lat, rope], 1)).view(1, 1, pos.size, -1)
        v = torch.from_numpy(lat).view(1, 1, pos.size, -1)
        for h in range(w.num_qo_heads):
            qv = np.concatenate([w.q[r, h], w.q_extra[r, h]]).astype(np.float64)
            qt = torch.from_numpy(qv).view(1, 1, 1, -1)
            ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=w.sm_scale)
            np.testing.assert_allclose(out[r, h], ref.view(-1).numpy(), rtol=0, atol=1e-12)
            lref = float(torch.logsumexp(w.sm_scale * (k.view(pos.size, -1) @ qt.view(-1)), 0))
            assert abs(lse[r, h] - lref * LOG2E) < 1e-12


def test_closed_forms(orc):
    w = _small(seed=3)
    csr = _csr(orc, w)
    zq, zx = np.zeros_like(w.q), np.zeros_like(w.q_extra)
    out, lse = orc.attention_mla(zq, zx, w.k_pool, w.k_extra_pool, csr, w.page_size,
                                 w.sm_scale)
    ps = w.page_size
    for r in range(w.batch):
        pos = np.arange(int(w.logical_start[r]), int(w.written_len[r]))
        if pos.size == 0:
            continue
        t = w.block_tables[r]
        mean = w.k_pool[t[pos // ps], pos % ps, :w.dim].astype(np.float64).mean(0)
        for h in range(w.num_qo_heads):
            np.testing.assert_allclose(out[r, h], mean, rtol=0, atol=1e-13)
            assert abs(lse[r, h] - math.log2(pos.size)) < 1e-12
    # no rope query: the rope keys do not matter, bit for bit
    a = orc.attention_mla(w.q, zx, w.k_pool, w.k_extra_pool, csr, w.page_size, w.sm_scale)
    kx2 = (w.k_extra_pool * np.float16(-3)).astype(np.float16)
    b = orc.attention_mla(w.q, zx, w.k_pool, kx2, csr, w.page_size, w.sm_scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # ...but with a rope query they do (a dropped second term would not notice)
    c = orc.attention_mla(w.q, w.q_extra, w.k_pool, kx2, csr, w.page_size, w.sm_scale)
    d = orc.attention_mla(w.q, w.q_extra, w.k_pool, w.k_extra_pool, csr, w.page_size,
                          w.sm_scale)
    assert np.max(np.abs(c[0] - d[0])) > 1e-3


@pytest.mark.parametrize("c", [1, 2, 3, 5])
def test_split_invariance(orc, c):
    w = _small(seed=4)
    csr = _csr(orc, w)
    whole = orc.attention_mla(w.q, w.q_extra, w.k_pool, w.k_extra_pool, csr, w.page_size,
                              w.sm_scale)
    plan = orc.plan(csr["indptr"], 1, 1, fixed_pages_per_chunk=c)
    pv, pl = orc.attention_mla(w.q, w.q_extra, w.k_pool, w.k_extra_pool, csr, w.page_size,
                               w.sm_scale, chunks=(plan["request_indices"],
                                                   plan["kv_tile_indices"], c))
    mv, ml = orc.merge(pv, pl, plan["o_indptr"])
    np.testing.assert_allclose(mv, whole[0], rtol=0, atol=1e-12)
    fin = np.isfinite(whole[1])
    assert np.array_equal(fin, np.isfinite(ml))
    np.testing.assert_allclose(ml[fin], whole[1][fin], rtol=0, atol=1e-12)


def test_indexer_columns_never_read(orc):
    w = _small(seed=5)
    p = _small(seed=5, poison_indexer=True, poison_unused=True)
    csr = _csr(orc, w)
    a = orc.attention_mla(w.q, w.q_extra, w.k_pool, w.k_extra_pool, csr, w.page_size,
                          w.sm_scale)
    b = orc.attention_mla(p.q, p.q_extra, p.k_pool, p.k_extra_pool, csr, p.page_size,
                          p.sm_scale)
    assert np.all(np.isfinite(b[0]))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
