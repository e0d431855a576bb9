"""CPU pins for the oracle's block-selection helpers (no GPU).

`block_positions` (the positions a list of selected blocks covers, sparse
paged decode doc, "Selection from blocks") and `attention_dense_f64` (one
query over gathered rows) serve the block-sparse parity test.  Pins:
- block_positions: a hand-worked selection (out-of-order blocks, a final
  block cut at the live length), and the count rule on random selections;
- attention_dense_f64: the closed forms (q = 0, identical keys, one row,
  no rows) and torch's scaled_dot_product_attention in float64.
"""
import math

import numpy as np
import pytest

LOG2E = 1.0 / math.log(2.0)


def test_block_positions_hand_worked(orc):
    # blocks of 4 positions, live length 22: block 5 holds positions 20, 21 only
    got = orc.block_positions([3, 0, 5], 4, 22)
    assert got.tolist() == [12, 13, 14, 15, 0, 1, 2, 3, 20, 21]
    # a final block that is exactly full contributes all of its positions
    assert orc.block_positions([1, 2], 8, 24).tolist() == list(range(8, 24))
    assert orc.block_positions([], 8, 24).tolist() == []


def test_block_positions_count_rule(orc):
    rng = np.random.default_rng(11)
    for _ in range(200):
        c = int(rng.integers(1, 40))
        kv_len = int(rng.integers(1, 2000))
        nblk = (kv_len + c - 1) // c
        ids = rng.choice(nblk, size=int(rng.integers(1, nblk + 1)), replace=False)
        pos = orc.block_positions(ids, c, kv_len)
        want = sum(min(c, kv_len - int(j) * c) for j in ids)
        assert len(pos) == want
        assert np.all(pos < kv_len) and len(set(pos.tolist())) == want
        assert np.all(np.isin(pos // c, ids))


def test_attention_dense_closed_forms(orc):
    rng = np.random.default_rng(12)
    n, d = 37, 16
    v = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    # q = 0: uniform weights
    out, lse = orc.attention_dense_f64(np.zeros(d), k, v, 0.25)
    np.testing.assert_allclose(out, v.mean(0), rtol=0, atol=1e-13)
    assert abs(lse - math.log2(n)) < 1e-12
    # identical keys: uniform weights, LSE2 = s * log2 e + log2 n
    q = rng.standard_normal(d)
    kk = np.tile(k[:1], (n, 1))
    out, lse = orc.attention_dense_f64(q, kk, v, 0.25)
    s = 0.25 * float(k[0] @ q)
    np.testing.assert_allclose(out, v.mean(0), rtol=0, atol=1e-13)
    assert abs(lse - (s * LOG2E + math.log2(n))) < 1e-12
    # one row: that row's value
    out, lse = orc.attention_dense_f64(q, k[:1], v[:1], 0.25)
    np.testing.assert_allclose(out, v[0], rtol=0, atol=0)
    assert abs(lse - s * LOG2E) < 1e-12
    # no rows: zeros and -inf
    out, lse = orc.attention_dense_f64(q, k[:0], v[:0], 0.25)
    assert np.all(out == 0) and lse == -np.inf


def test_attention_dense_matches_torch_sdpa_float64(orc):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    for n, d in ((1, 8), (5, 32), (300, 128)):
        q = rng.standard_normal(d)
        k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, d))
        scale = 1.0 / math.sqrt(d)
        out, lse = orc.attention_dense_f64(q, k, v, scale)
        qt = torch.from_numpy(q).view(1, 1, 1, d)
        kt = torch.from_numpy(k).view(1, 1, n, d)
        vt = torch.from_numpy(v).view(1, 1, n, d)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        np.testing.assert_allclose(out, ref.view(-1).numpy(), rtol=0, atol=1e-12)
        lref = float(torch.logsumexp(scale * (kt.view(n, d) @ qt.view(d)), 0)) * LOG2E
        assert abs(lse - lref) < 1e-12
