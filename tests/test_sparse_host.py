"""CPU tests of the block-selection page table's shape (sparse-paged-decode
doc, the two granularities): token-exact tables hold one one-token page per
selected position, block-granular tables one page per block with the final
block's written positions as last_page_len, and tables in between name each
block by block_size / page_size pages."""
import numpy as np
import pytest

from paged_attention_decode_amd import binding as B


def test_sparse_csr_token_exact_and_block_granular():
    tail = np.array([91, 128, 1], np.int32)
    t = B.paged_sparse_csr(16, 128, tail, page_size=1)
    counts = np.diff(t["indptr"])
    assert counts.tolist() == [15 * 128 + 91, 16 * 128, 15 * 128 + 1]
    assert np.all(t["last_page_len"] == 1) and np.all(t["first_page_offset"] == 0)
    b = B.paged_sparse_csr(16, 128, tail, page_size=128)
    assert b["indptr"].tolist() == [0, 16, 32, 48]
    assert b["last_page_len"].tolist() == [91, 128, 1]
    # 32-row pages: 4 per block; the final block's 91 positions fill 3 pages,
    # the last holding 91 - 64 = 27; 128 positions fill 4; 1 position 1
    m = B.paged_sparse_csr(16, 128, tail, page_size=32)
    assert np.diff(m["indptr"]).tolist() == [15 * 4 + 3, 16 * 4, 15 * 4 + 1]
    assert m["last_page_len"].tolist() == [27, 32, 1]
    # every table satisfies the geometry identity with the selected position counts
    for csr, ps in ((t, 1), (b, 128), (m, 32)):
        nnz = int(csr["indptr"][-1])
        B.csr_validate(3, ps, nnz, csr["indptr"], np.arange(nnz, dtype=np.int32),
                       csr["last_page_len"], csr["first_page_offset"],
                       seq_lens=15 * 128 + tail)


def test_sparse_csr_page_sizes_against_brute_force():
    """Every page size dividing the block, random tails: the page count and
    last page length equal those of cutting the selected positions (block by
    block, the final block cut to its tail) into pages of page_size rows."""
    rng = np.random.default_rng(5)
    for c in (16, 64, 96):
        for ps in [p for p in range(1, c + 1) if c % p == 0]:
            blocks = int(rng.integers(1, 6))
            tail = rng.integers(1, c + 1, size=4).astype(np.int32)
            t = B.paged_sparse_csr(blocks, c, tail, page_size=ps)
            for r in range(4):
                sizes = [ps] * ((blocks - 1) * (c // ps))
                rest = int(tail[r])
                while rest > 0:
                    sizes.append(min(ps, rest))
                    rest -= ps
                assert t["indptr"][r + 1] - t["indptr"][r] == len(sizes)
                assert t["last_page_len"][r] == sizes[-1]


def test_sparse_csr_rejects_bad_tail_and_page_size():
    for tail in ([0], [129]):
        with pytest.raises(B.PagedDecodeError) as e:
            B.paged_sparse_csr(4, 128, np.array(tail, np.int32), page_size=1)
        assert e.value.name == "PD_E_ARG"
    for ps in (0, 3, 256):
        with pytest.raises(B.PagedDecodeError) as e:
            B.paged_sparse_csr(4, 128, np.array([5], np.int32), page_size=ps)
        assert e.value.name == "PD_E_ARG"
