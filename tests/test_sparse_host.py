"""CPU tests of the block-selection page table's shape (sparse-paged-decode
doc, the two granularities): token-exact tables hold one one-token page per
selected position, block-granular tables one page per block with the final
block's written positions as last_page_len."""
import numpy as np
import pytest

from paged_attention_decode_amd import binding as B


def test_sparse_csr_token_exact_and_block_granular():
    tail = np.array([91, 128, 1], np.int32)
    t = B.paged_sparse_csr(16, 128, tail, token_exact=True)
    counts = np.diff(t["indptr"])
    assert counts.tolist() == [15 * 128 + 91, 16 * 128, 15 * 128 + 1]
    assert np.all(t["last_page_len"] == 1) and np.all(t["first_page_offset"] == 0)
    b = B.paged_sparse_csr(16, 128, tail, token_exact=False)
    assert b["indptr"].tolist() == [0, 16, 32, 48]
    assert b["last_page_len"].tolist() == [91, 128, 1]
    # both tables satisfy the geometry identity with the selected position counts
    for csr, ps in ((t, 1), (b, 128)):
        nnz = int(csr["indptr"][-1])
        B.csr_validate(3, ps, nnz, csr["indptr"], np.arange(nnz, dtype=np.int32),
                       csr["last_page_len"], csr["first_page_offset"],
                       seq_lens=15 * 128 + tail)


def test_sparse_csr_rejects_bad_tail():
    for tail in ([0], [129]):
        with pytest.raises(B.PagedDecodeError) as e:
            B.paged_sparse_csr(4, 128, np.array(tail, np.int32), token_exact=True)
        assert e.value.name == "PD_E_ARG"
