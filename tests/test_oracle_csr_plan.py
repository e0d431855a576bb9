"""CPU pins for the oracle's page-table builder and plan (no GPU).

The builder enumerates tokens; here it is checked against hand-worked
fixtures and against the closed form of the geometry (a different formula).
The plan scans every chunk size; here it is checked against hand-worked
fixtures and against the properties the plan is defined by.
"""
import json
import os

import numpy as np
import pytest


GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _tables_for_case(case):
    if isinstance(case["block_tables"], str):
        ps, ls, wl = case["page_size"], case["logical_start"][0], case["written_len"][0]
        nblk = -(-wl // ps)
        t = np.full(nblk, -1, np.int32)
        t[ls // ps:] = np.arange(1000, 1000 + nblk - ls // ps)
        return [t]
    return [np.array(t, np.int32) for t in case["block_tables"]]


@pytest.mark.parametrize("case", _load("csr_cases.json")["cases"], ids=lambda c: c["name"])
def test_csr_golden(orc, case):
    tables = _tables_for_case(case)
    csr = orc.csr_from_block_tables(tables, case["logical_start"], case["written_len"],
                                    case["page_size"])
    for key in ("indptr", "indices", "last_page_len", "first_page_offset", "seq_lens",
                "rope_offsets"):
        if key in case:
            assert csr[key].tolist() == case[key], key


def _closed_form(ls, wl, ps):
    """Geometry closed form, independent of token enumeration."""
    if wl == ls:
        return 0, 0, 0
    first_blk, last_blk = ls // ps, (wl - 1) // ps
    return last_blk - first_blk + 1, wl - last_blk * ps, ls - first_blk * ps


def test_csr_random_sweep_identity_and_closed_form(orc):
    rng = np.random.default_rng(7)
    for case in range(600):
        ps = int(rng.choice([1, 2, 3, 4, 7, 16, 32, 64]))
        b = int(rng.integers(1, 6))
        ls, wl, tables = [], [], []
        for _ in range(b):
            w = int(rng.integers(0, 300))
            mode = rng.random()
            s = w if mode < 0.1 else (int(rng.integers(0, w + 1)) if mode < 0.5 else 0)
            if rng.random() < 0.2 and s == 0 and w >= ps:
                w = (w // ps) * ps
            nblk = -(-w // ps)
            t = rng.permutation(10_000)[:nblk].astype(np.int32)
            t[: s // ps] = -1
            ls.append(s)
            wl.append(w)
            tables.append(t)
        csr = orc.csr_from_block_tables(tables, ls, wl, ps)
        ip = csr["indptr"]
        for r in range(b):
            pages = ip[r + 1] - ip[r]
            lpl, fpo, n = csr["last_page_len"][r], csr["first_page_offset"][r], csr["seq_lens"][r]
            assert n == wl[r] - ls[r]
            assert (pages, lpl, fpo) == _closed_form(ls[r], wl[r], ps), (case, r)
            if pages:
                assert (pages - 1) * ps + lpl - fpo == n
                assert 1 <= lpl <= ps and 0 <= fpo < ps
                assert csr["indices"][ip[r]:ip[r + 1]].tolist() == \
                    tables[r][ls[r] // ps:(wl[r] - 1) // ps + 1].tolist()
            assert csr["rope_offsets"][r] == wl[r]


def test_csr_rejects_visible_token_in_released_page(orc):
    with pytest.raises(ValueError):
        orc.csr_from_block_tables([np.array([-1, 3], np.int32)], [10], [20], 16)


def test_csr_long_context_config(orc):
    # the table geometry alone (no pool) is enough here
    ps = 16
    ls = [0, 0, 0, 32768 + 7 - 4096]
    wl = [32768, 32768, 32768, 32768 + 7]
    tables = []
    base = 0
    for s, e in zip(ls, wl):
        nb = -(-e // ps)
        t = np.full(nb, -1, np.int32)
        t[s // ps:] = np.arange(base, base + nb - s // ps)
        base += nb - s // ps
        tables.append(t)
    csr = orc.csr_from_block_tables(tables, ls, wl, ps)
    assert (np.diff(csr["indptr"])).tolist() == [2048, 2048, 2048, 257]
    assert csr["last_page_len"].tolist() == [16, 16, 16, 7]
    assert csr["first_page_offset"].tolist() == [0, 0, 0, 7]
    assert csr["seq_lens"].tolist() == [32768, 32768, 32768, 4096]
    assert csr["indptr"][-1] == 6401


@pytest.mark.parametrize("case", _load("plan_cases.json")["cases"], ids=lambda c: c["name"])
def test_plan_golden(orc, case):
    indptr = np.concatenate([[0], np.cumsum(case["pages"])]).astype(np.int32)
    p = orc.plan(indptr, case["num_kv_heads"], case["target"])
    assert p["pages_per_chunk"] == case["pages_per_chunk"]
    assert p["num_chunks"] == case["num_chunks"]
    for key in ("request_indices", "kv_tile_indices", "o_indptr"):
        if key in case:
            assert p[key].tolist() == case[key], key


def _chunks(pages, c):
    return sum(max(1, -(-p // c)) for p in pages)


def test_plan_defining_properties_random(orc):
    rng = np.random.default_rng(11)
    for _ in range(300):
        b = int(rng.integers(1, 9))
        pages = rng.integers(0, 200, size=b)
        pages[rng.random(b) < 0.15] = 0
        hkv = int(rng.choice([1, 2, 4, 8]))
        target = int(rng.integers(1, 3000))
        indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
        p = orc.plan(indptr, hkv, target)
        c, n = p["pages_per_chunk"], p["num_chunks"]
        cmax = max(1, int(pages.max()))
        assert 1 <= c <= cmax
        assert n == _chunks(pages, c)
        if n * hkv >= target:
            # maximal: the next larger size no longer reaches the target
            assert c == cmax or _chunks(pages, c + 1) * hkv < target
        else:
            # fallback only when even c = 1 does not reach it
            assert c == 1 and _chunks(pages, 1) * hkv < target
        # request-major emission, every request >= 1 chunk, tiles 0..k-1
        oi = p["o_indptr"]
        assert oi[0] == 0 and oi[-1] == n
        for r in range(b):
            k = oi[r + 1] - oi[r]
            assert k == max(1, -(-int(pages[r]) // c))
            assert p["request_indices"][oi[r]:oi[r + 1]].tolist() == [r] * k
            assert p["kv_tile_indices"][oi[r]:oi[r + 1]].tolist() == list(range(k))


def test_plan_fixed_chunk_and_infeasible(orc):
    indptr = np.array([0, 7, 7, 12], np.int32)
    p = orc.plan(indptr, 2, 1, fixed_pages_per_chunk=1)
    assert p["pages_per_chunk"] == 1 and p["num_chunks"] == 7 + 1 + 5
    # more requests than the launch bound admits: no plan at all
    big = np.arange(0, 70000, dtype=np.int32)
    with pytest.raises(ValueError):
        orc.plan(big, 1, 1)
