"""CPU tests of cascade decode's host side: detection of the shared span
(library against hand-worked fixtures and against the brute-force oracle,
bit-exact), the split of the page table into the shared level and the
per-request level, and the merge-input layout for mixed batches."""
import json
import os

import numpy as np
import pytest

from paged_attention_decode_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "cascade_detect_cases.json")))


def _csr(pages):
    indptr = np.cumsum([0] + [len(p) for p in pages]).astype(np.int32)
    idx = np.array([x for p in pages for x in p], np.int32)
    return indptr, idx


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=lambda c: c["name"])
def test_detect_golden(orc, case):
    indptr, idx = _csr(case["pages"])
    for fn in (orc.cascade_detect, B.paged_cascade_detect):
        m, s = fn(indptr, idx, case["fpo"], case["min_shared"], case["min_members"])
        assert [int(x) for x in m] == case["members"], (fn, case["why"])
        assert s == case["shared"], (fn, case["why"])


def _random_batch(rng):
    """Ragged batch with several groups of requests sharing leading pages,
    requests that start mid-page, empty requests and one-page requests."""
    pool = rng.permutation(4000).astype(np.int32)
    pos = 0
    pages, fpo = [], []
    ngroups = int(rng.integers(1, 4))
    for _ in range(ngroups):
        plen = int(rng.integers(1, 40))
        prefix = pool[pos:pos + plen]
        pos += plen
        for _ in range(int(rng.integers(1, 6))):
            keep = int(rng.integers(0, plen + 1)) if rng.random() < 0.3 else plen
            tail = int(rng.integers(0, 12))
            pages.append(np.concatenate([prefix[:keep], pool[pos:pos + tail]]))
            pos += tail
            fpo.append(int(rng.integers(1, 16)) if rng.random() < 0.15 else 0)
    for _ in range(int(rng.integers(0, 4))):
        n = int(rng.integers(0, 6))
        pages.append(pool[pos:pos + n])
        pos += n
        fpo.append(0)
    order = rng.permutation(len(pages))
    pages = [pages[i] for i in order]
    fpo = [fpo[i] if len(pages[k]) else 0 for k, i in enumerate(order)]
    return pages, np.asarray(fpo, np.int32)


def test_detect_matches_oracle_random(orc):
    rng = np.random.Generator(np.random.PCG64(70))
    hits = 0
    for _ in range(600):
        pages, fpo = _random_batch(rng)
        indptr, idx = _csr(pages)
        ms = int(rng.integers(1, 8))
        mm = int(rng.integers(2, 4))
        m0, s0 = orc.cascade_detect(indptr, idx, fpo, ms, mm)
        m1, s1 = B.paged_cascade_detect(indptr, idx, fpo, ms, mm)
        assert np.array_equal(m0, m1) and s0 == s1
        hits += s0 > 0
    assert 100 < hits < 590          # both outcomes are exercised


def _lpl(rng, pages, fpo, ps):
    out = []
    for p, f in zip(pages, fpo):
        if len(p) == 0:
            out.append(0)
        elif len(p) == 1:
            out.append(int(rng.integers(f + 1, ps + 1)))
        else:
            out.append(int(rng.integers(1, ps + 1)))
    return np.asarray(out, np.int32)


def test_split_rebuilds_every_page_list(orc):
    rng = np.random.Generator(np.random.PCG64(71))
    ps = 16
    done = 0
    for _ in range(300):
        pages, fpo = _random_batch(rng)
        indptr, idx = _csr(pages)
        members, span = B.paged_cascade_detect(indptr, idx, fpo, 1, 2)
        if span == 0:
            continue
        lpl = _lpl(rng, pages, fpo, ps)
        idx0, csr1 = B.paged_cascade_split(ps, indptr, idx, lpl, fpo, members, span)
        assert np.array_equal(idx0, pages[members[0]][:span])
        ip1, ix1 = csr1["indptr"], csr1["indices"]
        for r, p in enumerate(pages):
            own = ix1[ip1[r]:ip1[r + 1]]
            if r in members:
                assert np.array_equal(np.concatenate([idx0, own]), p)
                assert csr1["first_page_offset"][r] == 0 and len(own) >= 1
            else:
                assert np.array_equal(own, p)
                assert csr1["first_page_offset"][r] == fpo[r]
            assert csr1["last_page_len"][r] == lpl[r]
        # both levels are valid page tables that satisfy the geometry identity
        B.csr_validate(len(pages), ps, 4000, ip1, ix1, csr1["last_page_len"],
                       csr1["first_page_offset"])
        B.csr_validate(1, ps, 4000, np.array([0, span], np.int32), idx0,
                       np.array([ps], np.int32), np.array([0], np.int32))
        done += 1
    assert done > 50


def test_split_rejects_bad_members():
    pages = [[5, 6, 7, 8], [5, 6, 7, 9], [5, 6], [1, 2, 3]]
    indptr, idx = _csr(pages)
    lpl = np.full(4, 16, np.int32)
    fpo = np.zeros(4, np.int32)
    ok = B.paged_cascade_split(16, indptr, idx, lpl, fpo, [0, 1], 3)
    assert ok[1]["indptr"].tolist() == [0, 1, 2, 4, 7]
    bad = [([1, 0], 3),            # not ascending
           ([0, 1], 4),            # no page after the span
           ([0, 2], 2),            # member 2 holds no page after the span
           ([0, 3], 1)]            # member 3 does not hold the span
    for members, span in bad:
        with pytest.raises(B.PagedDecodeError) as e:
            B.paged_cascade_split(16, indptr, idx, lpl, fpo, members, span)
        assert e.value.name == "PD_E_ARG"
    fpo_bad = np.array([0, 7, 0, 0], np.int32)
    with pytest.raises(B.PagedDecodeError):
        B.paged_cascade_split(16, indptr, idx, lpl, fpo_bad, [0, 1], 3)


def test_layout_groups_level0_rows_before_own_rows():
    rng = np.random.Generator(np.random.PCG64(72))
    for _ in range(200):
        batch = int(rng.integers(1, 9))
        counts = rng.integers(1, 5, size=batch)
        o1 = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        k = int(rng.integers(1, batch + 1))
        members = np.sort(rng.choice(batch, size=k, replace=False)).astype(np.int32)
        n0 = int(rng.integers(1, 6))
        dst0, dst1, oi = B.paged_cascade_layout(members, n0, o1)
        rows = np.full(int(oi[-1]), -1)
        for m, r in enumerate(members):
            assert dst0[m] == oi[r]
            rows[oi[r]:oi[r] + n0] = 0
        for r in range(batch):
            lead = n0 if r in members else 0
            assert oi[r + 1] - oi[r] == lead + counts[r]
            for t in range(counts[r]):
                assert dst1[o1[r] + t] == oi[r] + lead + t
                rows[dst1[o1[r] + t]] = 1
        assert np.all(rows >= 0)       # every merge-input row is written exactly by one source


def test_merge_layout_locates_every_stacked_row():
    """The in-place merge's descriptors against an enumeration of the stacked
    launches' output: launch j stacks members j*per .. of member_req and writes
    [n0, S*Hq] rows after the earlier launches; member position p's head
    kv*G + g is stacked head kv*S*G + p*G + g (the head stacking)."""
    rng = np.random.Generator(np.random.PCG64(73))
    for _ in range(200):
        batch = int(rng.integers(1, 12))
        k = int(rng.integers(1, batch + 1))
        members = np.sort(rng.choice(batch, size=k, replace=False)).astype(np.int32)
        per = int(rng.integers(1, 5))
        n0 = int(rng.integers(1, 6))
        hkv = int(rng.integers(1, 4))
        g = int(rng.integers(1, 5))
        hq = hkv * g
        desc = B.paged_cascade_merge_layout(batch, members, per, n0, hq)
        where = {}
        row = 0
        for j in range(0, k, per):
            launch = members[j:j + per]
            s = launch.size
            for i in range(n0):
                for kv in range(hkv):
                    for p in range(s):
                        for gi in range(g):
                            where[(int(launch[p]), i, kv * g + gi)] = row
                            row += 1
        assert row == n0 * k * hq
        for r in range(batch):
            first, s, p = (int(x) for x in desc[r])
            if r not in members:
                assert (first, s, p) == (0, 0, -1)
                continue
            for i in range(n0):
                for h in range(hq):
                    kv, gi = divmod(h, g)
                    assert first + i * s * hq + kv * s * g + p * g + gi == where[(r, i, h)]


def test_merge_layout_rejects_bad_members():
    with pytest.raises(B.PagedDecodeError) as e:
        B.paged_cascade_merge_layout(4, [2, 1], 2, 3, 8)
    assert e.value.name == "PD_E_ARG"
    with pytest.raises(B.PagedDecodeError):
        B.paged_cascade_merge_layout(4, [0, 4], 2, 3, 8)
    with pytest.raises(B.PagedDecodeError) as e:
        B.paged_cascade_merge_layout(4, [0, 1], 2, 1 << 20, 1 << 12)   # rows past int32
    assert e.value.name == "PD_E_ARG"


@pytest.mark.parametrize("dtype,head_dim,g", [
    (B.PD_DTYPE_FP16, 128, 1), (B.PD_DTYPE_FP16, 128, 2), (B.PD_DTYPE_FP16, 128, 4),
    (B.PD_DTYPE_FP16, 128, 8), (B.PD_DTYPE_FP16, 128, 12), (B.PD_DTYPE_FP16, 128, 16),
    (B.PD_DTYPE_FP16, 64, 2), (B.PD_DTYPE_FP16, 64, 4), (B.PD_DTYPE_FP32, 128, 4),
    (B.PD_DTYPE_FP32, 64, 4), (B.PD_DTYPE_FP32, 64, 8)])
def test_cascade_subgroup_sizes_all_have_a_kernel(dtype, head_dim, g):
    """Every level-0 launch of a cascade step (per members stacked, the last
    launch the rest) has a partial kernel, for 2 to 32 members and page sizes
    1, 8, 16 and 64; and no other launch size needs fewer launches.  Before
    the remainder was checked, 13 members at G = 4 left a 5-member launch
    (stacked G = 20), which no kernel serves."""
    from paged_attention_decode_amd.decode import cascade_members_per_launch
    lib = B.load()
    kv_heads = 8

    def ok(k, ps):
        return lib.paged_decode_kernel_kind(dtype, head_dim, k * g, ps, kv_heads * head_dim) >= 0

    for ps in (1, 8, 16, 64):
        for m in range(2, 33):
            per = cascade_members_per_launch(m, g, head_dim, dtype, ps, kv_heads * head_dim)
            sizes = [min(per, m - i) for i in range(0, m, per)]
            assert sum(sizes) == m
            assert all(ok(s, ps) for s in sizes), (ps, m, per, sizes)
            for other in range(1, m + 1):
                n = -(-m // other)
                if ok(other, ps) and ok(m - (n - 1) * other, ps):
                    assert n >= len(sizes), (ps, m, per, other)
