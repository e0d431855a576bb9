"""CPU tests of the HIP library's host side (no GPU): it loads and exports
every symbol of include/paged_decode.h; CSR building and the plan match the
oracle bit-exactly; validation rejects every malformed table; the
fast-divide used for page indirection matches / and %."""
import os
import re

import numpy as np
import pytest

from paged_attention_decode_amd import binding as B
from paged_attention_decode_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_exports_every_declared_symbol(lib):
    text = open(os.path.join(ROOT, "include", "paged_decode.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    names.discard("typedef")
    assert {"csr_validate", "paged_decode_plan", "paged_decode_partial",
            "paged_merge_states"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert set(B.EXPORTED) == names


def test_version(lib):
    assert "gfx950" in B.version()


def _random_tables(rng, b, ps, max_len):
    ls, wl, tables = [], [], []
    for _ in range(b):
        w = int(rng.integers(0, max_len))
        u = rng.random()
        s = w if u < 0.1 else (int(rng.integers(0, w + 1)) if u < 0.5 else 0)
        if rng.random() < 0.2 and s == 0 and w >= ps:
            w = (w // ps) * ps
        nblk = -(-w // ps)
        t = rng.permutation(5000)[:nblk].astype(np.int32)
        t[: s // ps] = -1
        ls.append(s)
        wl.append(w)
        tables.append(t)
    return ls, wl, tables


def test_csr_build_matches_oracle_bit_exact(orc):
    rng = np.random.default_rng(21)
    for _ in range(600):
        ps = int(rng.choice([1, 2, 5, 8, 16, 32, 64]))
        b = int(rng.integers(1, 7))
        ls, wl, tables = _random_tables(rng, b, ps, 400)
        got = B.paged_csr_build(tables, ls, wl, ps, 5000)
        ref = orc.csr_from_block_tables(tables, ls, wl, ps)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), k


def test_csr_build_configs_match_oracle(orc):
    for w in (workloads.tiny_fp32(), workloads.batched_fp16()):
        got = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                                w.k_pool.shape[0])
        ref = orc.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                        w.page_size)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), k


def _good():
    # two requests: 3 pages (fpo 2, lpl 5), 1 page (fpo 1, lpl 3); page size 8
    return dict(indptr=[0, 3, 4], indices=[4, 0, 7, 2], last_page_len=[5, 3],
                first_page_offset=[2, 1], seq_lens=[2 * 8 + 5 - 2, 2])


@pytest.mark.parametrize("mutate,code,bad", [
    (lambda c: c.update(indptr=[1, 3, 4]), "PD_E_INDPTR", -1),
    (lambda c: c.update(indptr=[0, 3, 2]), "PD_E_INDPTR", 1),
    (lambda c: c["indices"].__setitem__(2, 9), "PD_E_INDEX_RANGE", 0),
    (lambda c: c["indices"].__setitem__(3, -1), "PD_E_INDEX_RANGE", 1),
    (lambda c: c["last_page_len"].__setitem__(0, 0), "PD_E_LAST_PAGE_LEN", 0),
    (lambda c: c["last_page_len"].__setitem__(0, 9), "PD_E_LAST_PAGE_LEN", 0),
    (lambda c: c["first_page_offset"].__setitem__(0, 8), "PD_E_FIRST_PAGE_OFFSET", 0),
    (lambda c: c["first_page_offset"].__setitem__(0, -1), "PD_E_FIRST_PAGE_OFFSET", 0),
    (lambda c: c["first_page_offset"].__setitem__(1, 3), "PD_E_FIRST_PAGE_OFFSET", 1),
    (lambda c: c["seq_lens"].__setitem__(1, 3), "PD_E_GEOMETRY", 1),
])
def test_csr_validate_rejections(lib, mutate, code, bad):
    c = {k: list(v) for k, v in _good().items()}
    assert B.csr_validate(2, 8, 8, **c)[0] == 0
    mutate(c)
    rc, where = B.csr_validate(2, 8, 8, raise_on_error=False, **c)
    assert B.ERRORS[rc] == code
    assert where == bad
    with pytest.raises(B.PagedDecodeError) as ei:
        B.csr_validate(2, 8, 8, **c)
    assert ei.value.name == code


def test_csr_validate_empty_request_encoding(lib):
    ok = dict(indptr=[0, 0, 2], indices=[1, 2], last_page_len=[0, 4], first_page_offset=[0, 0],
              seq_lens=[0, 12])
    assert B.csr_validate(2, 8, 8, **ok)[0] == 0
    bad = dict(ok, last_page_len=[1, 4])
    assert B.ERRORS[B.csr_validate(2, 8, 8, raise_on_error=False, **bad)[0]] == "PD_E_LAST_PAGE_LEN"
    bad = dict(ok, first_page_offset=[2, 0])
    assert B.ERRORS[B.csr_validate(2, 8, 8, raise_on_error=False, **bad)[0]] == \
        "PD_E_FIRST_PAGE_OFFSET"


def test_csr_build_rejects(lib):
    with pytest.raises(B.PagedDecodeError) as ei:
        B.paged_csr_build([np.array([-1, 3], np.int32)], [10], [20], 16, 8)
    assert ei.value.name == "PD_E_INDEX_RANGE"
    with pytest.raises(B.PagedDecodeError) as ei:
        B.paged_csr_build([np.array([0, 3], np.int32)], [0], [20], 8, 8)   # 3 blocks needed
    assert ei.value.name == "PD_E_ARG"
    with pytest.raises(B.PagedDecodeError) as ei:
        B.paged_csr_build([np.array([0, 9], np.int32)], [0], [10], 8, 8)   # page 9 not in pool
    assert ei.value.name == "PD_E_INDEX_RANGE"


def _plan_equal(orc, indptr, hkv, target, fixed=0, hq=None):
    hq = hq or hkv * 4
    info, ri, ti, oi = B.paged_decode_plan(indptr, hq, hkv, 128, target, fixed)
    ref = orc.plan(indptr, hkv, target, fixed_pages_per_chunk=fixed)
    assert info.pages_per_chunk == ref["pages_per_chunk"]
    assert info.num_chunks == ref["num_chunks"]
    assert np.array_equal(ri, ref["request_indices"])
    assert np.array_equal(ti, ref["kv_tile_indices"])
    assert np.array_equal(oi, ref["o_indptr"])
    assert info.num_wgs == info.num_chunks * hkv and info.q_groups == 1
    assert info.needs_merge == int(info.num_chunks != len(indptr) - 1)
    assert info.workspace_bytes == info.num_chunks * hq * (128 + 1) * 4
    return info


def test_plan_matches_oracle_random(orc):
    rng = np.random.default_rng(31)
    for _ in range(400):
        b = int(rng.integers(1, 10))
        pages = rng.integers(0, 400, size=b)
        pages[rng.random(b) < 0.15] = 0
        indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
        hkv = int(rng.choice([1, 2, 4, 8]))
        target = int(rng.integers(1, 5000))
        _plan_equal(orc, indptr, hkv, target)
        if rng.random() < 0.3:
            _plan_equal(orc, indptr, hkv, target, fixed=int(rng.integers(1, 50)))


def test_plan_long_context_targets(orc):
    indptr = np.array([0, 2048, 4096, 6144, 6401], np.int32)
    for t, (c, n) in {256: (227, 32), 512: (102, 66), 1024: (51, 129), 2048: (25, 257),
                      4096: (12, 535)}.items():
        info = _plan_equal(orc, indptr, 8, t)
        assert (info.pages_per_chunk, info.num_chunks) == (c, n)


def test_plan_launch_floor_and_infeasible(orc):
    info = _plan_equal(orc, np.array([0, 100000], np.int32), 1, 10 ** 9)
    assert info.pages_per_chunk == 2 and info.num_chunks == 50000
    big = np.arange(0, 70000, dtype=np.int32)
    with pytest.raises(B.PagedDecodeError) as ei:
        B.paged_decode_plan(big, 4, 1, 128, 1)
    assert ei.value.name == "PD_E_INFEASIBLE"
    with pytest.raises(B.PagedDecodeError) as ei:
        B.paged_decode_plan(np.array([0, 100000], np.int32), 4, 1, 128, 1, 1)
    assert ei.value.name == "PD_E_INFEASIBLE"


def test_plan_single_chunk_needs_no_merge(orc):
    indptr = np.array([0, 3, 5, 5], np.int32)
    info = _plan_equal(orc, indptr, 2, 1)
    assert info.needs_merge == 0 and info.num_chunks == 3


def test_q_heads_per_wg_and_unsupported(lib):
    for g in (1, 2, 4, 8, 12, 16):
        for d in (64, 128):
            for dt in (0, 1):
                assert B.paged_decode_q_heads_per_wg(g, d, dt) == g
    # 24 and 32 heads per KV head run on the MFMA kernel only: fp16, D = 128
    for g in (24, 32):
        assert B.paged_decode_q_heads_per_wg(g, 128, 0) == g
    for g, d, dt in ((3, 128, 0), (4, 96, 0), (32, 128, 1), (32, 64, 0), (24, 128, 1), (20, 128, 0),
                     (64, 128, 0)):
        with pytest.raises(B.PagedDecodeError) as ei:
            B.paged_decode_q_heads_per_wg(g, d, dt)
        assert ei.value.name == "PD_E_UNSUPPORTED"


@pytest.mark.parametrize("d", list(range(1, 257)))
def test_fastdiv_exhaustive_small(lib, d):
    n = np.arange(0, 1 << 16, dtype=np.uint32)
    q, r = B.paged_fastdiv_eval(d, n)
    assert np.array_equal(q, n // d) and np.array_equal(r, n % d)


def test_fastdiv_wide_and_random(lib):
    rng = np.random.default_rng(0)
    n = np.concatenate([np.arange(0, 1 << 20, dtype=np.uint32),
                        rng.integers(0, 1 << 31, size=1 << 20, dtype=np.uint32),
                        np.array([(1 << 31) - 1, (1 << 31) - 2], np.uint32)])
    for d in [1, 2, 3, 7, 16, 17, 64, 100, 128, 255, 256, 1000, 4096, 65537, (1 << 30) + 3]:
        q, r = B.paged_fastdiv_eval(d, n)
        assert np.array_equal(q, n // d) and np.array_equal(r, n % d), d


def test_plan_paged_mla_q_groups(orc):
    """head_dim 512 plans the paged-MLA kernel: (chunk, q group) units of 64
    query heads; the chunk list itself is the ordinary plan's."""
    indptr = np.array([0, 512, 1024, 1536, 2048], np.int32)
    for hq, qg in ((128, 2), (64, 1), (32, 1), (16, 1)):
        info, ri, ti, oi = B.paged_decode_plan(indptr, hq, 1, 512, 256, 0, page_size=64)
        ref = orc.plan(indptr, qg, 256)
        assert info.q_groups == qg and info.num_wgs == info.num_chunks * qg
        assert info.pages_per_chunk == ref["pages_per_chunk"]
        assert np.array_equal(ri, ref["request_indices"]) and np.array_equal(oi, ref["o_indptr"])
        assert info.workspace_bytes == info.num_chunks * hq * 513 * 4
    with pytest.raises(B.PagedDecodeError) as ei:
        B.paged_decode_plan(indptr, 128, 2, 512, 256, 0)
    assert ei.value.name == "PD_E_UNSUPPORTED"
    with pytest.raises(B.PagedDecodeError) as ei:
        B.paged_decode_plan(indptr, 48, 1, 512, 256, 0)
    assert ei.value.name == "PD_E_UNSUPPORTED"
    assert B.paged_decode_q_heads_per_wg(128, 512, B.PD_DTYPE_FP16) == 64
    assert B.paged_decode_q_heads_per_wg(32, 512, B.PD_DTYPE_FP16) == 32


def test_mla_partial_argument_errors_before_launch():
    """Argument checks of paged_mla_decode_partial return before any launch
    (no device needed)."""
    lib = B.load()
    one = 16  # any non-null, 16-byte aligned address: nothing is dereferenced
    args = [one] * 4 + [640 * 64, 640, 64 * 64, 64, 512, 64, B.PD_DTYPE_FP16] + [one] * 6 + \
        [1, 1, 1, 128, 64, 0.04, one, one, None]
    assert lib.paged_mla_decode_partial(*([None] + args[1:])) == B.CODES["PD_E_NULL"]
    bad_dim = list(args)
    bad_dim[8] = 256
    assert lib.paged_mla_decode_partial(*bad_dim) == B.CODES["PD_E_UNSUPPORTED"]
    bad_heads = list(args)
    bad_heads[20] = 48
    assert lib.paged_mla_decode_partial(*bad_heads) == B.CODES["PD_E_UNSUPPORTED"]
    bad_stride = list(args)
    bad_stride[5] = 641                  # a row start off a 16-byte boundary
    assert lib.paged_mla_decode_partial(*bad_stride) == B.CODES["PD_E_UNSUPPORTED"]
    fp32 = list(args)
    fp32[10] = B.PD_DTYPE_FP32
    assert lib.paged_mla_decode_partial(*fp32) == B.CODES["PD_E_UNSUPPORTED"]


def test_kernel_wrappers_refuse_host_tensors():
    """The binding refuses a CPU tensor where a kernel takes a device pointer,
    before any call into the library."""
    torch = pytest.importorskip("torch")
    v = torch.zeros(2, 1, 4)
    lse = torch.zeros(2, 1)
    oi = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensors"):
        B.paged_merge_states(v, lse, oi, 1, 1, 4, v[:1], lse[:1], stream=0)


def test_fused_noalloc_refuses_before_touching_the_device(lib):
    """Size errors of the no-allocation entry point come back before any
    device call: a workspace larger than the library's 16 MiB array is
    PD_E_CAPACITY, bad sizes PD_E_ARG."""
    f = lib.paged_decode_fused_noalloc
    args = [None] * 3 + [0, 0, 0, 0] + [None] * 6
    tail = [None, None, None]
    # 4096 chunks x 32 heads x 128 dims x 4 B = 64 MiB of partial rows
    rc = f(*args, 4096, 1, 4, 32, 8, 128, 16, 0.1, *tail)
    assert rc == -8 and b"scratch" in lib.pd_last_error()
    rc = f(*args, 4096, 1, 0, 32, 8, 128, 16, 0.1, *tail)
    assert rc == -2


def test_cascade_partial_argument_errors_before_launch():
    """paged_cascade_partial refuses bad arguments before any launch (no
    device needed: every case below fails a host-side check)."""
    import ctypes
    lib = B.load()
    one = 16  # any non-null, 16-byte aligned address: nothing is dereferenced

    def level(batch, chunks, v=one):
        return B.CascadeLevel(one, one, one, one, one, one, batch, chunks, 2, v, one)

    def call(q=one, batch=4, members=4, per=4, dtype=B.PD_DTYPE_FP16, d=128, hpw=0,
             l0=None, l1=None):
        l0 = B.cascade_levels([level(1, 4)]) if l0 is None else l0
        l1 = level(batch, 8) if l1 is None else l1
        return lib.paged_cascade_partial(q, batch, one, members, per, one, one, 16 * 8 * d,
                                         8 * d, d, dtype, 32, 8, d, 16, 0.088, l0,
                                         ctypes.byref(l1), hpw, None)

    assert call(q=None) == B.CODES["PD_E_NULL"]
    assert call(members=5) == B.CODES["PD_E_ARG"]                 # more members than requests
    assert call(hpw=3) == B.CODES["PD_E_ARG"]
    assert call(l1=level(3, 8)) == B.CODES["PD_E_ARG"]            # level 1 misses a request
    assert call(l0=B.cascade_levels([level(1, 4, v=None)])) == B.CODES["PD_E_NULL"]
    assert call(l0=B.cascade_levels([level(1, -1)])) == B.CODES["PD_E_ARG"]
    assert call(dtype=7) == B.CODES["PD_E_UNSUPPORTED"]
    assert call(d=96) == B.CODES["PD_E_UNSUPPORTED"]              # no kernel for this head dim
    # with 2 members per table the call reads two level-0 tables: the second
    # one is checked too
    two = B.cascade_levels([level(1, 4), level(1, 4, v=None)])
    assert call(per=2, l0=two) == B.CODES["PD_E_NULL"]


def test_read_probe_argument_errors_before_launch():
    lib = B.load()
    assert lib.paged_hbm_read_probe(None, 1024, 4, 1, 16, None) == B.CODES["PD_E_NULL"]
    assert lib.paged_hbm_read_probe(16, 1000, 4, 1, 16, None) == B.CODES["PD_E_ARG"]
    assert lib.paged_hbm_read_probe(16, 1024, 0, 1, 16, None) == B.CODES["PD_E_ARG"]
    assert lib.paged_hbm_read_probe(8, 1024, 4, 1, 16, None) == B.CODES["PD_E_UNSUPPORTED"]


def test_decode_objects_refuse_mis_shaped_step_inputs():
    """The decode objects check q and the pools against the shapes they were
    planned for before any launch: the C-ABI sees only addresses, so a
    mis-shaped or mistyped tensor would be read out of bounds.  Built on the
    host (device='cpu'); every call below raises before the binding's
    device-pointer check would."""
    torch = pytest.importorskip("torch")
    from paged_attention_decode_amd import decode as PD

    w = workloads.generic("shape_checks", seed=5, dtype=workloads.FP16, page_size=8,
                          num_qo_heads=8, num_kv_heads=2, head_dim=64,
                          logical_start=[0, 3], written_len=[40, 29])
    pages = w.k_pool.shape[0]
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, 8, pages)
    dec = PD.PagedDecode(csr, page_size=8, num_pool_pages=pages, num_qo_heads=8,
                         num_kv_heads=2, head_dim=64, target_wgs=8, device="cpu")
    q = torch.from_numpy(w.q)
    k, v = torch.from_numpy(w.k_pool), torch.from_numpy(w.v_pool)
    dec.check_step(q, k, v)                                   # the planned shapes pass
    bad = [
        ((q[:1], k, v), ValueError),                          # batch
        ((q[:, :4], k, v), ValueError),                       # heads
        ((q.transpose(0, 1).contiguous().transpose(0, 1), k, v), ValueError),   # not contiguous
        ((q.float(), k, v), TypeError),                       # dtype against the pools
        ((q, k[: pages - 1], v[: pages - 1]), ValueError),    # fewer pages than the table names
        ((q, k[:, :4], v[:, :4]), ValueError),                # page size
        ((q, k[:, :, :1], v[:, :, :1]), ValueError),          # KV heads
        ((q, k[..., :32], v[..., :32]), ValueError),          # head dim
    ]
    for call in (dec.partial, dec.fused_step, dec.run):
        for args, err in bad:
            with pytest.raises(err):
                call(*args, w.sm_scale)

    m = workloads.mla_paged("shape_checks_mla", seed=6, logical_start=[0], written_len=[70],
                            num_qo_heads=16)
    mcsr = B.paged_csr_build(m.block_tables, m.logical_start, m.written_len, m.page_size,
                             m.k_pool.shape[0])
    mdec = PD.MlaDecode(mcsr, page_size=m.page_size, num_pool_pages=m.k_pool.shape[0],
                        num_qo_heads=16, target_wgs=8, device="cpu")
    mq, mqx = torch.from_numpy(m.q), torch.from_numpy(m.q_extra)
    mk, mkx = torch.from_numpy(m.k_pool), torch.from_numpy(m.k_extra_pool)
    mdec.check_step(mq, mqx, mk, mkx)
    for args, err in [((mq[:, :8], mqx, mk, mkx), ValueError),
                      ((mq, mqx[..., :32], mk, mkx), ValueError),
                      ((mq.float(), mqx, mk, mkx), TypeError),
                      ((mq, mqx, mk[..., :256], mkx), ValueError),
                      ((mq, mqx, mk, mkx[:1]), ValueError)]:
        for call in (mdec.partial, mdec.run):
            with pytest.raises(err):
                call(*args, m.sm_scale)
