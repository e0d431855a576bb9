"""f64 CPU oracle for fused paged-attention decode v2 -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It is the plain, slow, obviously
correct definition that the HIP library is checked against, and it shares no
code with that library (its arithmetic lives in ``oracle.c``, compiled with
plain gcc; this file only marshals numpy arrays).

Functions and the passages of the mlxcel pages they follow:

- ``csr_from_block_tables``: PR #984 commit "cache::paged_csr" (CSR view with
  first_page_offset, retired pages dropped, exactly-full last page) -- built
  by enumerating every visible token.
- ``attention``: naive two-pass softmax over each request's visible tokens,
  gathered one by one through the page table (sparse-paged-decode doc,
  "Indirection"); query head h reads KV head h // (Hq/Hkv) (same doc, the
  ContiguousCacheLayout query reshape).  LSE reported in log2 units (PR #984
  body, item 2).
- ``partial``: the same attention restricted to one chunk's pages (PR #984
  body, items 2 and 4).
- ``merge``: the variable-length merge of normalized states (issue #898 item
  3; cascade-attention doc "Softmax states compose"; PR #984 body item 3 for
  -inf rows and all-empty groups).
- ``plan``: exhaustive scan over pages-per-chunk (PR #984 body item 4, the
  commit "plan + launch": largest chunk size whose workgroup count reaches the
  target, 65535-chunk launch bound, >= 1 chunk per request, request order).
- ``attention_mla``: decode with a second key stream (sparse-paged-decode
  doc, DSA section): score = scale*(q . k[0:Dim]) + scale*(q_extra .
  k_extra) over rows gathered one by one through the page table, one KV
  head, the latent rows k[0:Dim] as values; whole requests or chunk ranges.
- ``block_positions``: the positions a selection of KV blocks covers
  (sparse-paged-decode doc, selection from blocks).
- ``cascade_detect``: brute-force search for the shared page span that
  cascade decode attends once (cascade-attention doc, detection section:
  positional comparison of page ids, groups by first page, span capped one
  page short of every member's last page, requests starting mid-page left
  out, minimum span and member count, largest span * (members - 1) wins).

Every function is pinned by CPU tests in ``tests/test_oracle_*.py`` against
closed forms, library special cases and hand-worked fixtures.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB names another build of oracle.c (the sanitizer test's)
_LIB = os.environ.get("ORACLE_LIB", os.path.join(_HERE, "liboracle.so"))
_lib = None

MAX_CHUNKS = 65535

i32p = ctypes.POINTER(ctypes.c_int32)
f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (next to the source)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.orc_half_to_double.restype = ctypes.c_double
        lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
        _lib = lib
    return _lib


def _p(a, t=i32p):
    return a.ctypes.data_as(t)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def half_to_double(bits: int) -> float:
    return _load().orc_half_to_double(ctypes.c_uint16(bits))


def csr_from_block_tables(block_tables: Sequence[np.ndarray], logical_start, written_len,
                          page_size: int):
    """Returns dict(indptr, indices, last_page_len, first_page_offset,
    seq_lens, rope_offsets), all int32."""
    lib = _load()
    b = len(block_tables)
    off = np.zeros(b + 1, np.int32)
    for r, t in enumerate(block_tables):
        off[r + 1] = off[r] + len(t)
    bt = _i32(np.concatenate([np.asarray(t, np.int32) for t in block_tables])
              if b and off[-1] else np.zeros(1, np.int32))
    ls, wl = _i32(logical_start), _i32(written_len)
    cap = max(1, int(off[-1]))
    indptr = np.zeros(b + 1, np.int32)
    indices = np.zeros(cap, np.int32)
    lpl, fpo, sl, ro = (np.zeros(b, np.int32) for _ in range(4))
    rc = lib.orc_csr_from_block_tables(ctypes.c_int32(b), ctypes.c_int32(page_size),
                                       _p(off), _p(bt), _p(ls), _p(wl), ctypes.c_int32(cap),
                                       _p(indptr), _p(indices), _p(lpl), _p(fpo), _p(sl),
                                       _p(ro))
    if rc != 0:
        raise ValueError("oracle: invalid block tables (rc=%d)" % rc)
    return dict(indptr=indptr, indices=indices[:indptr[-1]].copy(), last_page_len=lpl,
                first_page_offset=fpo, seq_lens=sl, rope_offsets=ro)


def _dtype_code(arr):
    if arr.dtype == np.float16:
        return 0
    if arr.dtype == np.float32:
        return 1
    raise TypeError("oracle takes fp16 or fp32 inputs")


def _pool_strides(pool):
    # element strides of a [pages, page_size, heads, D] array, D contiguous
    if pool.strides[-1] != pool.itemsize:
        raise ValueError("head dim must be contiguous")
    return tuple(s // pool.itemsize for s in pool.strides[:3])


def attention(q, k_pool, v_pool, csr, page_size: int, sm_scale: float,
              nthreads: int = 1):
    """q [B, Hq, D]; pools [pages, page_size, Hkv, D] (fp16 or fp32, same
    dtype as q).  Returns (out [B, Hq, D] f64, lse2 [B, Hq] f64)."""
    lib = _load()
    q = np.ascontiguousarray(q)
    assert k_pool.dtype == q.dtype == v_pool.dtype and k_pool.shape == v_pool.shape
    assert _pool_strides(k_pool) == _pool_strides(v_pool)
    b, hq, d = q.shape
    hkv = k_pool.shape[2]
    ps_, ts_, hs_ = _pool_strides(k_pool)
    out = np.zeros((b, hq, d), np.float64)
    lse = np.zeros((b, hq), np.float64)
    indptr, indices = _i32(csr["indptr"]), _i32(csr["indices"])
    if indices.size == 0:
        indices = np.zeros(1, np.int32)
    lpl, fpo = _i32(csr["last_page_len"]), _i32(csr["first_page_offset"])
    rc = lib.orc_attention(ctypes.c_int32(b), ctypes.c_int32(hq), ctypes.c_int32(hkv),
                           ctypes.c_int32(d), ctypes.c_int32(page_size),
                           ctypes.c_int32(_dtype_code(q)), _p(indptr), _p(indices),
                           _p(lpl), _p(fpo), ctypes.c_void_p(q.ctypes.data),
                           ctypes.c_void_p(k_pool.ctypes.data), ctypes.c_void_p(v_pool.ctypes.data),
                           ctypes.c_int64(ps_), ctypes.c_int64(ts_), ctypes.c_int64(hs_),
                           ctypes.c_double(sm_scale), _p(out, f64p), _p(lse, f64p),
                           ctypes.c_int32(nthreads))
    if rc != 0:
        raise ValueError("oracle attention failed (rc=%d)" % rc)
    return out, lse


def partial(q, k_pool, v_pool, csr, page_size: int, sm_scale: float,
            request_indices, kv_tile_indices, pages_per_chunk: int, nthreads: int = 1):
    """Per-chunk attention.  Returns (v [N, Hq, D] f64, lse2 [N, Hq] f64)."""
    lib = _load()
    q = np.ascontiguousarray(q)
    b, hq, d = q.shape
    hkv = k_pool.shape[2]
    ps_, ts_, hs_ = _pool_strides(k_pool)
    ri, ti = _i32(request_indices), _i32(kv_tile_indices)
    n = ri.size
    out = np.zeros((n, hq, d), np.float64)
    lse = np.zeros((n, hq), np.float64)
    indptr, indices = _i32(csr["indptr"]), _i32(csr["indices"])
    if indices.size == 0:
        indices = np.zeros(1, np.int32)
    lpl, fpo = _i32(csr["last_page_len"]), _i32(csr["first_page_offset"])
    rc = lib.orc_partial(ctypes.c_int32(n), _p(ri), _p(ti), ctypes.c_int32(pages_per_chunk),
                         ctypes.c_int32(hq), ctypes.c_int32(hkv), ctypes.c_int32(d),
                         ctypes.c_int32(page_size), ctypes.c_int32(_dtype_code(q)),
                         _p(indptr), _p(indices), _p(lpl), _p(fpo), ctypes.c_void_p(q.ctypes.data),
                         ctypes.c_void_p(k_pool.ctypes.data), ctypes.c_void_p(v_pool.ctypes.data),
                         ctypes.c_int64(ps_), ctypes.c_int64(ts_), ctypes.c_int64(hs_),
                         ctypes.c_double(sm_scale), _p(out, f64p), _p(lse, f64p),
                         ctypes.c_int32(nthreads))
    if rc != 0:
        raise ValueError("oracle partial failed (rc=%d)" % rc)
    return out, lse


def merge(v_in, lse_in, o_indptr):
    """v_in [N, H, D], lse_in [N, H] (log2 units), o_indptr [M+1].  Returns
    (v_out [M, H, D] f64, lse_out [M, H] f64)."""
    lib = _load()
    v_in = np.ascontiguousarray(v_in, dtype=np.float64)
    lse_in = np.ascontiguousarray(lse_in, dtype=np.float64)
    oi = _i32(o_indptr)
    m = oi.size - 1
    _, h, d = v_in.shape if v_in.ndim == 3 else (0, lse_in.shape[1], 1)
    out = np.zeros((m, h, d), np.float64)
    lse = np.zeros((m, h), np.float64)
    if v_in.size == 0:
        v_in = np.zeros((1, h, d), np.float64)
        lse_in = np.zeros((1, h), np.float64)
    rc = lib.orc_merge(ctypes.c_int32(m), ctypes.c_int32(h), ctypes.c_int32(d),
                       _p(v_in, f64p), _p(lse_in, f64p), _p(oi), _p(out, f64p),
                       _p(lse, f64p))
    if rc != 0:
        raise ValueError("oracle merge failed (rc=%d)" % rc)
    return out, lse


def plan(indptr, num_kv_heads: int, target: int, q_groups: int = 1,
         fixed_pages_per_chunk: int = 0, max_chunks: int = MAX_CHUNKS):
    """Returns dict(pages_per_chunk, num_chunks, request_indices,
    kv_tile_indices, o_indptr) or raises ValueError when no plan exists."""
    lib = _load()
    indptr = _i32(indptr)
    b = indptr.size - 1
    cap = int(sum(max(1, int(indptr[r + 1] - indptr[r])) for r in range(b)))
    ri = np.zeros(max(1, cap), np.int32)
    ti = np.zeros(max(1, cap), np.int32)
    oi = np.zeros(b + 1, np.int32)
    c = ctypes.c_int32(0)
    n = ctypes.c_int32(0)
    rc = lib.orc_plan(ctypes.c_int32(b), _p(indptr), ctypes.c_int64(num_kv_heads * q_groups),
                      ctypes.c_int64(target), ctypes.c_int32(fixed_pages_per_chunk),
                      ctypes.c_int64(max_chunks), ctypes.byref(c), ctypes.byref(n),
                      _p(ri), _p(ti), _p(oi), ctypes.c_int32(max(1, cap)))
    if rc != 0:
        raise ValueError("oracle: no plan (rc=%d)" % rc)
    return dict(pages_per_chunk=c.value, num_chunks=n.value,
                request_indices=ri[:n.value].copy(), kv_tile_indices=ti[:n.value].copy(),
                o_indptr=oi)


def cascade_detect(indptr, indices, first_page_offset, min_shared_pages=16, min_members=2):
    """Brute-force cascade detection: returns (members int32 array in request
    order, shared_pages); empty and 0 when nothing qualifies."""
    lib = _load()
    indptr = _i32(indptr)
    b = indptr.size - 1
    idx = _i32(indices) if np.asarray(indices).size else np.zeros(1, np.int32)
    fpo = _i32(first_page_offset)
    out = np.zeros(max(1, b), np.int32)
    nm = ctypes.c_int32(0)
    sp = ctypes.c_int32(0)
    rc = lib.orc_cascade_detect(ctypes.c_int32(b), _p(indptr), _p(idx), _p(fpo),
                                ctypes.c_int32(min_shared_pages), ctypes.c_int32(min_members),
                                _p(out), ctypes.byref(nm), ctypes.byref(sp))
    if rc != 0:
        raise ValueError("oracle cascade detection failed (rc=%d)" % rc)
    return out[:nm.value].copy(), sp.value


def block_positions(block_ids, block_size: int, kv_len: int):
    """Positions a list of selected blocks covers: block j holds positions
    [j*C, (j+1)*C), and nothing at or past the live length kv_len
    (sparse-paged-decode doc, selection from blocks)."""
    out = []
    for j in np.asarray(block_ids, np.int64):
        lo = int(j) * block_size
        out.extend(range(lo, min(lo + block_size, int(kv_len))))
    return np.asarray(out, np.int64)


def attention_dense_f64(q_rows, k_rows, v_rows, sm_scale):
    """Dense attention of one query over gathered rows, for tiny cross-checks
    (numpy, f64): returns (out [D], lse2)."""
    q = np.asarray(q_rows, np.float64)
    k = np.asarray(k_rows, np.float64)
    v = np.asarray(v_rows, np.float64)
    if k.shape[0] == 0:
        return np.zeros(q.shape[-1]), -np.inf
    s = sm_scale * (k @ q)
    m = s.max()
    w = np.exp(s - m)
    z = w.sum()
    return (w[:, None] * v).sum(0) / z, (m + np.log(z)) / np.log(2.0)


def _row_strides(pool):
    # element strides (page, entry) of a [pages, page_size, row] fp16 array
    if pool.ndim != 3 or pool.strides[-1] != pool.itemsize:
        raise ValueError("pool must be [pages, page_size, row] with contiguous rows")
    return pool.strides[0] // pool.itemsize, pool.strides[1] // pool.itemsize


def attention_mla(q, q_extra, k_pool, k_extra_pool, csr, page_size: int, sm_scale: float,
                  chunks=None, nthreads: int = 1):
    """q [B, Hq, Dim] and q_extra [B, Hq, E] fp16; k_pool [pages, page_size,
    RowStride >= Dim] and k_extra_pool [pages, page_size, >= E] fp16.
    chunks = (request_indices, kv_tile_indices, pages_per_chunk) selects
    chunk mode.  Returns (out [rows, Hq, Dim] f64, lse2 [rows, Hq] f64)."""
    lib = _load()
    q = np.ascontiguousarray(q)
    qx = np.ascontiguousarray(q_extra)
    for a in (q, qx, k_pool, k_extra_pool):
        if a.dtype != np.float16:
            raise TypeError("attention_mla takes fp16 arrays")
    b, hq, dim = q.shape
    ex = qx.shape[2]
    if k_pool.shape[2] < dim or k_extra_pool.shape[2] < ex:
        raise ValueError("pool rows narrower than the query")
    kps, kts = _row_strides(k_pool)
    xps, xts = _row_strides(k_extra_pool)
    indptr, indices = _i32(csr["indptr"]), _i32(csr["indices"])
    if indices.size == 0:
        indices = np.zeros(1, np.int32)
    lpl, fpo = _i32(csr["last_page_len"]), _i32(csr["first_page_offset"])
    if chunks is None:
        rows, ri, ti, c = b, None, None, 0
    else:
        ri, ti = _i32(chunks[0]), _i32(chunks[1])
        rows, c = ri.size, int(chunks[2])
    out = np.zeros((rows, hq, dim), np.float64)
    lse = np.zeros((rows, hq), np.float64)
    u16 = ctypes.POINTER(ctypes.c_uint16)
    rc = lib.orc_attention_mla(
        ctypes.c_int32(rows), ctypes.c_int32(hq), ctypes.c_int32(dim), ctypes.c_int32(ex),
        ctypes.c_int32(page_size), _p(indptr), _p(indices), _p(lpl), _p(fpo),
        q.ctypes.data_as(u16), qx.ctypes.data_as(u16), ctypes.c_void_p(k_pool.ctypes.data),
        ctypes.c_void_p(k_extra_pool.ctypes.data), ctypes.c_int64(kps), ctypes.c_int64(kts),
        ctypes.c_int64(xps), ctypes.c_int64(xts), ctypes.c_double(sm_scale),
        _p(ri) if ri is not None else None, _p(ti) if ti is not None else None,
        ctypes.c_int32(c), _p(out, f64p), _p(lse, f64p), ctypes.c_int32(nthreads))
    if rc != 0:
        raise ValueError("oracle attention_mla failed (rc=%d)" % rc)
    return out, lse
