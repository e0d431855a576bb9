"""Seeded synthetic workloads for paged-attention decode.

This module only draws random numbers and lays them out: query vectors, K/V page
pools, and per-request block tables with a logical start and a written length.
It computes nothing the decode method computes (no page-table compression, no
chunk plan, no attention).  Both the HIP path and the f64 oracle consume what it
produces, each building its own page table from the block tables.

Block-table convention: ``block_tables[r][b]`` is the physical pool page that
holds logical tokens ``[b*page_size, (b+1)*page_size)`` of request ``r``; a page
that was released after a front trim holds ``-1``.  Tokens
``[logical_start[r], written_len[r])`` are visible.

The five workloads follow the decode-v2 correctness and performance configs of
the mlxcel pages (PR #984 "fused paged-attention decode v2" correctness
harness: pages assigned out of a pool with 2x slack, partial last pages,
windows that start mid-page; sparse-paged-decode doc "ContiguousCacheLayout";
cascade-attention doc "head stacking").
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

FP16 = "fp16"
FP32 = "fp32"


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                      # "fp16" or "fp32": q, K and V share it
    page_size: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    sm_scale: float                 # natural-units softmax scale
    q: np.ndarray                   # [B, Hq, D]
    k_pool: np.ndarray              # [num_pages, page_size, Hkv, D]
    v_pool: np.ndarray              # same shape as k_pool
    block_tables: List[np.ndarray]  # per request, int32, -1 = released page
    logical_start: np.ndarray       # [B] int32
    written_len: np.ndarray         # [B] int32
    target_wgs: Optional[int] = None
    extra: dict = dataclasses.field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def visible_tokens(self) -> np.ndarray:
        return (self.written_len - self.logical_start).astype(np.int64)

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode step reads: every visible token's
        row once per KV head, for both K and V."""
        esz = 2 if self.dtype == FP16 else 4
        return int(self.visible_tokens.sum()) * self.num_kv_heads * self.head_dim * 2 * esz


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == FP16:
        return x.astype(np.float16)   # IEEE round-to-nearest-even
    return x


def _pool(rng, num_pages, page_size, hkv, d, dtype, poison_unused, used_pages):
    k = _normal(rng, (num_pages, page_size, hkv, d), dtype)
    v = _normal(rng, (num_pages, page_size, hkv, d), dtype)
    if poison_unused:
        unused = np.ones(num_pages, dtype=bool)
        unused[np.asarray(used_pages, dtype=np.int64)] = False
        k[unused] = np.nan
        v[unused] = np.nan
    return k, v


def poison_invisible(w: "Workload") -> "Workload":
    """Set every pool entry that is not a visible token of some request to
    NaN: unused pages, entries before a window's first token in its first
    page, entries past the last written token in a last page.  A decode that
    reads any of them (outside the masked slots) produces NaN."""
    ps = w.page_size
    visible = np.zeros(w.k_pool.shape[:2], dtype=bool)
    for t, s, e in zip(w.block_tables, w.logical_start, w.written_len):
        pos = np.arange(int(s), int(e))
        if pos.size:
            visible[t[pos // ps], pos % ps] = True
    w.k_pool[~visible] = np.nan
    w.v_pool[~visible] = np.nan
    return w


def _tables_from_lengths(rng, lengths_start_end, page_size, pool_pages):
    """Draw distinct physical pages for every logical block a request still
    holds (blocks wholly before the logical start are released = -1)."""
    need = []
    for ls, wl in lengths_start_end:
        nblk = -(-wl // page_size) if wl > 0 else 0
        first_live = ls // page_size
        need.append((nblk, first_live))
    total = sum(max(0, nb - fl) for nb, fl in need)
    if total > pool_pages:
        raise ValueError("pool too small")
    perm = rng.permutation(pool_pages).astype(np.int32)
    tables, used, pos = [], [], 0
    for nb, fl in need:
        t = np.full(nb, -1, dtype=np.int32)
        live = max(0, nb - fl)
        t[fl:nb] = perm[pos:pos + live]
        used.extend(perm[pos:pos + live].tolist())
        pos += live
        tables.append(t)
    return tables, used


def generic(name, *, seed, dtype, page_size, num_qo_heads, num_kv_heads, head_dim,
            logical_start, written_len, pool_slack=2.0, pool_pages=None,
            poison_unused=False, reverse_pages=False, sm_scale=None, target_wgs=None):
    """Any geometry: per-request (logical_start, written_len)."""
    rng = _rng(seed)
    ls = np.asarray(logical_start, dtype=np.int32)
    wl = np.asarray(written_len, dtype=np.int32)
    nlive = sum(max(0, (-(-int(w) // page_size) if w > 0 else 0) - int(s) // page_size)
                for s, w in zip(ls, wl))
    if pool_pages is None:
        pool_pages = max(1, int(np.ceil(pool_slack * max(1, nlive))))
    tables, used = _tables_from_lengths(rng, list(zip(ls.tolist(), wl.tolist())),
                                        page_size, pool_pages)
    if reverse_pages:
        # physical pages in reverse logical order across the whole batch: a
        # kernel that ignored the page table would read the wrong rows
        live = [p for t in tables for p in t if p >= 0]
        rev = iter(sorted(live, reverse=True))
        tables = [np.array([next(rev) if p >= 0 else -1 for p in t], dtype=np.int32)
                  for t in tables]
    q = _normal(rng, (len(ls), num_qo_heads, head_dim), dtype)
    k, v = _pool(rng, pool_pages, page_size, num_kv_heads, head_dim, dtype,
                 poison_unused, used)
    w = Workload(name=name, dtype=dtype, page_size=page_size,
                 num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim,
                 sm_scale=float(sm_scale if sm_scale is not None else 1.0 / np.sqrt(head_dim)),
                 q=q, k_pool=k, v_pool=v, block_tables=tables,
                 logical_start=ls, written_len=wl, target_wgs=target_wgs)
    return poison_invisible(w) if poison_unused else w


def tiny_fp32(seed=1, poison_unused=False):
    """Tiny fp32 decode: B=1, Hq=8, Hkv=2, D=64, page_size=16, 500 visible
    tokens (last page holds 4), pool of 64 pages, the request's 32 pages the
    first 32 entries of a random permutation of the pool."""
    rng = _rng(seed)
    ps, hq, hkv, d, n = 16, 8, 2, 64, 500
    perm = rng.permutation(64).astype(np.int32)
    table = perm[:32].copy()
    q = _normal(rng, (1, hq, d), FP32)
    k, v = _pool(rng, 64, ps, hkv, d, FP32, poison_unused, table)
    w = Workload(name="tiny_fp32", dtype=FP32, page_size=ps, num_qo_heads=hq,
                 num_kv_heads=hkv, head_dim=d, sm_scale=1.0 / np.sqrt(d),
                 q=q, k_pool=k, v_pool=v, block_tables=[table],
                 logical_start=np.zeros(1, np.int32),
                 written_len=np.array([n], np.int32), target_wgs=8)
    return poison_invisible(w) if poison_unused else w


def batched_fp16(seed=2, poison_unused=False):
    """Batched fp16 decode: B=4, Hq=32, Hkv=8, D=128, page_size=16, lengths
    uniform in [1024, 4096] with request 0 rounded down to a whole number of
    pages (an exactly-full last page), pages drawn without replacement from a
    2048-page pool."""
    rng = _rng(seed)
    ps, hq, hkv, d, b = 16, 32, 8, 128, 4
    lens = rng.integers(1024, 4097, size=b).astype(np.int32)
    lens[0] = (lens[0] // ps) * ps
    tables, used = _tables_from_lengths(rng, [(0, int(x)) for x in lens], ps, 2048)
    q = _normal(rng, (b, hq, d), FP16)
    k, v = _pool(rng, 2048, ps, hkv, d, FP16, poison_unused, used)
    w = Workload(name="batched_fp16", dtype=FP16, page_size=ps, num_qo_heads=hq,
                 num_kv_heads=hkv, head_dim=d, sm_scale=1.0 / np.sqrt(d),
                 q=q, k_pool=k, v_pool=v, block_tables=tables,
                 logical_start=np.zeros(b, np.int32), written_len=lens)
    return poison_invisible(w) if poison_unused else w


def long_context_fp16(seed=3, poison_unused=False, num_qo_heads=32, page_size=16, head_dim=128):
    """Long-context split-KV: B=4, Hq=32, Hkv=8, D=128, page_size=16, fp16.
    Requests 0-2 see 32768 tokens from position 0.  Request 3 is a sliding
    window of 4096 visible tokens whose first visible token sits at entry 7 of
    its first page: written length 32768+7, logical start 32768+7-4096, so
    the 1792 pages before the window are released.  Pool = 2x the live
    pages, drawn without replacement.  num_qo_heads other than 32 gives the
    same KV geometry with larger query groups (G = num_qo_heads / 8), and
    page_size other than 16 the same token windows in pages of that size, and
    head_dim other than 128 rows of that many halves."""
    rng = _rng(seed)
    ps, hq, hkv, d = page_size, num_qo_heads, 8, head_dim
    wl = np.array([32768, 32768, 32768, 32768 + 7], np.int32)
    ls = np.array([0, 0, 0, 32768 + 7 - 4096], np.int32)
    live = sum(-(-int(w) // ps) - int(s) // ps for w, s in zip(wl, ls))
    pool_pages = 2 * live
    tables, used = _tables_from_lengths(rng, list(zip(ls.tolist(), wl.tolist())), ps,
                                        pool_pages)
    q = _normal(rng, (4, hq, d), FP16)
    k, v = _pool(rng, pool_pages, ps, hkv, d, FP16, poison_unused, used)
    w = Workload(name="long_context_fp16", dtype=FP16, page_size=ps,
                 num_qo_heads=hq, num_kv_heads=hkv, head_dim=d,
                 sm_scale=1.0 / np.sqrt(d), q=q, k_pool=k, v_pool=v,
                 block_tables=tables, logical_start=ls, written_len=wl)
    return poison_invisible(w) if poison_unused else w


@dataclasses.dataclass
class SparseWorkload:
    """Token-sparse selection over a dense [B, Hkv, Cap, D] allocation."""
    k_dense: np.ndarray     # [1, Hkv, Cap, D] fp16
    v_dense: np.ndarray
    q: np.ndarray           # [1, Hq, 1, D] fp16
    positions: List[np.ndarray]  # per KV head, sorted distinct positions
    sm_scale: float

    @property
    def kv_bytes(self) -> int:
        return sum(len(p) for p in self.positions) * self.k_dense.shape[-1] * 2 * 2


def token_sparse_fp16(seed=4, cap=131072, topk=2048, hq=24, hkv=2, d=128):
    """Token-sparse selection at page_size=1: dense [1, 2, 131072, 128] fp16
    per side, per KV head a sorted random top-k of 2048 distinct positions."""
    rng = _rng(seed)
    k = _normal(rng, (1, hkv, cap, d), FP16)
    v = _normal(rng, (1, hkv, cap, d), FP16)
    q = _normal(rng, (1, hq, 1, d), FP16)
    pos = [np.sort(rng.choice(cap, size=topk, replace=False)).astype(np.int32)
           for _ in range(hkv)]
    return SparseWorkload(k_dense=k, v_dense=v, q=q, positions=pos,
                          sm_scale=1.0 / np.sqrt(d))


def folded_sparse(s: SparseWorkload, name="token_sparse_fp16") -> Workload:
    """The same selection laid out as a page_size-1 paged workload: the
    dense [1, Hkv, Cap, D] allocation read as a pool of Hkv*Cap one-token
    pages with one KV head, one request per KV head holding its selected
    rows, and the query [1, Hq, 1, D] read as [Hkv, Hq/Hkv, D] (query head i
    under KV head i // (Hq/Hkv)).  Pure relayout: no values change."""
    _, hkv, cap, d = s.k_dense.shape
    hq = s.q.shape[1]
    k = s.k_dense.reshape(hkv * cap, 1, 1, d)
    v = s.v_dense.reshape(hkv * cap, 1, 1, d)
    q = s.q.reshape(hkv, hq // hkv, d)
    tables = [(h * cap + np.asarray(p, np.int64)).astype(np.int32)
              for h, p in enumerate(s.positions)]
    lens = np.array([len(p) for p in s.positions], np.int32)
    return Workload(name=name, dtype=FP16, page_size=1, num_qo_heads=hq // hkv,
                    num_kv_heads=1, head_dim=d, sm_scale=s.sm_scale, q=q, k_pool=k,
                    v_pool=v, block_tables=tables, logical_start=np.zeros(hkv, np.int32),
                    written_len=lens)


@dataclasses.dataclass
class BlockSparseWorkload:
    """A selection of KV blocks per (sequence, KV head) over a dense
    [B, Hkv, Cap, D] allocation; each request's final, partially written
    block is listed last."""
    k_dense: np.ndarray     # [B, Hkv, Cap, D] fp16
    v_dense: np.ndarray
    q: np.ndarray           # [B, Hq, D] fp16
    block_ids: np.ndarray   # [B*Hkv, blocks] int32
    block_size: int
    kv_len: np.ndarray      # [B] visible positions of each sequence
    sm_scale: float
    name: str = "block_sparse_fp16"


def block_sparse_fp16(seed=7, hq=64, hkv=4, cap=65536, block_size=128, blocks=16,
                      kv_len=65536 - 37, d=128):
    """Block-sparse decode in the geometry of the sparse-paged-decode doc's
    MiniMax-M3 example (64 query heads, 4 KV heads, head dim 128, blocks of
    128 positions, 16 selected blocks): one sequence whose live window holds
    kv_len positions of a Cap-position allocation; per KV head 15 distinct
    blocks drawn from the scored set (every block but the final one) plus the
    final block, listed last.  Positions at or past kv_len are NaN, so a
    decode that reads past the final block's written positions produces NaN."""
    rng = _rng(seed)
    k = _normal(rng, (1, hkv, cap, d), FP16)
    v = _normal(rng, (1, hkv, cap, d), FP16)
    k[:, :, kv_len:] = np.nan
    v[:, :, kv_len:] = np.nan
    q = _normal(rng, (1, hq, d), FP16)
    final = (kv_len - 1) // block_size
    ids = np.stack([np.concatenate([rng.choice(final, size=blocks - 1, replace=False),
                                    [final]]) for _ in range(hkv)]).astype(np.int32)
    return BlockSparseWorkload(k_dense=k, v_dense=v, q=q, block_ids=ids, block_size=block_size,
                               kv_len=np.array([kv_len], np.int64), sm_scale=1.0 / np.sqrt(d))


def cascade_fp16(seed=5, members=4, prefix_tokens=8192, suffix_lo=256, suffix_hi=2048,
                 hq=32, hkv=8, d=128, ps=16, poison_unused=False):
    """Cascade shared prefix: ``members`` requests share the same physical
    pages for an 8192-token prefix, followed by private suffixes of uniform
    [256, 2048] tokens.  Pool = 2x the live pages."""
    rng = _rng(seed)
    suffix = rng.integers(suffix_lo, suffix_hi + 1, size=members).astype(np.int32)
    pre_pages = prefix_tokens // ps
    suf_pages = [-(-int(s) // ps) for s in suffix]
    live = pre_pages + sum(suf_pages)
    pool_pages = 2 * live
    perm = rng.permutation(pool_pages).astype(np.int32)
    prefix = perm[:pre_pages]
    tables, pos = [], pre_pages
    for sp in suf_pages:
        tables.append(np.concatenate([prefix, perm[pos:pos + sp]]).astype(np.int32))
        pos += sp
    used = perm[:pos]
    q = _normal(rng, (members, hq, d), FP16)
    k, v = _pool(rng, pool_pages, ps, hkv, d, FP16, poison_unused, used)
    wl = (prefix_tokens + suffix).astype(np.int32)
    w = Workload(name="cascade_fp16", dtype=FP16, page_size=ps, num_qo_heads=hq,
                 num_kv_heads=hkv, head_dim=d, sm_scale=1.0 / np.sqrt(d),
                 q=q, k_pool=k, v_pool=v, block_tables=tables,
                 logical_start=np.zeros(members, np.int32), written_len=wl,
                 extra={"shared_pages": pre_pages, "suffix_tokens": suffix})
    return poison_invisible(w) if poison_unused else w


def random_geometry(seed, *, batch, page_size, max_len, dtype=FP16, num_qo_heads=8,
                    num_kv_heads=2, head_dim=128, p_empty=0.1, p_trim=0.4,
                    poison_unused=True, reverse_pages=False):
    """Random ragged batch: empty requests, front-trimmed windows that start
    mid-page, partial and exactly-full last pages."""
    rng = _rng(seed)
    ls, wl = [], []
    for _ in range(batch):
        w = int(rng.integers(0, max_len + 1))
        u = rng.random()
        if u < p_empty:
            s = w                                   # nothing visible
        elif u < p_empty + p_trim and w > 0:
            s = int(rng.integers(0, w + 1))         # front trim, any offset
        else:
            s = 0
        if rng.random() < 0.2 and w > 0 and s == 0:
            w = max(page_size, (w // page_size) * page_size)   # exactly full
        ls.append(s)
        wl.append(w)
    return generic(f"random_{seed}", seed=seed + 1000, dtype=dtype, page_size=page_size,
                   num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                   head_dim=head_dim, logical_start=ls, written_len=wl,
                   poison_unused=poison_unused, reverse_pages=reverse_pages)


ALL = {
    "tiny_fp32": tiny_fp32,
    "batched_fp16": batched_fp16,
    "long_context_fp16": long_context_fp16,
    "cascade_fp16": cascade_fp16,
}


@dataclasses.dataclass
class MlaWorkload:
    """Decode with a second key stream (the DSA / paged-MLA shape of the
    sparse-paged-decode doc): one KV head; k_pool rows hold the latent
    (dim elements, also the values) followed by an indexer key up to
    row_stride; k_extra_pool holds the rope keys; both share the page table."""
    name: str
    page_size: int
    num_qo_heads: int
    dim: int
    extra_dim: int
    row_stride: int
    sm_scale: float
    q: np.ndarray                   # [B, Hq, dim] fp16
    q_extra: np.ndarray             # [B, Hq, extra_dim] fp16
    k_pool: np.ndarray              # [pages, page_size, row_stride] fp16
    k_extra_pool: np.ndarray        # [pages, page_size, extra_dim] fp16
    block_tables: List[np.ndarray]
    logical_start: np.ndarray
    written_len: np.ndarray
    dtype: str = FP16

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def visible_tokens(self) -> np.ndarray:
        return (self.written_len - self.logical_start).astype(np.int64)

    def kv_bytes(self) -> int:
        """Algorithmic bytes one decode step reads: every visible token's
        latent and rope keys once (the latent doubles as the value)."""
        return int(self.visible_tokens.sum()) * (self.dim + self.extra_dim) * 2


def mla_paged(name="mla_paged", *, seed, logical_start, written_len, num_qo_heads=128,
              page_size=64, dim=512, extra_dim=64, row_stride=640, pool_slack=2.0,
              poison_unused=False, poison_indexer=False):
    """A paged latent cache: per-request (logical_start, written_len), pages
    drawn without replacement from a pool with 2x slack.  poison_unused sets
    unused pages to NaN; poison_indexer sets the row columns past `dim` (the
    indexer key, never read by the decode) to NaN."""
    rng = _rng(seed)
    ls = np.asarray(logical_start, dtype=np.int32)
    wl = np.asarray(written_len, dtype=np.int32)
    nlive = sum(max(0, (-(-int(w) // page_size) if w > 0 else 0) - int(s) // page_size)
                for s, w in zip(ls, wl))
    pool_pages = max(1, int(np.ceil(pool_slack * max(1, nlive))))
    tables, used = _tables_from_lengths(rng, list(zip(ls.tolist(), wl.tolist())), page_size,
                                        pool_pages)
    b = ls.size
    k = _normal(rng, (pool_pages, page_size, row_stride), FP16)
    kx = _normal(rng, (pool_pages, page_size, extra_dim), FP16)
    q = _normal(rng, (b, num_qo_heads, dim), FP16)
    qx = _normal(rng, (b, num_qo_heads, extra_dim), FP16)
    if poison_unused:
        unused = np.ones(pool_pages, dtype=bool)
        unused[np.asarray(used, dtype=np.int64)] = False
        k[unused] = np.nan
        kx[unused] = np.nan
    if poison_indexer:
        k[:, :, dim:] = np.nan
    return MlaWorkload(name=name, page_size=page_size, num_qo_heads=num_qo_heads, dim=dim,
                       extra_dim=extra_dim, row_stride=row_stride,
                       sm_scale=1.0 / np.sqrt(dim + extra_dim), q=q, q_extra=qx, k_pool=k,
                       k_extra_pool=kx, block_tables=tables, logical_start=ls, written_len=wl)


def mla_paged_fp16(seed=9, batch=4, context=32768, **kw):
    """Paged MLA decode in DeepSeek-V3.2's attention geometry (128 query
    heads, latent 512, rope 64, indexer key 128, so rows of 640): `batch`
    requests of `context` visible tokens in 64-token pages."""
    return mla_paged("mla_paged_fp16", seed=seed, logical_start=[0] * batch,
                     written_len=[context] * batch, **kw)


def dsa_sparse_fp16(seed=10, batch=8, capacity=32768, kv_len=32768 - 29, topk=2048,
                    num_qo_heads=128, dim=512, extra_dim=64, row_stride=640,
                    poison_unselected=False):
    """DSA decode over a dense latent cache: per sequence a [capacity,
    row_stride] latent allocation and a [capacity, extra_dim] rope allocation,
    read as page_size-1 pools (row = b * capacity + position); each sequence
    selects `topk` distinct positions below kv_len (sorted).  The page table
    lists the selected rows.  poison_unselected sets every unselected row (and
    the indexer-key columns) to NaN."""
    rng = _rng(seed)
    k = _normal(rng, (batch * capacity, 1, row_stride), FP16)
    kx = _normal(rng, (batch * capacity, 1, extra_dim), FP16)
    q = _normal(rng, (batch, num_qo_heads, dim), FP16)
    qx = _normal(rng, (batch, num_qo_heads, extra_dim), FP16)
    tables = []
    for s in range(batch):
        pos = np.sort(rng.choice(kv_len, size=topk, replace=False)).astype(np.int32)
        tables.append(s * capacity + pos)
    if poison_unselected:
        keep = np.zeros(batch * capacity, dtype=bool)
        keep[np.concatenate(tables)] = True
        k[~keep] = np.nan
        kx[~keep] = np.nan
        k[:, :, dim:] = np.nan
    return MlaWorkload(name="dsa_sparse_fp16", page_size=1, num_qo_heads=num_qo_heads,
                       dim=dim, extra_dim=extra_dim, row_stride=row_stride,
                       sm_scale=1.0 / np.sqrt(dim + extra_dim), q=q, q_extra=qx, k_pool=k,
                       k_extra_pool=kx, block_tables=tables,
                       logical_start=np.zeros(batch, np.int32),
                       written_len=np.full(batch, topk, np.int32))
