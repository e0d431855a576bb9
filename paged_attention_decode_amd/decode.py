"""Decode steps over the C-ABI: flat split-KV decode, cascade, token-sparse.

Host work here is the pages' run step (mlxcel PR #984 body item 5 and the
commit adding plan + launch): validate the CSR view, build the plan once, keep
the int32 arrays and workspace resident on the device, then each step is one
partial launch plus a merge launch when some request was split.  Every
arithmetic step runs in the library's HIP kernels; this module only moves
arguments and allocates caller-owned buffers with torch.
"""
from __future__ import annotations

import time

import numpy as np
import torch

from . import binding as B


def _pd_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return B.PD_DTYPE_FP16
    if t.dtype == torch.float32:
        return B.PD_DTYPE_FP32
    raise TypeError("q and pools must be float16 or float32")


def pool_strides(k_pool: torch.Tensor, v_pool: torch.Tensor):
    """Element strides (page, token, head) of a [pages, page_size, Hkv, D]
    pool pair; D must be contiguous and both pools laid out alike."""
    if k_pool.dim() != 4 or k_pool.shape != v_pool.shape:
        raise ValueError("pools must be [pages, page_size, Hkv, D] and of one shape")
    if k_pool.stride() != v_pool.stride() or k_pool.stride(3) != 1:
        raise ValueError("K and V pools need identical strides and a contiguous head dim")
    return k_pool.stride(0), k_pool.stride(1), k_pool.stride(2)


def _dev_i32(a, device):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(device)


class PagedDecode:
    """One batch's validated page table, plan and workspace, reusable across
    decode steps until a request crosses a page boundary."""

    def __init__(self, csr: dict, *, page_size: int, num_pool_pages: int, num_qo_heads: int,
                 num_kv_heads: int, head_dim: int, target_wgs: int = 0,
                 fixed_pages_per_chunk: int = 0, fused: bool = False, dtype=torch.float16,
                 device="cuda"):
        indptr = np.asarray(csr["indptr"], np.int32)
        self.indptr = indptr
        self.batch = indptr.size - 1
        self.page_size = page_size
        self.num_qo_heads, self.num_kv_heads, self.head_dim = num_qo_heads, num_kv_heads, head_dim
        B.csr_validate(self.batch, page_size, num_pool_pages, indptr, csr["indices"],
                       csr["last_page_len"], csr["first_page_offset"], csr.get("seq_lens"))
        pd_dtype = B.PD_DTYPE_FP32 if dtype == torch.float32 else B.PD_DTYPE_FP16
        info, ri, ti, oi = B.paged_decode_plan(indptr, num_qo_heads, num_kv_heads, head_dim,
                                               target_wgs, fixed_pages_per_chunk,
                                               dtype=pd_dtype, page_size=page_size)
        self.info, self.request_indices, self.kv_tile_indices, self.o_indptr = info, ri, ti, oi
        self.fixed_pages_per_chunk = fixed_pages_per_chunk
        self.num_pool_pages = num_pool_pages
        self.device = torch.device(device)
        idx = np.asarray(csr["indices"], np.int32)
        self.d_indices = _dev_i32(idx if idx.size else np.zeros(1, np.int32), self.device)
        self.d_indptr = _dev_i32(indptr, self.device)
        self.d_lpl = _dev_i32(csr["last_page_len"], self.device)
        self.d_fpo = _dev_i32(csr["first_page_offset"], self.device)
        self.d_req = _dev_i32(ri, self.device)
        self.d_tile = _dev_i32(ti, self.device)
        self.d_oindptr = _dev_i32(oi, self.device)
        n = info.num_chunks
        self.v_partial = torch.empty((n, num_qo_heads, head_dim), dtype=torch.float32,
                                     device=self.device)
        self.lse_partial = torch.empty((n, num_qo_heads), dtype=torch.float32, device=self.device)
        self.fused = fused
        if info.needs_merge or fused:
            self.out = torch.empty((self.batch, num_qo_heads, head_dim), dtype=torch.float32,
                                   device=self.device)
            self.lse = torch.empty((self.batch, num_qo_heads), dtype=torch.float32,
                                   device=self.device)
        else:   # write-O-directly: the partial, in request order, is the answer
            self.out, self.lse = self.v_partial, self.lse_partial
        # per-(request, KV head) arrival counters of the fused launch; every
        # completed launch leaves them at zero
        self.counters = (torch.zeros(self.batch * num_kv_heads, dtype=torch.int32,
                                     device=self.device) if fused else None)

    def plan_summary(self) -> dict:
        i = self.info
        return dict(pages_per_chunk=i.pages_per_chunk, num_chunks=i.num_chunks,
                    num_wgs=i.num_wgs, needs_merge=bool(i.needs_merge),
                    target_wgs=i.target_wgs, workspace_bytes=i.workspace_bytes)

    def use_workspace(self, v_partial, lse_partial):
        """Write the partial rows into caller-owned fp32 tensors of shape
        [num_chunks, Hq, D] and [num_chunks, Hq] (e.g. views of a larger
        buffer) instead of this object's own."""
        n = self.info.num_chunks
        if tuple(v_partial.shape) != (n, self.num_qo_heads, self.head_dim) or \
                tuple(lse_partial.shape) != (n, self.num_qo_heads) or \
                v_partial.dtype != torch.float32 or lse_partial.dtype != torch.float32 or \
                not v_partial.is_contiguous() or not lse_partial.is_contiguous():
            raise ValueError("workspace must be contiguous fp32 [%d, %d, %d] and [%d, %d]"
                             % (n, self.num_qo_heads, self.head_dim, n, self.num_qo_heads))
        if self.out is self.v_partial:
            self.out, self.lse = v_partial, lse_partial
        self.v_partial, self.lse_partial = v_partial, lse_partial

    def check_step(self, q, k_pool, v_pool):
        """The shapes the kernels index by: q a contiguous [B, Hq, D] tensor
        and pools [>= num_pool_pages, page_size, Hkv, D] (strided views
        allowed), all of one dtype.  The C-ABI sees only addresses, so a
        mis-shaped tensor is refused here rather than read out of bounds."""
        if tuple(q.shape) != (self.batch, self.num_qo_heads, self.head_dim) or \
                not q.is_contiguous():
            raise ValueError("q must be a contiguous [B, Hq, D] = [%d, %d, %d] tensor (got %s)"
                             % (self.batch, self.num_qo_heads, self.head_dim, tuple(q.shape)))
        if q.dtype != k_pool.dtype or q.dtype != v_pool.dtype:
            raise TypeError("q and pools must share a dtype")
        if k_pool.dim() != 4 or k_pool.shape[0] < self.num_pool_pages or \
                tuple(k_pool.shape[1:]) != (self.page_size, self.num_kv_heads, self.head_dim):
            raise ValueError("pools must be [>= %d pages, %d, %d, %d] (got %s)"
                             % (self.num_pool_pages, self.page_size, self.num_kv_heads,
                                self.head_dim, tuple(k_pool.shape)))

    def partial(self, q, k_pool, v_pool, sm_scale, stream=None):
        self.check_step(q, k_pool, v_pool)
        ps_, ts_, hs_ = pool_strides(k_pool, v_pool)
        B.paged_decode_partial(q, k_pool, v_pool, ps_, ts_, hs_, _pd_dtype(q), self.d_indices,
                               self.d_indptr, self.d_lpl, self.d_fpo, self.d_req, self.d_tile,
                               self.info.num_chunks, self.info.pages_per_chunk, self.batch,
                               self.num_qo_heads, self.num_kv_heads, self.head_dim,
                               self.page_size, sm_scale, self.v_partial, self.lse_partial,
                               stream)

    def merge(self, stream=None):
        if self.info.needs_merge:
            B.paged_merge_states(self.v_partial, self.lse_partial, self.d_oindptr, self.batch,
                                 self.num_qo_heads, self.head_dim, self.out, self.lse, stream)

    def fused_step(self, q, k_pool, v_pool, sm_scale, stream=None):
        self.check_step(q, k_pool, v_pool)
        ps_, ts_, hs_ = pool_strides(k_pool, v_pool)
        B.paged_decode_fused(q, k_pool, v_pool, ps_, ts_, hs_, _pd_dtype(q), self.d_indices,
                             self.d_indptr, self.d_lpl, self.d_fpo, self.d_req, self.d_tile,
                             self.info.num_chunks, self.info.pages_per_chunk, self.batch,
                             self.num_qo_heads, self.num_kv_heads, self.head_dim,
                             self.page_size, sm_scale, self.v_partial, self.lse_partial,
                             self.counters, self.out, self.lse, stream)

    def run(self, q, k_pool, v_pool, sm_scale, stream=None):
        """One decode step: returns (out [B, Hq, D] fp32, lse [B, Hq] fp32,
        log2 units); the tensors are this object's buffers."""
        if self.fused:
            self.fused_step(q, k_pool, v_pool, sm_scale, stream)
        else:
            self.partial(q, k_pool, v_pool, sm_scale, stream)
            self.merge(stream)
        return self.out, self.lse


def cascade_members_per_launch(members: int, group_size: int, head_dim: int, pd_dtype: int,
                               page_size: int, token_stride: int) -> int:
    """Members stacked per level-0 launch of a cascade step.  Launches stack
    `per` members each in member order and the last one the rest, so both
    per * G and the remainder's stacked group must have a partial kernel
    (for this dtype, head dim and page size).  Among the sizes that satisfy
    that, the one with the fewest launches wins (each launch reads the shared
    span once), then the one whose last launch stacks the most members.  A
    single member is always a supported launch (its group is the flat
    decode's), so some size always qualifies."""
    lib = B.load()

    def ok(k):
        return k == 0 or lib.paged_decode_kernel_kind(pd_dtype, head_dim, k * group_size,
                                                      page_size, token_stride) >= 0

    if not ok(1):
        raise ValueError("no partial kernel for group size %d, head_dim %d"
                         % (group_size, head_dim))
    best = None
    for per in range(1, members + 1):
        launches = -(-members // per)
        last = members - (launches - 1) * per
        if ok(per) and ok(last):
            key = (launches, -last)
            if best is None or key < best[0]:
                best = (key, per)
    return best[1]


class CascadeDecode:
    """Cascade decode of one batch (cascade-attention doc).

    Detection over the page table (``paged_cascade_detect``) picks the
    requests that share leading pages and the shared span, unless members and
    shared_pages are given.  Level 0 attends the span once per subgroup of
    members with their query heads stacked (a launch stacks at most 32 query
    heads per KV head, 16 off the MFMA kernel, so a larger M*G splits the
    members into subgroups that each read the span); level 1 attends every
    request's own pages -- the members' pages after the span and the other
    requests' whole lists; one merge finishes every request.  The merge reads
    the level-0 rows where the stacked launches wrote them
    (``paged_cascade_merge_states``; head_dim a multiple of 32), or, with
    merge_in_place=False or another head size, from a copy that un-stacks
    them into the host-computed layout (``paged_cascade_gather_states`` +
    ``paged_merge_states``).  With no qualifying span the step is the flat
    decode.
    """

    def __init__(self, csr: dict, *, page_size: int, num_pool_pages: int, num_qo_heads: int,
                 num_kv_heads: int, head_dim: int, members=None, shared_pages: int = 0,
                 min_shared_pages: int = 16, min_members: int = 2, target_wgs: int = 0,
                 target_wgs_level0: int = 0, min_level0_tokens: int = 64,
                 merge_in_place: bool = True, pair_launch: bool = True,
                 heads_per_workgroup: int = 0, fixed_pages_level0: int = 0,
                 fixed_pages_level1: int = 0, dtype=torch.float16, device="cuda"):
        indptr = np.asarray(csr["indptr"], np.int32)
        indices = np.asarray(csr["indices"], np.int32)
        lpl = np.asarray(csr["last_page_len"], np.int32)
        fpo = np.asarray(csr["first_page_offset"], np.int32)
        self.batch = indptr.size - 1
        self.num_qo_heads, self.num_kv_heads, self.head_dim = num_qo_heads, num_kv_heads, head_dim
        B.csr_validate(self.batch, page_size, num_pool_pages, indptr, indices, lpl, fpo,
                       csr.get("seq_lens"))
        if members is None:
            members, shared_pages = B.paged_cascade_detect(indptr, indices, fpo,
                                                           min_shared_pages, min_members)
        self.member_req = np.asarray(members, np.int32)
        self.shared_pages = int(shared_pages)
        self.dtype = dtype
        self.device = torch.device(device)
        kw = dict(page_size=page_size, num_pool_pages=num_pool_pages, num_kv_heads=num_kv_heads,
                  head_dim=head_dim, dtype=dtype, device=device)
        self.flat = None
        if self.member_req.size == 0 or self.shared_pages == 0:
            self.flat = PagedDecode(csr, num_qo_heads=num_qo_heads, target_wgs=target_wgs, **kw)
            self.out, self.lse = self.flat.out, self.flat.lse
            return
        idx0, csr1 = B.paged_cascade_split(page_size, indptr, indices, lpl, fpo, self.member_req,
                                           self.shared_pages)
        csr0 = dict(indptr=np.array([0, self.shared_pages], np.int32), indices=idx0,
                    last_page_len=np.array([page_size], np.int32),
                    first_page_offset=np.array([0], np.int32))
        # subgroups of members whose stacked group size a launch supports
        g = num_qo_heads // num_kv_heads
        pd_dtype = B.PD_DTYPE_FP32 if dtype == torch.float32 else B.PD_DTYPE_FP16
        per = cascade_members_per_launch(self.member_req.size, g, head_dim, pd_dtype, page_size,
                                         num_kv_heads * head_dim)
        self.subgroups = [self.member_req[i:i + per] for i in range(0, self.member_req.size, per)]
        self.pair_launch = pair_launch
        self.heads_per_workgroup = heads_per_workgroup
        self.level0 = []
        fixed = fixed_pages_level0
        # Level 0's chunks hold at least min_level0_tokens tokens unless a
        # level-0 target (target_wgs_level0) is given; a target_wgs given for
        # the whole step still gets the floor.  A stacked chunk writes M*G
        # partial rows per KV head, so the occupancy plan's smallest chunks
        # (2 pages of 16 at 8K shared tokens) write half as many bytes as they
        # read.  Measured on MI355X (graph-replayed steps): 4-page chunks took
        # 4 x 8K from 34.4 to 33.4 us and 16 x 8K from 68.8 to 67.0 us; from
        # 32K shared tokens on the plan's chunks are larger anyway.
        floor = 0 if target_wgs_level0 else min(self.shared_pages,
                                                  -(-min_level0_tokens // page_size))
        # When the first level-0 launch and level 1 run as one grid (pair
        # launch: both on the MFMA kernel), they share the GPU.  By default
        # level 0 is planned for about two (chunk, KV head) units per CU (its
        # chunks are few and long, and each adds members*Hq partial rows to
        # the merge), and level 1 for as many units.  Sweeps on MI355X (4 to
        # 16 members, 8K to 32K shared tokens; level-1 chunks of 1 to 33
        # pages) put this within about 10% of the best chunking, where either
        # level planned for the whole GPU was up to 1.5x slower.  The
        # workgroups hold one KV head each: at the same chunking that was as
        # fast as two or faster (graph-replayed, 4 x 8K shared tokens 19.1
        # against 20.1 us, 16 x 8K 46.9 against 47.7, 4 x 32K 36.6 against
        # 37.8-38.4, equal at 8 x 8K and 8 x 16K).
        t0, t1 = target_wgs_level0 or target_wgs, target_wgs
        g0 = self.subgroups[0].size * g
        self.pair_eligible = pair_launch and g <= 16 and B.load().paged_decode_kernel_kind(
            pd_dtype, head_dim, g0, page_size, num_kv_heads * head_dim) == 2
        if self.pair_eligible and not heads_per_workgroup:
            self.heads_per_workgroup = 1
        if self.pair_eligible and not (target_wgs_level0 or target_wgs):
            cus = torch.cuda.get_device_properties(self.device).multi_processor_count
            t0 = 2 * cus
            t1 = t0
        self.targets = (t0, t1)
        for sub in self.subgroups:
            lv = PagedDecode(csr0, num_qo_heads=sub.size * num_qo_heads, target_wgs=t0,
                             fixed_pages_per_chunk=fixed, **kw)
            if not fixed and lv.info.pages_per_chunk < floor:
                fixed = floor
                lv = PagedDecode(csr0, num_qo_heads=sub.size * num_qo_heads, target_wgs=t0,
                                 fixed_pages_per_chunk=fixed, **kw)
            fixed = fixed or lv.info.pages_per_chunk      # one level-0 chunking for all
            self.level0.append(lv)
        self.level1 = PagedDecode(csr1, num_qo_heads=num_qo_heads, target_wgs=t1,
                                  fixed_pages_per_chunk=fixed_pages_level1, **kw)
        self.n0 = self.level0[0].info.num_chunks
        self.n1 = self.level1.info.num_chunks
        self.rows0 = None
        if merge_in_place and head_dim % 32 == 0:
            # the merge reads the level-0 rows in place: the launches write one
            # buffer, one after another
            total = sum(self.n0 * sub.size * num_qo_heads for sub in self.subgroups)
            self.rows0 = (torch.empty((total, head_dim), dtype=torch.float32, device=self.device),
                          torch.empty(total, dtype=torch.float32, device=self.device))
            first = 0
            for lv, sub in zip(self.level0, self.subgroups):
                rows = self.n0 * sub.size * num_qo_heads
                lv.use_workspace(
                    self.rows0[0][first:first + rows].view(self.n0, sub.size * num_qo_heads,
                                                           head_dim),
                    self.rows0[1][first:first + rows].view(self.n0, sub.size * num_qo_heads))
                first += rows
            self.d_l0_desc = _dev_i32(
                B.paged_cascade_merge_layout(self.batch, self.member_req, per, self.n0,
                                             num_qo_heads), self.device)
        # the C-ABI's view of each level (device addresses of the tensors above)
        self.l0_levels = B.cascade_levels(
            [B.cascade_level(lv.d_indices, lv.d_indptr, lv.d_lpl, lv.d_fpo, lv.d_req, lv.d_tile,
                             1, lv.info.num_chunks, lv.info.pages_per_chunk, lv.v_partial,
                             lv.lse_partial) for lv in self.level0])
        self.members_per_launch = per
        self.d_member_req = _dev_i32(self.member_req, self.device)
        l1 = self.level1
        self.l1_level = B.cascade_level(l1.d_indices, l1.d_indptr, l1.d_lpl, l1.d_fpo, l1.d_req,
                                        l1.d_tile, self.batch, l1.info.num_chunks,
                                        l1.info.pages_per_chunk, l1.v_partial, l1.lse_partial)
        self.page_size = page_size
        dst0, dst1, oi = B.paged_cascade_layout(self.member_req, self.n0, self.level1.o_indptr)
        self.o_indptr = oi
        self.d_oindptr = _dev_i32(oi, self.device)
        self.d_dst1 = _dev_i32(dst1 if dst1.size else np.zeros(1, np.int32), self.device)
        self.d_members, self.d_dst0 = [], []
        pos = 0
        for sub in self.subgroups:
            self.d_members.append(_dev_i32(sub, self.device))
            self.d_dst0.append(_dev_i32(dst0[pos:pos + sub.size], self.device))
            pos += sub.size
        rows = int(oi[-1])
        self.v_cat = self.lse_cat = None            # the gathered merge input
        if self.rows0 is None:
            self.v_cat = torch.empty((rows, num_qo_heads, head_dim), dtype=torch.float32,
                                     device=self.device)
            self.lse_cat = torch.empty((rows, num_qo_heads), dtype=torch.float32,
                                       device=self.device)
        self.out = torch.empty((self.batch, num_qo_heads, head_dim), dtype=torch.float32,
                               device=self.device)
        self.lse = torch.empty((self.batch, num_qo_heads), dtype=torch.float32,
                               device=self.device)

    @property
    def active(self) -> bool:
        return self.flat is None

    def plan_summary(self) -> dict:
        if self.flat is not None:
            return dict(cascade=False, flat=self.flat.plan_summary())
        return dict(cascade=True, members=[int(x) for x in self.member_req],
                    shared_pages=self.shared_pages, subgroups=len(self.subgroups),
                    pair_launch=self.pair_launch, heads_per_workgroup=self.heads_per_workgroup,
                    targets=list(self.targets), level0=self.level0[0].plan_summary(),
                    level1=self.level1.plan_summary())

    def run(self, q, k_pool, v_pool, sm_scale, stream=None):
        """One decode step: returns (out [B, Hq, D] fp32, lse [B, Hq] fp32)."""
        if self.flat is not None:
            return self.flat.run(q, k_pool, v_pool, sm_scale, stream)
        hq, d, hkv = self.num_qo_heads, self.head_dim, self.num_kv_heads
        if q.shape != (self.batch, hq, d) or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B, Hq, D] tensor")
        if q.dtype != self.dtype or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
            raise TypeError("q and pools must share the dtype the cascade was planned for")
        if not (q.is_cuda and k_pool.is_cuda and v_pool.is_cuda):
            raise ValueError("q and pools must be device tensors")
        self.level1.check_step(q, k_pool, v_pool)       # level 1 holds every request's q
        ps_, ts_, hs_ = pool_strides(k_pool, v_pool)
        # level 0 reads the members' queries in place (stacked heads, no
        # copy); one grid carries every level-0 launch and level 1 unless
        # pair_launch is off
        B.paged_cascade_partial(q, self.batch, self.d_member_req, self.member_req.size,
                                self.members_per_launch, k_pool, v_pool, ps_, ts_, hs_,
                                _pd_dtype(q), hq, hkv, d, self.page_size, sm_scale,
                                self.l0_levels, self.l1_level if self.pair_launch else None,
                                self.heads_per_workgroup, stream)
        if not self.pair_launch:
            self.level1.partial(q, k_pool, v_pool, sm_scale, stream)
        if self.rows0 is not None:
            B.paged_cascade_merge_states(self.rows0[0], self.rows0[1], self.n0, self.d_l0_desc,
                                         self.level1.v_partial, self.level1.lse_partial,
                                         self.level1.d_oindptr, self.batch, hq, hkv, d,
                                         self.out, self.lse, stream)
            return self.out, self.lse
        for j, sub in enumerate(self.subgroups):
            last = j == len(self.subgroups) - 1       # the last call also moves level 1
            B.paged_cascade_gather_states(
                self.level0[j].v_partial, self.level0[j].lse_partial, self.n0, sub.size,
                self.d_dst0[j], self.level1.v_partial if last else None,
                self.level1.lse_partial if last else None, self.n1 if last else 0,
                self.d_dst1 if last else None, hq, hkv, d, self.v_cat, self.lse_cat, stream)
        B.paged_merge_states(self.v_cat, self.lse_cat, self.d_oindptr, self.batch, hq, d,
                             self.out, self.lse, stream)
        return self.out, self.lse


def sparse_pool_view(k_dense: torch.Tensor, v_dense: torch.Tensor):
    """Token-sparse decode over a dense [B, Hkv, Cap, D] allocation
    (sparse-paged-decode doc, ContiguousCacheLayout): at page_size 1 and one
    pool head the allocation is the pool [B*Hkv*Cap, 1, 1, D] -- a view, no
    copy.  Request r = b*Hkv + h selects rows r*Cap + position."""
    b, hkv, cap, d = k_dense.shape
    if v_dense.shape != k_dense.shape or not k_dense.is_contiguous() or not v_dense.is_contiguous():
        raise ValueError("K and V allocations must be contiguous and of one shape "
                         "(shared row mapping)")
    return k_dense.view(b * hkv * cap, 1, 1, d), v_dense.view(b * hkv * cap, 1, 1, d)


def sparse_fold_query(q: torch.Tensor, num_kv_heads: int):
    """[B, Hq, 1, D] -> [B*Hkv, Hq/Hkv, D]: query head i sits under KV head
    i // (Hq/Hkv), so folding the KV-head axis into the request axis is a
    reshape."""
    b, hq, one, d = q.shape
    return q.reshape(b * num_kv_heads, hq // num_kv_heads, d)


def sparse_block_tables(positions, cap: int, batch: int = 1):
    """Per folded request r = b*Hkv + h: its selected pool rows."""
    del batch
    return [(r * cap + np.asarray(pos, np.int64)).astype(np.int32)
            for r, pos in enumerate(positions)]


class BlockSparseDecode:
    """Decode over a selection of KV blocks per (sequence, KV head) on a dense
    [B, Hkv, Cap, D] allocation (sparse-paged-decode doc: the two page-table
    granularities).

    Every (sequence, KV head) is one request of the page table, holding its
    query heads i // G == h (the ContiguousCacheLayout folding).  Each request
    lists `blocks_per_request` block ids, its partially written final block
    last; that block holds kv_len - final*block_size positions.

    token_exact=False (block-granular, needs Cap % block_size == 0): the
    allocation is read as a pool of pages of page_size rows, page_size
    dividing block_size, and each selected block becomes its block_size /
    page_size pages -- the same whole blocks are read.  page_size =
    block_size is one page per block; the default, 16 where it divides the
    block (else the block), lets the plan cut a small selection into chunks
    smaller than a block, so that it spreads over the GPU.
    token_exact=True: the allocation is read as one-token pages and the block
    ids are expanded into token rows.  Either way the ids are a device value
    turned into the table's rows by one device pass per step; the table's
    shape depends only on the selection size, so nothing is read back.
    """

    def __init__(self, k_dense, v_dense, *, num_qo_heads: int, block_size: int,
                 blocks_per_request: int, kv_len, token_exact: bool = False,
                 page_size: int = 0, target_wgs: int = 0, fixed_pages_per_chunk: int = 0,
                 device="cuda"):
        b, hkv, cap, d = k_dense.shape
        if v_dense.shape != k_dense.shape or not k_dense.is_contiguous() or \
                not v_dense.is_contiguous():
            raise ValueError("K and V allocations must be contiguous and of one shape")
        if num_qo_heads % hkv:
            raise ValueError("query heads must be a multiple of KV heads")
        if not token_exact and cap % block_size:
            raise ValueError("block-granular pages need Cap % block_size == 0")
        kv_len = np.broadcast_to(np.asarray(kv_len, np.int64), (b,))
        if np.any(kv_len < 1) or np.any(kv_len > cap):
            raise ValueError("kv_len must be in [1, Cap]")
        self.batch, self.num_kv_heads, self.num_qo_heads, self.head_dim = b, hkv, num_qo_heads, d
        self.requests = b * hkv
        self.blocks = blocks_per_request
        self.block_size = block_size
        self.token_exact = token_exact
        if token_exact:
            ps = 1
        else:
            ps = page_size or (16 if block_size % 16 == 0 else block_size)
            if ps < 1 or block_size % ps:
                raise ValueError("page_size must divide block_size")
        final = (kv_len - 1) // block_size
        tail = np.repeat((kv_len - final * block_size).astype(np.int32), hkv)
        csr = B.paged_sparse_csr(blocks_per_request, block_size, tail, ps)
        nnz = int(csr["indptr"][-1])
        self.page_size, self.span = ps, block_size // ps
        self.k_pool = k_dense.view(b * hkv * cap // ps, ps, 1, d)
        self.v_pool = v_dense.view(b * hkv * cap // ps, ps, 1, d)
        base = np.arange(self.requests, dtype=np.int64) * (cap // ps)
        if int(base[-1]) + cap // ps > np.iinfo(np.int32).max:
            raise ValueError("the allocation has more pages than int32 page ids can name")
        self.num_blocks = cap // block_size
        # the table's rows are written on the device every step; placeholder
        # rows (valid pool rows) let the host check the table's shape now
        csr["indices"] = np.zeros(max(1, nnz), np.int32)[:nnz]
        self.dec = PagedDecode(csr, page_size=self.page_size,
                               num_pool_pages=self.k_pool.shape[0],
                               num_qo_heads=num_qo_heads // hkv, num_kv_heads=1, head_dim=d,
                               target_wgs=target_wgs,
                               fixed_pages_per_chunk=fixed_pages_per_chunk, device=device)
        dev = self.dec.device
        self.d_base = _dev_i32(base.astype(np.int32), dev)
        # pages of the final block that hold its written positions
        self.d_final = _dev_i32(((tail + ps - 1) // ps).astype(np.int32), dev)

    def plan_summary(self) -> dict:
        return dict(self.dec.plan_summary(), page_size=self.page_size,
                    token_exact=self.token_exact)

    def run(self, q, block_ids, sm_scale, stream=None):
        """q [B, Hq, D]; block_ids [B*Hkv, blocks_per_request] int32 on the
        device.  Returns (out [B, Hq, D], lse [B, Hq]) fp32, log2 LSE."""
        if block_ids.dtype != torch.int32 or block_ids.numel() != self.requests * self.blocks:
            raise ValueError("block_ids must be int32 [B*Hkv, blocks_per_request]")
        B.paged_sparse_expand_blocks(block_ids, self.requests, self.blocks, self.d_base,
                                     self.span, self.d_final, self.dec.d_indptr,
                                     self.num_blocks, self.dec.d_indices, stream)
        qf = q.reshape(self.requests, self.num_qo_heads // self.num_kv_heads, self.head_dim)
        out, lse = self.dec.run(qf, self.k_pool, self.v_pool, sm_scale, stream)
        return (out.view(self.batch, self.num_qo_heads, self.head_dim),
                lse.view(self.batch, self.num_qo_heads))




def _row_pool_strides(pool: torch.Tensor):
    """Element strides (page, entry) of a [pages, page_size, row] pool with
    contiguous rows."""
    if pool.dim() != 3 or pool.stride(2) != 1:
        raise ValueError("MLA pools must be [pages, page_size, row] with contiguous rows")
    return pool.stride(0), pool.stride(1)


class MlaDecode:
    """Paged MLA / DSA decode of one batch (sparse-paged-decode doc, the DSA
    section): one KV head; scores over the latent (the first `dim` elements
    of each k_pool row) plus a second key stream (k_extra_pool); the latent
    rows are the values.  The plan is paged_decode_plan's with head_dim =
    dim (q groups of 64 heads); each step is one partial launch plus a merge
    when a request was split."""

    def __init__(self, csr: dict, *, page_size: int, num_pool_pages: int, num_qo_heads: int,
                 dim: int = 512, extra_dim: int = 64, target_wgs: int = 0,
                 fixed_pages_per_chunk: int = 0, device="cuda"):
        indptr = np.asarray(csr["indptr"], np.int32)
        self.indptr = indptr
        self.batch = indptr.size - 1
        self.page_size, self.num_qo_heads = page_size, num_qo_heads
        self.dim, self.extra_dim = dim, extra_dim
        self.num_pool_pages = num_pool_pages
        B.csr_validate(self.batch, page_size, num_pool_pages, indptr, csr["indices"],
                       csr["last_page_len"], csr["first_page_offset"], csr.get("seq_lens"))
        info, ri, ti, oi = B.paged_decode_plan(indptr, num_qo_heads, 1, dim, target_wgs,
                                               fixed_pages_per_chunk, dtype=B.PD_DTYPE_FP16,
                                               page_size=page_size)
        self.info, self.request_indices, self.kv_tile_indices, self.o_indptr = info, ri, ti, oi
        self.device = torch.device(device)
        idx = np.asarray(csr["indices"], np.int32)
        self.d_indices = _dev_i32(idx if idx.size else np.zeros(1, np.int32), self.device)
        self.d_indptr = _dev_i32(indptr, self.device)
        self.d_lpl = _dev_i32(csr["last_page_len"], self.device)
        self.d_fpo = _dev_i32(csr["first_page_offset"], self.device)
        self.d_req = _dev_i32(ri, self.device)
        self.d_tile = _dev_i32(ti, self.device)
        self.d_oindptr = _dev_i32(oi, self.device)
        n = info.num_chunks
        self.v_partial = torch.empty((n, num_qo_heads, dim), dtype=torch.float32,
                                     device=self.device)
        self.lse_partial = torch.empty((n, num_qo_heads), dtype=torch.float32, device=self.device)
        if info.needs_merge:
            self.out = torch.empty((self.batch, num_qo_heads, dim), dtype=torch.float32,
                                   device=self.device)
            self.lse = torch.empty((self.batch, num_qo_heads), dtype=torch.float32,
                                   device=self.device)
        else:   # write-O-directly
            self.out, self.lse = self.v_partial, self.lse_partial

    def plan_summary(self) -> dict:
        i = self.info
        return dict(pages_per_chunk=i.pages_per_chunk, num_chunks=i.num_chunks,
                    num_wgs=i.num_wgs, q_groups=i.q_groups, needs_merge=bool(i.needs_merge),
                    target_wgs=i.target_wgs, workspace_bytes=i.workspace_bytes)

    def check_step(self, q, q_extra, k_pool, k_extra_pool):
        """Shapes and dtypes the kernel indexes by (the C-ABI sees only
        addresses)."""
        if q.shape != (self.batch, self.num_qo_heads, self.dim) or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B, Hq, dim] tensor")
        if q_extra.shape != (self.batch, self.num_qo_heads, self.extra_dim) or \
                not q_extra.is_contiguous():
            raise ValueError("q_extra must be a contiguous [B, Hq, extra_dim] tensor")
        if not (q.dtype == q_extra.dtype == k_pool.dtype == k_extra_pool.dtype == torch.float16):
            raise TypeError("paged MLA decode takes fp16 queries and pools")
        for pool, width in ((k_pool, self.dim), (k_extra_pool, self.extra_dim)):
            if pool.dim() != 3 or pool.shape[0] < self.num_pool_pages or \
                    pool.shape[1] != self.page_size or pool.shape[2] < width:
                raise ValueError("pools must be [>= %d pages, %d, >= row width] (got %s)"
                                 % (self.num_pool_pages, self.page_size, tuple(pool.shape)))

    def partial(self, q, q_extra, k_pool, k_extra_pool, sm_scale, stream=None):
        self.check_step(q, q_extra, k_pool, k_extra_pool)
        kps, kts = _row_pool_strides(k_pool)
        xps, xts = _row_pool_strides(k_extra_pool)
        B.paged_mla_decode_partial(q, q_extra, k_pool, k_extra_pool, kps, kts, xps, xts,
                                   self.dim, self.extra_dim, _pd_dtype(q), self.d_indices,
                                   self.d_indptr, self.d_lpl, self.d_fpo, self.d_req,
                                   self.d_tile, self.info.num_chunks, self.info.pages_per_chunk,
                                   self.batch, self.num_qo_heads, self.page_size, sm_scale,
                                   self.v_partial, self.lse_partial, stream)

    def merge(self, stream=None):
        if self.info.needs_merge:
            B.paged_merge_states(self.v_partial, self.lse_partial, self.d_oindptr, self.batch,
                                 self.num_qo_heads, self.dim, self.out, self.lse, stream)

    def run(self, q, q_extra, k_pool, k_extra_pool, sm_scale, stream=None):
        """One decode step: returns (out [B, Hq, dim] fp32, lse [B, Hq] fp32,
        log2 units); the tensors are this object's buffers."""
        self.partial(q, q_extra, k_pool, k_extra_pool, sm_scale, stream)
        self.merge(stream)
        return self.out, self.lse


def graph_time(fn, n: int = 120, per_graph: int = 30, settle_s: float = 0.05) -> float:
    """GPU seconds per call of fn(i): per_graph calls are captured once in a
    HIP graph and the graph is replayed n // per_graph times between events
    on the current stream, so the host's per-launch cost is not counted.  fn
    must launch work only (no allocation, no synchronization).  Before the
    timed replays the graph is replayed, untimed, for settle_s seconds of
    wall time: capture leaves the GPU idle, and a GPU coming out of idle runs
    its first milliseconds of work measurably slower (on MI355X a kernel
    trace of the long-context step showed each of four timed 30-step replays
    faster than the one before without it, 71.2 down to 69.8 us per step)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fn(i)
    torch.cuda.synchronize()
    reps = max(1, n // per_graph)
    t_end = time.time() + settle_s
    while True:
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        if time.time() >= t_end:
            break
    cur = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for _ in range(reps):
        g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * per_graph)


def chunk_candidates(indptr, default_c: int):
    """Pages-per-chunk values worth timing for one batch: the powers of two
    below the longest request's page count, that count itself, and the
    default plan's choice."""
    max_pages = max(1, int(np.max(np.diff(np.asarray(indptr)))))
    cands = {max_pages, default_c}
    c = 1
    while c < max_pages:
        cands.add(c)
        c *= 2
    return sorted(cands)


def _autotune(make, run, indptr, candidates, n):
    """Times run(dec) for make(0) (the device-default plan) and make(c) for
    each candidate c (default: chunk_candidates()); returns (the fastest
    decoder, [{pages_per_chunk, num_chunks, step_us}, ...])."""
    base = make(0)
    if candidates is None:
        candidates = chunk_candidates(indptr, base.info.pages_per_chunk)
    best, table = None, []
    for c in candidates:
        dec = base if c == base.info.pages_per_chunk else make(int(c))
        t = graph_time(lambda i: run(dec), n)
        table.append(dict(pages_per_chunk=dec.info.pages_per_chunk,
                          num_chunks=dec.info.num_chunks, step_us=round(t * 1e6, 2)))
        if best is None or t < best[0]:
            best = (t, dec)
    return best[1], table


def autotune(csr: dict, q, k_pool, v_pool, sm_scale, *, page_size: int, num_pool_pages: int,
             num_qo_heads: int, num_kv_heads: int, head_dim: int, candidates=None,
             n: int = 120, device="cuda"):
    """Chunk-size autotune for one batch on this GPU: times a decode step
    (partial + merge) at each candidate pages-per-chunk -- by default
    chunk_candidates(), i.e. the powers of two within the batch's range plus
    the device-default plan's choice -- and returns (the fastest PagedDecode,
    [{pages_per_chunk, num_chunks, step_us}, ...]).  Every candidate reads
    the given q and pools; the result does not depend on the choice beyond
    rounding (split-KV is exact in real arithmetic)."""
    dtype = q.dtype
    make = lambda c: PagedDecode(  # noqa: E731
        csr, page_size=page_size, num_pool_pages=num_pool_pages, num_qo_heads=num_qo_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, fixed_pages_per_chunk=c, dtype=dtype,
        device=device)
    return _autotune(make, lambda dec: dec.run(q, k_pool, v_pool, sm_scale), csr["indptr"],
                     candidates, n)


def autotune_mla(csr: dict, q, q_extra, k_pool, k_extra_pool, sm_scale, *, page_size: int,
                 num_pool_pages: int, num_qo_heads: int, candidates=None, n: int = 120,
                 device="cuda"):
    """The chunk-size autotune of autotune() for the paged-MLA / DSA decode
    (MlaDecode): returns (the fastest MlaDecode, its table)."""
    make = lambda c: MlaDecode(  # noqa: E731
        csr, page_size=page_size, num_pool_pages=num_pool_pages, num_qo_heads=num_qo_heads,
        fixed_pages_per_chunk=c, device=device)
    return _autotune(make, lambda dec: dec.run(q, q_extra, k_pool, k_extra_pool, sm_scale),
                     csr["indptr"], candidates, n)
