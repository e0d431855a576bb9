"""Thin ctypes binding of libpaged_decode.so (the C-ABI in include/paged_decode.h).

Each function has the C name and only marshals arguments: host arrays are
numpy int32, device buffers are torch tensors (or raw device addresses), the
stream defaults to torch's current stream.  A non-zero status raises
``PagedDecodeError`` carrying the library's message.  The library must be
built (``python -m paged_attention_decode_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PAGED_DECODE_LIB", os.path.join(HERE, "libpaged_decode.so"))

PD_DTYPE_FP16 = 0
PD_DTYPE_FP32 = 1
PD_MAX_CHUNKS = 65535

ERRORS = {
    0: "PD_OK", -1: "PD_E_NULL", -2: "PD_E_ARG", -3: "PD_E_INDPTR", -4: "PD_E_INDEX_RANGE",
    -5: "PD_E_LAST_PAGE_LEN", -6: "PD_E_FIRST_PAGE_OFFSET", -7: "PD_E_GEOMETRY",
    -8: "PD_E_CAPACITY", -9: "PD_E_INFEASIBLE", -10: "PD_E_UNSUPPORTED", -11: "PD_E_HIP",
}
CODES = {v: k for k, v in ERRORS.items()}

EXPORTED = ["pd_last_error", "pd_version", "csr_validate", "paged_csr_build",
            "paged_decode_plan", "paged_decode_partial", "paged_decode_fused",
            "paged_decode_fused_noalloc", "paged_merge_states", "paged_decode_kernel_kind", "paged_decode_set_kernel_choice",
            "paged_cascade_detect", "paged_cascade_split", "paged_cascade_layout",
            "paged_cascade_partial",
            "paged_cascade_stack_q", "paged_cascade_gather_states",
            "paged_cascade_merge_layout", "paged_cascade_merge_states",
            "paged_sparse_csr", "paged_sparse_expand_blocks", "paged_mla_decode_partial",
            "paged_decode_q_heads_per_wg", "paged_decode_default_target_wgs",
            "paged_fastdiv_eval", "paged_hbm_read_probe"]


class PagedDecodeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, message))
        self.code = code
        self.name = ERRORS.get(code, "?")


class PlanInfo(ctypes.Structure):
    _fields_ = [("pages_per_chunk", ctypes.c_int32), ("num_chunks", ctypes.c_int32),
                ("num_wgs", ctypes.c_int32), ("q_groups", ctypes.c_int32),
                ("needs_merge", ctypes.c_int32), ("target_wgs", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]


class CascadeLevel(ctypes.Structure):
    _fields_ = [("indices", ctypes.c_void_p), ("indptr", ctypes.c_void_p),
                ("last_page_len", ctypes.c_void_p), ("first_page_offset", ctypes.c_void_p),
                ("request_indices", ctypes.c_void_p), ("kv_tile_indices", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("num_chunks", ctypes.c_int32),
                ("pages_per_chunk", ctypes.c_int32), ("v_partial", ctypes.c_void_p),
                ("lse_partial", ctypes.c_void_p)]


i32p = ctypes.POINTER(ctypes.c_int32)
u32p = ctypes.POINTER(ctypes.c_uint32)
vp = ctypes.c_void_p
i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float

_SIGS = {
    "pd_last_error": (ctypes.c_char_p, []),
    "pd_version": (ctypes.c_char_p, []),
    "csr_validate": (i32, [i32, i32, i32, i32p, i32p, i32p, i32p, i32p, i32p]),
    "paged_csr_build": (i32, [i32, i32, i32, i32p, i32p, i32p, i32p, i32, i32p, i32p, i32p,
                              i32p, i32p, i32p]),
    "paged_decode_plan": (i32, [i32, i32p, i32, i32, i32, i32, i32, i32, i32, i32, i32p, i32p,
                                i32p, ctypes.POINTER(PlanInfo)]),
    "paged_decode_partial": (i32, [vp, vp, vp, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp,
                                   i32, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp]),
    "paged_decode_fused": (i32, [vp, vp, vp, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp,
                                 i32, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp,
                                 vp]),
    "paged_decode_fused_noalloc": (i32, [vp, vp, vp, i64, i64, i64, i32, vp, vp, vp, vp, vp,
                                         vp, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp,
                                         vp]),
    "paged_merge_states": (i32, [vp, vp, vp, i32, i32, i32, vp, vp, vp]),
    "paged_mla_decode_partial": (i32, [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, vp,
                                       vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp,
                                       vp]),
    "paged_decode_kernel_kind": (i32, [i32, i32, i32, i32, i64]),
    "paged_decode_set_kernel_choice": (i32, [i32]),
    "paged_cascade_detect": (i32, [i32, i32p, i32p, i32p, i32, i32, i32p, i32p, i32p]),
    "paged_cascade_split": (i32, [i32, i32, i32p, i32p, i32p, i32p, i32p, i32, i32, i32p, i32p,
                                  i32p, i32p, i32p]),
    "paged_cascade_layout": (i32, [i32, i32p, i32, i32, i32p, i32p, i32p, i32p]),
    "paged_cascade_stack_q": (i32, [vp, i32, vp, i32, i32, i32, i32, vp, vp]),
    "paged_cascade_partial": (i32, [vp, i32, vp, i32, i32, vp, vp, i64, i64, i64, i32, i32, i32,
                                    i32, i32, f32, ctypes.POINTER(CascadeLevel),
                                    ctypes.POINTER(CascadeLevel), i32, vp]),
    "paged_cascade_gather_states": (i32, [vp, vp, i32, i32, vp, vp, vp, i32, vp, i32, i32, i32,
                                          vp, vp, vp]),
    "paged_cascade_merge_layout": (i32, [i32, i32p, i32, i32, i32, i32, i32p]),
    "paged_cascade_merge_states": (i32, [vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, vp,
                                         vp, vp]),
    "paged_sparse_csr": (i32, [i32, i32, i32, i32, i32p, i32p, i32p, i32p]),
    "paged_sparse_expand_blocks": (i32, [vp, i32, i32, vp, i32, vp, vp, i32, vp, vp]),
    "paged_decode_q_heads_per_wg": (i32, [i32, i32, i32]),
    "paged_decode_default_target_wgs": (i32, [i32, i32, i32, i32, i32]),
    "paged_fastdiv_eval": (i32, [i32, u32p, i64, u32p, u32p]),
    "paged_hbm_read_probe": (i32, [vp, i64, i32, i32, vp, vp]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError("libpaged_decode.so is not built (run "
                               "`python -m paged_attention_decode_amd.build`); there is no "
                               "fallback path")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != 0:
        msg = load().pd_last_error().decode()
        raise PagedDecodeError(rc, msg)
    return rc


def _host_i32(a) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a


def _hp(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(i32p)


def _dev(x) -> Optional[int]:
    """Device address of a torch tensor (or an int address, or None).  A
    tensor that is not in GPU memory is refused: the kernels would read its
    host address as a device address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise ValueError("paged_decode: kernel arguments must be GPU tensors (got %s on %s)"
                         % (type(x).__name__, getattr(x, "device", "host")))
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def version() -> str:
    return load().pd_version().decode()


def csr_validate(batch, page_size, num_pool_pages, indptr, indices, last_page_len,
                 first_page_offset, seq_lens=None, raise_on_error=True):
    """Returns (status, bad_request); raises PagedDecodeError by default."""
    lib = load()
    ip, ix = _host_i32(indptr), _host_i32(indices)
    lp, fo = _host_i32(last_page_len), _host_i32(first_page_offset)
    sl = None if seq_lens is None else _host_i32(seq_lens)
    if ix.size == 0:
        ix = np.zeros(1, np.int32)
    bad = ctypes.c_int32(-2)
    rc = lib.csr_validate(batch, page_size, num_pool_pages, _hp(ip), _hp(ix), _hp(lp), _hp(fo),
                          _hp(sl), ctypes.byref(bad))
    if raise_on_error:
        _check(rc)
    return rc, bad.value


def paged_csr_build(block_tables, logical_start, written_len, page_size, num_pool_pages):
    """Block tables (list of int32 arrays, -1 = released) -> CSR dict."""
    lib = load()
    b = len(block_tables)
    off = np.zeros(b + 1, np.int32)
    for r, t in enumerate(block_tables):
        off[r + 1] = off[r] + len(t)
    bt = _host_i32(np.concatenate([np.asarray(t, np.int32) for t in block_tables])
                   if off[-1] else np.zeros(1, np.int32))
    ls, wl = _host_i32(logical_start), _host_i32(written_len)
    cap = max(1, int(off[-1]))
    indptr = np.zeros(b + 1, np.int32)
    indices = np.zeros(cap, np.int32)
    lpl, fpo, sl, ro = (np.zeros(b, np.int32) for _ in range(4))
    _check(lib.paged_csr_build(b, page_size, num_pool_pages, _hp(off), _hp(bt), _hp(ls),
                               _hp(wl), cap, _hp(indptr), _hp(indices), _hp(lpl), _hp(fpo),
                               _hp(sl), _hp(ro)))
    return dict(indptr=indptr, indices=indices[:indptr[-1]].copy(), last_page_len=lpl,
                first_page_offset=fpo, seq_lens=sl, rope_offsets=ro)


def paged_decode_plan(indptr, num_qo_heads, num_kv_heads, head_dim, target_wgs=0,
                      fixed_pages_per_chunk=0, sizes_only=False, dtype=PD_DTYPE_FP16,
                      page_size=16):
    """Returns (info: PlanInfo, request_indices, kv_tile_indices, o_indptr).
    page_size only matters for the device-default target (target_wgs <= 0)."""
    lib = load()
    ip = _host_i32(indptr)
    b = ip.size - 1
    info = PlanInfo()
    oi = np.zeros(b + 1, np.int32)
    _check(lib.paged_decode_plan(b, _hp(ip), num_qo_heads, num_kv_heads, head_dim, dtype,
                                 page_size, target_wgs, fixed_pages_per_chunk, 0, None, None,
                                 _hp(oi), ctypes.byref(info)))
    if sizes_only:
        return info, None, None, oi
    cap = max(1, info.num_chunks)
    ri = np.zeros(cap, np.int32)
    ti = np.zeros(cap, np.int32)
    _check(lib.paged_decode_plan(b, _hp(ip), num_qo_heads, num_kv_heads, head_dim, dtype,
                                 page_size, target_wgs, fixed_pages_per_chunk, cap, _hp(ri),
                                 _hp(ti), _hp(oi), ctypes.byref(info)))
    return info, ri[:info.num_chunks], ti[:info.num_chunks], oi


def paged_decode_partial(q, k_pool, v_pool, page_stride, token_stride, head_stride, dtype,
                         indices, indptr, last_page_len, first_page_offset, request_indices,
                         kv_tile_indices, num_chunks, pages_per_chunk, batch, num_qo_heads,
                         num_kv_heads, head_dim, page_size, sm_scale, v_partial, lse_partial,
                         stream=None):
    lib = load()
    _check(lib.paged_decode_partial(
        _dev(q), _dev(k_pool), _dev(v_pool), page_stride, token_stride, head_stride, dtype,
        _dev(indices), _dev(indptr), _dev(last_page_len), _dev(first_page_offset),
        _dev(request_indices), _dev(kv_tile_indices), num_chunks, pages_per_chunk, batch,
        num_qo_heads, num_kv_heads, head_dim, page_size, float(sm_scale), _dev(v_partial),
        _dev(lse_partial), _stream(stream)))


def paged_mla_decode_partial(q, q_extra, k_pool, k_extra_pool, k_page_stride, k_token_stride,
                             x_page_stride, x_token_stride, dim, extra_dim, dtype, indices,
                             indptr, last_page_len, first_page_offset, request_indices,
                             kv_tile_indices, num_chunks, pages_per_chunk, batch, num_qo_heads,
                             page_size, sm_scale, v_partial, lse_partial, stream=None):
    lib = load()
    _check(lib.paged_mla_decode_partial(
        _dev(q), _dev(q_extra), _dev(k_pool), _dev(k_extra_pool), k_page_stride, k_token_stride,
        x_page_stride, x_token_stride, dim, extra_dim, dtype, _dev(indices), _dev(indptr),
        _dev(last_page_len), _dev(first_page_offset), _dev(request_indices),
        _dev(kv_tile_indices), num_chunks, pages_per_chunk, batch, num_qo_heads, page_size,
        float(sm_scale), _dev(v_partial), _dev(lse_partial), _stream(stream)))


def paged_decode_fused(q, k_pool, v_pool, page_stride, token_stride, head_stride, dtype,
                       indices, indptr, last_page_len, first_page_offset, request_indices,
                       kv_tile_indices, num_chunks, pages_per_chunk, batch, num_qo_heads,
                       num_kv_heads, head_dim, page_size, sm_scale, v_partial, lse_partial,
                       counters, out, lse_out, stream=None):
    lib = load()
    _check(lib.paged_decode_fused(
        _dev(q), _dev(k_pool), _dev(v_pool), page_stride, token_stride, head_stride, dtype,
        _dev(indices), _dev(indptr), _dev(last_page_len), _dev(first_page_offset),
        _dev(request_indices), _dev(kv_tile_indices), num_chunks, pages_per_chunk, batch,
        num_qo_heads, num_kv_heads, head_dim, page_size, float(sm_scale), _dev(v_partial),
        _dev(lse_partial), _dev(counters), _dev(out), _dev(lse_out), _stream(stream)))


def paged_decode_fused_noalloc(q, k_pool, v_pool, page_stride, token_stride, head_stride,
                               dtype, indices, indptr, last_page_len, first_page_offset,
                               request_indices, kv_tile_indices, num_chunks, pages_per_chunk,
                               batch, num_qo_heads, num_kv_heads, head_dim, page_size, sm_scale,
                               out, lse_out, stream=None):
    lib = load()
    _check(lib.paged_decode_fused_noalloc(
        _dev(q), _dev(k_pool), _dev(v_pool), page_stride, token_stride, head_stride, dtype,
        _dev(indices), _dev(indptr), _dev(last_page_len), _dev(first_page_offset),
        _dev(request_indices), _dev(kv_tile_indices), num_chunks, pages_per_chunk, batch,
        num_qo_heads, num_kv_heads, head_dim, page_size, float(sm_scale), _dev(out),
        _dev(lse_out), _stream(stream)))


def paged_decode_kernel_kind(dtype, head_dim, group_size, page_size, token_stride):
    return _check_nonneg(load().paged_decode_kernel_kind(dtype, head_dim, group_size, page_size,
                                                         token_stride))


def paged_decode_set_kernel_choice(choice):
    """0 (or False): default choice; 1 (or True): every shape on the token
    kernel; 2: no MFMA kernel (VALU page or token kernel)."""
    _check(load().paged_decode_set_kernel_choice(int(choice)))


def paged_merge_states(v_in, lse_in, o_indptr, num_out_rows, num_heads, head_dim, v_out,
                       lse_out, stream=None):
    lib = load()
    _check(lib.paged_merge_states(_dev(v_in), _dev(lse_in), _dev(o_indptr), num_out_rows,
                                  num_heads, head_dim, _dev(v_out), _dev(lse_out),
                                  _stream(stream)))


def paged_cascade_detect(indptr, indices, first_page_offset, min_shared_pages=16,
                         min_members=2):
    """Returns (member_req int32 array, shared_pages); empty / 0 if nothing
    qualifies."""
    indptr = _host_i32(indptr)
    batch = indptr.size - 1
    indices = _host_i32(indices if np.asarray(indices).size else np.zeros(1, np.int32))
    fpo = _host_i32(first_page_offset)
    members = np.zeros(max(1, batch), np.int32)
    nm, sp = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().paged_cascade_detect(batch, _hp(indptr), _hp(indices), _hp(fpo),
                                       min_shared_pages, min_members, _hp(members),
                                       ctypes.byref(nm), ctypes.byref(sp)))
    return members[:nm.value].copy(), sp.value


def paged_cascade_split(page_size, indptr, indices, last_page_len, first_page_offset,
                        member_req, shared_pages):
    """Returns (indices0, csr1) with csr1 a dict of the level-1 page table."""
    indptr = _host_i32(indptr)
    batch = indptr.size - 1
    indices = _host_i32(indices)
    member_req = _host_i32(member_req)
    nnz1 = int(indptr[-1]) - member_req.size * shared_pages
    indices0 = np.zeros(max(1, shared_pages), np.int32)
    indptr1 = np.zeros(batch + 1, np.int32)
    indices1 = np.zeros(max(1, nnz1), np.int32)
    lpl1 = np.zeros(batch, np.int32)
    fpo1 = np.zeros(batch, np.int32)
    _check(load().paged_cascade_split(batch, page_size, _hp(indptr), _hp(indices),
                                      _hp(_host_i32(last_page_len)),
                                      _hp(_host_i32(first_page_offset)), _hp(member_req),
                                      member_req.size, shared_pages, _hp(indices0), _hp(indptr1),
                                      _hp(indices1), _hp(lpl1), _hp(fpo1)))
    return indices0[:shared_pages].copy(), dict(indptr=indptr1, indices=indices1[:max(0, nnz1)],
                                                last_page_len=lpl1, first_page_offset=fpo1)


def paged_cascade_layout(member_req, level0_rows, o_indptr1):
    """Returns (dst0, dst1, o_indptr) of the cascade merge input."""
    member_req = _host_i32(member_req)
    o1 = _host_i32(o_indptr1)
    batch = o1.size - 1
    dst0 = np.zeros(max(1, member_req.size), np.int32)
    dst1 = np.zeros(max(1, int(o1[-1])), np.int32)
    oi = np.zeros(batch + 1, np.int32)
    _check(load().paged_cascade_layout(batch, _hp(member_req), member_req.size, level0_rows,
                                       _hp(o1), _hp(dst0), _hp(dst1), _hp(oi)))
    return dst0[:member_req.size].copy(), dst1[:int(o1[-1])].copy(), oi


def paged_cascade_stack_q(q, dtype, member_req, members, num_qo_heads, num_kv_heads, head_dim,
                          q0, stream=None):
    _check(load().paged_cascade_stack_q(_dev(q), dtype, _dev(member_req), members, num_qo_heads,
                                        num_kv_heads, head_dim, _dev(q0), _stream(stream)))


def cascade_level(indices, indptr, last_page_len, first_page_offset, request_indices,
                  kv_tile_indices, batch, num_chunks, pages_per_chunk, v_partial, lse_partial):
    """A paged_cascade_level struct of device addresses (the tensors must
    outlive every call that uses it)."""
    return CascadeLevel(_dev(indices), _dev(indptr), _dev(last_page_len),
                        _dev(first_page_offset), _dev(request_indices), _dev(kv_tile_indices),
                        batch, num_chunks, pages_per_chunk, _dev(v_partial), _dev(lse_partial))


def cascade_levels(levels):
    """A ctypes array of paged_cascade_level structs (level 0's tables)."""
    return (CascadeLevel * len(levels))(*levels)


def paged_cascade_partial(q, batch, member_req, members, members_per_launch, k_pool, v_pool,
                          page_stride, token_stride, head_stride, dtype, num_qo_heads,
                          num_kv_heads, head_dim, page_size, sm_scale, level0, level1=None,
                          heads_per_workgroup=0, stream=None):
    """level0: the array from cascade_levels(); level1: a CascadeLevel or None."""
    _check(load().paged_cascade_partial(
        _dev(q), batch, _dev(member_req), members, members_per_launch, _dev(k_pool),
        _dev(v_pool), page_stride, token_stride, head_stride, dtype, num_qo_heads, num_kv_heads,
        head_dim, page_size, float(sm_scale), level0,
        ctypes.byref(level1) if level1 is not None else None, int(heads_per_workgroup),
        _stream(stream)))


def paged_cascade_gather_states(v0, lse0, n0, members, dst0, v1, lse1, n1, dst1, num_qo_heads,
                                num_kv_heads, head_dim, v_dst, lse_dst, stream=None):
    _check(load().paged_cascade_gather_states(_dev(v0), _dev(lse0), n0, members, _dev(dst0),
                                              _dev(v1), _dev(lse1), n1, _dev(dst1),
                                              num_qo_heads, num_kv_heads, head_dim, _dev(v_dst),
                                              _dev(lse_dst), _stream(stream)))


def paged_cascade_merge_layout(batch, member_req, members_per_launch, level0_rows,
                               num_qo_heads):
    """Returns l0_desc [batch, 3] int32: (first level-0 row of the request's
    launch, members stacked in it, position in it; -1 for a non-member)."""
    member_req = _host_i32(member_req)
    desc = np.zeros((batch, 3), np.int32)
    _check(load().paged_cascade_merge_layout(batch, _hp(member_req), member_req.size,
                                             members_per_launch, level0_rows, num_qo_heads,
                                             _hp(desc)))
    return desc


def paged_cascade_merge_states(v0, lse0, n0, l0_desc, v1, lse1, o_indptr1, batch,
                               num_qo_heads, num_kv_heads, head_dim, v_out, lse_out,
                               stream=None):
    _check(load().paged_cascade_merge_states(_dev(v0), _dev(lse0), n0, _dev(l0_desc), _dev(v1),
                                             _dev(lse1), _dev(o_indptr1), batch, num_qo_heads,
                                             num_kv_heads, head_dim, _dev(v_out), _dev(lse_out),
                                             _stream(stream)))


def paged_sparse_csr(blocks_per_request, block_size, tail, page_size):
    """Returns dict(indptr, last_page_len, first_page_offset) of a selection's
    page table in pages of page_size rows (host arrays)."""
    tail = _host_i32(tail)
    r = tail.size
    indptr = np.zeros(r + 1, np.int32)
    lpl = np.zeros(r, np.int32)
    fpo = np.zeros(r, np.int32)
    _check(load().paged_sparse_csr(r, blocks_per_request, block_size, page_size,
                                   _hp(tail), _hp(indptr), _hp(lpl), _hp(fpo)))
    return dict(indptr=indptr, last_page_len=lpl, first_page_offset=fpo)


def paged_sparse_expand_blocks(block_ids, num_requests, blocks_per_request, base, span,
                               final_rows, out_indptr, num_blocks, rows, stream=None):
    _check(load().paged_sparse_expand_blocks(_dev(block_ids), num_requests, blocks_per_request,
                                             _dev(base), span, _dev(final_rows), _dev(out_indptr),
                                             num_blocks, _dev(rows), _stream(stream)))


def paged_decode_q_heads_per_wg(group_size, head_dim, dtype):
    return _check_nonneg(load().paged_decode_q_heads_per_wg(group_size, head_dim, dtype))


def paged_decode_default_target_wgs(device, group_size, head_dim, dtype, num_kv_heads=1):
    return _check_nonneg(load().paged_decode_default_target_wgs(device, group_size, head_dim,
                                                                dtype, num_kv_heads))


def _check_nonneg(v):
    if v < 0:
        _check(v)
    return v


def paged_fastdiv_eval(d, n):
    n = np.ascontiguousarray(np.asarray(n, dtype=np.uint32))
    q = np.zeros_like(n)
    r = np.zeros_like(n)
    _check(load().paged_fastdiv_eval(d, n.ctypes.data_as(u32p), n.size, q.ctypes.data_as(u32p),
                                     r.ctypes.data_as(u32p)))
    return q, r


def paged_hbm_read_probe(buf, nbytes, num_wgs, sink, nontemporal=True, stream=None):
    """One read pass over nbytes of the device tensor buf (measurement)."""
    _check(load().paged_hbm_read_probe(_dev(buf), int(nbytes), int(num_wgs), int(nontemporal),
                                       _dev(sink), _stream(stream)))
