"""Thin ctypes binding over libddt.so (include/ddt.h).

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch CUDA tensors (torch supplies device memory and the
current stream); host-side arrays (prefix lengths for planning) are numpy
arrays or lists.  Outputs that are not passed in are allocated with torch.
The library must be built (``python -m mla_tree_verify_parents_amd.build``);
loading fails loudly otherwise -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from .build import LIB

DDT_F32, DDT_BF16 = 0, 1
DDT_OK, DDT_EINVAL, DDT_EUNSUPPORTED, DDT_EWORKSPACE, DDT_EHIP = 0, -1, -2, -3, -4
MAX_NODES = 1024
MAX_BATCH = 128

_lib = None


class DdtError(RuntimeError):
    pass


class AttnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int),
                ("d_lat", ctypes.c_int), ("d_rope", ctypes.c_int), ("dtype", ctypes.c_int),
                ("scale", ctypes.c_float), ("kv_chunk", ctypes.c_int),
                ("ld_ql", ctypes.c_int64), ("ld_qp", ctypes.c_int64),
                ("ld_ckv", ctypes.c_int64), ("ld_kpe", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("bt_ld", ctypes.c_int64), ("page_size", ctypes.c_int),
                ("prefix_len_dev", ctypes.c_void_p)]


class ArgmaxTask(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("dtype", ctypes.c_int), ("rows", ctypes.c_int64),
                ("V", ctypes.c_int64), ("ld", ctypes.c_int64), ("idx", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class AcceptTask(ctypes.Structure):
    _fields_ = [("draft_ids", ctypes.c_void_p), ("parents", ctypes.c_void_p), ("accept_len", ctypes.c_void_p),
                ("path", ctypes.c_void_p), ("tokens", ctypes.c_void_p), ("prefix_len", ctypes.c_void_p),
                ("new_prefix_len", ctypes.c_void_p), ("src_slot", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise DdtError(f"{LIB} is not built; run `python -m mla_tree_verify_parents_amd.build`")
        L = ctypes.CDLL(LIB)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.ddt_version.argtypes = []
        L.ddt_status_string.argtypes = [i32]
        L.ddt_status_string.restype = ctypes.c_char_p
        L.ddt_build_mask.argtypes = [P, i32, i32, P, P, P, P]
        L.ddt_verify_workspace.argtypes = [ctypes.POINTER(AttnDesc), P, ctypes.POINTER(sz)]
        L.ddt_verify_plan.argtypes = [ctypes.POINTER(AttnDesc), P, ctypes.POINTER(i32), ctypes.POINTER(i32), P, P, i32,
                                      ctypes.POINTER(i32)]
        L.ddt_verify_attn.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P, P, sz, P]
        L.ddt_verify_attn_noalloc.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P, P]
        L.ddt_verify_noalloc_scratch_bytes.argtypes = []
        L.ddt_verify_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.ddt_argmax_workspace.argtypes = [i64, i64, ctypes.POINTER(sz)]
        L.ddt_argmax.argtypes = [P, i32, i64, i64, i64, P, P, sz, P]
        L.ddt_greedy_accept.argtypes = [P, P, P, i32, i32, P, P, P, P]
        L.ddt_compact_kv.argtypes = [P, i64, P, i64, i32, i32, i32, P, P, P, P, i32, i32, P, P]
        L.ddt_compact_kv_paged.argtypes = [P, i64, P, i64, i32, i32, i32, P, i64, i32, P, P, P, i32, i32, P, P]
        L.ddt_accept_compact.argtypes = [P, P, P, i32, i32, P, P, P, P, i64, P, i64, i32, i32, i32, P, P, P, P, P]
        L.ddt_accept_compact_paged.argtypes = [P, P, P, i32, i32, P, P, P, P, i64, P, i64, i32, i32, i32, P, i64, i32,
                                               P, P, P, P]
        L.ddt_verify_attn_argmax.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P, P, sz,
                                             ctypes.POINTER(ArgmaxTask), P]
        L.ddt_verify_step.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P, P, sz,
                                      ctypes.POINTER(ArgmaxTask), ctypes.POINTER(AcceptTask), P]
        L.ddt_draft_topk_workspace.argtypes = [i64, i64, i32, ctypes.POINTER(sz)]
        L.ddt_draft_topk.argtypes = [P, i64, i64, i64, i32, P, P, P, sz, P]
        L.ddt_best_first_tree.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P, P]
        L.ddt_proj_pack_weight.argtypes = [P, i32, i32, i32, i32, P, P]
        L.ddt_head_proj.argtypes = [P, i64, P, i32, i32, i32, i32, i32, P, i64, P]
        L.ddt_probe_mfma_bf16.argtypes = [P, P, P, i32, i32, P]
        L.ddt_probe_read.argtypes = [P, sz, P, i32, P]
        L.ddt_probe_copy.argtypes = [P, P, sz, i32, P]
        for f in ("ddt_version", "ddt_build_mask", "ddt_verify_workspace", "ddt_verify_plan", "ddt_verify_attn",
                  "ddt_verify_attn_noalloc",
                  "ddt_argmax_workspace", "ddt_argmax", "ddt_greedy_accept", "ddt_compact_kv", "ddt_compact_kv_paged",
                  "ddt_accept_compact", "ddt_accept_compact_paged", "ddt_verify_attn_argmax", "ddt_verify_step",
                  "ddt_draft_topk_workspace", "ddt_draft_topk", "ddt_best_first_tree",
                  "ddt_proj_pack_weight", "ddt_head_proj",
                  "ddt_probe_mfma_bf16", "ddt_probe_read", "ddt_probe_copy"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        raise DdtError(f"{what}: {lib().ddt_status_string(rc).decode()} ({rc})")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _contig(t, dtype, name):
    _dev(t, dtype, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _holds(t, n, name):
    """A contiguous tensor the library reads or writes n consecutive elements of."""
    if t.numel() < n:
        raise ValueError(f"{name} must hold at least {n} elements, got {t.numel()}")
    return t


def _src_slot(src_slot, B, N):
    """The optional [B, N] int32 src_slot output: the library writes B*N entries."""
    if src_slot is not None:
        _contig(src_slot, torch.int32, "src_slot")
        if tuple(src_slot.shape) != (B, N):
            raise ValueError(f"src_slot must be [B, N] = [{B}, {N}], got {tuple(src_slot.shape)}")
    return src_slot


def _rows(t, name):
    """2-D view with unit column stride -> row stride in elements."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D view with unit column stride")
    return t.stride(0)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return DDT_F32
    if t.dtype == torch.bfloat16:
        return DDT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def build_mask(parents, mask=None, depth=None, tree_err=None, stream=None):
    """parents [B, N] int32 -> (mask [B, N, W] int64 bit words, depth [B, N], tree_err [B])."""
    _contig(parents, torch.int32, "parents")
    if parents.dim() != 2:
        raise ValueError("parents must be [B, N]")
    B, N = parents.shape
    W = (N + 63) // 64
    dev = parents.device
    if mask is None:
        mask = torch.empty((B, N, W), dtype=torch.int64, device=dev)
    if depth is None:
        depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    if tree_err is None:
        tree_err = torch.empty((B,), dtype=torch.int32, device=dev)
    _holds(_contig(mask, torch.int64, "mask"), B * N * W, "mask")
    _holds(_contig(depth, torch.int32, "depth"), B * N, "depth")
    _holds(_contig(tree_err, torch.int32, "tree_err"), B, "tree_err")
    _check(lib().ddt_build_mask(_p(parents), B, N, _p(mask), _p(depth), _p(tree_err), _stream(stream)),
           "ddt_build_mask")
    return mask, depth, tree_err


def attn_desc(q_lat, q_pe, ckv, kpe, *, B, H, N, scale, kv_chunk=0, pages=None, prefix_len_dev=None):
    """pages: None (contiguous cache from kv_base) or (block_table [B, bt_ld]
    int32 device, page_size): slot t of request b is pool row
    block_table[b, t // page_size] * page_size + t % page_size.
    prefix_len_dev: None, or [B] int32 device committed lengths read by the
    kernels when they run; the host lengths are then upper bounds."""
    d = AttnDesc(B, H, N, q_lat.shape[1], q_pe.shape[1], _dtype_code(q_lat), float(scale), int(kv_chunk),
                 _rows(q_lat, "q_lat"), _rows(q_pe, "q_pe"), _rows(ckv, "ckv"), _rows(kpe, "kpe"))
    if pages is not None:
        table, page_size = pages
        _contig(table, torch.int32, "block_table")
        if table.dim() != 2 or table.shape[0] != B:
            raise ValueError("block_table must be [B, bt_ld]")
        d.block_table, d.bt_ld, d.page_size = table.data_ptr(), table.shape[1], int(page_size)
    if prefix_len_dev is not None:
        _contig(prefix_len_dev, torch.int32, "prefix_len_dev")
        if tuple(prefix_len_dev.shape) != (B,):
            raise ValueError("prefix_len_dev must be [B]")
        d.prefix_len_dev = prefix_len_dev.data_ptr()
    return d


def _host_lengths(prefix_len_host, B: int) -> np.ndarray:
    """The [B] host committed lengths (or their bounds) as the library reads
    them: int32, one per request (the library reads exactly B entries)."""
    a = np.asarray(prefix_len_host)
    if a.shape != (B,):
        raise ValueError(f"prefix_len_host must have B = {B} entries, got shape {a.shape}")
    if a.size and (a.min() < np.iinfo(np.int32).min or a.max() > np.iinfo(np.int32).max):
        raise ValueError("prefix_len_host values must fit int32")
    return np.ascontiguousarray(a, dtype=np.int32)


def verify_workspace_bytes(desc: AttnDesc, prefix_len_host) -> int:
    pl = _host_lengths(prefix_len_host, desc.B)
    n = ctypes.c_size_t(0)
    _check(lib().ddt_verify_workspace(ctypes.byref(desc), pl.ctypes.data, ctypes.byref(n)),
           "ddt_verify_workspace")
    return n.value


def verify_plan(desc: AttnDesc, prefix_len_host):
    """ddt_verify_plan: (n_blocks, chunk, nsplit [B], items [n_items, 6]) of
    the attention launch for this shape and these host lengths; an item is
    (workgroup, request, split, row tile, first key, end key)."""
    pl = _host_lengths(prefix_len_host, desc.B)
    nb, ch, ni = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    nsplit = np.zeros(desc.B, np.int32)
    _check(lib().ddt_verify_plan(ctypes.byref(desc), pl.ctypes.data, ctypes.byref(nb), ctypes.byref(ch),
                                 nsplit.ctypes.data, None, 0, ctypes.byref(ni)), "ddt_verify_plan")
    items = np.zeros((max(ni.value, 1), 6), np.int32)
    _check(lib().ddt_verify_plan(ctypes.byref(desc), pl.ctypes.data, ctypes.byref(nb), ctypes.byref(ch),
                                 nsplit.ctypes.data, items.ctypes.data, items.shape[0], ctypes.byref(ni)),
           "ddt_verify_plan")
    return nb.value, ch.value, nsplit, items[:ni.value]


def _attn_args(q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, H, scale, out, lse, workspace, kv_chunk,
               BN=None, pages=None, alloc_workspace=True, prefix_len_dev=None):
    for t, n in ((q_lat, "q_lat"), (q_pe, "q_pe"), (ckv, "ckv"), (kpe, "kpe")):
        _dev(t, q_lat.dtype, n)
    if pages is None or kv_base is not None:
        _contig(kv_base, torch.int64, "kv_base")
    if mask is None:  # (B, N) given instead: the kernel derives the ancestor bits
        B, N = BN
    else:
        _contig(mask, torch.int64, "mask")
        if mask.dim() != 3 or mask.shape[2] != (mask.shape[1] + 63) // 64:
            raise ValueError("mask must be [B, N, ceil(N/64)] (from build_mask)")
        B, N = mask.shape[0], mask.shape[1]
    if kv_base is not None:
        _holds(kv_base, B, "kv_base")
    rows = B * N * H
    if q_lat.shape[0] != rows or q_pe.shape[0] != rows:
        raise ValueError("q rows must be B*N*H")
    pl = _host_lengths(prefix_len_host, B)
    desc = attn_desc(q_lat, q_pe, ckv, kpe, B=B, H=H, N=N, scale=scale, kv_chunk=kv_chunk, pages=pages,
                     prefix_len_dev=prefix_len_dev)
    if out is None:
        out = torch.empty((rows, q_lat.shape[1]), dtype=q_lat.dtype, device=q_lat.device)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=q_lat.device)
    _holds(_contig(out, q_lat.dtype, "out"), rows * q_lat.shape[1], "out")
    _holds(_contig(lse, torch.float32, "lse"), rows, "lse")
    if workspace is None and alloc_workspace:  # (a caller's workspace is checked by the library)
        need = verify_workspace_bytes(desc, pl)
        if need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=q_lat.device)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return desc, pl, out, lse, workspace, ws_n


def verify_attn(q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, *, H, scale, out=None, lse=None,
                workspace=None, kv_chunk=0, pages=None, prefix_len_dev=None, stream=None):
    """Tree-verify attention.  q_lat [B*N*H, d_lat], q_pe [B*N*H, d_rope] (2-D views),
    ckv [pool, d_lat], kpe [pool, d_rope] (2-D views of the cache pool), kv_base [B]
    int64 (device; may be None with pages), prefix_len_host [B] (host), mask [B, N, W]
    from build_mask; pages and prefix_len_dev as for attn_desc.
    Returns (out [B*N*H, d_lat], lse [B*N*H] fp32)."""
    desc, pl, out, lse, workspace, ws_n = _attn_args(q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, H,
                                                     scale, out, lse, workspace, kv_chunk, pages=pages,
                                                     prefix_len_dev=prefix_len_dev)
    _check(lib().ddt_verify_attn(ctypes.byref(desc), _p(q_lat), _p(q_pe), _p(ckv), _p(kpe), _p(kv_base),
                                 pl.ctypes.data, _p(mask), _p(out), _p(lse), _p(workspace), ws_n,
                                 _stream(stream)), "ddt_verify_attn")
    return out, lse


def verify_attn_noalloc(q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, *, H, scale, out, lse, kv_chunk=0,
                        pages=None, prefix_len_dev=None, stream=None):
    """verify_attn without a workspace and without allocating: the library
    keeps the split partials in its own per-device scratch
    (noalloc_scratch_bytes()); out and lse must be given.  Calls on one
    device share that scratch and must not overlap."""
    if out is None or lse is None:
        raise ValueError("verify_attn_noalloc allocates nothing: pass out and lse")
    desc, pl, out, lse, _, _ = _attn_args(q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, H, scale, out, lse,
                                          None, kv_chunk, pages=pages, alloc_workspace=False,
                                          prefix_len_dev=prefix_len_dev)
    _check(lib().ddt_verify_attn_noalloc(ctypes.byref(desc), _p(q_lat), _p(q_pe), _p(ckv), _p(kpe), _p(kv_base),
                                         pl.ctypes.data, _p(mask), _p(out), _p(lse), _stream(stream)),
           "ddt_verify_attn_noalloc")
    return out, lse


def noalloc_scratch_bytes() -> int:
    return int(lib().ddt_verify_noalloc_scratch_bytes())


def _argmax_task(logits, idx, argmax_workspace):
    _dev(logits, None, "logits")
    ld = _rows(logits, "logits")
    rows, V = logits.shape
    if idx is None:
        idx = torch.empty((rows,), dtype=torch.int32, device=logits.device)
    _holds(_contig(idx, torch.int32, "idx"), rows, "idx")
    need = argmax_workspace_bytes(rows, V)
    if argmax_workspace is None and need > 0:
        argmax_workspace = torch.zeros((need,), dtype=torch.uint8, device=logits.device)  # zero before first use
    am_n = 0 if argmax_workspace is None else argmax_workspace.numel() * argmax_workspace.element_size()
    return ArgmaxTask(_p(logits), _dtype_code(logits), rows, V, ld, _p(idx), _p(argmax_workspace), am_n), idx


def verify_attn_argmax(q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, logits, *, H, scale, out=None,
                       lse=None, workspace=None, idx=None, argmax_workspace=None, kv_chunk=0, pages=None,
                       prefix_len_dev=None, stream=None):
    """verify_attn and argmax(logits) in one launch -> (out, lse, idx)."""
    desc, pl, out, lse, workspace, ws_n = _attn_args(q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, H,
                                                     scale, out, lse, workspace, kv_chunk, pages=pages,
                                                     prefix_len_dev=prefix_len_dev)
    task, idx = _argmax_task(logits, idx, argmax_workspace)
    _check(lib().ddt_verify_attn_argmax(ctypes.byref(desc), _p(q_lat), _p(q_pe), _p(ckv), _p(kpe), _p(kv_base),
                                        pl.ctypes.data, _p(mask), _p(out), _p(lse), _p(workspace), ws_n,
                                        ctypes.byref(task), _stream(stream)), "ddt_verify_attn_argmax")
    return out, lse, idx


def _accept_outputs(parents, accept_len, path, tokens):
    B, N = parents.shape
    dev = parents.device
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if path is None:
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    for t, n in ((accept_len, "accept_len"), (path, "path"), (tokens, "tokens")):
        _contig(t, torch.int32, n)
    _holds(accept_len, B, "accept_len")
    for t, n in ((path, "path"), (tokens, "tokens")):
        if tuple(t.shape) != (B, N):
            raise ValueError(f"{n} must be [B, N] = [{B}, {N}], got {tuple(t.shape)}")
    return accept_len, path, tokens


def _tree_inputs(parents, named):
    """parents [B, N] int32 and per-node int32 inputs of B*N entries each."""
    _contig(parents, torch.int32, "parents")
    if parents.dim() != 2:
        raise ValueError("parents must be [B, N]")
    B, N = parents.shape
    for t, n in named:
        _contig(t, torch.int32, n)
        if t.numel() != B * N:
            raise ValueError(f"{n} must hold B*N = {B * N} entries (one per tree node), got {t.numel()}")
    return B, N


def verify_step(q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, logits, draft_ids, parents, prefix_len, *,
                H, scale, new_prefix_len=None, out=None, lse=None, workspace=None, idx=None, argmax_workspace=None,
                accept_len=None, path=None, tokens=None, src_slot=None, kv_chunk=0, pages=None,
                device_lengths=False, stream=None):
    """Attention + argmax, then acceptance + compaction, in two launches.

    mask: from build_mask, or None for trees of at most 128 nodes (the
    attention then derives each row's ancestor bits from parents itself);
    logits [B*N, V] (one target row per tree node); draft_ids, parents [B, N]
    int32; prefix_len [B] int32 device (same values as prefix_len_host);
    new_prefix_len [B] int32 device receives the advanced lengths (default:
    prefix_len itself, updated in place).  The cache views ckv / kpe are
    compacted in place (through the block table with pages).
    device_lengths: the attention reads the committed lengths from
    prefix_len on the device, and prefix_len_host holds upper bounds of them
    (so steps can be enqueued or captured without reading lengths back).
    -> (out, lse, idx, accept_len, path, tokens, new_prefix_len)."""
    desc, pl, out, lse, workspace, ws_n = _attn_args(q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, H,
                                                     scale, out, lse, workspace, kv_chunk, BN=tuple(parents.shape),
                                                     pages=pages, prefix_len_dev=prefix_len if device_lengths else None)
    task, idx = _argmax_task(logits, idx, argmax_workspace)
    for t, n in ((draft_ids, "draft_ids"), (parents, "parents"), (prefix_len, "prefix_len")):
        _contig(t, torch.int32, n)
    if tuple(parents.shape) != (desc.B, desc.N) or tuple(draft_ids.shape) != (desc.B, desc.N):
        raise ValueError("draft_ids and parents must be [B, N]")
    _holds(prefix_len, desc.B, "prefix_len")
    if new_prefix_len is None:
        new_prefix_len = prefix_len
    _holds(_contig(new_prefix_len, torch.int32, "new_prefix_len"), desc.B, "new_prefix_len")
    accept_len, path, tokens = _accept_outputs(parents, accept_len, path, tokens)
    _src_slot(src_slot, desc.B, desc.N)
    acc = AcceptTask(_p(draft_ids), _p(parents), _p(accept_len), _p(path), _p(tokens), _p(prefix_len),
                     _p(new_prefix_len), _p(src_slot))
    _check(lib().ddt_verify_step(ctypes.byref(desc), _p(q_lat), _p(q_pe), _p(ckv), _p(kpe), _p(kv_base),
                                 pl.ctypes.data, _p(mask), _p(out), _p(lse), _p(workspace), ws_n,
                                 ctypes.byref(task), ctypes.byref(acc), _stream(stream)), "ddt_verify_step")
    return out, lse, idx, accept_len, path, tokens, new_prefix_len


def argmax_workspace_bytes(rows: int, V: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ddt_argmax_workspace(rows, V, ctypes.byref(n)), "ddt_argmax_workspace")
    return n.value


def argmax(logits, idx=None, workspace=None, stream=None):
    """logits [rows, V] fp32/bf16 (2-D view) -> idx [rows] int32.

    workspace: argmax_workspace_bytes(rows, V) bytes of device memory,
    zero-filled before its first use (every call leaves it zeroed again).
    """
    _dev(logits, None, "logits")
    ld = _rows(logits, "logits")
    rows, V = logits.shape
    if idx is None:
        idx = torch.empty((rows,), dtype=torch.int32, device=logits.device)
    _holds(_contig(idx, torch.int32, "idx"), rows, "idx")
    need = argmax_workspace_bytes(rows, V)
    if workspace is None and need > 0:
        workspace = torch.zeros((need,), dtype=torch.uint8, device=logits.device)  # zero before first use
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ddt_argmax(_p(logits), _dtype_code(logits), rows, V, ld, _p(idx), _p(workspace), ws_n,
                            _stream(stream)), "ddt_argmax")
    return idx


def greedy_accept(target_ids, draft_ids, parents, accept_len=None, path=None, tokens=None, stream=None):
    """-> (accept_len [B], path [B, N], tokens [B, N]) int32 device tensors."""
    B, N = _tree_inputs(parents, ((target_ids, "target_ids"), (draft_ids, "draft_ids")))
    accept_len, path, tokens = _accept_outputs(parents, accept_len, path, tokens)
    _check(lib().ddt_greedy_accept(_p(target_ids), _p(draft_ids), _p(parents), B, N, _p(accept_len), _p(path),
                                   _p(tokens), _stream(stream)), "ddt_greedy_accept")
    return accept_len, path, tokens


def compact_kv(ckv, kpe, kv_base, prefix_len, path, accept_len, src_slot=None, pages=None, stream=None):
    """In-place compaction of the cache pool views; prefix_len [B] int32 (device) is updated.
    pages: None (contiguous from kv_base) or (block_table [B, bt_ld] int32, page_size); kv_base
    is then unused (may be None)."""
    _dev(ckv, None, "ckv")
    _dev(kpe, ckv.dtype, "kpe")
    _contig(path, torch.int32, "path")
    if path.dim() != 2:
        raise ValueError("path must be [B, N]")
    B, N = path.shape
    _holds(_contig(prefix_len, torch.int32, "prefix_len"), B, "prefix_len")
    _holds(_contig(accept_len, torch.int32, "accept_len"), B, "accept_len")
    _src_slot(src_slot, B, N)
    if pages is not None:
        table, page_size = pages
        _contig(table, torch.int32, "block_table")
        if table.dim() != 2 or table.shape[0] != B:
            raise ValueError("block_table must be [B, bt_ld]")
        _check(lib().ddt_compact_kv_paged(_p(ckv), _rows(ckv, "ckv"), _p(kpe), _rows(kpe, "kpe"), _dtype_code(ckv),
                                          ckv.shape[1], kpe.shape[1], _p(table), table.shape[1], int(page_size),
                                          _p(prefix_len), _p(path), _p(accept_len), B, N, _p(src_slot),
                                          _stream(stream)), "ddt_compact_kv_paged")
        return prefix_len, src_slot
    _holds(_contig(kv_base, torch.int64, "kv_base"), B, "kv_base")
    _check(lib().ddt_compact_kv(_p(ckv), _rows(ckv, "ckv"), _p(kpe), _rows(kpe, "kpe"), _dtype_code(ckv),
                                ckv.shape[1], kpe.shape[1], _p(kv_base), _p(prefix_len), _p(path),
                                _p(accept_len), B, N, _p(src_slot), _stream(stream)), "ddt_compact_kv")
    return prefix_len, src_slot


def accept_compact(target_ids, draft_ids, parents, ckv, kpe, kv_base, prefix_len, accept_len=None, path=None,
                   tokens=None, src_slot=None, new_prefix_len=None, pages=None, stream=None):
    """greedy_accept + compact_kv in one launch -> (accept_len, path, tokens).

    The advanced lengths go to new_prefix_len (default: prefix_len, in place).
    pages: None (contiguous from kv_base) or (block_table [B, bt_ld] int32,
    page_size); kv_base is then unused (may be None)."""
    B, N = _tree_inputs(parents, ((target_ids, "target_ids"), (draft_ids, "draft_ids")))
    _dev(ckv, None, "ckv")
    _dev(kpe, ckv.dtype, "kpe")
    if pages is None:
        _holds(_contig(kv_base, torch.int64, "kv_base"), B, "kv_base")
    _holds(_contig(prefix_len, torch.int32, "prefix_len"), B, "prefix_len")
    if new_prefix_len is None:
        new_prefix_len = prefix_len
    _holds(_contig(new_prefix_len, torch.int32, "new_prefix_len"), B, "new_prefix_len")
    accept_len, path, tokens = _accept_outputs(parents, accept_len, path, tokens)
    _src_slot(src_slot, B, N)
    if pages is not None:
        table, page_size = pages
        _contig(table, torch.int32, "block_table")
        if table.dim() != 2 or table.shape[0] != B:
            raise ValueError("block_table must be [B, bt_ld]")
        _check(lib().ddt_accept_compact_paged(_p(target_ids), _p(draft_ids), _p(parents), B, N, _p(accept_len),
                                              _p(path), _p(tokens), _p(ckv), _rows(ckv, "ckv"), _p(kpe),
                                              _rows(kpe, "kpe"), _dtype_code(ckv), ckv.shape[1], kpe.shape[1],
                                              _p(table), table.shape[1], int(page_size), _p(prefix_len),
                                              _p(new_prefix_len), _p(src_slot), _stream(stream)),
               "ddt_accept_compact_paged")
        return accept_len, path, tokens
    _check(lib().ddt_accept_compact(_p(target_ids), _p(draft_ids), _p(parents), B, N, _p(accept_len), _p(path),
                                    _p(tokens), _p(ckv), _rows(ckv, "ckv"), _p(kpe), _rows(kpe, "kpe"),
                                    _dtype_code(ckv), ckv.shape[1], kpe.shape[1], _p(kv_base), _p(prefix_len),
                                    _p(new_prefix_len), _p(src_slot), _stream(stream)), "ddt_accept_compact")
    return accept_len, path, tokens


def draft_topk_workspace_bytes(rows: int, V: int, K: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ddt_draft_topk_workspace(rows, V, K, ctypes.byref(n)), "ddt_draft_topk_workspace")
    return n.value


def draft_topk(logits, K, ids=None, logp=None, workspace=None, stream=None):
    """fp32 draft logits [rows, V] (row view) -> (ids [rows, K] int32, logp [rows, K] fp32)."""
    _dev(logits, torch.float32, "logits")
    ld = _rows(logits, "logits")
    rows, V = logits.shape
    dev = logits.device
    if ids is None:
        ids = torch.empty((rows, K), dtype=torch.int32, device=dev)
    if logp is None:
        logp = torch.empty((rows, K), dtype=torch.float32, device=dev)
    _holds(_contig(ids, torch.int32, "ids"), rows * K, "ids")
    _holds(_contig(logp, torch.float32, "logp"), rows * K, "logp")
    if workspace is None:
        workspace = torch.empty((max(16, draft_topk_workspace_bytes(rows, V, K)),), dtype=torch.uint8, device=dev)
    ws_n = workspace.numel() * workspace.element_size()
    _check(lib().ddt_draft_topk(_p(logits), rows, V, ld, K, _p(ids), _p(logp), _p(workspace), ws_n,
                                _stream(stream)), "ddt_draft_topk")
    return ids, logp


def best_first_tree(ids, logp, root_tokens, budget, parents=None, tokens=None, depth=None, stream=None):
    """ids [B, D, K] int32, logp [B, D, K] fp32, root_tokens [B] int32 ->
    (parents, tokens, depth) [B, budget+1] int32."""
    _contig(ids, torch.int32, "ids")
    _contig(logp, torch.float32, "logp")
    _contig(root_tokens, torch.int32, "root_tokens")
    B, D, K = ids.shape
    if tuple(logp.shape) != (B, D, K) or tuple(root_tokens.shape) != (B,):
        raise ValueError("logp must be [B, D, K] and root_tokens [B]")
    dev = ids.device
    outs = []
    for t, n in ((parents, "parents"), (tokens, "tokens"), (depth, "depth")):
        if t is None:
            t = torch.empty((B, budget + 1), dtype=torch.int32, device=dev)
        _holds(_contig(t, torch.int32, n), B * (budget + 1), n)
        outs.append(t)
    _check(lib().ddt_best_first_tree(_p(ids), _p(logp), B, D, K, budget, _p(root_tokens), _p(outs[0]), _p(outs[1]),
                                     _p(outs[2]), _stream(stream)), "ddt_best_first_tree")
    return tuple(outs)


def proj_pack_weight(w, packed=None, stream=None):
    """Per-head projection weights [H, K, n_out] bf16 ([in, out] per head)
    -> the packed operand order ddt_head_proj reads (same shape and bytes)."""
    _contig(w, torch.bfloat16, "w")
    if w.dim() != 3:
        raise ValueError("w must be [H, K, n_out]")
    H, K, n_out = w.shape
    if packed is None:
        packed = torch.empty_like(w)
    _contig(packed, torch.bfloat16, "packed")
    if packed.numel() != w.numel():
        raise ValueError("packed must hold H*K*n_out elements")
    _check(lib().ddt_proj_pack_weight(_p(w), H, K, n_out, DDT_BF16, _p(packed), _stream(stream)),
           "ddt_proj_pack_weight")
    return packed


def head_proj(x, w_packed, H, y=None, stream=None):
    """y[t*H + h] = x[t*H + h] @ W[h] for bf16 row views x [M*H, K] (rows
    token-major, head-minor); w_packed from proj_pack_weight ([H, K, n_out]).
    y: None (a new [M*H, n_out] tensor) or a row view [M*H, >= n_out] whose
    first n_out columns are written."""
    _dev(x, torch.bfloat16, "x")
    ld_x = _rows(x, "x")
    _contig(w_packed, torch.bfloat16, "w_packed")
    Hw, K, n_out = w_packed.shape
    if Hw != H or x.shape[1] != K or x.shape[0] % H != 0:
        raise ValueError("x must be [M*H, K] with w_packed [H, K, n_out]")
    M = x.shape[0] // H
    if y is None:
        y = torch.empty((M * H, n_out), dtype=torch.bfloat16, device=x.device)
    _dev(y, torch.bfloat16, "y")
    ld_y = _rows(y, "y")
    if y.shape[0] != M * H or y.shape[1] < n_out:
        raise ValueError("y must have M*H rows of at least n_out columns")
    _check(lib().ddt_head_proj(_p(x), ld_x, _p(w_packed), M, H, K, n_out, DDT_BF16, _p(y), ld_y, _stream(stream)),
           "ddt_head_proj")
    return y


# ---------------------------------------------------------------- probes ----
# include/ddt_probe.h: the device's achievable MFMA rate and HBM bandwidth,
# measured by the library's own kernels beside the datasheet peaks.
PROBE_THREADS = 256
PROBE_MFMA_OPERANDS = 4096
PROBE_MFMA_FLOP_PER_WAVE_ITER = 524288


def probe_mfma_bf16(ops, blocks, iters, sink=None, clk=None, stream=None):
    """bf16 MFMA loop over the operand fragments in `ops` (4096 bf16);
    performs blocks * 4 * iters * PROBE_MFMA_FLOP_PER_WAVE_ITER flop.
    Returns (sink, clk): clk[b] = (core-clock ticks, 100 MHz ticks) of
    workgroup b's loop."""
    _contig(ops, torch.bfloat16, "ops")
    if ops.numel() != PROBE_MFMA_OPERANDS:
        raise ValueError(f"ops must hold {PROBE_MFMA_OPERANDS} values")
    if sink is None:
        sink = torch.empty((blocks * PROBE_THREADS,), dtype=torch.float32, device=ops.device)
    if clk is None:
        clk = torch.empty((blocks, 2), dtype=torch.int64, device=ops.device)
    _contig(sink, torch.float32, "sink")
    _contig(clk, torch.int64, "clk")
    if sink.numel() < blocks * PROBE_THREADS or clk.numel() < 2 * blocks:
        raise ValueError("sink or clk too small")
    _check(lib().ddt_probe_mfma_bf16(_p(ops), _p(sink), _p(clk), blocks, iters, _stream(stream)),
           "ddt_probe_mfma_bf16")
    return sink, clk


def probe_read(src, blocks, sink=None, stream=None):
    """Streaming read of every byte of `src` (contiguous, 16-byte multiple)."""
    _dev(src, None, "src")
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    if sink is None:
        sink = torch.empty((blocks * PROBE_THREADS,), dtype=torch.int32, device=src.device)
    _contig(sink, torch.int32, "sink")
    if sink.numel() < blocks * PROBE_THREADS:
        raise ValueError("sink too small")
    nbytes = src.numel() * src.element_size()
    _check(lib().ddt_probe_read(_p(src), nbytes, _p(sink), blocks, _stream(stream)), "ddt_probe_read")
    return sink


def probe_copy(src, dst, blocks, stream=None):
    """Streaming copy of `src` into `dst` (contiguous, same byte size)."""
    for t, n in ((src, "src"), (dst, "dst")):
        _dev(t, None, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    _check(lib().ddt_probe_copy(_p(src), _p(dst), nbytes, blocks, _stream(stream)), "ddt_probe_copy")
