"""ctypes shim over ``liboracle.so``, the fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this module.  The product path (the
HIP library and its binding) never imports, links or calls it.

Each wrapper takes numpy arrays.  Floating point arrays are either float32
(fp32 data) or uint16 (bf16 bit patterns); 2-D views may have a row stride
larger than their width (for example the c_kv and k_pe column ranges of one
interleaved cache pool).  The definitions are in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain C11, OpenMP, -O2)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_build_mask.argtypes = [P, i32, i32, P, P, P]
        L.orc_verify_attn.argtypes = [i32, i32, i32, i32, i32, i32, dbl,
                                      P, i64, P, i64, P, i64, P, i64,
                                      P, P, P, P, i64, P, P, P]
        L.orc_argmax.argtypes = [P, i32, i64, i64, i64, P]
        L.orc_greedy_accept.argtypes = [P, P, P, i32, i32, P, P, P]
        L.orc_compact_kv.argtypes = [P, i64, P, i64, i32, i32, i32, P, P, P, P, i32, i32, P]
        L.orc_num_threads.argtypes = []
        L.orc_draft_topk.argtypes = [P, i64, i64, i64, i32, P, P]
        L.orc_best_first_tree.argtypes = [P, P, i32, i32, i32, i32, P, P, P]
        L.orc_head_proj.argtypes = [i64, i32, i32, i32, P, i32, i64, P, i32, P]
        for f in (L.orc_build_mask, L.orc_verify_attn, L.orc_argmax, L.orc_greedy_accept,
                  L.orc_compact_kv, L.orc_num_threads, L.orc_draft_topk, L.orc_best_first_tree,
                  L.orc_head_proj):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {a.dtype}")


def _ld(a: np.ndarray) -> int:
    assert a.ndim == 2 and a.strides[1] == a.itemsize, "rows must be unit-stride"
    return a.strides[0] // a.itemsize


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def num_threads() -> int:
    return lib().orc_num_threads()


def build_mask(parents: np.ndarray):
    """parents [B, N] int32 -> (mask [B, N, W] uint64, depth [B, N] int32, tree_err [B] int32)."""
    par = _c(parents, np.int32)
    B, N = par.shape
    W = (N + 63) // 64
    mask = np.zeros((B, N, W), np.uint64)
    depth = np.zeros((B, N), np.int32)
    err = np.zeros((B,), np.int32)
    rc = lib().orc_build_mask(_ptr(par), B, N, _ptr(mask), _ptr(depth), _ptr(err))
    if rc != 0:
        raise RuntimeError(f"orc_build_mask failed: {rc}")
    return mask, depth, err


def verify_attn(q_lat, q_pe, ckv, kpe, kv_base, prefix_len, parents, *, H: int,
                scale: float, rows=None, with_wsum: bool = False):
    """Tree-verify attention for all (or the listed) flat rows r = (b*N + i)*H + h.

    q_lat [B*N*H, d_lat], q_pe [B*N*H, d_rope]: 2-D (views allowed).
    ckv [pool, d_lat], kpe [pool, d_rope]: 2-D views of the cache pool.
    Returns (out [R, d_lat] float64, lse [R] float64[, wsum [R]]).
    """
    par = _c(parents, np.int32)
    B, N = par.shape
    dt = _dtype_code(q_lat)
    for a in (q_pe, ckv, kpe):
        assert _dtype_code(a) == dt
    d_lat, d_rope = q_lat.shape[1], q_pe.shape[1]
    assert ckv.shape[1] == d_lat and kpe.shape[1] == d_rope
    assert q_lat.shape[0] == B * N * H
    kvb = _c(kv_base, np.int64)
    pl = _c(prefix_len, np.int32)
    if rows is not None:
        rows = _c(rows, np.int64)
        R = rows.shape[0]
    else:
        R = B * N * H
    out = np.zeros((R, d_lat), np.float64)
    lse = np.zeros((R,), np.float64)
    wsum = np.zeros((R,), np.float64)
    rc = lib().orc_verify_attn(B, H, N, d_lat, d_rope, dt, float(scale),
                               _ptr(q_lat), _ld(q_lat), _ptr(q_pe), _ld(q_pe),
                               _ptr(ckv), _ld(ckv), _ptr(kpe), _ld(kpe),
                               _ptr(kvb), _ptr(pl), _ptr(par), _ptr(rows), R,
                               _ptr(out), _ptr(lse), _ptr(wsum))
    if rc != 0:
        raise RuntimeError(f"orc_verify_attn failed: {rc}")
    return (out, lse, wsum) if with_wsum else (out, lse)


def head_proj(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-head projection y[t*H + h] = x[t*H + h] @ w[h].

    x [M*H, K] (2-D, row views allowed), w [H, K, n_out]; each float32,
    uint16 (bf16 bits) or float64.  Returns y [M*H, n_out] float64."""
    def code(a):
        return F64 if a.dtype == np.float64 else _dtype_code(a)
    w = np.ascontiguousarray(w)
    H, K, n_out = w.shape
    assert x.ndim == 2 and x.shape[1] == K and x.shape[0] % H == 0
    M = x.shape[0] // H
    y = np.zeros((M * H, n_out), np.float64)
    rc = lib().orc_head_proj(M, H, K, n_out, _ptr(x), code(x), _ld(x), _ptr(w), code(w), _ptr(y))
    if rc != 0:
        raise RuntimeError(f"orc_head_proj failed: {rc}")
    return y


def argmax(logits: np.ndarray) -> np.ndarray:
    """logits [rows, V] float32 or uint16(bf16) -> int32 [rows]."""
    dt = _dtype_code(logits)
    rows, V = logits.shape
    idx = np.zeros((rows,), np.int32)
    rc = lib().orc_argmax(_ptr(logits), dt, rows, V, _ld(logits), _ptr(idx))
    if rc != 0:
        raise RuntimeError(f"orc_argmax failed: {rc}")
    return idx


def greedy_accept(target_ids, draft_ids, parents):
    """-> (accept_len [B], path [B, N], tokens [B, N]) int32."""
    t = _c(target_ids, np.int32)
    d = _c(draft_ids, np.int32)
    p = _c(parents, np.int32)
    B, N = p.shape
    acc = np.zeros((B,), np.int32)
    path = np.zeros((B, N), np.int32)
    tok = np.zeros((B, N), np.int32)
    rc = lib().orc_greedy_accept(_ptr(t), _ptr(d), _ptr(p), B, N, _ptr(acc), _ptr(path), _ptr(tok))
    if rc != 0:
        raise RuntimeError(f"orc_greedy_accept failed: {rc}")
    return acc, path, tok


def compact_kv(ckv, kpe, kv_base, prefix_len, path, accept_len):
    """In-place compaction of the (views of the) cache pool.

    Returns (new prefix_len [B] int32, src_slot [B, N] int32).
    """
    dt = _dtype_code(ckv)
    p = _c(path, np.int32)
    B, N = p.shape
    pl = np.array(prefix_len, dtype=np.int32, copy=True)
    kvb = _c(kv_base, np.int64)
    acc = _c(accept_len, np.int32)
    src = np.zeros((B, N), np.int32)
    rc = lib().orc_compact_kv(_ptr(ckv), _ld(ckv), _ptr(kpe), _ld(kpe), dt, ckv.shape[1],
                              kpe.shape[1], _ptr(kvb), _ptr(pl), _ptr(p), _ptr(acc), B, N, _ptr(src))
    if rc != 0:
        raise RuntimeError(f"orc_compact_kv failed: {rc}")
    return pl, src


def draft_topk(logits: np.ndarray, K: int):
    """fp32 draft logits [rows, V] (row view) -> (ids [rows, K] int32, logp [rows, K] float64)."""
    assert logits.dtype == np.float32
    rows, V = logits.shape
    ids = np.zeros((rows, K), np.int32)
    logp = np.zeros((rows, K), np.float64)
    rc = lib().orc_draft_topk(_ptr(logits), rows, V, _ld(logits), K, _ptr(ids), _ptr(logp))
    if rc != 0:
        raise RuntimeError(f"orc_draft_topk failed: {rc}")
    return ids, logp


def best_first_tree(ids: np.ndarray, lp: np.ndarray, budget: int, root: int):
    """ids [D, K] int32, lp [D, K] float32 -> (parents, tokens, depth) [budget+1] int32."""
    ids = _c(ids, np.int32)
    lp = _c(lp, np.float32)
    D, K = ids.shape
    par = np.zeros(budget + 1, np.int32)
    tok = np.zeros(budget + 1, np.int32)
    dep = np.zeros(budget + 1, np.int32)
    rc = lib().orc_best_first_tree(_ptr(ids), _ptr(lp), D, K, budget, int(root), _ptr(par), _ptr(tok), _ptr(dep))
    if rc != 0:
        raise RuntimeError(f"orc_best_first_tree failed: {rc}")
    return par, tok, dep
