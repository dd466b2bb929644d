"""Python binding of libcsa.so (include/csa.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors are torch
tensors on the current GPU; the call is enqueued on torch's current stream.
Outputs are allocated with torch when ``out`` is None.  There is no fallback:
if libcsa.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")
# the same library built with device-side input checks (synchronizes each checked call)
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa_debug.so")
CSA_F32, CSA_BF16 = 0, 1
_lib = None


class CompressPass(ctypes.Structure):
    """csa_compress_pass_t: one csa_compress call's arguments."""
    _fields_ = [("x", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("slot_bias", ctypes.c_void_p), ("pool", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("D", ctypes.c_int32),
                ("m", ctypes.c_int32), ("overlap", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("cs", ctypes.c_void_p), ("n_pos", ctypes.c_int32), ("pos0", ctypes.c_int32)]


class CachePass(ctypes.Structure):
    """csa_cache_pass_t: one csa_cache_append call's arguments."""
    _fields_ = [("x", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("slot_bias", ctypes.c_void_p), ("ring_x", ctypes.c_void_p),
                ("ring_g", ctypes.c_void_p), ("pool", ctypes.c_void_p), ("win", ctypes.c_void_p),
                ("count", ctypes.c_void_p), ("B", ctypes.c_int32), ("n", ctypes.c_int32),
                ("D", ctypes.c_int32), ("m", ctypes.c_int32), ("overlap", ctypes.c_int32),
                ("T_cap", ctypes.c_int32), ("W", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("cs", ctypes.c_void_p), ("n_pos", ctypes.c_int32)]


def lib():
    """The loaded libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load(_LIB_PATH)
    return _lib


def use_library(which):
    """Make the bindings call another build: a path (e.g. DEBUG_LIB_PATH) or a
    handle that load() or use_library() returned.  Returns the handle they
    called before (None if none was loaded yet)."""
    global _lib
    prev = _lib
    _lib = load(which) if isinstance(which, str) else which
    return prev


def load(path: str):
    """A libcsa build at `path` with every entry point's signature set."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m sparse_long_context_pool_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
                             ctypes.c_double, ctypes.c_size_t)
    sig = {
        "csa_last_error": ([], ctypes.c_char_p),
        "csa_version": ([], ctypes.c_char_p),
        "csa_rope_table": ([vp, i32, i32, f64, vp], ctypes.c_int),
        "csa_rope_table_yarn": ([vp, i32, i32, f64, f64, i32, f64, f64, vp], ctypes.c_int),
        "csa_compress": ([vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, i32,
                          i32, vp], ctypes.c_int),
        "csa_compress_many": ([ctypes.POINTER(CompressPass), i32, i32, vp], ctypes.c_int),
        "csa_cache_append_many": ([ctypes.POINTER(CachePass), i32, i32, vp], ctypes.c_int),
        "csa_cache_append": ([vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                              i32, i32, i32, vp, i32, i32, vp], ctypes.c_int),
        "csa_index_scores": ([vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                              vp], ctypes.c_int),
        "csa_topk": ([vp, vp, vp, i32, i32, i32, i32, i32, vp], ctypes.c_int),
        "csa_index_topk": ([vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, sz,
                            i32, vp], ctypes.c_int),
        "csa_index_topk_workspace_size": ([i32] * 8, sz),
        "csa_sparse_attn": ([vp, vp, vp, i32, vp, i32, vp, i32, vp, vp, vp, i32, i32,
                             i32, i32, i32, i32, vp, i32, i32, f32, vp, sz, i32, vp],
                            ctypes.c_int),
        "csa_sparse_attn_noalloc": ([vp, vp, vp, i32, vp, i32, vp, i32, vp, vp, vp, i32,
                                     i32, i32, i32, i32, i32, vp, i32, i32, f32, i32, vp],
                                    ctypes.c_int),
        "csa_sparse_attn_workspace_size": ([i32] * 9, sz),
        "hca_attn": ([vp, vp, vp, i32, vp, i32, i32, vp, vp, vp, i32, i32, i32, i32,
                      i32, i32, vp, i32, i32, f32, vp, sz, i32, vp], ctypes.c_int),
        "hca_attn_workspace_size": ([i32] * 9, sz),
        "csa_grouped_out_proj": ([vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp],
                                 ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


EXPORTS = ("csa_last_error", "csa_version", "csa_rope_table", "csa_rope_table_yarn",
           "csa_compress", "csa_compress_many",
           "csa_cache_append", "csa_cache_append_many",
           "csa_index_scores", "csa_topk", "csa_index_topk", "csa_index_topk_workspace_size",
           "csa_sparse_attn", "csa_sparse_attn_noalloc",
           "csa_sparse_attn_workspace_size", "hca_attn", "hca_attn_workspace_size",
           "csa_grouped_out_proj")


def _check(status: int, fn: str):
    if status != 0:
        msg = lib().csa_last_error().decode()
        raise RuntimeError(f"{fn} failed (status {status}): {msg}")


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype == torch.float32:
        return CSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def version() -> str:
    return lib().csa_version().decode()


def csa_rope_table(n_pos: int, rope_dim: int, theta: float, device=None) -> torch.Tensor:
    """cos/sin table [n_pos, rope_dim/2, 2] fp32 (angle in fp64)."""
    cs = torch.empty((n_pos, rope_dim // 2, 2), dtype=torch.float32,
                     device=device or torch.device("cuda"))
    _check(lib().csa_rope_table(_ptr(cs), n_pos, rope_dim, float(theta), _stream()),
           "csa_rope_table")
    return cs


def csa_rope_table_yarn(n_pos: int, rope_dim: int, theta: float, factor: float,
                        original_max_pos: int, beta_fast: float = 32.0, beta_slow: float = 1.0,
                        device=None) -> torch.Tensor:
    """cos/sin table [n_pos, rope_dim/2, 2] fp32 with YaRN-scaled pair frequencies."""
    cs = torch.empty((n_pos, rope_dim // 2, 2), dtype=torch.float32,
                     device=device or torch.device("cuda"))
    _check(lib().csa_rope_table_yarn(_ptr(cs), n_pos, rope_dim, float(theta), float(factor),
                                     int(original_max_pos), float(beta_fast), float(beta_slow),
                                     _stream()),
           "csa_rope_table_yarn")
    return cs


def csa_compress(x, gate=None, slot_bias=None, *, m: int, overlap: int, rope_dim: int = 0,
                 cs=None, pos0: int = 0, out=None) -> torch.Tensor:
    """x [B, S, D] (+ gate [B, S, D], slot_bias [(1+overlap)*m, D] fp32) -> pool [B, S//m, D]."""
    B, S, D = x.shape
    if gate is not None:
        assert gate.shape == x.shape and gate.dtype == x.dtype
    if slot_bias is not None:
        assert slot_bias.dtype == torch.float32 and slot_bias.shape == ((1 + overlap) * m, D)
    if out is None:
        out = torch.empty((B, S // m, D), dtype=x.dtype, device=x.device)
    n_pos = 0 if cs is None else cs.shape[0]
    _check(lib().csa_compress(_ptr(x), _ptr(gate), _ptr(slot_bias), _ptr(out), B, S, D, m,
                              overlap, rope_dim, _ptr(cs), n_pos, pos0, _dtype(x), _stream()),
           "csa_compress")
    return out


def csa_compress_many(passes) -> list:
    """Several csa_compress passes in one call.  ``passes`` is a sequence of
    dicts with csa_compress's arguments (keys x, gate, slot_bias, m, overlap,
    rope_dim, cs, pos0, out); all x share one dtype.  Returns the pools."""
    passes = list(passes)
    arr = (CompressPass * max(len(passes), 1))()
    outs = []
    dtype = _dtype(passes[0]["x"]) if passes else CSA_BF16
    for q, p in enumerate(passes):
        x, gate, sb = p["x"], p.get("gate"), p.get("slot_bias")
        m, overlap = p["m"], p.get("overlap", 0)
        B, S, D = x.shape
        if _dtype(x) != dtype:
            raise TypeError("csa_compress_many: all passes must share one dtype")
        if gate is not None:
            assert gate.shape == x.shape and gate.dtype == x.dtype
        if sb is not None:
            assert sb.dtype == torch.float32 and sb.shape == ((1 + overlap) * m, D)
        out = p.get("out")
        if out is None:
            out = torch.empty((B, S // m, D), dtype=x.dtype, device=x.device)
        cs = p.get("cs")
        c = arr[q]
        c.x, c.gate, c.slot_bias, c.pool, c.cs = (
            None if t is None else _ptr(t).value for t in (x, gate, sb, out, cs))
        c.B, c.S, c.D, c.m, c.overlap = B, S, D, m, overlap
        c.rope_dim = p.get("rope_dim", 0)
        c.n_pos = 0 if cs is None else cs.shape[0]
        c.pos0 = p.get("pos0", 0)
        outs.append(out)
    _check(lib().csa_compress_many(arr, len(passes), dtype, _stream()), "csa_compress_many")
    return outs


def csa_cache_append(x, gate, slot_bias, count, ring_x, ring_g, pool, win=None, *, m: int,
                     overlap: int, rope_dim: int = 0, cs=None) -> None:
    """Append x [B, n, D] (+ gate) to a decode cache: ring_x/ring_g [B, (1+overlap)m, D]
    (compressor buffer and overlap state), pool [B, T_cap, D], win [B, W, D] or None
    (the sliding window as a ring); count [B] int32 = tokens appended before (the
    caller adds n afterwards)."""
    B, n, D = x.shape
    if gate is not None:
        assert gate.shape == x.shape and gate.dtype == x.dtype
    assert count.dtype == torch.int32 and count.numel() == B
    T_cap = pool.shape[1]
    W = 0 if win is None else win.shape[1]
    n_pos = 0 if cs is None else cs.shape[0]
    _check(lib().csa_cache_append(_ptr(x), _ptr(gate), _ptr(slot_bias), _ptr(ring_x),
                                  _ptr(ring_g), _ptr(pool), _ptr(win), _ptr(count), B, n, D, m,
                                  overlap, T_cap, W, rope_dim, _ptr(cs), n_pos, _dtype(x),
                                  _stream()),
           "csa_cache_append")


def csa_cache_append_many(passes) -> None:
    """Several csa_cache_append updates in one call.  ``passes`` is a sequence
    of dicts with csa_cache_append's arguments (keys x, gate, slot_bias, count,
    ring_x, ring_g, pool, win, m, overlap, rope_dim, cs); all x share one dtype
    and every pass updates its own cache."""
    passes = list(passes)
    arr = (CachePass * max(len(passes), 1))()
    dtype = _dtype(passes[0]["x"]) if passes else CSA_BF16
    for q, p in enumerate(passes):
        x, gate, count = p["x"], p.get("gate"), p["count"]
        B, n, D = x.shape
        if _dtype(x) != dtype:
            raise TypeError("csa_cache_append_many: all passes must share one dtype")
        if gate is not None:
            assert gate.shape == x.shape and gate.dtype == x.dtype
        assert count.dtype == torch.int32 and count.numel() == B
        pool, win, cs = p["pool"], p.get("win"), p.get("cs")
        c = arr[q]
        c.x, c.gate, c.slot_bias, c.ring_x, c.ring_g, c.pool, c.win, c.count, c.cs = (
            None if t is None else _ptr(t).value
            for t in (x, gate, p.get("slot_bias"), p["ring_x"], p.get("ring_g"), pool, win,
                      count, cs))
        c.B, c.n, c.D, c.m, c.overlap = B, n, D, p["m"], p.get("overlap", 0)
        c.T_cap, c.W = pool.shape[1], 0 if win is None else win.shape[1]
        c.rope_dim = p.get("rope_dim", 0)
        c.n_pos = 0 if cs is None else cs.shape[0]
    _check(lib().csa_cache_append_many(arr, len(passes), dtype, _stream()),
           "csa_cache_append_many")


def csa_index_scores(q_idx, w_idx, k_pool, q_pos, *, m: int, out=None) -> torch.Tensor:
    """q_idx [B, S, nI, cI], w_idx [B, S, nI] fp32, k_pool [B, T, cI] -> scores [B, S, T] fp32.

    Entries w >= R(t) are not written."""
    B, S, nI, cI = q_idx.shape
    T = k_pool.shape[1]
    assert w_idx.dtype == torch.float32 and k_pool.dtype == q_idx.dtype
    assert q_pos.dtype == torch.int32 and q_pos.numel() == B
    if out is None:
        out = torch.empty((B, S, T), dtype=torch.float32, device=q_idx.device)
    _check(lib().csa_index_scores(_ptr(q_idx), _ptr(w_idx), _ptr(k_pool), _ptr(out),
                                  _ptr(q_pos), B, S, T, nI, cI, m, _dtype(q_idx), _stream()),
           "csa_index_scores")
    return out


def csa_topk(scores, q_pos, *, k: int, m: int, out=None) -> torch.Tensor:
    """scores [B, S, T] fp32 -> idx [B, S, k] int32 (ascending, -1 padded)."""
    B, S, T = scores.shape
    assert scores.dtype == torch.float32 and q_pos.dtype == torch.int32
    if out is None:
        out = torch.empty((B, S, k), dtype=torch.int32, device=scores.device)
    _check(lib().csa_topk(_ptr(scores), _ptr(out), _ptr(q_pos), B, S, T, k, m, _stream()),
           "csa_topk")
    return out


def csa_index_topk(q_idx, w_idx, k_pool, q_pos, *, k: int, m: int, out=None,
                   workspace=None) -> torch.Tensor:
    """csa_topk(csa_index_scores(...)) in one call -> idx [B, S, k] int32."""
    B, S, nI, cI = q_idx.shape
    T = k_pool.shape[1]
    assert w_idx.dtype == torch.float32 and k_pool.dtype == q_idx.dtype
    assert q_pos.dtype == torch.int32 and q_pos.numel() == B
    if out is None:
        out = torch.empty((B, S, k), dtype=torch.int32, device=q_idx.device)
    dt = _dtype(q_idx)
    need = lib().csa_index_topk_workspace_size(B, S, T, nI, cI, k, m, dt)
    ws, ws_bytes = _ws(need, q_idx.device, workspace)
    _check(lib().csa_index_topk(_ptr(q_idx), _ptr(w_idx), _ptr(k_pool), _ptr(out), _ptr(q_pos),
                                B, S, T, nI, cI, k, m, _ptr(ws), ws_bytes, dt, _stream()),
           "csa_index_topk")
    return out


def _ws(size: int, device, workspace):
    if size == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(size, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def csa_sparse_attn(q, kv_win, win_pos0, pool, idx, sink, q_pos, *, rope_dim: int, cs,
                    window: int, scale: float, dv: int | None = None, out=None,
                    workspace=None) -> torch.Tensor:
    """q [B, S, H, D]; kv_win [B, L, D] (rotated); pool [B, T, D] (rotated);
    idx [B, S, k] int32; sink [H] fp32 or None -> out [B, S, H, dv]."""
    B, S, H, D = q.shape
    dv = D if dv is None else dv
    L = 0 if kv_win is None else kv_win.shape[1]
    T = 0 if pool is None else pool.shape[1]
    k = 0 if idx is None else idx.shape[2]
    if out is None:
        out = torch.empty((B, S, H, dv), dtype=q.dtype, device=q.device)
    dt = _dtype(q)
    need = lib().csa_sparse_attn_workspace_size(B, S, H, D, dv, rope_dim, k, window, dt)
    ws, ws_bytes = _ws(need, q.device, workspace)
    n_pos = 0 if cs is None else cs.shape[0]
    _check(lib().csa_sparse_attn(_ptr(q), _ptr(kv_win), _ptr(win_pos0), L, _ptr(pool), T,
                                 _ptr(idx), k, _ptr(sink), _ptr(out), _ptr(q_pos), B, S, H, D,
                                 dv, rope_dim, _ptr(cs), n_pos, window, float(scale),
                                 _ptr(ws), ws_bytes, dt, _stream()),
           "csa_sparse_attn")
    return out


def csa_sparse_attn_noalloc(q, kv_win, win_pos0, pool, idx, sink, q_pos, *, rope_dim: int, cs,
                            window: int, scale: float, dv: int | None = None,
                            out=None) -> torch.Tensor:
    """csa_sparse_attn with the split workspace in the library's own device array
    (the C call allocates nothing; `out` is allocated here when None)."""
    B, S, H, D = q.shape
    dv = D if dv is None else dv
    L = 0 if kv_win is None else kv_win.shape[1]
    T = 0 if pool is None else pool.shape[1]
    k = 0 if idx is None else idx.shape[2]
    if out is None:
        out = torch.empty((B, S, H, dv), dtype=q.dtype, device=q.device)
    n_pos = 0 if cs is None else cs.shape[0]
    _check(lib().csa_sparse_attn_noalloc(_ptr(q), _ptr(kv_win), _ptr(win_pos0), L, _ptr(pool),
                                         T, _ptr(idx), k, _ptr(sink), _ptr(out), _ptr(q_pos), B,
                                         S, H, D, dv, rope_dim, _ptr(cs), n_pos, window,
                                         float(scale), _dtype(q), _stream()),
           "csa_sparse_attn_noalloc")
    return out


def hca_attn(q, kv_win, win_pos0, pool, sink, q_pos, *, m: int, rope_dim: int, cs,
             window: int, scale: float, dv: int | None = None, out=None,
             workspace=None) -> torch.Tensor:
    """As csa_sparse_attn with every ready pool entry w < min(T, (t+1)//m)."""
    B, S, H, D = q.shape
    dv = D if dv is None else dv
    L = 0 if kv_win is None else kv_win.shape[1]
    T = 0 if pool is None else pool.shape[1]
    if out is None:
        out = torch.empty((B, S, H, dv), dtype=q.dtype, device=q.device)
    dt = _dtype(q)
    need = lib().hca_attn_workspace_size(B, S, H, D, dv, rope_dim, T, window, dt)
    ws, ws_bytes = _ws(need, q.device, workspace)
    n_pos = 0 if cs is None else cs.shape[0]
    _check(lib().hca_attn(_ptr(q), _ptr(kv_win), _ptr(win_pos0), L, _ptr(pool), T, m,
                          _ptr(sink), _ptr(out), _ptr(q_pos), B, S, H, D, dv, rope_dim,
                          _ptr(cs), n_pos, window, float(scale), _ptr(ws), ws_bytes, dt,
                          _stream()),
           "hca_attn")
    return out


def csa_grouped_out_proj(o, w_a, w_b, *, mid=None, out=None):
    """o [M, groups*group_in] (or [B, S, H, dv], flattened), w_a [groups, rank, group_in],
    w_b [hidden, groups*rank] -> (mid [M, groups*rank], out [M, hidden])."""
    groups, rank, group_in = w_a.shape
    hidden = w_b.shape[0]
    M = o.numel() // (groups * group_in)
    assert o.numel() == M * groups * group_in and w_b.shape[1] == groups * rank
    assert w_a.dtype == o.dtype and w_b.dtype == o.dtype
    if mid is None:
        mid = torch.empty((M, groups * rank), dtype=o.dtype, device=o.device)
    if out is None:
        out = torch.empty((M, hidden), dtype=o.dtype, device=o.device)
    _check(lib().csa_grouped_out_proj(_ptr(o), _ptr(w_a), _ptr(w_b), _ptr(mid), _ptr(out), M,
                                      groups, group_in, rank, hidden, _dtype(o), _stream()),
           "csa_grouped_out_proj")
    return mid, out
