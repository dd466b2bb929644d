"""CPU oracle for the CSA / HCA / DSA hot path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports it and shares no code with it.

The arithmetic lives in ``csa_oracle.c`` (plain fp32, sequential sums, one
OpenMP loop over query rows); this module only marshals numpy arrays.  Every
function follows the Hugging Face Transformers model pages:

* "DeepSeek-V4", section "Hybrid attention (§2.3)": CSA pool (m=4, overlapping
  windows) plus Lightning Indexer and top-k; HCA pool (m'=128, non-overlapping,
  no indexer); shared K=V single-head MQA; partial interleaved RoPE with the
  output rope slice rotated at -i (eq. 26); per-head sink (eq. 27); sliding
  window K=V branch.
* "DeepSeek-V4", section "Attention mask layout": readiness w < (t+1)//m and
  the -1 sentinel for unfilled top-k slots.
* "DeepSeek-V3.2", section "DeepSeek Sparse Attention (DSA)": token-level
  indexer (m=1) and attention over the selected tokens.

* "DeepSeek-V4", DeepseekV4Config: compress_rope_theta used with rope scaling
  for YaRN (``yarn_freqs``: the published YaRN frequency interpolation).
* "DeepSeek-V4", section "Hybrid attention (§2.3)", grouped low-rank output
  projection (o_groups, o_lora_rank): ``grouped_out_proj`` (float64 numpy).

Functions without a pin on the pages are marked "parity unpinned" in
``csa_oracle.c``'s header (the ReLU of the index score, the compressor's gating
form, the pool RoPE position, theta per layer, the softmax scale).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Portable flags: the library is built here and may run on another host CPU.
# No FMA contraction, so every a*b+c is two roundings, exactly as written.
GCC_CMD = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-o", _LIB, _SRC, "-lm"]


def build() -> str:
    """Compile liboracle.so from csa_oracle.c (always rebuilds)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


def ensure_built() -> str:
    if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(ensure_built())
        f32p = ctypes.POINTER(ctypes.c_float)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_long)
        ci, cl, cd, cf = ctypes.c_int, ctypes.c_long, ctypes.c_double, ctypes.c_float
        lib.orc_round_bf16.argtypes = [cf]
        lib.orc_round_bf16.restype = cf
        lib.orc_round_bf16_array.argtypes = [f32p, cl]
        lib.orc_round_bf16_array.restype = None
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.orc_rope_table_f.argtypes = [f32p, ci, ci, cd, f64p]
        lib.orc_rope_table_f.restype = None
        lib.orc_yarn_freqs.argtypes = [f64p, ci, cd, cd, cl, cd, cd]
        lib.orc_yarn_freqs.restype = None
        lib.orc_rope_apply_f.argtypes = [f32p, cl, ci, ci, cd, f64p, i64p, ci]
        lib.orc_rope_apply_f.restype = None
        lib.orc_compress_f.argtypes = [f32p, f32p, f32p, f32p, ci, ci, ci, ci, ci,
                                       cd, f64p, cl, ci]
        lib.orc_compress_f.restype = ci
        lib.orc_ready_count.argtypes = [cl, ci, ci]
        lib.orc_ready_count.restype = cl
        lib.orc_index_scores.argtypes = [f32p, f32p, i64p, ci, f32p, ci, ci, ci,
                                         ci, f32p]
        lib.orc_index_scores.restype = ci
        lib.orc_topk.argtypes = [f32p, i64p, ci, ci, ci, ci, i32p]
        lib.orc_topk.restype = ci
        lib.orc_attention_f.argtypes = [f32p, i64p, ci, ci, ci, ci, f32p, cl, ci,
                                        ci, f32p, ci, i32p, ci, ci, f32p, ci, cd,
                                        f64p, cf, f32p]
        lib.orc_attention_f.restype = ci
        _lib = lib
    return _lib


def _f32(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a, ctype=ctypes.c_float):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (status {rc})")


def round_bf16(a) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32."""
    out = _f32(a).copy()
    _load().orc_round_bf16_array(_ptr(out), out.size)
    return out


def _freqs(freqs, rope_dim):
    if freqs is None:
        return None
    f = np.ascontiguousarray(freqs, dtype=np.float64)
    assert f.shape == (rope_dim // 2,)
    return f


def yarn_freqs(rope_dim: int, theta: float, factor: float, original_max_pos: int,
               beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """Per-pair YaRN frequencies (fp64), see orc_yarn_freqs in csa_oracle.c."""
    f = np.empty(rope_dim // 2, dtype=np.float64)
    _load().orc_yarn_freqs(_ptr(f, ctypes.c_double), rope_dim, float(theta), float(factor),
                           int(original_max_pos), float(beta_fast), float(beta_slow))
    return f


def rope_table(n_pos: int, rope_dim: int, theta: float, freqs=None) -> np.ndarray:
    """cs[p, i, 0/1] = cos/sin(p * f_i), f_i = theta**(-2i/rope_dim) or freqs[i];
    fp64 angle, fp32 store."""
    cs = np.empty((n_pos, rope_dim // 2, 2), dtype=np.float32)
    f = _freqs(freqs, rope_dim)
    _load().orc_rope_table_f(_ptr(cs), n_pos, rope_dim, float(theta),
                             _ptr(f, ctypes.c_double))
    return cs


def rope_apply(v, rope_dim: int, theta: float, pos, sign: int = +1,
               freqs=None) -> np.ndarray:
    """Rotate the trailing rope_dim channels of the last axis of v.

    pos is a scalar or one position per leading row of v; sign=-1 rotates
    at -pos; freqs: per-pair frequencies (None: theta**(-2i/rope_dim))."""
    v = _f32(v).copy()
    D = v.shape[-1]
    flat = v.reshape(-1, D)
    pos = np.broadcast_to(np.asarray(pos, dtype=np.int64), (flat.shape[0],))
    pos = np.ascontiguousarray(pos)
    f = _freqs(freqs, rope_dim)
    _load().orc_rope_apply_f(_ptr(flat), flat.shape[0], D, rope_dim, float(theta),
                             _ptr(f, ctypes.c_double), _ptr(pos, ctypes.c_long), int(sign))
    return flat.reshape(v.shape)


def ready_count(t: int, m: int, T: int) -> int:
    return int(_load().orc_ready_count(int(t), int(m), int(T)))


def compress(x, gate=None, slot_bias=None, *, m: int, overlap: int,
             rope_dim: int = 0, theta: float = 1.0, pos0: int = 0,
             round_bf16: bool = False, freqs=None) -> np.ndarray:
    """Pool one sequence x[S, D] into [S//m, D] (see csa_oracle.c)."""
    x = _f32(x)
    S, D = x.shape
    gate = _f32(gate)
    slot_bias = _f32(slot_bias)
    if gate is not None:
        assert gate.shape == (S, D)
    if slot_bias is not None:
        assert slot_bias.shape == ((1 + overlap) * m, D)
    pool = np.zeros((S // m, D), dtype=np.float32)
    f = _freqs(freqs, rope_dim)
    rc = _load().orc_compress_f(_ptr(x), _ptr(gate), _ptr(slot_bias), _ptr(pool), S, D,
                                m, overlap, rope_dim, float(theta), _ptr(f, ctypes.c_double),
                                int(pos0), 1 if round_bf16 else 0)
    _check(rc, "compress")
    return pool


def cache_state(x, gate=None, slot_bias=None, *, count: int, m: int, overlap: int,
                rope_dim: int = 0, theta: float = 1.0, W: int = 0,
                bf16: bool = False):
    """The decode cache of one sequence after its first `count` tokens x[:count]
    (page "DeepSeek-V4", section "Cache layers": a sliding window of K=V rows and
    the compressor's buffer / pool / count with overlap state), written out from
    its definition rather than updated step by step:

    * pool: the compressor over those tokens -- the count // m entries whose
      window has closed, positions counted from token 0;
    * ring_x / ring_g: raw rows of the last L = (1+overlap) m tokens, token p at
      row p mod L (the compressor's buffer and overlap state);
    * win: the last W tokens rotated at their own positions, token p at row
      p mod W.

    Returns (pool, ring_x, ring_g, win, ring_rows, win_rows): the row lists give
    the ring / window rows that hold a token (the others hold nothing yet)."""
    x = _f32(x)
    D = x.shape[1]
    g = _f32(gate)
    L = (1 + overlap) * m
    pool = compress(x[:count], None if g is None else g[:count], slot_bias, m=m,
                    overlap=overlap, rope_dim=rope_dim, theta=theta, pos0=0,
                    round_bf16=bf16)
    ring_x = np.zeros((L, D), np.float32)
    ring_g = np.zeros((L, D), np.float32) if g is not None else None
    ring_rows = []
    for p in range(max(0, count - L), count):
        ring_x[p % L] = x[p]
        if g is not None:
            ring_g[p % L] = g[p]
        ring_rows.append(p % L)
    win = np.zeros((max(W, 1), D), np.float32)
    win_rows = []
    for p in range(max(0, count - W), count):
        r = rope_apply(x[p:p + 1], rope_dim, theta, np.array([p]), +1)[0] if rope_dim else x[p]
        win[p % W] = round_bf16(r) if bf16 else r
        win_rows.append(p % W)
    return pool, ring_x, ring_g, win[:W], sorted(ring_rows), sorted(win_rows)


def index_scores(qI, wI, tpos, kI, *, m: int) -> np.ndarray:
    """qI[n, nI, cI], wI[n, nI], tpos[n], kI[T, cI] -> scores[n, T] (-inf if not ready)."""
    qI, wI, kI = _f32(qI), _f32(wI), _f32(kI)
    tpos = np.ascontiguousarray(tpos, dtype=np.int64)
    n, nI, cI = qI.shape
    T = kI.shape[0]
    assert wI.shape == (n, nI) and kI.shape == (T, cI) and tpos.shape == (n,)
    scores = np.empty((n, T), dtype=np.float32)
    rc = _load().orc_index_scores(_ptr(qI), _ptr(wI), _ptr(tpos, ctypes.c_long), n,
                                  _ptr(kI), T, nI, cI, m, _ptr(scores))
    _check(rc, "index_scores")
    return scores


def topk(scores, tpos, *, k: int, m: int) -> np.ndarray:
    """scores[n, T] -> idx[n, k] int32: best min(k, R) ready entries, ascending, -1 pad."""
    scores = _f32(scores)
    tpos = np.ascontiguousarray(tpos, dtype=np.int64)
    n, T = scores.shape
    idx = np.empty((n, k), dtype=np.int32)
    rc = _load().orc_topk(_ptr(scores), _ptr(tpos, ctypes.c_long), n, T, k, m,
                          _ptr(idx, ctypes.c_int32))
    _check(rc, "topk")
    return idx


def index_topk(qI, wI, tpos, kI, *, k: int, m: int) -> np.ndarray:
    """The fused indexer step ("DeepSeek-V3.2", section "DeepSeek Sparse
    Attention": score every earlier key, keep the top-k): top-k of the index
    scores, by definition the composition of the two."""
    return topk(index_scores(qI, wI, tpos, kI, m=m), tpos, k=k, m=m)


def attention(q, tpos, *, kv_win=None, win_pos0: int = 0, window: int = 0,
              pool=None, idx=None, m: int = 1, sink=None, rope_dim: int = 0,
              theta: float = 1.0, scale: float, dv: int | None = None,
              freqs=None) -> np.ndarray:
    """q[n, H, D] at positions tpos[n] -> out[n, H, dv].

    idx[n, k] selects pool rows (CSA/DSA); idx=None attends every ready pool
    row w < min(T, (t+1)//m) (HCA).
    """
    q = _f32(q)
    tpos = np.ascontiguousarray(tpos, dtype=np.int64)
    n, H, D = q.shape
    dv = D if dv is None else dv
    kv_win = _f32(kv_win)
    L_win = 0 if kv_win is None else kv_win.shape[0]
    pool = _f32(pool) if pool is not None else np.zeros((0, D), np.float32)
    T = pool.shape[0]
    k = 0
    if idx is not None:
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        assert idx.shape[0] == n
        k = idx.shape[1]
    sink = _f32(sink)
    out = np.empty((n, H, dv), dtype=np.float32)
    f = _freqs(freqs, rope_dim)
    rc = _load().orc_attention_f(
        _ptr(q), _ptr(tpos, ctypes.c_long), n, H, D, dv, _ptr(kv_win), int(win_pos0),
        L_win, int(window), _ptr(pool), T,
        None if idx is None else _ptr(idx, ctypes.c_int32), k, int(m), _ptr(sink),
        int(rope_dim), float(theta), _ptr(f, ctypes.c_double), float(scale), _ptr(out))
    _check(rc, "attention")
    return out


def grouped_out_proj(o, w_a, w_b, *, round_mid_bf16: bool = False, mid=None):
    """Grouped low-rank output projection ("DeepSeek-V4", section "Hybrid
    attention (§2.3)": the heads split into o_groups groups, each group's
    concatenated head outputs projected to o_lora_rank values by its own map
    (o_a_proj), the groups concatenated and mapped to hidden_size (o_b_proj);
    DeepseekV4Config: no bias).

    o [M, G*Kg] (heads g*H/G .. (g+1)*H/G - 1 of each row form group g),
    w_a [G, r, Kg], w_b [hidden, G*r] -> (mid [M, G*r], out [M, hidden]) in
    float64.  round_mid_bf16 rounds mid to bf16 before the second product, as
    a bf16 pipeline stores it.  Given `mid` (e.g. another implementation's
    stored mid), only the second product is taken (o and w_a are unused)."""
    w_b = np.asarray(w_b, np.float64)
    if mid is not None:
        mid = np.asarray(mid, np.float64)
        return mid, mid @ w_b.T
    o = np.asarray(o, np.float64)
    w_a = np.asarray(w_a, np.float64)
    M = o.shape[0]
    G, r, Kg = w_a.shape
    assert o.shape == (M, G * Kg) and w_b.shape[1] == G * r
    mid = np.empty((M, G * r), np.float64)
    for g in range(G):
        # group g: its own input columns, its own projection
        mid[:, g * r:(g + 1) * r] = o[:, g * Kg:(g + 1) * Kg] @ w_a[g].T
    if round_mid_bf16:
        mid = round_bf16(mid.astype(np.float32)).astype(np.float64)
    out = mid @ w_b.T
    return mid, out
