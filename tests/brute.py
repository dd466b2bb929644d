"""Independent fp64 brute-force formulations used to pin the oracle.

These are written from the mask-based description of the Hugging Face
Transformers "DeepSeek-V4" page (section "Attention mask layout": the sliding
causal mask concatenated with the compressor's block bias, then eager softmax
attention) and the "DeepSeek-V3.2" page (section "DeepSeek Sparse Attention":
attention restricted to the selected tokens through an additive mask).  They
share nothing with ``oracle/``: RoPE here is complex multiplication, attention
is one dense softmax over every key column with -inf where the mask forbids.
"""
from __future__ import annotations

import numpy as np


def rope_complex(v, rope_dim: int, theta: float, pos, sign: int = +1):
    """Rotate trailing interleaved pairs as complex numbers: (a + ib) * e^{i*sign*pos*f_i}."""
    v = np.array(v, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return v
    D = v.shape[-1]
    half = rope_dim // 2
    f = theta ** (-2.0 * np.arange(half) / rope_dim)
    pos = np.asarray(pos, dtype=np.float64)
    ang = sign * pos[..., None] * f            # [..., half]
    z = v[..., D - rope_dim::2] + 1j * v[..., D - rope_dim + 1::2]
    z = z * np.exp(1j * ang)
    v[..., D - rope_dim::2] = z.real
    v[..., D - rope_dim + 1::2] = z.imag
    return v


def ready(t: int, m: int, T: int) -> int:
    """Entries w with w < (t+1)//m are visible (page rule), at most T of them."""
    return max(0, min(T, (t + 1) // m))


def dense_masked_attention(q, tpos, *, kv_win, win_pos0, window, pool, allowed_pool,
                           sink, rope_dim, theta, scale, dv):
    """One dense softmax per (row, head) over [window rows ; pool rows ; sink].

    q[n, H, D]; kv_win[L, D] with row r at position win_pos0 + r (already
    rotated); pool[T, D] (already rotated); allowed_pool(t, row_index) -> bool
    array over the T pool rows.  The sink column adds e^{z_h} to the
    denominator and carries no value.
    """
    q = np.asarray(q, np.float64)
    n, H, D = q.shape
    L = 0 if kv_win is None else kv_win.shape[0]
    T = 0 if pool is None else pool.shape[0]
    keys = np.zeros((L + T, D))
    if L:
        keys[:L] = kv_win
    if T:
        keys[L:] = pool
    out = np.zeros((n, H, dv))
    for r in range(n):
        t = int(tpos[r])
        mask = np.full(L + T, -np.inf)
        for rr in range(L):
            s = win_pos0 + rr
            if t - window < s <= t and s >= 0:
                mask[rr] = 0.0
        if T:
            ok = allowed_pool(t, r)
            mask[L:][ok] = 0.0
        qr = rope_complex(q[r], rope_dim, theta, np.full(H, t), +1)   # [H, D]
        logits = scale * qr @ keys.T + mask[None, :]                    # [H, L+T]
        if sink is not None:
            logits = np.concatenate([logits, np.asarray(sink, np.float64)[:, None]], 1)
        mx = np.max(logits, axis=1, keepdims=True)
        mx = np.where(np.isfinite(mx), mx, 0.0)
        e = np.exp(logits - mx)
        den = e.sum(1, keepdims=True)
        p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
        o = p[:, :L + T] @ keys[:, :dv]
        if dv == D:
            o = rope_complex(o, rope_dim, theta, np.full(H, t), -1)
        out[r] = o
    return out
