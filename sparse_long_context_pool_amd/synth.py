"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

Holds none of the attention method's arithmetic: only random draws, a scale
factor and the fp32 -> bf16 storage conversion (done by torch, round to
nearest even).  Every tensor is drawn in fixed chunks of leading rows from
``numpy.random.default_rng([seed, tensor_id, chunk])``, so any subset of rows
can be regenerated on its own (the CPU checks recompute sampled rows of
tensors that are several GiB on the device).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

CHUNK_ROWS = 64

# Stable tensor ids: changing one changes that tensor's values only.
TID = {
    "q": 1, "x": 2, "gate": 3, "x_idx": 4, "gate_idx": 5, "q_idx": 6, "w_idx": 7,
    "sink": 8, "pool": 9, "k_idx": 10, "kv_win": 11, "slot_bias": 12,
    "slot_bias_idx": 13, "scores": 14,
    # decode caches: compressor buffers and the step's new token
    "ring_x": 15, "ring_g": 16, "ring_xi": 17, "ring_gi": 18, "x_new": 19, "g_new": 20,
    "xi_new": 21, "gi_new": 22,
    # grouped output projection: the attention output and the two weights
    "attn_out": 23, "o_a_proj": 24, "o_b_proj": 25,
}


def _chunk(seed: int, tid: int, c: int, nrows: int, row_size: int) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, c])
    return rng.standard_normal((nrows, row_size), dtype=np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal(seed: int, name: str, n_rows: int, row_shape=(), *, scale: float = 1.0,
           rows=None, bf16: bool = False) -> np.ndarray:
    """N(0, scale^2) draws shaped [n_rows, *row_shape] (or [len(rows), ...]).

    bf16=True returns the fp32 values of the bf16-rounded draws.
    """
    tid = TID[name]
    row_shape = tuple(row_shape)
    row_size = int(np.prod(row_shape)) if row_shape else 1
    if rows is None:
        out = np.empty((n_rows, row_size), dtype=np.float32)
        nch = (n_rows + CHUNK_ROWS - 1) // CHUNK_ROWS

        def fill(c):
            r0 = c * CHUNK_ROWS
            r1 = min(n_rows, r0 + CHUNK_ROWS)
            out[r0:r1] = _chunk(seed, tid, c, r1 - r0, row_size)

        if nch > 8:
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(fill, range(nch)))
        else:
            for c in range(nch):
                fill(c)
    else:
        rows = np.asarray(rows, dtype=np.int64)
        out = np.empty((rows.size, row_size), dtype=np.float32)
        cache = {}
        for j, r in enumerate(rows):
            c = int(r) // CHUNK_ROWS
            if c not in cache:
                r0 = c * CHUNK_ROWS
                cache[c] = _chunk(seed, tid, c, min(n_rows, r0 + CHUNK_ROWS) - r0, row_size)
            out[j] = cache[c][int(r) - c * CHUNK_ROWS]
    if scale != 1.0:
        out *= np.float32(scale)
    if bf16:
        out = torch.from_numpy(out).to(torch.bfloat16).to(torch.float32).numpy()
    return out.reshape((out.shape[0],) + row_shape)


def normal_torch(seed: int, name: str, n_rows: int, row_shape=(), *, scale: float = 1.0,
                 dtype=torch.bfloat16) -> torch.Tensor:
    """Same values as ``normal`` (all rows), built chunk-wise into a host tensor
    of ``dtype`` without materialising the whole fp32 array (multi-GiB inputs)."""
    tid = TID[name]
    row_shape = tuple(row_shape)
    row_size = int(np.prod(row_shape)) if row_shape else 1
    host = torch.empty((n_rows, row_size), dtype=dtype)
    nch = (n_rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def fill(c):
        r0 = c * CHUNK_ROWS
        r1 = min(n_rows, r0 + CHUNK_ROWS)
        a = _chunk(seed, tid, c, r1 - r0, row_size)
        if scale != 1.0:
            a *= np.float32(scale)
        host[r0:r1] = torch.from_numpy(a).to(dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nch)))
    return host.reshape((n_rows,) + row_shape)
