"""The debug build (libcsa_debug.so: the same kernels, the C ABI compiled with
CSA_DEBUG) checks attention index rows on the device before the launch: an
entry outside [-1, T) is reported as an invalid argument instead of being
read as an empty slot; valid inputs give the release library's bits."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    from sparse_long_context_pool_amd import csa
    assert torch.cuda.is_available()
    csa.lib()
    return csa


def _inputs(seed, B=1, S=40, H=64, D=512, T=60, k=24, window=16, m=4, qp=(100,)):
    r = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).cuda()
    q = bf(r.standard_normal((B, S, H, D)))
    L = max(qp) + S
    kv = bf(r.standard_normal((B, L, D)))
    pool = bf(r.standard_normal((B, T, D)))
    idx = np.full((B, S, k), -1, np.int32)
    for b in range(B):
        for i in range(S):
            R = oracle.ready_count(qp[b] + i, m, T)
            sel = np.sort(r.choice(R, size=min(k, R), replace=False)) if R else []
            idx[b, i, :len(sel)] = sel
    sink = torch.from_numpy(r.standard_normal(H).astype(np.float32)).cuda()
    return q, kv, pool, idx, sink, qp


def _call(csa, fn, q, kv, pool, idx, sink, qp, window=16, rope=64):
    B, S, H, D = q.shape
    cs = csa.csa_rope_table(max(qp) + S + 1, rope, 160000.0)
    q_pos = torch.tensor(qp, dtype=torch.int32, device="cuda")
    win_pos0 = torch.zeros(B, dtype=torch.int32, device="cuda")
    return fn(q, kv, win_pos0, pool, dev(idx, torch.int32), sink, q_pos, rope_dim=rope, cs=cs,
              window=window, scale=1.0 / math.sqrt(D), dv=D)


@pytest.mark.parametrize("entry", ["csa_sparse_attn", "csa_sparse_attn_noalloc"])
def test_debug_build_matches_release_and_rejects_bad_index_rows(csa, entry):
    q, kv, pool, idx, sink, qp = _inputs(5)
    release = host(_call(csa, getattr(csa, entry), q, kv, pool, idx, sink, qp))
    prev = csa.use_library(csa.DEBUG_LIB_PATH)
    try:
        assert b"debug" in csa.lib().csa_version()
        got = host(_call(csa, getattr(csa, entry), q, kv, pool, idx, sink, qp))
        assert np.array_equal(got.view(np.uint32), release.view(np.uint32))
        T = pool.shape[1]
        for bad in (T, -2, 1 << 30):
            b_idx = idx.copy()
            b_idx[0, 7, 3] = bad                 # element 7 * k + 3
            with pytest.raises(RuntimeError, match=r"outside \[-1, T=60\).*element 171"):
                _call(csa, getattr(csa, entry), q, kv, pool, b_idx, sink, qp)
        # the library still works after a rejected call
        again = host(_call(csa, getattr(csa, entry), q, kv, pool, idx, sink, qp))
        assert np.array_equal(again.view(np.uint32), release.view(np.uint32))
    finally:
        csa.use_library(prev)
